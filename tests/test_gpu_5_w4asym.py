"""GPU parity for W4A16 with per-group zero points and activation-order groups.

Pack and unpack must match the oracle bit for bit (codes, scales, zero
points, column order); the product must stay within 2e-3 * sum_k |a_k w_k| +
1e-3 of the oracle's fp64 product with the dequantized weights, taken in the
input column order; one-hot activations must give single dequantized weights
exactly.
"""
import numpy as np
import pytest

import oracle.rne as OR
import oracle.w4 as OW
import oracle.w4asym as OA
import synth
from gpu_common import bits16, check_close, log, require_gpu

pytestmark = pytest.mark.gpu

S = 2.0 ** -8  # an exact binary16 scale for the hand-built groups


def _special_groups(huge=True):
    """128-wide groups that stress the quantizer: all positive (z = 0), all
    negative (z = 15), all zero (s = 0), code ties, a zero-point tie, an
    underflowing scale, one nonzero value and (huge) values near the binary16
    range, whose products overflow an fp16 output."""
    gs = []
    gs.append(np.linspace(0.001, 0.05, 128))
    gs.append(-np.linspace(0.001, 0.05, 128))
    gs.append(np.zeros(128))
    ties = np.array([-7.0, 8.0] + [k + 0.5 for k in range(-7, 7)] * 9, dtype=np.float64)[:128]
    gs.append(ties * S)                                   # s = 2^-8, z = 7, w / s on .5
    zt = np.concatenate([[-2.5, 12.5], np.linspace(-2.5, 12.5, 126)])
    gs.append(zt * S)                                     # -lo / s = 2.5 -> z = 2
    gs.append(np.linspace(-1, 1, 128) * 1e-9)             # scale underflows
    if huge:
        gs.append(np.where(np.arange(128) % 3 == 0, -60000.0, 60000.0))
    one = np.zeros(128)
    one[77] = -0.5
    gs.append(one)
    return [g.astype(np.float32) for g in gs]


def _weights(N, K, seed, huge=True):
    """Gaussian rows with a per-row offset (so zero points spread over 0..15),
    the first rows replaced by special groups tiled across the row."""
    rng = np.random.default_rng(seed)
    W = synth.weights(N, K, seed) + rng.uniform(-0.03, 0.03, (N, 1)).astype(np.float32)
    sp = _special_groups(huge)
    G = K // 128
    for r in range(min(N, len(sp))):
        W[r] = np.concatenate([sp[(r + g) % len(sp)] for g in range(G)])
    return W


def _g_idx(K, tag):
    return synth.group_index(K, synth.seed_for("gidx", tag, K))


def _pack_both(W, g_idx, dev):
    """Pack on the device and in the oracle; assert bit-identical results."""
    import torch
    import bit_weight_only_tq_amd as tq
    gi = None if g_idx is None else torch.from_numpy(g_idx).to(dev)
    q, s, z, perm = tq.w4a16_pack_asym(torch.from_numpy(W).to(dev), gi)
    rq, rs, rz, rp = OA.w4a_pack(W, g_idx)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(bits16(s), rs)
    np.testing.assert_array_equal(z.cpu().numpy(), rz)
    if g_idx is None:
        assert perm is None
    else:
        np.testing.assert_array_equal(perm.cpu().numpy(), rp)
    return (q, s, z, perm), (rq, rs, rz, rp)


@pytest.mark.parametrize("N,K,order", [
    (8, 128, False), (8, 128, True), (64, 1024, False), (300, 1024, True), (1024, 4096, True),
    (100, 14336, True),
])
def test_w4a_pack_parity(N, K, order):
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"w4a16_pack_asym N={N} K={K} act_order={order}")
    W = _weights(N, K, synth.seed_for("w4ap", N, K))
    g = _g_idx(K, "pack") if order else None
    (q, s, z, perm), (rq, rs, rz, rp) = _pack_both(W, g, dev)
    qo, wdq = tq.w4a16_unpack_asym(q, s, z, K, perm)
    np.testing.assert_array_equal(qo.cpu().numpy(), OA.w4a_unpack(rq, K))
    np.testing.assert_array_equal(bits16(wdq), OA.w4a_dequant_f16_bits(rq, rs, rz, K, rp if order else None))


def test_w4a_pack_full_size_sampled_rows():
    """4096 x 14336 with activation order: every packed row from the device,
    the oracle on a sample of rows (rows are packed independently)."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 4096, 14336
    log(f"w4a16_pack_asym full N={N} K={K}")
    W = synth.weights_device(N, K, synth.seed_for("w4apf", N, K), dev)
    g = _g_idx(K, "full")
    q, s, z, perm = tq.w4a16_pack_asym(W, torch.from_numpy(g).to(dev))
    rows = np.sort(np.random.default_rng(5).choice(N, 96, replace=False))
    idx = torch.from_numpy(rows).to(dev)
    rq, rs, rz, rp = OA.w4a_pack(W.index_select(0, idx).cpu().numpy(), g)
    np.testing.assert_array_equal(perm.cpu().numpy(), rp)
    np.testing.assert_array_equal(q.index_select(0, idx).cpu().numpy(), rq)
    np.testing.assert_array_equal(bits16(s.index_select(0, idx)), rs)
    np.testing.assert_array_equal(z.index_select(0, idx).cpu().numpy(), rz)


def test_w4a_pack_errors():
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log("w4a16_pack_asym errors")
    K = 384
    W = torch.zeros((4, K), dtype=torch.float32, device=dev)
    g = _g_idx(K, "err")
    bad = g.copy()
    bad[np.flatnonzero(bad == 0)[0]] = 1                   # group 0 has 127 columns, group 1 has 129
    for gi in (bad, np.where(g == 2, 3, g).astype(np.int32), np.where(g == 2, -1, g).astype(np.int32)):
        with pytest.raises(tq.TQError) as e:
            tq.w4a16_pack_asym(W, torch.from_numpy(gi).to(dev))
        assert e.value.name == "TQ_ERR_GROUP"
    W[2, 5] = float("nan")
    with pytest.raises(tq.TQError) as e:
        tq.w4a16_pack_asym(W, torch.from_numpy(g).to(dev))
    assert e.value.name == "TQ_ERR_NONFINITE"
    W[2, 5] = 1e6                                          # (1e6 - 0) / 15 > 65504
    with pytest.raises(tq.TQError) as e:
        tq.w4a16_pack_asym(W)
    assert e.value.name == "TQ_ERR_RANGE"


_CACHE = {}


def _packed(N, K, order, dev):
    key = (N, K, order)
    if key not in _CACHE:
        W = _weights(N, K, synth.seed_for("w4ag", N, K), huge=False)
        g = _g_idx(K, "gemm") if order else None
        dev_t, ref = _pack_both(W, g, dev)
        rq, rs, rz, rp = ref
        _CACHE.clear()
        _CACHE[key] = dev_t, OA.w4a_dequant(rq, rs, rz, K, rp if order else None)
    return _CACHE[key]


@pytest.mark.parametrize("order", [False, True])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16, 24, 40])
def test_w4a_gemm(M, dt, order):
    """Every kernel the dispatcher picks for 1 <= M <= 40 (streaming,
    per-lane FMA, blocks of 16 rows at M = 24, the matrix-core GEMM at
    M = 40), ragged N, with bias."""
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 300, 1024
    log(f"w4a16_gemm_asym M={M} N={N} K={K} {dt} act_order={order}")
    (q, s, z, perm), wdq = _packed(N, K, order, dev)
    A = synth.activations(M, K, synth.seed_for("w4aa", M, K), dt)
    bias = synth.activations(1, N, synth.seed_for("w4ab", N), dt)[0]
    C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev), zeros=z, perm=perm)
    check_close(C, A, wdq, bias=bias, label=f"w4a {M}x{N}x{K} {dt} order={order}")


@pytest.mark.parametrize("M", [1, 16])
def test_w4a_one_hot_bit_exact(M):
    """A = rows of the identity: C[m, n] = wdq[n, k_m] exactly, (q - z) * s
    rounded once to fp16 and placed at input column perm[i]; pins the zero
    point, the nibble order and the direction of the column order."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 300, 1024
    log(f"w4a one-hot M={M}")
    (q, s, z, perm), wdq = _packed(N, K, True, dev)
    ks = [0, 1, 2, 7, 8, 100, 127, 128, 129, 255, 256, 511, 640, 900, 1000, 1023][:M] if M > 1 else [517]
    A = torch.zeros((len(ks), K), dtype=torch.float16)
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = tq.w4a16_gemm(A.to(dev), q, s, zeros=z, perm=perm)
    np.testing.assert_array_equal(bits16(C), OR.f16_bits(wdq[:, ks].T))


def test_w4a_order_without_zeros():
    """Column order with the symmetric format: the matrix packed by
    w4a16_pack after permuting its columns, applied with perm and no zero
    points (zero point 8)."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K, M = 200, 512, 4
    log("w4 act order, symmetric")
    W = synth.weights(N, K, synth.seed_for("w4so", N, K))
    perm = OA.order_from_g_idx(_g_idx(K, "sym"), K)
    q, s = tq.w4a16_pack(torch.from_numpy(np.ascontiguousarray(W[:, perm])).to(dev))
    rq, rs = OW.w4_pack(np.ascontiguousarray(W[:, perm]))
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    wdq = np.empty((N, K))
    wdq[:, perm] = OW.w4_dequant(rq, rs, K)
    A = synth.activations(M, K, synth.seed_for("w4soa", M), "f16")
    C = tq.w4a16_gemm(A.to(dev), q, s, perm=torch.from_numpy(perm).to(dev))
    check_close(C, A, wdq, label="w4 act order symmetric")


@pytest.mark.parametrize("M,N,K", [
    (1, 4096, 14336), (4, 4096, 14336), (16, 4096, 14336), (1, 14336, 4096), (16, 28672, 4096), (40, 1024, 4096),
    (1, 28672, 4096), (2, 4096, 14336), (2, 6144, 4096),
])
def test_w4a_decode_shapes(M, N, K):
    """Llama-3-8B shapes with activation order: the workspace the query asks
    for (counters + gather + split partials), exactly the counters and the
    gather (no split) and none (rejected); sampled output columns within the
    tolerance; a repeated call is bit-identical."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    need = tq.w4a16_gemm_asym_workspace_bytes(M, N, K, with_perm=True)
    log(f"w4a decode M={M} N={N} K={K} workspace={need}")
    W = synth.weights_device(N, K, synth.seed_for("w4ad", N, K), dev)
    g = _g_idx(K, "dec")
    q, s, z, perm = tq.w4a16_pack_asym(W, torch.from_numpy(g).to(dev))
    cols = np.sort(np.random.default_rng(N + K + 3).choice(N, min(N, 160), replace=False))
    idx = torch.from_numpy(cols).to(dev)
    rq, rs, rz, rp = OA.w4a_pack(W.index_select(0, idx).cpu().numpy(), g)
    np.testing.assert_array_equal(q.index_select(0, idx).cpu().numpy(), rq)
    np.testing.assert_array_equal(z.index_select(0, idx).cpu().numpy(), rz)
    del W
    wdq = OA.w4a_dequant(rq, rs, rz, K, rp)
    A = synth.activations(M, K, synth.seed_for("w4ada", M, K), "f16")
    bias = synth.activations(1, N, synth.seed_for("w4adb", N), "f16")[0]
    gather = tq.TQ_WORKSPACE_FLAG_BYTES + (M * K * 2 + 255) // 256 * 256  # counters + gathered activations
    outs = []
    for nbytes in ("auto", gather):
        ws = nbytes if nbytes == "auto" else tq.new_workspace(nbytes, dev)
        C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev), zeros=z, perm=perm, workspace=ws)
        check_close(C.index_select(1, idx), A, wdq, bias=bias[torch.from_numpy(cols)],
                    label=f"w4a {M}x{N}x{K} ws={nbytes}")
        outs.append(C)
    with pytest.raises(tq.TQError) as e:
        tq.w4a16_gemm(A.to(dev), q, s, zeros=z, perm=perm, workspace=None)
    assert e.value.name == "TQ_ERR_SHAPE"
    C2 = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev), zeros=z, perm=perm)
    assert torch.equal(outs[0].view(torch.int16), C2.view(torch.int16))


@pytest.mark.parametrize("case", ["odd_groups", "scales_offset", "zeros_offset"])
def test_w4_pair_fallbacks(case):
    """Two groups per wave read scales and zero points in pairs, which needs
    even offsets and aligned arrays; otherwise the plan takes another split or
    kernel.  Odd G (K = 17 * 128), a scale array 2 bytes past 4-byte
    alignment and a zero-point array 1 byte past 2-byte alignment must all
    still match the oracle, with and without zero points."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, M = 300, 4
    K = 17 * 128 if case == "odd_groups" else 4096
    log(f"w4 pair fallback {case} K={K}")
    W = _weights(N, K, synth.seed_for("w4pf", K), huge=False)
    (q, s, z, _), (rq, rs, rz, _) = _pack_both(W, None, dev)
    if case == "scales_offset":
        buf = torch.empty((s.numel() + 1,), dtype=torch.float16, device=dev)
        buf[1:].copy_(s.reshape(-1))
        s = buf[1:].view(s.shape)
    if case == "zeros_offset":
        buf = torch.empty((z.numel() + 1,), dtype=torch.uint8, device=dev)
        buf[1:].copy_(z.reshape(-1))
        z = buf[1:].view(z.shape)
    A = synth.activations(M, K, synth.seed_for("w4pfa", K), "f16")
    C = tq.w4a16_gemm(A.to(dev), q, s, zeros=z)
    check_close(C, A, OA.w4a_dequant(rq, rs, rz, K), label=f"w4a pair fallback {case}")
    sq, ss = tq.w4a16_pack(torch.from_numpy(W).to(dev))
    rsq, rss = OW.w4_pack(W)
    np.testing.assert_array_equal(sq.cpu().numpy(), rsq)
    if case == "scales_offset":
        buf = torch.empty((ss.numel() + 1,), dtype=torch.float16, device=dev)
        buf[1:].copy_(ss.reshape(-1))
        ss = buf[1:].view(ss.shape)
    C = tq.w4a16_gemm(A.to(dev), sq, ss)
    check_close(C, A, OW.w4_dequant(rsq, rss, K), label=f"w4 pair fallback {case}")


@pytest.mark.parametrize("N,K,order", [(320, 4096, True), (320, 4096, False), (160, 14336, True)])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_w4a_m1_kernel_one_hot(N, K, order, dt):
    """The W4A16 M = 1 kernel with zero points (4 and 8 groups per wave): a
    one-hot row gives C[0, n] = wdq[n, k] bit for bit, (q - z) * s rounded
    once, at columns in every nibble position and in first and last groups
    of several waves; with activation order the one-hot column is an input
    column and lands wherever perm puts it."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"w4a M=1 kernel one-hot N={N} K={K} order={order} {dt}")
    (q, s, z, perm), wdq = _packed(N, K, order, dev)
    to_bits = OR.f16_bits if dt == "f16" else OR.bf16_bits
    for k in sorted({0, 1, 3, 4, 7, 9, 31, 33, 127, 128, 517, 1023, 2048 + 70, K - 129, K - 1}):
        A = torch.zeros((1, K), dtype=torch.float16 if dt == "f16" else torch.bfloat16)
        A[0, k] = 1.0
        C = tq.w4a16_gemm(A.to(dev), q, s, zeros=z, perm=perm if order else None)
        np.testing.assert_array_equal(bits16(C)[0], to_bits(wdq[:, k]), err_msg=f"k={k}")


@pytest.mark.parametrize("M", [1, 16, 300])
def test_w4a_perm_out_of_range_clamped(M):
    """A perm that is not the pack's (entries below 0, at K and far past it):
    the gather clamps such an index to its own column, so an identity perm
    with bad entries gives exactly the product without perm, on the decode
    kernels and on the prefill GEMM, with no access outside A."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 200, 1024
    log(f"w4 perm out of range M={M}")
    W = synth.weights(N, K, synth.seed_for("w4pbad", N, K))
    q, s = tq.w4a16_pack(torch.from_numpy(W).to(dev))
    perm = np.arange(K, dtype=np.int32)
    perm[[3, 100, 640, K - 1]] = [-5, K, K + 7, 2 ** 31 - 1]
    A = synth.activations(M, K, synth.seed_for("w4pbada", M, K), "f16").to(dev)
    ref = tq.w4a16_gemm(A, q, s)
    C = tq.w4a16_gemm(A, q, s, perm=torch.from_numpy(perm).to(dev))
    np.testing.assert_array_equal(bits16(C), bits16(ref))
