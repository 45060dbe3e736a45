"""GPU parity: quantized GEMV / GEMM outputs against the fp64 oracle.

Each output element must be finite and within 2e-3 * sum_k |a_k w_k| + 1e-3
of the oracle's fp64 product with the dequantized weights.  One-hot
activations must reproduce single dequantized weights bit for bit.
"""
import numpy as np
import pytest

import oracle.rne as OR
import oracle.ternary as OT
import oracle.w4 as OW
import synth
from gpu_common import bits16, check_close, log, require_gpu

pytestmark = pytest.mark.gpu

_CACHE = {}


def _ternary(N, K, dev):
    """(W, codes, scale on device, oracle codes, oracle scale bits, wdq64) for a shape."""
    key = ("t", N, K)
    if key not in _CACHE:
        import torch
        import bit_weight_only_tq_amd as tq
        W = synth.smallest_case()[0] if (N, K) == (256, 256) else synth.weights(N, K, synth.seed_for("w", N, K))
        codes, scale = tq.tq_pack(torch.from_numpy(W).to(dev))
        rc, rs = OT.ternary_pack(W)
        np.testing.assert_array_equal(codes.cpu().numpy(), rc)
        np.testing.assert_array_equal(bits16(scale), rs)
        _CACHE.clear()
        _CACHE[key] = (codes, scale, rc, rs, OT.ternary_dequant(rc, rs, K))
    return _CACHE[key]


def _w4(N, K, dev):
    key = ("w4", N, K)
    if key not in _CACHE:
        import torch
        import bit_weight_only_tq_amd as tq
        W = synth.weights(N, K, synth.seed_for("w4", N, K))
        q, s = tq.w4a16_pack(torch.from_numpy(W).to(dev))
        rq, rs = OW.w4_pack(W)
        np.testing.assert_array_equal(q.cpu().numpy(), rq)
        _CACHE.clear()
        _CACHE[key] = (q, s, rq, rs, OW.w4_dequant(rq, rs, K))
    return _CACHE[key]


def test_smallest_case():
    """256 x 256 ternary layer, M = 1, fp16, seed 0."""
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log("smallest case 256x256 M=1")
    W, A = synth.smallest_case()
    codes, scale, rc, rs, wdq = _ternary(256, 256, dev)
    C = tq.tq_gemm(A.to(dev), codes, scale)
    check_close(C, A, wdq, label="smallest")


DECODE_SHAPES = [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)]


@pytest.mark.parametrize("N,K", DECODE_SHAPES)
@pytest.mark.parametrize("M", [1, 4, 16])
def test_ternary_decode(N, K, M):
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"tq_gemm decode N={N} K={K} M={M}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("a", N, K, M), "f16")
    assert tq.tq_select_path("ternary", M, N, K) == "gemv"
    C = tq.tq_gemm(A.to(dev), codes, scale)
    check_close(C, A, wdq, label=f"decode {N}x{K} M={M}")


@pytest.mark.parametrize("N,K", DECODE_SHAPES)
@pytest.mark.parametrize("M", [1, 4, 16])
def test_w4_decode(N, K, M):
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"w4a16_gemm decode N={N} K={K} M={M}")
    q, s, rq, rs, wdq = _w4(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("a4", N, K, M), "f16")
    C = tq.w4a16_gemm(A.to(dev), q, s)
    check_close(C, A, wdq, label=f"w4 {N}x{K} M={M}")


# Shapes of the M = 1 decode kernel: 4 waves of 4 chunk-sets, 14 waves of 4,
# 14 waves of 8, and two 16-row blocks per workgroup (from 3072 row-blocks).
M1_SHAPES = [(320, 4096), (4096, 14336), (1024, 28672), (49152, 4096)]


@pytest.mark.parametrize("N,K", M1_SHAPES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_m1_one_hot_and_bias(N, K, dt):
    """The M = 1 decode kernel (fp16 and bf16 forms: fields masked into the
    mantissa of 1024 or of 128): a one-hot row e_k gives C[0, n] = wdq[n, k]
    bit for bit, for columns k in the first and last chunk of several waves
    and at every code-field position; a dense row with a bias is within the
    tolerance."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"M=1 kernel one-hot and bias N={N} K={K} {dt}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    to_bits = OR.f16_bits if dt == "f16" else OR.bf16_bits
    ks = sorted({0, 5, 9, 14, 255, 256 + 77, 1023, 1024 + 130, 2048 + 3, K // 2 + 31, K - 257, K - 8, K - 1})
    for k in ks:
        A = torch.zeros((1, K), dtype=tdt)
        A[0, k] = 1.0
        C = tq.tq_gemm(A.to(dev), codes, scale, path="gemv")
        np.testing.assert_array_equal(bits16(C)[0], to_bits(wdq[:, k]), err_msg=f"k={k}")
    A = synth.activations(1, K, synth.seed_for("m1", N, K, dt), dt)
    bias = synth.activations(1, N, synth.seed_for("m1b", N, K, dt), dt)[0]
    C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev))
    check_close(C, A, wdq, bias=bias, label=f"M=1 kernel {N}x{K} {dt} with bias")


# Streaming decode kernels with 3, 5, 6 and 7 row-blocks per workgroup: the
# fewest that put at most one workgroup on each of 256 compute units
# (768, 1280, 1536 and 1792 row-blocks of 16 at K = 4096, no K split).
STREAM_T_SHAPES = [(12288, 4096), (20480, 4096), (24576, 4096), (28672, 4096)]


@pytest.mark.parametrize("N,K", STREAM_T_SHAPES)
@pytest.mark.parametrize("M", [4, 16])
@pytest.mark.parametrize("fmt", ["ternary", "w4"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_stream_row_blocks(N, K, M, fmt, dt):
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"stream row-blocks {fmt} N={N} K={K} M={M} {dt}")
    A = synth.activations(M, K, synth.seed_for("st", fmt, N, K, M), dt)
    bias = synth.activations(1, N, synth.seed_for("stb", fmt, N, K), dt)[0]
    if fmt == "ternary":
        codes, scale, rc, rs, wdq = _ternary(N, K, dev)
        C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev))
    else:
        q, s, rq, rs, wdq = _w4(N, K, dev)
        C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev))
    check_close(C, A, wdq, bias=bias, label=f"stream {fmt} {N}x{K} M={M} {dt}")


@pytest.mark.parametrize("N,K", [(14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_ternary_prefill_full(N, K, dt):
    """M = 2048, every output element checked."""
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    M = 2048
    log(f"tq_gemm prefill N={N} K={K} M={M} {dt}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("p", N, K, M, dt), dt)
    assert tq.tq_select_path("ternary", M, N, K, dt) == "gemm"
    C = tq.tq_gemm(A.to(dev), codes, scale)
    check_close(C, A, wdq, label=f"prefill {N}x{K} M={M} {dt}")


@pytest.mark.parametrize("N,K", [(14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M,dt", [(4096, "bf16"), (4096, "f16"), (8192, "bf16")])
def test_ternary_prefill_sampled(N, K, M, dt):
    """Large M: all columns of 256 sampled rows (fixed seed) checked."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"tq_gemm prefill sampled N={N} K={K} M={M} {dt}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("p", N, K, M, dt), dt)
    C = tq.tq_gemm(A.to(dev), codes, scale)
    rows = np.sort(np.random.default_rng(M + N).choice(M, 256, replace=False))
    idx = torch.from_numpy(rows)
    check_close(C.cpu()[idx], A[idx], wdq, label=f"prefill {N}x{K} M={M} {dt} sampled")


@pytest.mark.parametrize("M,N,K", [
    (1, 64, 64), (3, 100, 128), (17, 130, 192), (33, 257, 256), (130, 300, 64), (129, 513, 320),
    (5, 1000, 448), (2, 7, 64),
    (1, 300, 256), (4, 33, 512), (2, 70, 1280), (3, 31, 2304), (1, 5, 28672),
    (9, 45, 768), (16, 100, 2048), (12, 20, 4096), (2, 40, 512), (4, 9, 7168),
    # decode kernels with several 16-row blocks per workgroup and a partial
    # last workgroup, and a last wave with fewer chunk-sets than the others
    (3, 4200, 1024), (5, 16400, 2048), (4, 50, 4352), (6, 8300, 4352), (2, 8300, 4352),
])
@pytest.mark.parametrize("path", ["gemv", "stream_mfma", "gemm"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_ternary_ragged(M, N, K, path, dt):
    """Tiles with ragged edges in M and N, several K steps, every kernel family."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    if path == "gemv" and M > 16:
        pytest.skip("gemv handles M <= 16")
    log(f"tq_gemm ragged M={M} N={N} K={K} {path} {dt}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("r", M, N, K, dt), dt)
    bias = synth.activations(1, N, synth.seed_for("b", N, dt), dt)[0]
    C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev), path=path)
    check_close(C, A, wdq, bias=bias, label=f"ragged {M}x{N}x{K} {path} {dt}")


@pytest.mark.parametrize("path", ["gemv", "stream_mfma", "gemm"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_one_hot_bit_exact(path, dt):
    """A = rows of the identity: C[m, n] = wdq[n, k_m] exactly (one rounding of
    +-scale or 0 to the output dtype); pins indexing and bit order."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 300, 256
    log(f"one-hot {path} {dt}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    ks = [0, 5, 9, 255] if path == "gemv" else [0, 1, 2, 3, 4, 7, 8, 15, 16, 63, 64, 127, 200, 255]
    M = len(ks)
    A = torch.zeros((M, K), dtype=torch.float16 if dt == "f16" else torch.bfloat16)
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = tq.tq_gemm(A.to(dev), codes, scale, path=path)
    want = wdq[:, ks].T
    want_bits = OR.f16_bits(want) if dt == "f16" else OR.bf16_bits(want)
    np.testing.assert_array_equal(bits16(C), want_bits)


@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 16), ("stream_mfma", 40), ("stream_mfma", 100),
                                    ("gemm", 300)])
def test_deterministic_and_canary(path, M):
    """Two runs give bit-identical outputs; the bytes after C stay untouched."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 1024, 4096
    log(f"determinism {path} M={M}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("d", M), "f16").to(dev)
    buf = torch.full((M * N + 4096,), -12345.0, dtype=torch.float16, device=dev)
    C1 = buf[:M * N].view(M, N)
    tq.tq_gemm(A, codes, scale, out=C1, path=path)
    C2 = tq.tq_gemm(A, codes, scale, path=path)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    assert bool((buf[M * N:] == -12345.0).all())


@pytest.mark.parametrize("M,N,K,dt", [(17, 8192, 8192, "f16"), (64, 1024, 8192, "f16"), (32, 8192, 28672, "f16"),
                                      (100, 2000, 4096, "f16"), (48, 10240, 8192, "bf16"), (64, 8192, 28672, "bf16"),
                                      (40, 3000, 4160, "f16"), (200, 700, 4160, "bf16")])
def test_medium_split_k(M, N, K, dt):
    """Medium M with K split across workgroups (workspace from torch) and
    without a workspace (one pass over K): both within the tolerance, on
    sampled output columns at full 70B-like sizes; K % 256 != 0 takes the
    64-column-step kernel."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    nbytes = tq.tq_gemm_workspace_bytes(M, N, K, dt, path="stream_mfma")
    log(f"medium split-K M={M} N={N} K={K} {dt} workspace={nbytes}")
    W = synth.weights_device(N, K, synth.seed_for("msk", N, K), dev)
    codes, scale = tq.tq_pack(W)
    cols = np.sort(np.random.default_rng(N + K).choice(N, min(N, 192), replace=False))
    idx = torch.from_numpy(cols).to(dev)
    rc, rs = OT.ternary_pack(W.index_select(0, idx).cpu().numpy())
    del W
    wdq = OT.ternary_dequant(rc, rs, K)
    A = synth.activations(M, K, synth.seed_for("mska", M, K), dt)
    bias = synth.activations(1, N, synth.seed_for("mskb", N), dt)[0]
    for ws in ("auto", None):
        C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev), path="stream_mfma", workspace=ws)
        check_close(C.index_select(1, idx), A, wdq, bias=bias[torch.from_numpy(cols)],
                    label=f"medium {M}x{N}x{K} {dt} ws={ws}")


@pytest.mark.parametrize("M,N,K", [(2048, 4096, 14336), (300, 1000, 4096), (257, 300, 2048), (256, 4096, 4096)])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_gemm_split_k(M, N, K, dt):
    """Large-M kernel with K split across workgroups (workspace from torch)
    and without a workspace (one pass over K): both within the tolerance on
    sampled output columns, ragged M and N included, with bias."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    nbytes = tq.tq_gemm_workspace_bytes(M, N, K, dt, path="gemm")
    log(f"gemm split-K M={M} N={N} K={K} {dt} workspace={nbytes}")
    assert nbytes > 0
    W = synth.weights_device(N, K, synth.seed_for("gsk", N, K), dev)
    codes, scale = tq.tq_pack(W)
    cols = np.sort(np.random.default_rng(N + K).choice(N, min(N, 192), replace=False))
    idx = torch.from_numpy(cols).to(dev)
    rc, rs = OT.ternary_pack(W.index_select(0, idx).cpu().numpy())
    del W
    wdq = OT.ternary_dequant(rc, rs, K)
    A = synth.activations(M, K, synth.seed_for("gska", M, K, dt), dt)
    bias = synth.activations(1, N, synth.seed_for("gskb", N, dt), dt)[0]
    outs = []
    for ws in ("auto", None):
        C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev), path="gemm", workspace=ws)
        check_close(C.index_select(1, idx), A, wdq, bias=bias[torch.from_numpy(cols)],
                    label=f"gemm split {M}x{N}x{K} {dt} ws={ws}")
        outs.append(C)
    # a repeated split call is bit-identical (partials summed in a fixed order)
    C2 = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev), path="gemm")
    assert torch.equal(outs[0].view(torch.int16), C2.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(16, 4096, 14336), (3, 4100, 14336), (9, 8192, 28672), (5, 1000, 16384),
                                   (16, 57344, 8192), (12, 8200, 8192)])
def test_gemv_split_k(M, N, K):
    """Small-M streaming kernel with K split across workgroups (workspace from
    torch) and without a workspace (other kernels for K > 8192): both within
    the tolerance on sampled output columns, ragged N, with bias; a repeated
    split call is bit-identical."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    nbytes = tq.tq_gemm_workspace_bytes(M, N, K, path="gemv")
    log(f"gemv split-K M={M} N={N} K={K} workspace={nbytes}")
    W = synth.weights_device(N, K, synth.seed_for("vsk", N, K), dev)
    codes, scale = tq.tq_pack(W)
    cols = np.sort(np.random.default_rng(N + K + 1).choice(N, min(N, 192), replace=False))
    idx = torch.from_numpy(cols).to(dev)
    rc, rs = OT.ternary_pack(W.index_select(0, idx).cpu().numpy())
    del W
    wdq = OT.ternary_dequant(rc, rs, K)
    A = synth.activations(M, K, synth.seed_for("vska", M, K), "f16")
    bias = synth.activations(1, N, synth.seed_for("vskb", N), "f16")[0]
    outs = []
    for ws in ("auto", None):
        C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev), path="gemv", workspace=ws)
        check_close(C.index_select(1, idx), A, wdq, bias=bias[torch.from_numpy(cols)],
                    label=f"gemv split {M}x{N}x{K} ws={ws}")
        outs.append(C)
    C2 = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev), path="gemv")
    assert torch.equal(outs[0].view(torch.int16), C2.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(1, 20, 128), (3, 37, 384), (16, 300, 1024), (5, 16400, 256),
                                   (2, 64, 2048), (16, 17, 4096), (7, 1000, 14336)])
def test_w4_ragged_shapes(M, N, K):
    """W4A16 matrix-core kernel: one group per row (K = 128) up to 112, ragged
    N, two 16-row blocks per workgroup (N > 16384), M up to 16, with bias."""
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"w4 ragged M={M} N={N} K={K}")
    q, s, rq, rs, wdq = _w4(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("w4rs", M, N, K), "f16")
    bias = synth.activations(1, N, synth.seed_for("w4rsb", N), "f16")[0]
    C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev))
    check_close(C, A, wdq, bias=bias, label=f"w4 ragged {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(16, 4096, 14336), (5, 1000, 14336), (12, 8192, 28672), (3, 4100, 8192),
                                   (16, 28672, 4096), (40, 4096, 14336), (1, 28672, 4096), (1, 4100, 4096),
                                   (2, 4096, 14336), (2, 300, 1024)])
def test_w4_split_k(M, N, K):
    """W4A16 streaming kernel with the K groups split across workgroups
    (workspace from torch) and without a workspace: both within the tolerance
    on sampled output columns, ragged N, with bias; a repeated call is
    bit-identical.  M > 16 takes the matrix-core GEMM (its own K split) and,
    forced, the decode kernels over blocks of 16 rows through one workspace."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    nbytes = tq.w4a16_gemm_workspace_bytes(M, N, K)
    log(f"w4 split-K M={M} N={N} K={K} workspace={nbytes}")
    W = synth.weights_device(N, K, synth.seed_for("w4sk", N, K), dev)
    q, s = tq.w4a16_pack(W)
    cols = np.sort(np.random.default_rng(N + K + 2).choice(N, min(N, 160), replace=False))
    idx = torch.from_numpy(cols).to(dev)
    rq, rs = OW.w4_pack(W.index_select(0, idx).cpu().numpy())
    np.testing.assert_array_equal(q.index_select(0, idx).cpu().numpy(), rq)
    del W
    wdq = OW.w4_dequant(rq, rs, K)
    A = synth.activations(M, K, synth.seed_for("w4ska", M, K), "f16")
    bias = synth.activations(1, N, synth.seed_for("w4skb", N), "f16")[0]
    outs = []
    for ws in ("auto", None):
        C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev), workspace=ws)
        check_close(C.index_select(1, idx), A, wdq, bias=bias[torch.from_numpy(cols)],
                    label=f"w4 split {M}x{N}x{K} ws={ws}")
        outs.append(C)
    C2 = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev))
    assert torch.equal(outs[0].view(torch.int16), C2.view(torch.int16))
    if M > 16:
        ws = tq.new_workspace(64 << 20, dev)
        C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev), workspace=ws, path="gemv")
        check_close(C.index_select(1, idx), A, wdq, bias=bias[torch.from_numpy(cols)],
                    label=f"w4 row blocks {M}x{N}x{K}")


def test_w4_one_hot_bit_exact():
    """A = rows of the identity: C[m, n] = wdq[n, k_m] exactly (the group's
    value (q - 8) * s rounded once to fp16); pins nibble order and pairing."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 300, 256
    log("w4 one-hot")
    q, s, rq, rs, wdq = _w4(N, K, dev)
    ks = [0, 1, 2, 3, 4, 5, 6, 7, 8, 31, 32, 100, 127, 128, 200, 255]
    A = torch.zeros((len(ks), K), dtype=torch.float16)
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = tq.w4a16_gemm(A.to(dev), q, s)
    np.testing.assert_array_equal(bits16(C), OR.f16_bits(wdq[:, ks].T))


@pytest.mark.parametrize("M", [1, 20, 40])
def test_w4_ragged_and_blocked(M):
    """Ragged N = 200 at K = 384: the decode kernels (M = 1), blocks of 16
    rows (M = 20) and the matrix-core GEMM (M = 40), fp16 and bf16."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 200, 384
    log(f"w4 ragged M={M}")
    q, s, rq, rs, wdq = _w4(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("w4r", M), "f16")
    bias = synth.activations(1, N, synth.seed_for("w4b"), "f16")[0]
    C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev))
    check_close(C, A, wdq, bias=bias, label=f"w4 ragged M={M}")
    Ab = synth.activations(M, K, synth.seed_for("w4rb", M), "bf16")
    C = tq.w4a16_gemm(Ab.to(dev), q, s)
    check_close(C, Ab, wdq, label=f"w4 ragged bf16 M={M}")


# Shapes of the W4A16 M = 1 kernel: 8 waves of 4 groups, 14 waves of 8
# groups, 16 waves of 4, and two 16-row blocks per workgroup (1792 row-blocks
# of 8 waves would exceed 8 waves per SIMD on 256 compute units).
W4_M1_SHAPES = [(320, 4096), (1024, 14336), (512, 8192), (28672, 4096)]


@pytest.mark.parametrize("N,K", W4_M1_SHAPES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_w4_m1_one_hot_and_bias(N, K, dt):
    """The W4A16 M = 1 kernel (fp16, and bf16 with the odd nibbles shifted to
    bits 3..6): a one-hot row e_k gives C[0, n] = wdq[n, k] bit for bit for
    k at every nibble position of a word, every word of a lane slot and
    every slot of a group, in first and last groups of several waves; a
    dense row with a bias is within the tolerance."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"W4 M=1 kernel one-hot and bias N={N} K={K} {dt}")
    q, s, rq, rs, wdq = _w4(N, K, dev)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    to_bits = OR.f16_bits if dt == "f16" else OR.bf16_bits
    ks = sorted({0, 1, 2, 3, 4, 5, 6, 7, 8, 15, 31, 32, 63, 96 + 7, 127, 128, 640 + 45, 1023, 1024 + 77,
                 K // 2 + 19, K - 128, K - 33, K - 1})
    for k in ks:
        A = torch.zeros((1, K), dtype=tdt)
        A[0, k] = 1.0
        C = tq.w4a16_gemm(A.to(dev), q, s)
        np.testing.assert_array_equal(bits16(C)[0], to_bits(wdq[:, k]), err_msg=f"k={k}")
    A = synth.activations(1, K, synth.seed_for("w4m1", N, K, dt), dt)
    bias = synth.activations(1, N, synth.seed_for("w4m1b", N, K, dt), dt)[0]
    C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev))
    check_close(C, A, wdq, bias=bias, label=f"W4 M=1 kernel {N}x{K} {dt} with bias")


@pytest.mark.parametrize("M,N,K,path", [(5, 4096, 4096, "auto"), (16, 28672, 4096, "auto"), (11, 1024, 14336, "auto"),
                                        (24, 320, 4096, "auto"), (40, 320, 4096, "gemv"), (40, 320, 4096, "auto")])
def test_w4_bf16_row_blocks(M, N, K, path):
    """bf16 W4A16 past four rows: the streaming kernel's bf16 form (inside
    blocks of 16 rows when M > 16, the last block ragged; M = 40 also through
    the matrix-core GEMM); one-hot rows give C[m, n] = wdq[n, k_m] bit for
    bit, dense rows with a bias are within the tolerance, the row past M is
    untouched."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"W4 bf16 row blocks M={M} N={N} K={K}")
    q, s, rq, rs, wdq = _w4(N, K, dev)
    ks = [(37 * m + 5) % K for m in range(M)]
    A = torch.zeros((M, K), dtype=torch.bfloat16)
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = tq.w4a16_gemm(A.to(dev), q, s, path=path)
    np.testing.assert_array_equal(bits16(C), OR.bf16_bits(wdq[:, ks].T))
    A = synth.activations(M, K, synth.seed_for("w4bfr", M, N, K), "bf16")
    bias = synth.activations(1, N, synth.seed_for("w4bfrb", N, K), "bf16")[0]
    buf = torch.full((M + 1, N), -7.0, dtype=torch.bfloat16, device=dev)
    C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev), out=buf[:M], path=path)
    check_close(C, A, wdq, bias=bias, label=f"W4 bf16 row blocks M={M} {N}x{K}")
    assert bool((buf[M] == -7.0).all())


@pytest.mark.parametrize("N,K", [(320, 4096), (1024, 14336), (28672, 4096)])
@pytest.mark.parametrize("M", [2, 3, 4])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_w4_small_m_one_hot_and_bias(N, K, M, dt):
    """The W4A16 small-M kernel at M = 2..4 (two or four activation rows
    held; at M = 3 the fourth re-reads the third and is not stored): one-hot
    rows give C[m, n] = wdq[n, k_m] bit for bit; dense rows with a bias are
    within the tolerance; nothing is written past row M - 1."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"W4 small-M kernel one-hot and bias M={M} N={N} K={K} {dt}")
    q, s, rq, rs, wdq = _w4(N, K, dev)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    to_bits = OR.f16_bits if dt == "f16" else OR.bf16_bits
    sets = [[0, 9, 130, K - 1], [5, 127, 1024 + 33, K // 2 + 7], [2, 64 + 3, 2048 + 100, K - 200]]
    for ks in sets:
        ks = ks[:M]
        A = torch.zeros((M, K), dtype=tdt)
        for m, k in enumerate(ks):
            A[m, k] = 1.0
        buf = torch.full((M + 1, N), -7.0, dtype=tdt, device=dev)
        C = tq.w4a16_gemm(A.to(dev), q, s, out=buf[:M])
        np.testing.assert_array_equal(bits16(C), to_bits(wdq[:, ks].T), err_msg=f"ks={ks}")
        assert bool((buf[M] == -7.0).all())
    A = synth.activations(M, K, synth.seed_for("w4sm", M, N, K, dt), dt)
    bias = synth.activations(1, N, synth.seed_for("w4smb", N, K, dt), dt)[0]
    C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev))
    check_close(C, A, wdq, bias=bias, label=f"W4 small-M kernel M={M} {N}x{K} {dt} with bias")


@pytest.mark.parametrize("N,K", [(320, 4096), (4096, 14336), (1024, 28672)])
@pytest.mark.parametrize("M", [2, 3, 4])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_ternary_small_m_one_hot_and_bias(N, K, M, dt):
    """The ternary small-M kernel at M = 2..4 (two or four activation rows
    held; at M = 3 the fourth re-reads the third and is not stored; K = 28672
    holds four rows only within the LDS at M = 2, so M = 3, 4 stream in fp16;
    bf16 has no streaming kernel and stays on the small-M kernel): one-hot
    rows give C[m, n] = wdq[n, k_m] bit for bit; dense rows with a bias are
    within the tolerance; nothing is written past row M - 1."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"ternary small-M one-hot and bias M={M} N={N} K={K} {dt}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    to_bits = OR.f16_bits if dt == "f16" else OR.bf16_bits
    sets = [[0, 9, 130, K - 1], [5, 255, 1024 + 33, K // 2 + 7], [2, 64 + 3, 2048 + 100, K - 200]]
    for ks in sets:
        ks = ks[:M]
        A = torch.zeros((M, K), dtype=tdt)
        for m, k in enumerate(ks):
            A[m, k] = 1.0
        buf = torch.full((M + 1, N), -7.0, dtype=tdt, device=dev)
        C = tq.tq_gemm(A.to(dev), codes, scale, out=buf[:M])
        np.testing.assert_array_equal(bits16(C), to_bits(wdq[:, ks].T), err_msg=f"ks={ks}")
        assert bool((buf[M] == -7.0).all())
    A = synth.activations(M, K, synth.seed_for("tsm", M, N, K, dt), dt)
    bias = synth.activations(1, N, synth.seed_for("tsmb", N, K, dt), dt)[0]
    C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev))
    check_close(C, A, wdq, bias=bias, label=f"ternary small-M M={M} {N}x{K} {dt} with bias")


@pytest.mark.parametrize("M,N,K", [(5, 4096, 4096), (16, 28672, 4096), (9, 4096, 14336), (16, 1000, 4160)])
def test_bf16_decode_m_auto(M, N, K):
    """bf16 at M = 5..16 through the dispatcher: the streaming kernel's bf16
    form (K split with the queried workspace on long K), or the medium path's
    tiles where K % 256 != 0; every output against the oracle, with a bias;
    the rows past M untouched."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"bf16 decode-size M auto M={M} N={N} K={K}")
    assert tq.tq_select_path("ternary", M, N, K, "bf16") == ("gemv" if K % 256 == 0 else "stream_mfma")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("bfm", M, N, K), "bf16")
    bias = synth.activations(1, N, synth.seed_for("bfmb", N, K), "bf16")[0]
    buf = torch.full((M + 1, N), -7.0, dtype=torch.bfloat16, device=dev)
    C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev), out=buf[:M])
    check_close(C, A, wdq, bias=bias, label=f"bf16 auto M={M} {N}x{K}")
    assert bool((buf[M] == -7.0).all())


@pytest.mark.parametrize("M,N,K,dt", [(2560, 7168, 256, "f16"), (2500, 7000, 320, "bf16"), (4096, 14336, 256, "f16")])
def test_prefill_tail_split(M, N, K, dt):
    """Large M whose 256 x 256 tiles leave the last round of workgroups at
    most half full (280 and 896 tiles on 256 compute units): the first
    columns run as 256-row tiles and the rest as 128-row tiles in a second
    launch that writes its own columns of C; every output against the
    oracle, with a bias, ragged M, N and K steps, and the rows past M and
    columns past N untouched."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"prefill tail split M={M} N={N} K={K} {dt}")
    codes, scale, rc, rs, wdq = _ternary(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("pts", M, N, K, dt), dt)
    bias = synth.activations(1, N, synth.seed_for("ptsb", N, dt), dt)[0]
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    buf = torch.full((M * N + 4096,), -3.0, dtype=tdt, device=dev)
    C = tq.tq_gemm(A.to(dev), codes, scale, bias=bias.to(dev), out=buf[:M * N].view(M, N))
    assert bool((buf[M * N:] == -3.0).all())
    check_close(C, A, wdq, bias=bias, label=f"prefill tail split {M}x{N}x{K} {dt}")
