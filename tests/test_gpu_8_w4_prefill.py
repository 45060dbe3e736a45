"""GPU parity of the W4A16 matrix-core GEMM (256-row tiles from M = 256,
64-row tiles below; split K where the tiles leave compute units idle or K
holds more than 128 groups).

Symmetric (zero point 8) and asymmetric formats, with and without
activation order, fp16 and bf16 activations: every output at M = 2048 and
sampled rows at M = 4096 on the Llama-3-8B MLP shapes, ragged M and N with a
bias, the sparse edge-case groups, and one-hot rows that must reproduce
single dequantized weights bit for bit ((q - z) * s is exact in fp32 and
rounded once to the output format).
"""
import numpy as np
import pytest

import oracle.rne as OR
import oracle.w4 as OW
import oracle.w4asym as OA
import synth
from gpu_common import bits16, check_close, log, require_gpu

pytestmark = pytest.mark.gpu

_CACHE = {}


def _packed(N, K, fmt, dev, sparse=False):
    """Device packing and oracle dequant of one matrix; fmt in sym / asym / act."""
    key = (N, K, fmt, sparse)
    if key not in _CACHE:
        import torch
        import bit_weight_only_tq_amd as tq
        W = (synth.sparse_w4_weights(N, K, synth.seed_for("w4p-sp", N, K)) if sparse
             else synth.weights(N, K, synth.seed_for("w4p", N, K)))
        Wd = torch.from_numpy(W).to(dev)
        if fmt == "sym":
            q, s = tq.w4a16_pack(Wd)
            rq, rs = OW.w4_pack(W)
            z, perm, wdq = None, None, OW.w4_dequant(rq, rs, K)
        else:
            gidx = synth.group_index(K, synth.seed_for("w4p-g", K)) if fmt == "act" else None
            q, s, z, perm = tq.w4a16_pack_asym(Wd, None if gidx is None else torch.from_numpy(gidx).to(dev))
            rq, rs, rz, rperm = OA.w4a_pack(W, gidx)
            np.testing.assert_array_equal(z.cpu().numpy(), rz)
            wdq = OA.w4a_dequant(rq, rs, rz, K, rperm if gidx is not None else None)
        np.testing.assert_array_equal(q.cpu().numpy(), rq)
        _CACHE.clear()
        _CACHE[key] = (q, s, z, perm, wdq)
    return _CACHE[key]


@pytest.mark.parametrize("fmt", ["sym", "asym", "act"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("N,K", [(14336, 4096), (4096, 14336)])
def test_w4_prefill_full(N, K, dt, fmt):
    """M = 2048: every output element against the oracle."""
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    M = 2048
    log(f"w4 prefill M={M} N={N} K={K} {dt} {fmt}")
    assert tq.tq_select_path("w4a16", M, N, K, dt) == "gemm"
    q, s, z, perm, wdq = _packed(N, K, fmt, dev)
    A = synth.activations(M, K, synth.seed_for("w4pa", M, K, dt), dt)
    C = tq.w4a16_gemm(A.to(dev), q, s, zeros=z, perm=perm)
    check_close(C, A, wdq, label=f"w4 prefill {M}x{N}x{K} {dt} {fmt}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_w4_prefill_m4096_sampled(dt):
    """M = 4096 on 14336 x 4096: 256 sampled activation rows, all columns."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    M, N, K = 4096, 14336, 4096
    log(f"w4 prefill M={M} N={N} K={K} {dt} sampled")
    q, s, z, perm, wdq = _packed(N, K, "sym", dev)
    A = synth.activations(M, K, synth.seed_for("w4pa4", M, K, dt), dt)
    C = tq.w4a16_gemm(A.to(dev), q, s)
    rows = np.sort(np.random.default_rng(7).choice(M, 256, replace=False))
    check_close(C[torch.from_numpy(rows).to(dev)], A[torch.from_numpy(rows)], wdq, label=f"w4 prefill M=4096 {dt}")


@pytest.mark.parametrize("fmt", ["sym", "asym", "act"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(256, 128, 128), (300, 1000, 1024), (517, 260, 2048), (64, 384, 4096)])
def test_w4_prefill_ragged_bias(M, N, K, dt, fmt):
    """Ragged M and N (partial tiles, the scalar store path), a single group,
    a bias, and M below the dispatcher's threshold through the forced path;
    the row after C is left untouched."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"w4 prefill ragged M={M} N={N} K={K} {dt} {fmt}")
    q, s, z, perm, wdq = _packed(N, K, fmt, dev)
    A = synth.activations(M, K, synth.seed_for("w4pr", M, N, K, dt), dt)
    bias = synth.activations(1, N, synth.seed_for("w4prb", N, dt), dt)[0]
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    buf = torch.full((M + 1, N), -3.0, dtype=tdt, device=dev)
    C = tq.w4a16_gemm(A.to(dev), q, s, bias=bias.to(dev), zeros=z, perm=perm, path="gemm", out=buf[:M])
    check_close(C, A, wdq, bias=bias, label=f"w4 prefill ragged {M}x{N}x{K} {dt} {fmt}")
    assert bool((buf[M] == -3.0).all())


@pytest.mark.parametrize("regime", synth.ACT_REGIMES)
@pytest.mark.parametrize("fmt", ["sym", "asym"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_w4_prefill_edge(dt, fmt, regime):
    """Sparse groups (one nonzero value, one large value among values that
    quantize to zero) with dense, outlier and tiny activations."""
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    M, N, K = 512, 1024, 4096
    log(f"w4 prefill edge {dt} {fmt} {regime}")
    q, s, z, perm, wdq = _packed(N, K, fmt, dev, sparse=True)
    A = synth.activations_regime(M, K, synth.seed_for("w4pe", regime, dt), regime, dt)
    C = tq.w4a16_gemm(A.to(dev), q, s, zeros=z, perm=perm)
    check_close(C, A, wdq, label=f"w4 prefill edge {dt} {fmt} {regime}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("fmt", ["sym", "act"])
def test_w4_prefill_one_hot(dt, fmt):
    """Rows of the identity: C[m, n] = wdq[n, k_m] rounded once to the output
    format, bit for bit; pins the nibble order, the group of each column, the
    zero point and the scale index."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    N, K = 384, 2048
    log(f"w4 prefill one-hot {dt} {fmt}")
    q, s, z, perm, wdq = _packed(N, K, fmt, dev)
    ks = [0, 1, 2, 3, 4, 5, 6, 7, 8, 15, 16, 63, 64, 127, 128, 129, 255, 256, 1000, 1024, 1535, 2047]
    ks = ks + [k for k in range(300, 300 + 256 - len(ks))]
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    A = torch.zeros((len(ks), K), dtype=tdt)
    for m, k in enumerate(ks):
        A[m, k] = 1.0
    C = tq.w4a16_gemm(A.to(dev), q, s, zeros=z, perm=perm, path="gemm")
    to_bits = OR.f16_bits if dt == "f16" else OR.bf16_bits
    np.testing.assert_array_equal(bits16(C), to_bits(wdq[:, ks].T))


def test_w4_gemm_long_k_splits():
    """More than 128 groups (the scales one split can hold): with a workspace
    the GEMM splits K (at least two splits) and stays within the tolerance;
    forced without one it is refused with nothing launched, and the
    dispatcher then takes the decode kernels over row blocks."""
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    M, N, K = 300, 256, 16384 + 128
    assert tq.tq_select_path("w4a16", M, N, K) == "gemm"
    assert tq.w4a16_gemm_workspace_bytes(M, N, K) >= 2 * M * N * 4
    log(f"w4 long K M={M} N={N} K={K}")
    q, s, z, perm, wdq = _packed(N, K, "sym", dev)
    A = synth.activations(M, K, synth.seed_for("w4lk", M, K), "f16")
    C = tq.w4a16_gemm(A.to(dev), q, s)
    check_close(C, A, wdq, label="w4 long K, split")
    with pytest.raises(tq.TQError, match="TQ_ERR_PATH"):
        tq.w4a16_gemm(A.to(dev), q, s, path="gemm", workspace=None)
    C = tq.w4a16_gemm(A.to(dev)[:40], q, s, workspace=None)  # auto, no workspace: row blocks
    check_close(C, A[:40], wdq, label="w4 long K, row blocks")
