"""GPU parity at Llama-3-70B linear-layer shapes (hidden 8192, intermediate
28672, 8 KV heads of 128) for M in {1, 32, 64}.

Full-size weights are drawn on the device by the seeded generator and packed
by the library.  The oracle packs 256 sampled weight rows from the same
weights: their codes and scales must match bit for bit, and every output of
those rows must be within the tolerance of the fp64 oracle product.
"""
import numpy as np
import pytest

import oracle.ternary as OT
import synth
from gpu_common import bits16, check_close, log, require_gpu

pytestmark = pytest.mark.gpu

SHAPES_70B = [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)]
# the stacked layouts the decode benchmark runs: q,k,v and gate,up along N
FUSED_70B = [(10240, 8192), (57344, 8192)]
SAMPLE_ROWS = 256
_CACHE = {}


def _packed(N, K, dev):
    """(codes, scale, sampled rows, oracle dequant of those rows) for a shape."""
    key = (N, K)
    if key not in _CACHE:
        import torch
        import bit_weight_only_tq_amd as tq
        _CACHE.clear()
        W = synth.weights_device(N, K, synth.seed_for("w70b", N, K), dev)
        codes, scale = tq.tq_pack(W)
        rows = np.sort(np.random.default_rng(N + 7 * K).choice(N, SAMPLE_ROWS, replace=False))
        idx = torch.from_numpy(rows).to(dev)
        Wr = W.index_select(0, idx).cpu().numpy()
        del W
        torch.cuda.empty_cache()
        rc, rs = OT.ternary_pack(Wr)
        np.testing.assert_array_equal(codes.index_select(0, idx).cpu().numpy(), rc)
        np.testing.assert_array_equal(bits16(scale.index_select(0, idx)), rs)
        _CACHE[key] = (codes, scale, rows, OT.ternary_dequant(rc, rs, K))
    return _CACHE[key]


@pytest.mark.parametrize("N,K", SHAPES_70B)
@pytest.mark.parametrize("M", [1, 2, 32, 64])
def test_ternary_70b(N, K, M):
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"tq_gemm 70b N={N} K={K} M={M}")
    codes, scale, rows, wdq = _packed(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("a70b", N, K, M), "f16")
    assert tq.tq_select_path("ternary", M, N, K) == ("gemv" if M <= 16 else "stream_mfma")
    C = tq.tq_gemm(A.to(dev), codes, scale)
    check_close(C.index_select(1, torch.from_numpy(rows).to(dev)), A, wdq, label=f"70b {N}x{K} M={M}")


@pytest.mark.parametrize("N,K", FUSED_70B)
@pytest.mark.parametrize("M", [1, 2, 16])
def test_ternary_70b_fused(N, K, M):
    import torch
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"tq_gemm 70b fused N={N} K={K} M={M}")
    codes, scale, rows, wdq = _packed(N, K, dev)
    A = synth.activations(M, K, synth.seed_for("a70bf", N, K, M), "f16")
    C = tq.tq_gemm(A.to(dev), codes, scale)
    check_close(C.index_select(1, torch.from_numpy(rows).to(dev)), A, wdq, label=f"70b fused {N}x{K} M={M}")


@pytest.mark.parametrize("N,K", [(8192, 28672), (57344, 8192)])
def test_70b_m1_one_hot(N, K):
    """The M = 1 decode kernel with two row-blocks per workgroup (down with
    eight chunk-sets per wave, and the stacked gate/up): a one-hot row e_k
    gives C[0, n] = wdq[n, k] bit for bit on the sampled rows."""
    import torch
    import oracle.rne as OR
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    log(f"70b M=1 one-hot N={N} K={K}")
    codes, scale, rows, wdq = _packed(N, K, dev)
    idx = torch.from_numpy(rows).to(dev)
    for k in sorted({0, 7, 2047, 2048 + 5, K // 2 + 13, K - 129, K - 1}):
        A = torch.zeros((1, K), dtype=torch.float16)
        A[0, k] = 1.0
        C = tq.tq_gemm(A.to(dev), codes, scale)
        np.testing.assert_array_equal(bits16(C.index_select(1, idx))[0], OR.f16_bits(wdq[:, k]), err_msg=f"k={k}")
