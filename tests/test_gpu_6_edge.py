"""GPU parity on the method's edge cases, for every kernel family.

Ternary rows with one to eight kept entries (w_t = sign(w) * (|w| > 0.7
mean|w|) keeps exactly the nonzero entries of such a row) and scales from
1e-4 to 6e4, next to all-zero and dense rows; W4A16 groups with a single
nonzero value or one large value among values that quantize to zero.
Activations are dense N(0, 1), N(0, 1) with outliers of magnitude 200-1000,
or N(0, 1) * 2^-12.  Every output must stay within 2e-3 * sum_k |a_k w_k| +
1e-3 of the fp64 oracle: the error of a row has to scale with that row's
own sum, however few of its codes are nonzero.

Each case names the kernel family its shape and workspace route to
(comments); the dispatcher is deterministic, so the shapes below reach
every family: the small-M kernel (M <= 4), the LDS kernel (K < 4096), the
streaming kernel with and without a K split, the matrix-core GEMV (K > 8192
without a workspace), the per-lane FMA kernels (K % 256 != 0, or bf16 shapes
the others cannot take), the medium-M kernels (K % 256 == 0 or not) and the
prefill GEMM with and without a K split.
"""
import numpy as np
import pytest

import oracle.ternary as OT
import oracle.w4 as OW
import oracle.w4asym as OA
import synth
from gpu_common import bits16, check_close, log, require_gpu

pytestmark = pytest.mark.gpu

_CACHE = {}


def _ternary(N, K, dev):
    key = ("t", N, K)
    if key not in _CACHE:
        import torch
        import bit_weight_only_tq_amd as tq
        W = synth.sparse_ternary_weights(N, K, synth.seed_for("edge-t", N, K))
        codes, scale = tq.tq_pack(torch.from_numpy(W).to(dev))
        rc, rs = OT.ternary_pack(W)
        np.testing.assert_array_equal(codes.cpu().numpy(), rc)
        np.testing.assert_array_equal(bits16(scale), rs)
        _CACHE.clear()
        _CACHE[key] = (codes, scale, OT.ternary_dequant(rc, rs, K))
    return _CACHE[key]


def _w4(N, K, dev, asym):
    key = ("w4", N, K, asym)
    if key not in _CACHE:
        import torch
        import bit_weight_only_tq_amd as tq
        W = synth.sparse_w4_weights(N, K, synth.seed_for("edge-w4", N, K))
        Wd = torch.from_numpy(W).to(dev)
        if asym:
            q, s, z, _ = tq.w4a16_pack_asym(Wd)
            rq, rs, rz, _ = OA.w4a_pack(W)
            np.testing.assert_array_equal(z.cpu().numpy(), rz)
            wdq = OA.w4a_dequant(rq, rs, rz, K)
        else:
            q, s = tq.w4a16_pack(Wd)
            z = None
            rq, rs = OW.w4_pack(W)
            wdq = OW.w4_dequant(rq, rs, K)
        np.testing.assert_array_equal(q.cpu().numpy(), rq)
        np.testing.assert_array_equal(bits16(s), rs)
        _CACHE.clear()
        _CACHE[key] = (q, s, z, wdq)
    return _CACHE[key]


# (label, N, K, M, dtype, workspace, path): label names the kernel family
TERNARY_CASES = [
    ("small-M M=1", 1024, 4096, 1, "f16", "auto", "auto"),
    ("small-M M=1", 1024, 4096, 1, "bf16", "auto", "auto"),
    ("small-M M=2", 1024, 4096, 2, "f16", "auto", "auto"),
    ("small-M M=4", 1024, 4096, 4, "bf16", "auto", "auto"),
    ("small-M CSW=8", 512, 28672, 1, "f16", "auto", "auto"),
    ("LDS kernel", 1024, 2048, 1, "f16", "auto", "auto"),
    ("LDS kernel M=2", 1024, 2048, 2, "f16", None, "auto"),
    ("stream", 1024, 4096, 8, "f16", None, "auto"),
    ("stream", 1024, 4096, 16, "bf16", None, "auto"),
    ("stream split-K", 1024, 8192, 16, "f16", "auto", "auto"),
    ("stream split-K", 1024, 8192, 12, "bf16", "auto", "auto"),
    ("matrix-core GEMV", 1024, 16384, 8, "f16", None, "auto"),
    ("per-lane FMA K%256", 1024, 4160, 2, "f16", "auto", "auto"),
    ("per-lane FMA forced", 1024, 4160, 4, "bf16", "auto", "gemv"),
    ("medium mm K%256 at M=5", 1024, 4160, 5, "f16", "auto", "auto"),
    ("per-lane FMA bf16", 1024, 2048, 1, "bf16", "auto", "auto"),
    ("medium mm3", 1024, 4096, 32, "f16", "auto", "auto"),
    ("medium mm3", 1024, 4096, 64, "bf16", None, "auto"),
    ("medium mm K%256", 1024, 4160, 48, "f16", "auto", "auto"),
    ("medium mm K%256", 1024, 4160, 20, "bf16", None, "auto"),
    ("prefill split-K", 512, 4096, 300, "f16", "auto", "auto"),
    ("prefill split-K", 512, 4096, 300, "bf16", "auto", "auto"),
    ("prefill one pass", 768, 4096, 256, "f16", None, "auto"),
    ("prefill one pass", 768, 4096, 256, "bf16", None, "auto"),
]


@pytest.mark.parametrize("regime", synth.ACT_REGIMES)
@pytest.mark.parametrize("case", TERNARY_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-M{c[3]}-{c[4]}-ws{c[5]}")
def test_ternary_edge(case, regime):
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    label, N, K, M, dt, ws, path = case
    log(f"ternary edge {label} N={N} K={K} M={M} {dt} ws={ws} {regime}")
    codes, scale, wdq = _ternary(N, K, dev)
    A = synth.activations_regime(M, K, synth.seed_for("edge-a", N, K, M, regime), regime, dt)
    C = tq.tq_gemm(A.to(dev), codes, scale, path=path, workspace=ws)
    check_close(C, A, wdq, label=f"ternary edge {label} {N}x{K} M={M} {dt} {regime}")


W4_CASES = [
    ("small-M M=1", 1024, 4096, 1, "f16", "auto"),
    ("small-M M=1", 1024, 4096, 1, "bf16", "auto"),
    ("small-M M=4", 1024, 4096, 4, "f16", "auto"),
    ("small-M M=3", 1024, 4096, 3, "bf16", "auto"),
    ("stream", 1024, 4096, 8, "f16", None),
    ("stream", 1024, 4096, 16, "bf16", None),
    ("stream split-K", 1024, 8192, 16, "f16", "auto"),
    ("matrix-core GEMV", 1024, 16384, 8, "f16", None),
    ("per-lane FMA", 1024, 1024, 1, "f16", "auto"),
    ("per-lane FMA", 1024, 1024, 2, "bf16", "auto"),
    ("blocks of 16 rows", 1024, 4096, 24, "f16", "auto"),
    ("GEMM 64-row tiles, one pass", 1024, 4096, 40, "f16", None),
    ("GEMM 64-row tiles split-K", 1024, 8192, 20, "bf16", "auto"),
]


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
@pytest.mark.parametrize("regime", synth.ACT_REGIMES)
@pytest.mark.parametrize("case", W4_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-M{c[3]}-{c[4]}-ws{c[5]}")
def test_w4_edge(case, regime, asym):
    import bit_weight_only_tq_amd as tq
    dev = require_gpu()
    label, N, K, M, dt, ws = case
    if asym and label == "matrix-core GEMV":
        pytest.skip("the matrix-core W4 GEMV serves zero point 8 only")
    log(f"w4 edge {label} N={N} K={K} M={M} {dt} ws={ws} {regime} asym={asym}")
    q, s, z, wdq = _w4(N, K, dev, asym)
    A = synth.activations_regime(M, K, synth.seed_for("edge-a4", N, K, M, regime), regime, dt)
    C = tq.w4a16_gemm(A.to(dev), q, s, zeros=z, workspace=ws)
    check_close(C, A, wdq, label=f"w4 edge {label} {N}x{K} M={M} {dt} {regime} asym={asym}")
