"""tq_gemm_noalloc against tq_gemm_ws, through the C ABI.

The no-allocation entry point runs the schedule tq_gemm_ws takes with the
workspace tq_gemm_workspace_bytes() asks for, with the split partials in the
library's per-device scratch instead, so its output must match that call's
bit for bit.  Two calls in a row, the second on a smaller input, check that
the shared scratch carries nothing from one call to the next; both outputs
are also within the oracle's tolerance.
"""
import ctypes

import numpy as np
import pytest

import oracle.ternary as OT
import synth
from gpu_common import bits16, check_close, log, require_gpu

pytestmark = pytest.mark.gpu


def _layer(N, K, dev):
    import torch
    import bit_weight_only_tq_amd as tq
    W = synth.weights(N, K, synth.seed_for("noalloc", N, K))
    codes, scale = tq.tq_pack(torch.from_numpy(W).to(dev))
    rc, rs = OT.ternary_pack(W)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    return codes, scale, OT.ternary_dequant(rc, rs, K)


def _call_noalloc(lib, A, codes, scale, bias, C, dt):
    import torch
    M, K = A.shape
    N = codes.shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return lib.tq_gemm_noalloc(p(A), dt, M, N, K, p(codes), p(scale), p(bias), p(C), stream, 0)


def _call_ws(lib, A, codes, scale, bias, C, dt):
    import torch
    M, K = A.shape
    N = codes.shape[0]
    nbytes = lib.tq_gemm_workspace_bytes(M, N, K, dt, 0)
    ws = torch.zeros((max(nbytes, 1),), dtype=torch.uint8, device=A.device)  # counters zero
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.tq_gemm_ws(p(A), dt, M, N, K, p(codes), p(scale), p(bias), p(C), p(ws) if nbytes else None, nbytes,
                        stream, 0)
    return st, nbytes


# (M, N, K, dtype): decode split-K, then a smaller medium-M call, then a
# smaller decode call; each schedule uses the scratch (nonzero workspace)
SEQUENCES = [
    [(16, 1024, 8192, "f16"), (12, 768, 8192, "f16")],
    [(64, 2048, 4096, "bf16"), (32, 1024, 4096, "bf16")],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-".join(f"M{m}x{n}x{k}{d}" for m, n, k, d in s))
def test_noalloc_matches_workspace_entry_point(seq):
    import torch
    import bit_weight_only_tq_amd as tq
    from bit_weight_only_tq_amd import _lib
    dev = require_gpu()
    lib = _lib.load()
    for i, (M, N, K, dt) in enumerate(seq):
        log(f"tq_gemm_noalloc call {i}: M={M} N={N} K={K} {dt}")
        d = _lib.TQ_BF16 if dt == "bf16" else _lib.TQ_F16
        codes, scale, wdq = _layer(N, K, dev)
        A = synth.activations(M, K, synth.seed_for("noalloc-a", M, N, K), dt)
        bias = synth.activations(1, N, synth.seed_for("noalloc-b", N), dt)[0]
        Ad, bd = A.to(dev), bias.to(dev)
        C_ref = torch.empty((M, N), dtype=Ad.dtype, device=dev)
        st, nbytes = _call_ws(lib, Ad, codes, scale, bd, C_ref, d)
        assert st == 0 and 0 < nbytes <= lib.tq_gemm_noalloc_scratch_bytes(), (st, nbytes)
        C = torch.full((M, N), float("nan"), dtype=Ad.dtype, device=dev)
        assert _call_noalloc(lib, Ad, codes, scale, bd, C, d) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits16(C), bits16(C_ref))
        check_close(C, A, wdq, bias=bias, label=f"noalloc M={M} {N}x{K} {dt}")
    # the Python wrapper reaches the same entry point
    C2 = tq.tq_gemm_noalloc(Ad, codes, scale, bias=bd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits16(C2), bits16(C_ref))


def test_noalloc_without_split_and_rejection():
    """A schedule with no split (M = 1) needs no scratch; a prefill schedule
    whose partials exceed the scratch is rejected with nothing launched."""
    import torch
    from bit_weight_only_tq_amd import _lib
    dev = require_gpu()
    lib = _lib.load()
    codes, scale, wdq = _layer(1024, 4096, dev)
    A = synth.activations(1, 4096, synth.seed_for("noalloc-a1"), "f16")
    Ad = A.to(dev)
    C = torch.empty((1, 1024), dtype=torch.float16, device=dev)
    assert lib.tq_gemm_workspace_bytes(1, 1024, 4096, 0, 0) == 0
    assert _call_noalloc(lib, Ad, codes, scale, None, C, 0) == 0
    torch.cuda.synchronize()
    check_close(C, A, wdq, label="noalloc M=1")
    big_codes = torch.zeros((4096, 14336 // 4), dtype=torch.uint8, device=dev)
    big_scale = torch.zeros((4096,), dtype=torch.float16, device=dev)
    A2 = torch.zeros((2048, 14336), dtype=torch.float16, device=dev)
    C2 = torch.empty((2048, 4096), dtype=torch.float16, device=dev)
    st = _call_noalloc(lib, A2, big_codes, big_scale, None, C2, 0)
    assert _lib.STATUS_NAMES[st] == "TQ_ERR_SCRATCH"
