"""Helpers for the GPU parity tests: device checks and oracle comparisons."""
import numpy as np
import pytest

import oracle.check
import oracle.gemm
import oracle.rne
import oracle.ternary
import oracle.w4


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import bit_weight_only_tq_amd as tq
    tq.load()  # raises if libtq.so is missing: no silent fallback on a GPU machine
    return torch.device("cuda", 0)


def bits16(t):
    """uint16 bit patterns of a 16-bit torch tensor (any device) as numpy."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def a_f64(A):
    """Exact fp64 values of fp16 / bf16 activations (torch CPU tensor)."""
    return A.detach().cpu().double().numpy()


def check_close(C, A, wdq64, bias=None, label=""):
    """Tolerance verdict of a GEMM output against the fp64 oracle; asserts."""
    bias64 = None if bias is None else bias.detach().cpu().double().numpy()
    out, mag = oracle.gemm.gemm_ref64(a_f64(A), wdq64, bias64)
    import torch
    out_dtype = "bf16" if C.dtype == torch.bfloat16 else "f16"
    ok, st = oracle.check.tolerance_ok(C.detach().cpu().double().numpy(), out, mag, out_dtype=out_dtype)
    qc = oracle.check.quant_check(out, C.detach().cpu().double().numpy(), atol=1e-3, rtol=2e-3)
    assert ok, f"{label}: {st} quant_check={qc}"
    return st


def log(msg):
    print(f"[case] {msg}", flush=True)
