"""Tolerance verdict and error statistics (test infrastructure only).

* ``tolerance_ok``: an output element passes iff it is finite and
  |C - out64| <= rel * mag64 + abs_, with rel = 2e-3 and abs_ = 1e-3 by
  default, where mag64 = sum_k |a_k * w_k| (see ``oracle.gemm``).  A correctly
  rounded bf16 output is off by at most 2^-9 * |out| <= 1.953e-3 * mag64 and a
  fp16 one by 2^-11 * |out|, so any fp32-accumulating kernel that rounds its
  result once fits inside the bound with margin left for the fp32 sums.
* ``quant_check``: the four numbers [P3] section 10.6.3 asks for when
  comparing a quantized output with a reference (allclose verdict, max and
  mean absolute error, all finite).
"""

import numpy as np

REL_TOL = 2e-3
ABS_TOL = 1e-3


def tolerance_ok(C, out64, mag64, rel: float = REL_TOL, abs_: float = ABS_TOL):
    """(ok, stats) for output C against the fp64 reference."""
    C64 = np.asarray(C, dtype=np.float64)
    out64 = np.asarray(out64, dtype=np.float64)
    mag64 = np.asarray(mag64, dtype=np.float64)
    if C64.shape != out64.shape:
        raise ValueError(f"shape mismatch {C64.shape} vs {out64.shape}")
    finite = bool(np.isfinite(C64).all())
    err = np.abs(C64 - out64)
    bound = rel * mag64 + abs_
    with np.errstate(invalid="ignore"):
        ratio = np.where(np.isfinite(err), err / bound, np.inf)
    ok = finite and bool(np.all(err <= bound))
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    stats = {
        "ok": ok,
        "finite": finite,
        "max_abs": float(np.nanmax(err)) if err.size else 0.0,
        "mean_abs": float(np.nanmean(err)) if err.size else 0.0,
        "max_ratio_to_bound": float(ratio.max()) if ratio.size else 0.0,
        "worst_index": tuple(int(i) for i in worst),
        "n": int(C64.size),
    }
    return ok, stats


def quant_check(ref, test, atol: float, rtol: float):
    """allclose verdict plus max / mean absolute error and finiteness."""
    ref = np.asarray(ref, dtype=np.float64)
    test = np.asarray(test, dtype=np.float64)
    diff = np.abs(ref - test)
    return {
        "ok": bool(np.allclose(ref, test, atol=atol, rtol=rtol)),  # |ref-test| <= atol + rtol*|test|
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "mean_abs": float(diff.mean()) if diff.size else 0.0,
        "finite": bool(np.isfinite(test).all()),
    }
