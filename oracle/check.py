"""Tolerance verdict and error statistics (test infrastructure only).

* ``tolerance_ok``: an output element passes iff it is finite and
  |C - out64| <= rel * mag64 + abs_ (+ u * |out64| for bf16 outputs), with
  rel = 2e-3 and abs_ = 1e-3 by default, where mag64 = sum_k |a_k * w_k|
  (see ``oracle.gemm``), or iff it is an infinity of the sign of out64 and
  some value within that bound of out64 rounds to that infinity in the
  output format: the output is the fp32 result rounded once to the
  activation dtype, and a magnitude past the format's range rounds to
  infinity ([P1] section 4 writes half-precision outputs; the reading that
  overflow gives +-inf).  Rounding the exact result once to the output format
  costs up to u * |out| with u = 2^-11 for fp16 (always inside rel * mag64,
  since |out| <= mag64) but u = 2^-8 for bf16 (8 significant bits), which can
  exceed rel * mag64 when the terms of a short sum share one sign.  Since no
  implementation can beat the rounding of its own output format, bf16 outputs
  get that half-ulp allowance on top of the stated bound.
* ``quant_check``: the four numbers [P3] section 10.6.3 asks for when
  comparing a quantized output with a reference (allclose verdict, max and
  mean absolute error, all finite).
"""

import numpy as np

REL_TOL = 2e-3
ABS_TOL = 1e-3


BF16_UNIT_ROUNDOFF = 2.0 ** -8
# Smallest magnitudes that round to infinity (round to nearest even): the
# largest finite value plus half its unit in the last place.
F16_OVERFLOW = 65504.0 + 16.0
BF16_OVERFLOW = (2.0 - 2.0 ** -8) * 2.0 ** 127


def tolerance_ok(C, out64, mag64, rel: float = REL_TOL, abs_: float = ABS_TOL, out_dtype: str = "f16"):
    """(ok, stats) for output C (values of dtype ``out_dtype``) against the fp64 reference."""
    C64 = np.asarray(C, dtype=np.float64)
    out64 = np.asarray(out64, dtype=np.float64)
    mag64 = np.asarray(mag64, dtype=np.float64)
    if C64.shape != out64.shape:
        raise ValueError(f"shape mismatch {C64.shape} vs {out64.shape}")
    finite = bool(np.isfinite(C64).all())
    with np.errstate(invalid="ignore"):
        err = np.abs(C64 - out64)
    bound = rel * mag64 + abs_
    if out_dtype == "bf16":
        bound = bound + BF16_UNIT_ROUNDOFF * np.abs(out64)
        overflow = BF16_OVERFLOW
    elif out_dtype == "f16":
        overflow = F16_OVERFLOW
    else:
        raise ValueError(f"unknown output dtype {out_dtype!r}")
    inf_ok = np.isinf(C64) & (np.sign(C64) == np.sign(out64)) & (np.abs(out64) + bound >= overflow)
    with np.errstate(invalid="ignore"):
        ratio = np.where(inf_ok, 0.0, np.where(np.isfinite(err), err / bound, np.inf))
    ok = bool(np.all((np.isfinite(C64) & (err <= bound)) | inf_ok))
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
