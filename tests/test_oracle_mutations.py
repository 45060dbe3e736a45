"""Plant one plausible mistake at a time in a copy of the oracle; some pin must fail.

Each mutation is a textual edit of one oracle source file (a flipped
comparison, a swapped sign, a reversed bit order, a dropped term, a pairwise
sum instead of a running sum, double rounding, ...).  The edited copy is
imported as a separate package and every pin of ``oracle_pins`` is run on it
until one fails.  A mutation that no pin catches fails this test.  Nothing
here touches the real oracle or any GPU.
"""
import importlib
import os
import shutil
import sys

import pytest

from oracle_pins import ALL_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("ternary.py", "        if a > thr:", "        if a >= thr:"),
    ("ternary.py", "keep = a > thr[:, None]", "keep = a >= thr[:, None]"),
    ("ternary.py", "THRESHOLD_FACTOR = 0.7 ", "THRESHOLD_FACTOR = 0.75 "),
    ("ternary.py", "t.append(1 if v > 0 else -1)", "t.append(-1 if v > 0 else 1)"),
    ("ternary.py", "np.where(w > 0, 1, -1)", "np.where(w > 0, -1, 1)"),
    ("ternary.py", "byte |= code << (2 * k)", "byte |= code << (2 * (3 - k))"),
    ("ternary.py", "out |= c[:, :, k] << np.uint8(2 * k)", "out |= c[:, :, 3 - k] << np.uint8(2 * k)"),
    ("ternary.py", "kept_sum / np.maximum(kept, 1)", "s / K"),
    ("ternary.py", "scale64 = kept_sum / kept if kept else 0.0", "scale64 = s / K if kept else 0.0"),
    ("ternary.py", "s = np.cumsum(a, axis=1)[:, -1]", "s = a.sum(axis=1)"),
    ("ternary.py", "return (K + CODES_PER_BYTE - 1) // CODES_PER_BYTE", "return K // CODES_PER_BYTE"),
    ("ternary.py", "CODE_OF = {-1: 0, 0: 1, 1: 2}", "CODE_OF = {-1: 2, 0: 1, 1: 0}"),
    ("ternary.py", "VALUE_OF = {0: -1, 1: 0, 2: 1}", "VALUE_OF = {0: 1, 1: 0, 2: -1}"),
    ("ternary.py", "np.full((N, rb * CODES_PER_BYTE), CODE_OF[0]", "np.full((N, rb * CODES_PER_BYTE), CODE_OF[-1]"),
    ("ternary.py", "if np.any(fields == 3):", "if False:"),
    ("ternary.py", "thr = THRESHOLD_FACTOR * (s / K)\n        keep", "thr = THRESHOLD_FACTOR * (s / (K - 1))\n        keep"),
    ("ternary.py", "return fields.astype(np.int8) - 1", "return fields.astype(np.int8) - 2"),
    ("rne.py", "r = round(a / quantum)", "r = int(a / quantum + Fraction(1, 2))"),
    ("rne.py", "lsb = (u >> 16) & 1", "lsb = 0"),
    ("rne.py", ".astype(np.float16).view(np.uint16)", ".astype(np.float32).astype(np.float16).view(np.uint16)"),
    ("rne.py", "emin = 1 - bias", "emin = -bias"),
    ("w4.py", "sb = f16_bits(amax / 7.0)", "sb = f16_bits(amax / 8.0)"),
    ("w4.py", "r = np.rint(w / s)", "r = np.floor(w / s + 0.5)"),
    ("w4.py", "word |= q[:, :, i] << np.uint32(BITS * i)", "word |= q[:, :, 7 - i] << np.uint32(BITS * i)"),
    ("w4.py", "ZERO_POINT = 8", "ZERO_POINT = 7"),
    ("w4.py", "np.clip(r, QMIN, QMAX)", "np.clip(r, -7, 7)"),
    ("w4.py", "s = np.repeat(f16_values(scale_bits), group, axis=1)", "s = np.tile(f16_values(scale_bits), (1, group))"),
    ("w4.py", "rv = int(_round_half_even(v / s))", "rv = int(v / s)"),
    ("w4asym.py", "lo = np.minimum(w.min(axis=2), 0.0)", "lo = w.min(axis=2)"),
    ("w4asym.py", "hi = np.maximum(w.max(axis=2), 0.0)", "hi = w.max(axis=2)"),
    ("w4asym.py", "sb = f16_bits((hi - lo) / 15.0)", "sb = f16_bits((hi - lo) / 16.0)"),
    ("w4asym.py", "np.clip(np.rint(-lo / s), 0, QMAX)", "np.clip(np.floor(-lo / s), 0, QMAX)"),
    ("w4asym.py", "q = np.rint(w / s[:, :, None]) + z[:, :, None]", "q = np.rint(w / s[:, :, None]) - z[:, :, None]"),
    ("w4asym.py", "np.clip(q, 0, QMAX))", "np.clip(q, 0, 14))"),
    ("w4asym.py", 'return np.argsort(g, kind="stable")', 'return np.argsort(-g, kind="stable")'),
    ("w4asym.py", "packed = (q - z) * s", "packed = (q + z) * s"),
    ("w4asym.py", "out[:, np.asarray(perm)] = packed", "out = packed[:, np.asarray(perm)]"),
    ("w4asym.py", "word |= q[:, :, i] << np.uint32(BITS * i)", "word |= q[:, :, 7 - i] << np.uint32(BITS * i)"),
    ("w4asym.py", "z = int(min(max(_rint(-lo / s), 0), QMAX))", "z = int(min(max(_rint(lo / s), 0), QMAX))"),
    ("w4asym.py", "                if v < lo:", "                if v > lo:"),
    ("w4asym.py", "if np.any(np.bincount(g, minlength=G) != group):", "if False:"),
    ("w4asym.py", "row[perm[i]] = (q - z_row[g]) * f16_value_exact(s_row[g])", "row[i] = (q - z_row[g]) * f16_value_exact(s_row[g])"),
    ("gemm.py", "out = A64 @ wdq64.T", "out = A64 @ wdq64[::-1].T"),
    ("gemm.py", "mag = np.abs(A64) @ np.abs(wdq64).T", "mag = np.abs(A64 @ wdq64.T)"),
    ("gemm.py", "mag = mag + np.abs(b)[None, :]", "mag = mag + b[None, :]"),
    ("gemm.py", "                s += p\n", "                s -= p\n"),
    ("check.py", "bound = rel * mag64 + abs_", "bound = rel * mag64"),
    ("check.py", '"mean_abs": float(diff.mean())', '"mean_abs": float(diff.max())'),
    ("check.py", "BF16_UNIT_ROUNDOFF = 2.0 ** -8", "BF16_UNIT_ROUNDOFF = 2.0 ** -6"),
    ("check.py", 'if out_dtype == "bf16":', 'if out_dtype == "never":'),
    ("check.py", "(np.sign(C64) == np.sign(out64))", "(np.sign(C64) != 0)"),
    ("check.py", "(np.abs(out64) + bound >= overflow)", "(np.abs(out64) >= 0)"),
    ("check.py", "F16_OVERFLOW = 65504.0 + 16.0", "F16_OVERFLOW = 65504.0"),
    ("ternary.py", "return [[tv * f16_value_exact(sb) for tv in row] for row, sb in zip(t, scale_bits)]",
     "return [[tv * f16_value_exact(sb) for tv in row[::-1]] for row, sb in zip(t, scale_bits)]"),
    ("ternary.py", "t = ternary_unpack_loop(codes, K)\n    return", "t = [[-v for v in r] for r in ternary_unpack_loop(codes, K)]\n    return"),
    ("rne.py", "        return s * f * 2.0 ** -133", "        return s * f * 2.0 ** -126"),
    ("rne.py", "    return s * (128 + f) * 2.0 ** (e - 134)", "    return s * (128 + f) * 2.0 ** (e - 133)"),
    ("rne.py", "    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16", "    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15"),
]


def _load_mutant(tmp_path, idx, fname, old, new):
    name = f"oracle_mutant_{idx}"
    dst = tmp_path / name
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("__pycache__", "*.c", "*.so"))
    p = dst / fname
    src = p.read_text()
    assert src.count(old) == 1, f"mutation anchor not unique in {fname}: {old!r}"
    p.write_text(src.replace(old, new))
    sys.path.insert(0, str(tmp_path))
    try:
        pkg = importlib.import_module(name)
        for sub in ("errors", "rne", "ternary", "w4", "w4asym", "gemm", "check"):
            importlib.import_module(f"{name}.{sub}")
    finally:
        sys.path.remove(str(tmp_path))
    return pkg


@pytest.mark.parametrize("idx", range(len(MUTATIONS)),
                         ids=[f"{m[0]}:{m[1].strip()[:40]}" for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, idx):
    fname, old, new = MUTATIONS[idx]
    mutant = _load_mutant(tmp_path, idx, fname, old, new)
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # the pin caught the planted mistake
            return
    pytest.fail(f"no pin catches mutation {fname}: {old!r} -> {new!r}")
