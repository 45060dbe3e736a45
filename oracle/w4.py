"""W4A16 symmetric int4 weights - the reference definition (test infrastructure only).

What the pages fix
------------------
* [P2] section 5 (1): the checkpoint's quantization config is 4 bits, group
  size 128, no activation reordering, symmetric.
* [P2] section 5 (3) and section 4.2: eight int4 values are packed into one
  int32 (packed factor 8), the packed weight is [d_out, d_in/8] and the group
  scales are [d_out, d_in/128].

Readings where the pages are silent
-----------------------------------
* Symmetric int4 with the fixed zero point 8: stored code q = r + 8 with
  r in [-8, 7]; dequantized weight (q - 8) * s.
* Group scale s = max|w| / 7 over the 128 weights of a group along K, computed
  in fp64 and rounded once to binary16 (RANGE error if it overflows).
* r = round-half-even(w / s16) in fp64 with the stored binary16 scale, then
  clamped to [-8, 7].  fp64 division of a binary32 weight by a binary16 scale
  can neither create nor remove a tie, so this equals rounding the exact
  quotient.  A zero scale (an all-zero group) gives r = 0 everywhere.
* Nibble i (bits 4i..4i+3) of word j of a row holds column 8j + i (low nibble
  first); words are stored as int32 bit patterns, scales row-major [N, K/128].
"""

import numpy as np

from .errors import OracleError
from .rne import f16_bits, f16_bits_exact, f16_value_exact, f16_values

BITS = 4
GROUP = 128
ZERO_POINT = 8
QMIN, QMAX = -8, 7
PER_WORD = 8
F16_INF_BITS = 0x7C00


def _round_half_even(x: float) -> float:
    return float(round(x))  # Python rounds floats half to even


# ------------------------------------------------------------------ loop tier

def w4_pack_loop(W, group: int = GROUP):
    """W [N][K] -> (words [N][K/8] as unsigned 32-bit ints, scale bits [N][K/group])."""
    rows = [[float(v) for v in r] for r in W]
    N = len(rows)
    K = len(rows[0]) if N else 0
    if N <= 0 or K <= 0 or K % group or group % PER_WORD:
        raise OracleError("SHAPE", f"N={N} K={K} group={group}")
    for r in rows:
        for v in r:
            if v != v or v in (float("inf"), float("-inf")):
                raise OracleError("NONFINITE")
    words, scales = [], []
    for r in rows:
        q_row = []
        s_row = []
        for g in range(K // group):
            chunk = r[g * group:(g + 1) * group]
            amax = 0.0
            for v in chunk:
                if abs(v) > amax:
                    amax = abs(v)
            sb = f16_bits_exact(amax / 7.0)
            if sb & 0x7FFF == F16_INF_BITS:
                raise OracleError("RANGE", "group scale overflows binary16")
            s_row.append(sb)
            s = f16_value_exact(sb)
            for v in chunk:
                if s == 0.0:
                    rv = 0
                else:
                    rv = int(_round_half_even(v / s))
                    rv = min(max(rv, QMIN), QMAX)
                q_row.append(rv + ZERO_POINT)
        w_row = []
        for j in range(K // PER_WORD):
            word = 0
            for i in range(PER_WORD):
                word |= q_row[PER_WORD * j + i] << (BITS * i)
            w_row.append(word)
        words.append(w_row)
        scales.append(s_row)
    return words, scales


def w4_unpack_loop(words, K):
    """Packed words -> codes q in 0..15, [N][K]."""
    out = []
    for w_row in words:
        q = []
        for col in range(K):
            q.append((w_row[col // PER_WORD] >> (BITS * (col % PER_WORD))) & 0xF)
        out.append(q)
    return out


def w4_dequant_loop(words, scale_bits, K, group: int = GROUP):
    """(q - 8) * s as exact fp64 values [N][K]."""
    q = w4_unpack_loop(words, K)
    return [[(qv - ZERO_POINT) * f16_value_exact(s_row[col // group])
             for col, qv in enumerate(q_row)] for q_row, s_row in zip(q, scale_bits)]


# ----------------------------------------------------------------- numpy tier

def w4_pack(W, group: int = GROUP, row_block: int = 4096):
    """W float32 [N, K] -> (qweight int32 [N, K/8], scale bits uint16 [N, K/group])."""
    W = np.asarray(W)
    if W.ndim != 2 or W.dtype != np.float32:
        raise OracleError("SHAPE", f"weights must be 2-D float32, got {W.dtype} {W.shape}")
    N, K = W.shape
    if N <= 0 or K <= 0 or K % group or group % PER_WORD:
        raise OracleError("SHAPE", f"N={N} K={K} group={group}")
    if not np.isfinite(W).all():
        raise OracleError("NONFINITE")
    G = K // group
    qweight = np.empty((N, K // PER_WORD), dtype=np.uint32)
    scale_bits = np.empty((N, G), dtype=np.uint16)
    for r0 in range(0, N, row_block):
        w = W[r0:r0 + row_block].astype(np.float64).reshape(-1, G, group)
        amax = np.abs(w).max(axis=2)
        sb = f16_bits(amax / 7.0)
        if np.any(sb & 0x7FFF == F16_INF_BITS):
            raise OracleError("RANGE", "a group scale overflows binary16")
        s = f16_values(sb)[:, :, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.rint(w / s)                   # np.rint rounds half to even
        r = np.where(s == 0.0, 0.0, np.clip(r, QMIN, QMAX))
        q = (r + ZERO_POINT).astype(np.uint32).reshape(-1, K // PER_WORD, PER_WORD)
        word = np.zeros(q.shape[:2], dtype=np.uint32)
        for i in range(PER_WORD):
            word |= q[:, :, i] << np.uint32(BITS * i)
        qweight[r0:r0 + row_block] = word
        scale_bits[r0:r0 + row_block] = sb
    return qweight.view(np.int32), scale_bits


def w4_unpack(qweight, K: int):
    """int32 words [N, K/8] -> uint8 codes q in 0..15, [N, K]."""
    u = np.asarray(qweight).view(np.uint32)
    N = u.shape[0]
    if u.shape[1] * PER_WORD != K:
        raise OracleError("SHAPE", f"{u.shape[1]} words for K={K}")
    q = np.stack([(u >> np.uint32(BITS * i)) & np.uint32(0xF) for i in range(PER_WORD)], axis=2)
    return q.reshape(N, K).astype(np.uint8)


def w4_dequant(qweight, scale_bits, K: int, group: int = GROUP):
    """(q - 8) * s as exact fp64 [N, K]."""
    q = w4_unpack(qweight, K).astype(np.float64) - ZERO_POINT
    s = np.repeat(f16_values(scale_bits), group, axis=1)
    return q * s


def w4_dequant_f16_bits(qweight, scale_bits, K: int, group: int = GROUP):
    """Dequantized weights rounded once to binary16 (bit patterns)."""
    return f16_bits(w4_dequant(qweight, scale_bits, K, group))
