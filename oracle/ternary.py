"""Ternary (2-bit) weight quantization - the reference definition (test infrastructure only).

What the pages fix
------------------
* [P1] section 1, tip: ternary quantization is a scaled sign function,
  w_t = sign(w) * (|w| > threshold).  (The comparison operator was lost in the
  page's text; we read a strict ``>``.)
* [P1] section 3.1: the threshold is ``mean(|w|) * 0.7`` (explicitly not the
  standard deviation); the scale is one fp16 value per output row; a packed
  byte holds four codes, field k of byte j (bits 2k..2k+1) is column 4j+k, and
  the code table is 00 -> -1, 01 -> 0, 10 -> +1.
* [P1] section 4, naive kernel: the value of a field is ``code - 1``.
* [P1] sections 3.2-3.3: a packed row is ceil(K/4) bytes (4096 -> 1024);
  using floor instead drops the last weights of a row.

Readings where the pages are silent (each also listed in the design notes)
-------------------------------------------------------------------------
* The mean is taken per output row (the scale is per row).
* Sums are fp64 and sequential in ascending column order, so a GPU lane per
  row can reproduce every keep decision bit for bit.
* thr = 0.7 * (S / K) in fp64, exactly this sequence of operations.
* scale = mean |w| over the kept entries of the row (fp64 sum / count), rounded
  once to binary16; a row with no kept entry (only an all-zero row) gets +0.
* A scale that rounds to infinity is a RANGE error; a non-finite weight is a
  NONFINITE error.
* Tail columns of a row whose K is not a multiple of 4 are padded with the
  zero code 01.
* Unpack rejects the unused field 11 (BAD_CODE); fields past column K-1 (the
  padding) are not examined.
"""

import numpy as np

from .errors import OracleError
from .rne import f16_bits, f16_bits_exact, f16_value_exact, f16_values

THRESHOLD_FACTOR = 0.7       # [P1] section 3.1
CODE_OF = {-1: 0, 0: 1, 1: 2}  # [P1] section 3.1 table: 00 -> -1, 01 -> 0, 10 -> +1
VALUE_OF = {0: -1, 1: 0, 2: 1}
CODES_PER_BYTE = 4
F16_INF_BITS = 0x7C00


def row_bytes(K: int) -> int:
    """Bytes in one packed row: ceil(K / 4) ([P1] sections 3.2 and 3.3)."""
    return (K + CODES_PER_BYTE - 1) // CODES_PER_BYTE


# ------------------------------------------------------------------ loop tier

def ternarize_row_loop(w_row):
    """One row: (list of ternary values, fp16 scale bit pattern).  Pure Python."""
    K = len(w_row)
    if K <= 0:
        raise OracleError("SHAPE", "K must be positive")
    vals = [float(v) for v in w_row]
    for v in vals:
        if v != v or v in (float("inf"), float("-inf")):
            raise OracleError("NONFINITE")
    s = 0.0
    for v in vals:              # sequential, ascending column order
        s += abs(v)
    thr = THRESHOLD_FACTOR * (s / K)
    t = []
    kept_sum = 0.0
    kept = 0
    for v in vals:
        a = abs(v)
        if a > thr:
            t.append(1 if v > 0 else -1)
            kept_sum += a
            kept += 1
        else:
            t.append(0)
    scale64 = kept_sum / kept if kept else 0.0
    bits = f16_bits_exact(scale64)
    if bits & 0x7FFF == F16_INF_BITS:
        raise OracleError("RANGE", f"scale {scale64!r} overflows binary16")
    return t, bits


def pack_codes_loop(t_row, K):
    """Pack one row of ternary values into ceil(K/4) bytes (tail padded with 01)."""
    out = []
    for j in range(row_bytes(K)):
        byte = 0
        for k in range(CODES_PER_BYTE):
            col = CODES_PER_BYTE * j + k
            code = CODE_OF[t_row[col]] if col < K else CODE_OF[0]
            byte |= code << (2 * k)
        out.append(byte)
    return out


def ternary_pack_loop(W):
    """W: sequence of N rows of K weights -> (codes [N][ceil(K/4)], scale bits [N])."""
    rows = [list(r) for r in W]
    if not rows:
        raise OracleError("SHAPE", "N must be positive")
    K = len(rows[0])
    for r in rows:
        if len(r) != K:
            raise OracleError("SHAPE", "ragged rows")
    # a non-finite weight anywhere rejects the whole matrix
    for r in rows:
        for v in r:
            v = float(v)
            if v != v or v in (float("inf"), float("-inf")):
                raise OracleError("NONFINITE")
    codes, scales = [], []
    for r in rows:
        t, sb = ternarize_row_loop(r)
        codes.append(pack_codes_loop(t, K))
        scales.append(sb)
    return codes, scales


def ternary_unpack_loop(codes, K):
    """Packed rows -> ternary values [N][K]; BAD_CODE on a field 11 inside K."""
    out = []
    for row in codes:
        t = []
        for col in range(K):
            byte = row[col // CODES_PER_BYTE]
            field = (byte >> (2 * (col % CODES_PER_BYTE))) & 0x3
            if field not in VALUE_OF:
                raise OracleError("BAD_CODE", f"field 0b11 at column {col}")
            t.append(VALUE_OF[field])
        out.append(t)
    return out


def ternary_dequant_loop(codes, scale_bits, K):
    """Dequantized weights t * scale as fp64 values [N][K] (exact)."""
    t = ternary_unpack_loop(codes, K)
    return [[tv * f16_value_exact(sb) for tv in row] for row, sb in zip(t, scale_bits)]


# ----------------------------------------------------------------- numpy tier

def _check_matrix(W):
    W = np.asarray(W)
    if W.ndim != 2 or W.shape[0] <= 0 or W.shape[1] <= 0:
        raise OracleError("SHAPE", f"bad shape {W.shape}")
    if W.dtype != np.float32:
        raise OracleError("SHAPE", f"weights must be float32, got {W.dtype}")
    if not np.isfinite(W).all():
        raise OracleError("NONFINITE")
    return W


def ternarize(W, row_block: int = 4096, stats: dict = None):
    """Vectorized: W float32 [N, K] -> (t int8 [N, K], scale bits uint16 [N]).

    Same arithmetic and order as ``ternarize_row_loop``: ``np.cumsum`` along a
    row adds sequentially, so its last column equals the loop's running sum.
    If ``stats`` is a dict it receives the per-row fp64 values ``S`` (sum of
    |w|), ``thr``, ``kept_sum`` and ``kept``.
    """
    W = _check_matrix(W)
    N, K = W.shape
    t = np.empty((N, K), dtype=np.int8)
    scale_bits = np.empty(N, dtype=np.uint16)
    if stats is not None:
        for key in ("S", "thr", "kept_sum"):
            stats[key] = np.empty(N, dtype=np.float64)
        stats["kept"] = np.empty(N, dtype=np.int64)
    for r0 in range(0, N, row_block):
        w = W[r0:r0 + row_block].astype(np.float64)
        a = np.abs(w)
        s = np.cumsum(a, axis=1)[:, -1]
        thr = THRESHOLD_FACTOR * (s / K)
        keep = a > thr[:, None]
        t[r0:r0 + row_block] = np.where(keep, np.where(w > 0, 1, -1), 0)
        kept = keep.sum(axis=1)
        kept_sum = np.cumsum(np.where(keep, a, 0.0), axis=1)[:, -1]
        scale64 = np.where(kept > 0, kept_sum / np.maximum(kept, 1), 0.0)
        sb = f16_bits(scale64)
        if np.any(sb & 0x7FFF == F16_INF_BITS):
            raise OracleError("RANGE", "a row scale overflows binary16")
        scale_bits[r0:r0 + row_block] = sb
        if stats is not None:
            sl = slice(r0, r0 + row_block)
            stats["S"][sl], stats["thr"][sl] = s, thr
            stats["kept_sum"][sl], stats["kept"][sl] = kept_sum, kept
    return t, scale_bits


def pack_codes(t):
    """int8 ternary values [N, K] -> uint8 codes [N, ceil(K/4)] (tail code 01)."""
    t = np.asarray(t)
    N, K = t.shape
    rb = row_bytes(K)
    c = np.full((N, rb * CODES_PER_BYTE), CODE_OF[0], dtype=np.uint8)
    c[:, :K] = (t + 1).astype(np.uint8)        # 00 -> -1, 01 -> 0, 10 -> +1
    c = c.reshape(N, rb, CODES_PER_BYTE)
    out = np.zeros((N, rb), dtype=np.uint8)
    for k in range(CODES_PER_BYTE):
        out |= c[:, :, k] << np.uint8(2 * k)
    return out


def ternary_pack(W):
    """W float32 [N, K] -> (codes uint8 [N, ceil(K/4)], scale bits uint16 [N])."""
    t, sb = ternarize(W)
    return pack_codes(t), sb


def ternary_unpack(codes, K: int):
    """uint8 codes [N, ceil(K/4)] -> int8 ternary values [N, K]; BAD_CODE on 11."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, rb = codes.shape
    if rb != row_bytes(K):
        raise OracleError("SHAPE", f"row of {rb} bytes for K={K}")
    fields = np.stack([(codes >> np.uint8(2 * k)) & np.uint8(3)
                       for k in range(CODES_PER_BYTE)], axis=2).reshape(N, rb * CODES_PER_BYTE)[:, :K]
    if np.any(fields == 3):
        raise OracleError("BAD_CODE")
    return fields.astype(np.int8) - 1


def ternary_dequant(codes, scale_bits, K: int):
    """Dequantized weights t * scale as fp64 [N, K] (exact products)."""
    t = ternary_unpack(codes, K).astype(np.float64)
    return t * f16_values(scale_bits)[:, None]


def ternary_dequant_f16_bits(codes, scale_bits, K: int):
    """Dequantized weights as binary16 bit patterns [N, K].

    t * scale is exact in binary16 (+scale, -scale or zero); IEEE signs apply,
    so -1 * (+0) is -0 and 0 * scale is +0.
    """
    return f16_bits(ternary_dequant(codes, scale_bits, K))
