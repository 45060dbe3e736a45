"""W4A16 with per-group zero points and activation-order groups - the reference
definition (test infrastructure only).

What the pages fix
------------------
* [P2] section 5 (0), the GPTQ walk-through: the exporter writes INT4
  weights, a per-group scale and zero point, and optionally g_idx, the
  activation ordering of the input columns.
* [P2] section 5 (3): the layer holds a group zero-point parameter beside
  the group scale, group size 128; the packed weight is [d_out, d_in/8]
  (eight INT4 per INT32) and the scales [d_out, d_in/128].

Readings where the pages are silent
-----------------------------------
* Asymmetric min-max quantizer over each group's range widened to include 0:
  lo = min(0, min w), hi = max(0, max w), exact in fp64; scale
  s16 = RNE_binary16((hi - lo) / 15) (RANGE error if it overflows); zero point
  z = clamp(rint(-lo / s), 0, 15) and code q = clamp(rint(w / s) + z, 0, 15),
  both with s the stored binary16 value and round-half-even in fp64 (the
  quotient of a binary32 value by a binary16 one can neither create nor
  remove a tie).  A zero scale (all-zero group) gives z = 0 and q = 0.
* Dequantized weight (q - z) * s16.
* Zero points are stored one per byte: uint8 [N, K/128].
* Activation order: g_idx[k] in [0, K/128) names the group of input column k,
  and every group holds exactly 128 columns (else GROUP error).  The packed
  matrix stores the columns sorted by group, stably (ascending k within a
  group): packed column i is input column perm[i], so the groups are
  contiguous runs of 128, and codes, scales and zero points describe that
  packed order.  The product gathers the activations the same way:
  C = A[:, perm] @ dequant_packed^T = A @ dequant_original^T.
* Without g_idx, perm is the identity.
* Nibble order and words as the symmetric format (oracle.w4).
"""

import numpy as np

from .errors import OracleError
from .rne import f16_bits, f16_bits_exact, f16_value_exact, f16_values

BITS = 4
GROUP = 128
QMAX = 15
PER_WORD = 8
F16_INF_BITS = 0x7C00


def _rint(x: float) -> float:
    return float(round(x))  # Python rounds floats half to even


def order_from_g_idx(g_idx, K: int, group: int = GROUP):
    """Stable order of the input columns by group: perm (int32 [K])."""
    if g_idx is None:
        return np.arange(K, dtype=np.int32)
    g = np.asarray(g_idx).astype(np.int64).reshape(-1)
    G = K // group
    if g.shape[0] != K or np.any(g < 0) or np.any(g >= G):
        raise OracleError("GROUP", "g_idx must hold K group indices in [0, K/group)")
    if np.any(np.bincount(g, minlength=G) != group):
        raise OracleError("GROUP", "every group must hold exactly `group` columns")
    return np.argsort(g, kind="stable").astype(np.int32)


# ------------------------------------------------------------------ loop tier

def w4a_pack_loop(W, g_idx=None, group: int = GROUP):
    """W [N][K] -> (words [N][K/8] unsigned, scale bits [N][G], zeros [N][G], perm [K])."""
    rows = [[float(v) for v in r] for r in W]
    N = len(rows)
    K = len(rows[0]) if N else 0
    if N <= 0 or K <= 0 or K % group or group % PER_WORD:
        raise OracleError("SHAPE", f"N={N} K={K} group={group}")
    for r in rows:
        for v in r:
            if v != v or v in (float("inf"), float("-inf")):
                raise OracleError("NONFINITE")
    if g_idx is None:
        perm = list(range(K))
    else:
        G = K // group
        members = [[] for _ in range(G)]
        for k in range(K):
            gk = int(g_idx[k])
            if gk < 0 or gk >= G:
                raise OracleError("GROUP", "g_idx out of range")
            members[gk].append(k)
        for m in members:
            if len(m) != group:
                raise OracleError("GROUP", "every group must hold exactly `group` columns")
        perm = [k for m in members for k in m]
    words, scales, zeros = [], [], []
    for r in rows:
        packed = [r[perm[i]] for i in range(K)]
        q_row, s_row, z_row = [], [], []
        for g in range(K // group):
            chunk = packed[g * group:(g + 1) * group]
            lo, hi = 0.0, 0.0
            for v in chunk:
                if v < lo:
                    lo = v
                if v > hi:
                    hi = v
            sb = f16_bits_exact((hi - lo) / 15.0)
            if sb & 0x7FFF == F16_INF_BITS:
                raise OracleError("RANGE", "group scale overflows binary16")
            s = f16_value_exact(sb)
            if s == 0.0:
                z = 0
            else:
                z = int(min(max(_rint(-lo / s), 0), QMAX))
            s_row.append(sb)
            z_row.append(z)
            for v in chunk:
                if s == 0.0:
                    q = 0
                else:
                    q = int(min(max(_rint(v / s) + z, 0), QMAX))
                q_row.append(q)
        w_row = []
        for j in range(K // PER_WORD):
            word = 0
            for i in range(PER_WORD):
                word |= q_row[PER_WORD * j + i] << (BITS * i)
            w_row.append(word)
        words.append(w_row)
        scales.append(s_row)
        zeros.append(z_row)
    return words, scales, zeros, perm


def w4a_dequant_loop(words, scale_bits, zeros, perm, K, group: int = GROUP):
    """(q - z) * s as exact fp64 values [N][K], in the input column order."""
    out = []
    for w_row, s_row, z_row in zip(words, scale_bits, zeros):
        row = [0.0] * K
        for i in range(K):
            q = (w_row[i // PER_WORD] >> (BITS * (i % PER_WORD))) & 0xF
            g = i // group
            row[perm[i]] = (q - z_row[g]) * f16_value_exact(s_row[g])
        out.append(row)
    return out


# ----------------------------------------------------------------- numpy tier

def w4a_pack(W, g_idx=None, group: int = GROUP, row_block: int = 4096):
    """W float32 [N, K] -> (qweight int32 [N, K/8], scale bits uint16 [N, G],
    zeros uint8 [N, G], perm int32 [K])."""
    W = np.asarray(W)
    if W.ndim != 2 or W.dtype != np.float32:
        raise OracleError("SHAPE", f"weights must be 2-D float32, got {W.dtype} {W.shape}")
    N, K = W.shape
    if N <= 0 or K <= 0 or K % group or group % PER_WORD:
        raise OracleError("SHAPE", f"N={N} K={K} group={group}")
    if not np.isfinite(W).all():
        raise OracleError("NONFINITE")
    perm = order_from_g_idx(g_idx, K, group)
    G = K // group
    qweight = np.empty((N, K // PER_WORD), dtype=np.uint32)
    scale_bits = np.empty((N, G), dtype=np.uint16)
    zeros = np.empty((N, G), dtype=np.uint8)
    for r0 in range(0, N, row_block):
        w = W[r0:r0 + row_block][:, perm].astype(np.float64).reshape(-1, G, group)
        lo = np.minimum(w.min(axis=2), 0.0)
        hi = np.maximum(w.max(axis=2), 0.0)
        sb = f16_bits((hi - lo) / 15.0)
        if np.any(sb & 0x7FFF == F16_INF_BITS):
            raise OracleError("RANGE", "a group scale overflows binary16")
        s = f16_values(sb)
        with np.errstate(divide="ignore", invalid="ignore"):
            z = np.where(s == 0.0, 0.0, np.clip(np.rint(-lo / s), 0, QMAX))
            q = np.rint(w / s[:, :, None]) + z[:, :, None]
        q = np.where(s[:, :, None] == 0.0, 0.0, np.clip(q, 0, QMAX))
        q = q.astype(np.uint32).reshape(-1, K // PER_WORD, PER_WORD)
        word = np.zeros(q.shape[:2], dtype=np.uint32)
        for i in range(PER_WORD):
            word |= q[:, :, i] << np.uint32(BITS * i)
        qweight[r0:r0 + row_block] = word
        scale_bits[r0:r0 + row_block] = sb
        zeros[r0:r0 + row_block] = z.astype(np.uint8)
    return qweight.view(np.int32), scale_bits, zeros, perm


def w4a_unpack(qweight, K: int):
    """int32 words [N, K/8] -> uint8 codes in 0..15, [N, K], packed column order."""
    u = np.asarray(qweight).view(np.uint32)
    N = u.shape[0]
    if u.shape[1] * PER_WORD != K:
        raise OracleError("SHAPE", f"{u.shape[1]} words for K={K}")
    q = np.stack([(u >> np.uint32(BITS * i)) & np.uint32(0xF) for i in range(PER_WORD)], axis=2)
    return q.reshape(N, K).astype(np.uint8)


def w4a_dequant(qweight, scale_bits, zeros, K: int, perm=None, group: int = GROUP):
    """(q - z) * s as exact fp64 [N, K], in the input column order."""
    q = w4a_unpack(qweight, K).astype(np.float64)
    s = np.repeat(f16_values(scale_bits), group, axis=1)
    z = np.repeat(np.asarray(zeros).astype(np.float64), group, axis=1)
    packed = (q - z) * s
    if perm is None:
        return packed
    out = np.empty_like(packed)
    out[:, np.asarray(perm)] = packed
    return out


def w4a_dequant_f16_bits(qweight, scale_bits, zeros, K: int, perm=None, group: int = GROUP):
    """Dequantized weights rounded once to binary16 (bit patterns), input column order."""
    return f16_bits(w4a_dequant(qweight, scale_bits, zeros, K, perm, group))
