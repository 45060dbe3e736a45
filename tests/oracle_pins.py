"""Pins that tie the oracle to something other than itself.

Each ``pin_*`` function takes an oracle package object ``o`` (with submodules
``rne``, ``ternary``, ``w4``, ``gemm``, ``check``) and raises AssertionError
when the oracle disagrees with a fact the pages or the mathematics fix:
values the pages print (``tests/golden``), hand-derived examples, closed
forms, brute force over tiny inputs, exact rational arithmetic, or library
routines for the special cases that reduce to them.

``test_oracle_pins.py`` runs every pin on the real oracle; the mutation test
runs them on copies of the oracle with one plausible mistake planted each and
requires that some pin fails.
"""

import itertools
import math
import os
import random
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ------------------------------------------------------------------ rounding

def _f16_all_finite_bits():
    b = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 10) & 0x1F
    return b[exp != 31]


def pin_f16_exact_roundtrip_all_patterns(o):
    """Every finite binary16 value converts back to its own bit pattern."""
    for b in _f16_all_finite_bits()[::7].tolist() + [0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF]:
        v = float(np.uint16(b).view(np.float16))
        got = o.rne.f16_bits_exact(v)
        assert got == b, f"f16 exact {b:#06x} -> {got:#06x}"
        assert o.rne.f16_value_exact(b) == v or (v != v)


def pin_f16_numpy_tier_all_patterns(o):
    """numpy tier equals the library cast on every finite pattern and all midpoints."""
    b = _f16_all_finite_bits()
    v = b.view(np.float16).astype(np.float64)
    assert np.array_equal(o.rne.f16_bits(v), b)
    assert np.array_equal(o.rne.f16_values(b), v)


def pin_f16_hand_values(o):
    """Values derived by hand from the binary16 definition."""
    cases = {
        1.0: 0x3C00, -2.0: 0xC000, 65504.0: 0x7BFF, 65519.99: 0x7BFF, 65520.0: 0x7C00,
        2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000, 1.5 * 2.0 ** -25: 0x0001, 2.0 ** -14: 0x0400,
        0.25: 0x3400, 11.0: 0x4980, 11 * 2.0 ** -9: 0x2580,
        1 + 2.0 ** -11: 0x3C00,                   # tie -> even (1.0)
        1 + 3 * 2.0 ** -11: 0x3C02,               # tie -> even (1 + 2^-9)
        1 + 2.0 ** -11 + 2.0 ** -40: 0x3C01,      # just above the tie: rounded once, up
        -0.0: 0x8000, float("inf"): 0x7C00,
    }
    for x, want in cases.items():
        assert o.rne.f16_bits_exact(x) == want, f"exact {x!r}"
        assert int(o.rne.f16_bits(np.float64(x))) == want, f"numpy {x!r}"


def pin_f16_random_vs_fraction(o):
    """Random fp64 values and near-midpoints against rounding of the exact rational."""
    rng = np.random.default_rng(11)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-28, 17, 3000)))
    b = _f16_all_finite_bits()
    v = b.view(np.float16).astype(np.float64)
    pos = np.sort(v[v > 0])[::37]
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        xs += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)]
    for x in xs:
        x = float(x)
        want = _round_to_grid_f16(Fraction(x))
        got = o.rne.f16_bits_exact(x)
        assert got == want, f"{x!r}: {got:#06x} vs {want:#06x}"
        assert int(o.rne.f16_bits(np.float64(x))) == want


def _round_to_grid_f16(a: Fraction) -> int:
    """Independent RNE: scan the sorted list of binary16 values for the nearest."""
    s = 0x8000 if a < 0 else 0
    a = abs(a)
    if a >= Fraction(65520):
        return s | 0x7C00
    # the value grid of non-negative finite binary16, indexable by bit pattern
    lo, hi = 0, 0x7BFF
    while hi - lo > 1:                      # largest pattern with value <= a
        mid = (lo + hi) // 2
        if _f16_frac(mid) <= a:
            lo = mid
        else:
            hi = mid
    if _f16_frac(hi) <= a:
        lo = hi
    if lo == 0x7BFF:
        return s | lo
    d_lo = a - _f16_frac(lo)
    d_hi = _f16_frac(lo + 1) - a
    if d_lo < d_hi or (d_lo == d_hi and lo % 2 == 0):
        return s | lo
    return s | (lo + 1)


def _f16_frac(b: int) -> Fraction:
    e = (b >> 10) & 0x1F
    f = b & 0x3FF
    if e == 0:
        return Fraction(f, 2 ** 24)
    return Fraction(1024 + f) * Fraction(2) ** (e - 25)


def pin_bf16_vs_torch_and_hand(o):
    """bf16 rounding: hand ties, and torch's CPU cast from binary32."""
    import torch
    hand = {1.0: 0x3F80, 1 + 2.0 ** -8: 0x3F80, 1 + 3 * 2.0 ** -8: 0x3F82,
            -0.25: 0xBE80, 11 * 2.0 ** -9: 0x3CB0}
    for x, want in hand.items():
        assert o.rne.bf16_bits_exact(x) == want, x
        assert int(o.rne.bf16_bits(np.float64(x))) == want, x
    rng = np.random.default_rng(5)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, 20000))).astype(np.float32)
    f = np.concatenate([f, np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, 3.4e38, -1e-40])])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.rne.bf16_bits(f.astype(np.float64)), ref)
    for x, r in zip(f[::50].tolist(), ref[::50].tolist()):
        assert o.rne.bf16_bits_exact(x) == r, x


# ------------------------------------------------------------------ ternary

def pin_code_table_from_pages(o):
    """The code table and bit order the pages print (golden fixture)."""
    rows = _golden_lines("ternary_code_table.txt")
    table = {int(r[0], 2): int(r[1]) for r in rows if len(r) == 2 and set(r[0]) <= {"0", "1"}}
    assert table == {0: -1, 1: 0, 2: 1}
    # one byte per valid 4-code combination; field k of the byte is column k
    for t in itertools.product((-1, 0, 1), repeat=4):
        byte = sum(({v: c for c, v in table.items()}[tv]) << (2 * k) for k, tv in enumerate(t))
        codes = np.array([[byte]], dtype=np.uint8)
        got = o.ternary.ternary_unpack(codes, 4)[0].tolist()
        assert got == list(t), (byte, got, t)
        assert o.ternary.ternary_unpack_loop([[byte]], 4)[0] == list(t)


def pin_unpack_rejects_unused_field(o):
    """The 175 byte values with a 0b11 field are rejected; the 81 others decode."""
    ok = 0
    for byte in range(256):
        has11 = any(((byte >> (2 * k)) & 3) == 3 for k in range(4))
        try:
            o.ternary.ternary_unpack(np.array([[byte]], dtype=np.uint8), 4)
            rejected = False
        except o.OracleError as e:
            rejected = e.kind == "BAD_CODE"
        assert rejected == has11, byte
        ok += not has11
    assert ok == 81


def pin_row_bytes_from_pages(o):
    """ceil(K/4) bytes per row; the pages print 4096 -> 1024."""
    for K, rb in ((int(a), int(b)) for a, b in _golden_lines("ternary_layout.txt")):
        assert o.ternary.row_bytes(K) == rb
    for K in range(1, 40):
        assert o.ternary.row_bytes(K) == -(-K // 4)
        W = np.full((2, K), 0.01, dtype=np.float32)
        codes, _ = o.ternary.ternary_pack(W)
        assert codes.shape == (2, -(-K // 4))


def pin_threshold_constant_from_pages(o):
    rows = _golden_lines("ternary_threshold.txt")
    assert rows == [["mean_abs", "0.7"]]
    assert o.ternary.THRESHOLD_FACTOR == 0.7


def pin_worked_example(o):
    """Hand-derived: w = [0.1, -0.2, 0.01, 0.3] (fp32).

    mean|w| = 0.1525 (fp32 inputs: S = 0.6100000161677599), threshold
    0.7 * mean = 0.10675000282935798.  Kept: -0.2 and 0.3 (0.1 and 0.01 are
    below).  Codes [01, 00, 01, 10] -> byte 0b10_01_00_01 = 0x91.  Scale =
    mean of the kept magnitudes = 0.25000000745 -> binary16 0.25 = 0x3400.
    """
    W = np.array([[0.1, -0.2, 0.01, 0.3]], dtype=np.float32)
    codes, sb = o.ternary.ternary_pack(W)
    assert codes.tolist() == [[0x91]] and sb.tolist() == [0x3400]
    c2, s2 = o.ternary.ternary_pack_loop(W.tolist())
    assert c2 == [[0x91]] and s2 == [0x3400]


def pin_strict_threshold(o):
    """Hand-derived: a weight exactly at the threshold is dropped (strict >).

    Row [7, 11, 11, 11] * 2^-9: mean 10 * 2^-9; 0.7 * 10 in fp64 is the exact
    tie 7 - 2^-51 between two doubles and rounds (to even) to exactly 7, so
    the threshold equals the first weight.  Strict: codes [01, 10, 10, 10] =
    0xA9, scale 11 * 2^-9 = 0x2580.  With a sign flip on two weights:
    [-7, 11, -11, 11] -> [01, 10, 00, 10] = 0x89, same scale.
    """
    for row, byte in (([7, 11, 11, 11], 0xA9), ([-7, 11, -11, 11], 0x89)):
        W = (np.array([row], dtype=np.float64) * 2.0 ** -9).astype(np.float32)
        codes, sb = o.ternary.ternary_pack(W)
        assert codes.tolist() == [[byte]] and sb.tolist() == [0x2580], (codes, sb)
        c2, s2 = o.ternary.ternary_pack_loop(W.tolist())
        assert c2 == [[byte]] and s2 == [0x2580]


def pin_brute_force_roundtrip(o):
    """pack(s * t) == (t, s) for every t in {-1,0,1}^K, K <= 8, fp16 scales s.

    For such a row every kept magnitude is s and the threshold is
    0.7 * cnt * s / K < s, so exactly the nonzero entries are kept with their
    signs, and the scale (cnt * s / cnt) is s.  An all-zero row gives codes 01
    and scale +0.
    """
    for K in (1, 3, 4, 5, 8):
        T = np.array(list(itertools.product((-1, 0, 1), repeat=K)), dtype=np.int8)
        for s in (0.25, 0.0236968994140625, 2.0 ** -20, 60000.0):
            W = (T.astype(np.float64) * s).astype(np.float32)
            codes, sb = o.ternary.ternary_pack(W)
            t_back = o.ternary.ternary_unpack(codes, K)
            assert np.array_equal(t_back, T), (K, s)
            nz = np.any(T != 0, axis=1)
            want = np.where(nz, np.float16(s).view(np.uint16), 0)
            assert np.array_equal(sb, want), (K, s)
            if K <= 5 and s == 0.25:
                c2, s2 = o.ternary.ternary_pack_loop(W.tolist())
                assert np.array_equal(np.array(c2, dtype=np.uint8), codes)
                assert s2 == sb.tolist()


def pin_tail_padding_and_no_unused_code(o):
    """Ragged K: padded fields are 01; no 0b11 field is ever emitted."""
    rng = np.random.default_rng(3)
    for K in (1, 2, 3, 5, 6, 7, 13, 255, 257):
        W = rng.normal(0, 0.02, (9, K)).astype(np.float32)
        codes, _ = o.ternary.ternary_pack(W)
        fields = np.stack([(codes >> (2 * k)) & 3 for k in range(4)], axis=2).reshape(9, -1)
        assert not np.any(fields == 3)
        assert np.all(fields[:, K:] == 1)


def pin_sequential_sums(o):
    """Threshold and scale sums run sequentially in ascending column order.

    On wide-range data the pairwise sum numpy's ``sum`` uses differs from the
    running sum on most rows; the oracle's row statistics must equal running
    sums bit for bit, and both tiers must take the same decisions.
    """
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((64, 997)) * np.exp2(rng.integers(-24, 8, (64, 997)))).astype(np.float32)
    st = {}
    t_np, s_np = o.ternary.ternarize(W, stats=st)
    differs = 0
    for n in range(W.shape[0]):
        a = [abs(float(v)) for v in W[n]]
        run = 0.0
        for v in a:
            run += v
        assert st["S"][n] == run, n
        differs += run != float(np.sum(np.array(a)))
        thr = 0.7 * (run / len(a))
        kept_run = 0.0
        for v in a:
            if v > thr:
                kept_run += v
        assert st["thr"][n] == thr and st["kept_sum"][n] == kept_run, n
        t_loop, s_loop = o.ternary.ternarize_row_loop(W[n].tolist())
        assert t_loop == t_np[n].tolist() and s_loop == int(s_np[n]), n
    assert differs > 10      # the data does separate the two summation orders


def pin_idempotent_and_closed_form_stats(o):
    """pack(dequant(pack(W))) == pack(W); kept fraction and mean scale match
    the closed forms for W ~ N(0, s^2): P(|w| > 0.7 s sqrt(2/pi)) and
    E[|w| | kept] / s, from scipy's normal distribution."""
    from scipy.stats import norm
    from synth import weights
    W = weights(512, 4096, seed=99)
    codes, sb = o.ternary.ternary_pack(W)
    wdq = o.ternary.ternary_dequant(codes, sb, 4096).astype(np.float32)
    c2, s2 = o.ternary.ternary_pack(wdq)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sb)
    t = o.ternary.ternary_unpack(codes, 4096)
    c = 0.7 * math.sqrt(2 / math.pi)
    frac = float(np.mean(t != 0))
    assert abs(frac - 2 * (1 - norm.cdf(c))) < 0.003, frac
    ratio = float(np.mean(o.rne.f16_values(sb))) / 0.02
    assert abs(ratio - norm.pdf(c) / (1 - norm.cdf(c))) < 0.003, ratio


def pin_pack_errors(o):
    W = np.full((3, 8), 0.1, dtype=np.float32)
    for bad in (np.nan, np.inf, -np.inf):
        W2 = W.copy()
        W2[1, 5] = bad
        for f in (o.ternary.ternary_pack, lambda x: o.ternary.ternary_pack_loop(x.tolist())):
            try:
                f(W2)
                raise AssertionError("non-finite accepted")
            except o.OracleError as e:
                assert e.kind == "NONFINITE"
    big = np.full((1, 8), 70000.0, dtype=np.float32)       # scale 70000 overflows binary16
    for f in (o.ternary.ternary_pack, lambda x: o.ternary.ternary_pack_loop(x.tolist())):
        try:
            f(big)
            raise AssertionError("overflowing scale accepted")
        except o.OracleError as e:
            assert e.kind == "RANGE"
    ok = np.full((1, 8), 65504.0, dtype=np.float32)
    assert o.ternary.ternary_pack(ok)[1].tolist() == [0x7BFF]


def pin_dequant_signs(o):
    """-1 * (+0) is -0 in binary16; 0 * s is +0; +-1 * s is +-s."""
    # a scale that underflows binary16 to +0 with kept entries of both signs
    W = np.array([[1e-9, -1e-9, 0.0, 1e-9]], dtype=np.float32)
    codes, sb = o.ternary.ternary_pack(W)
    assert sb.tolist() == [0]
    bits = o.ternary.ternary_dequant_f16_bits(codes, sb, 4)
    assert bits.tolist() == [[0x0000, 0x8000, 0x0000, 0x0000]]
    W = np.array([[0.3, -0.3, 0.0, 0.3]], dtype=np.float32)
    codes, sb = o.ternary.ternary_pack(W)
    s = int(sb[0])
    assert o.ternary.ternary_dequant_f16_bits(codes, sb, 4).tolist() == [[s, s | 0x8000, 0, s]]


# ----------------------------------------------------------------------- W4

def pin_w4_format_from_pages(o):
    kv = dict(_golden_lines("w4a16_format.txt"))
    assert int(kv["bits"]) == o.w4.BITS and int(kv["group_size"]) == o.w4.GROUP
    assert int(kv["packed_factor"]) == o.w4.PER_WORD == 32 // o.w4.BITS
    assert kv["sym"] == "true" and o.w4.ZERO_POINT == 8
    W = np.random.default_rng(0).normal(0, 0.02, (6, 384)).astype(np.float32)
    q, s = o.w4.w4_pack(W)
    assert q.shape == (6, 384 // 8) and q.dtype == np.int32
    assert s.shape == (6, 384 // 128) and s.dtype == np.uint16


def pin_w4_hand_words(o):
    """Hand-derived nibble order: a group whose weights are r * s with r the
    repeating pattern -7..7, 0 (s a binary16 value, so max|w| / 7 = s exactly)
    has codes q = r + 8 = 1..15, 8, and words 0x87654321, 0x8FEDCBA9."""
    s = 0.0234375  # 3 * 2^-7, exact in binary16
    r = np.tile(np.array(list(range(-7, 8)) + [0]), 8)  # 128 values
    W = (r.astype(np.float64) * s).astype(np.float32)[None, :]
    q, sb = o.w4.w4_pack(W)
    words = q.view(np.uint32)[0].tolist()
    assert words == [0x87654321, 0x8FEDCBA9] * 8, [hex(w) for w in words[:2]]
    assert sb.tolist() == [[int(np.float16(s).view(np.uint16))]]
    wl, sl = o.w4.w4_pack_loop(W.tolist())
    assert wl[0] == words and sl == sb.tolist()
    assert o.w4.w4_unpack(q, 128)[0].tolist() == (r + 8).tolist()


def pin_w4_vs_fraction(o):
    """Codes equal round-half-even of the exact quotient w / s16 (Fraction),
    clamped to [-8, 7], including constructed exact ties (k + 1/2) * s16."""
    rng = np.random.default_rng(21)
    for trial in range(40):
        w = (rng.standard_normal(128) * 10.0 ** rng.integers(-6, 3)).astype(np.float32)
        if trial % 2:
            s16 = np.float16(np.abs(w.astype(np.float64)).max() / 7.0)
            w = np.clip(w, -6.9 * np.float64(s16), 6.9 * np.float64(s16)).astype(np.float32)
            ks = rng.integers(-7, 7, 40)
            w[:40] = ((ks + 0.5) * np.float64(s16)).astype(np.float32)   # exact ties
            w[40] = np.float32(7 * np.float64(s16))       # max|w| = 7 * s16 keeps s16
            assert sum(Fraction(float(v)) / Fraction(float(s16)) % 1 == Fraction(1, 2) for v in w) >= 40
        q, sb = o.w4.w4_pack(w[None, :])
        s = Fraction(float(np.uint16(sb[0, 0]).view(np.float16)))
        assert s == Fraction(float(np.float16(np.abs(w.astype(np.float64)).max() / 7.0)))
        codes = o.w4.w4_unpack(q, 128)[0]
        for k in range(128):
            want = 0 if s == 0 else max(-8, min(7, round(Fraction(float(w[k])) / s)))
            assert int(codes[k]) == want + 8, (trial, k, float(w[k]), float(s))


def pin_w4_closed_form_and_idempotent(o):
    """The element at max|w| gets |q - 8| = 7; normal-range codes lie in 1..15;
    pack(dequant(pack(W))) == pack(W) (the new max is 7 * s16, so s16 repeats)."""
    from synth import weights
    W = weights(64, 1024, seed=5)
    q, sb = o.w4.w4_pack(W)
    codes = o.w4.w4_unpack(q, 1024).astype(np.int64).reshape(64, 8, 128)
    arg = np.abs(W.reshape(64, 8, 128)).argmax(axis=2)
    at_max = np.take_along_axis(codes, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(at_max - 8) == 7)
    assert codes.min() >= 1 and codes.max() <= 15
    wdq = o.w4.w4_dequant(q, sb, 1024).astype(np.float32)
    q2, s2 = o.w4.w4_pack(wdq)
    assert np.array_equal(q2, q) and np.array_equal(s2, sb)
    wl, sl = o.w4.w4_pack_loop(W[:2].tolist())
    assert np.array_equal(np.array(wl, dtype=np.uint32), q[:2].view(np.uint32))
    assert sl == sb[:2].tolist()
    dl = o.w4.w4_dequant_loop(wl, sl, 1024)
    assert np.array_equal(np.array(dl), o.w4.w4_dequant(q[:2], sb[:2], 1024))


def pin_w4_errors_and_zero_group(o):
    W = np.zeros((1, 256), dtype=np.float32)
    W[0, 200] = 0.5
    q, sb = o.w4.w4_pack(W)
    assert o.w4.w4_unpack(q, 256)[0, :128].tolist() == [8] * 128 and sb[0, 0] == 0
    assert int(o.w4.w4_unpack(q, 256)[0, 200]) == 15
    W2 = np.full((1, 128), 5e5, dtype=np.float32)   # 5e5 / 7 overflows binary16
    try:
        o.w4.w4_pack(W2)
        raise AssertionError("overflow accepted")
    except o.OracleError as e:
        assert e.kind == "RANGE"
    # Hand-derived clamp case: max|w| = 9.8 * 2^-24, so max|w| / 7 = 1.4 * 2^-24
    # rounds to the subnormal scale 2^-24 (pattern 0x0001); then w / s = -9.8
    # rounds to -10 and clamps to -8 (code 0), +9.8 clamps to +7 (code 15),
    # and 2^-24 * 2.5 is a tie that rounds to 2 (code 10).
    W4 = np.zeros((1, 128), dtype=np.float32)
    W4[0, :3] = np.array([-9.8, 9.8, 2.5]) * 2.0 ** -24
    q, sb = o.w4.w4_pack(W4)
    assert sb.tolist() == [[0x0001]]
    assert o.w4.w4_unpack(q, 128)[0, :4].tolist() == [0, 15, 10, 8]
    wl, sl = o.w4.w4_pack_loop(W4.tolist())
    assert wl == q.view(np.uint32).tolist() and sl == sb.tolist()
    W3 = np.zeros((1, 128), dtype=np.float32)
    W3[0, 3] = np.nan
    try:
        o.w4.w4_pack(W3)
        raise AssertionError("NaN accepted")
    except o.OracleError as e:
        assert e.kind == "NONFINITE"


# --------------------------------------------------------------------- GEMM

def pin_gemm_hand_example(o):
    """Hand-computed: A = [[1, 2], [3, 4]], W = [[1, 0], [0, -1], [1, 1]]:
    C = A W^T = [[1, -2, 3], [3, -4, 7]]; mag = [[1, 2, 3], [3, 4, 7]]."""
    A = np.array([[1.0, 2.0], [3.0, 4.0]])
    Wd = np.array([[1.0, 0.0], [0.0, -1.0], [1.0, 1.0]])
    out, mag = o.gemm.gemm_ref64(A, Wd)
    assert out.tolist() == [[1, -2, 3], [3, -4, 7]] and mag.tolist() == [[1, 2, 3], [3, 4, 7]]
    out, mag = o.gemm.gemm_ref64(A, Wd, bias64=np.array([0.5, -1.0, 0.0]))
    assert out.tolist() == [[1.5, -3, 3], [3.5, -5, 7]] and mag.tolist() == [[1.5, 3, 3], [3.5, 5, 7]]
    lo, lm = o.gemm.gemm_ref64_loop(A.tolist(), Wd.tolist(), [0.5, -1.0, 0.0])
    assert lo == out.tolist() and lm == mag.tolist()


def pin_gemm_vs_exact_rational(o):
    """fp64 product against exact Fraction dot products on tiny random inputs."""
    rng = np.random.default_rng(8)
    A = rng.standard_normal((3, 37)).astype(np.float16).astype(np.float64)
    Wd = (rng.integers(-1, 2, (5, 37)) * 0.0234375)
    out, mag = o.gemm.gemm_ref64(A, Wd)
    for m in range(3):
        for n in range(5):
            ex = sum(Fraction(float(A[m, k])) * Fraction(float(Wd[n, k])) for k in range(37))
            exm = sum(abs(Fraction(float(A[m, k])) * Fraction(float(Wd[n, k]))) for k in range(37))
            assert abs(Fraction(out[m, n]) - ex) <= Fraction(1, 10 ** 12) * (exm + 1)
            assert abs(Fraction(mag[m, n]) - exm) <= Fraction(1, 10 ** 12) * (exm + 1)


def pin_gemm_ones_and_one_hot(o):
    """All-ones activation: out[n] = scale[n] * (#plus - #minus), counted from
    the packed bytes directly.  One-hot e_k: out[n] = wdq[n, k] exactly."""
    from synth import weights
    W = weights(64, 256, seed=17)
    codes, sb = o.ternary.ternary_pack(W)
    plus = np.zeros(64)
    minus = np.zeros(64)
    for n in range(64):
        for byte in codes[n].tolist():
            for k in range(4):
                f = (byte >> (2 * k)) & 3
                plus[n] += f == 2
                minus[n] += f == 0
    wdq = o.ternary.ternary_dequant(codes, sb, 256)
    out, _ = o.gemm.gemm_ref64(np.ones((1, 256)), wdq)
    s = sb.view(np.float16).astype(np.float64)
    assert np.array_equal(out[0], s * (plus - minus))
    for k in (0, 1, 127, 255):
        e = np.zeros((1, 256))
        e[0, k] = 1.0
        out, _ = o.gemm.gemm_ref64(e, wdq)
        assert np.array_equal(out[0], wdq[:, k])


def pin_tolerance_check(o):
    """The verdict: finite and |C - ref| <= 2e-3 * mag + 1e-3 element-wise."""
    ref = np.array([[1.0, -2.0]])
    mag = np.array([[10.0, 100.0]])
    ok, st = o.check.tolerance_ok(np.array([[1.0 + 0.021, -2.0 - 0.2009]]), ref, mag)
    assert ok, st
    ok, _ = o.check.tolerance_ok(np.array([[1.0 + 0.0211, -2.0]]), ref, mag)
    assert not ok
    ok, st = o.check.tolerance_ok(np.array([[np.nan, -2.0]]), ref, mag)
    assert not ok and not st["finite"]
    # bf16 outputs: the exact value 2 + 2^-7 (mag 2 + 2^-7) is a tie between the
    # bf16 neighbours 2 and 2 + 2^-6; either is a correct rounding, off by 2^-7,
    # which exceeds 2e-3 * mag + 1e-3 = 0.00504 but not the added 2^-8 * |out|.
    x = 2 + 2.0 ** -7
    ok, _ = o.check.tolerance_ok(np.array([[2.0]]), np.array([[x]]), np.array([[x]]))
    assert not ok
    for c in (2.0, 2 + 2.0 ** -6):
        ok, st = o.check.tolerance_ok(np.array([[c]]), np.array([[x]]), np.array([[x]]), out_dtype="bf16")
        assert ok, st
    ok, _ = o.check.tolerance_ok(np.array([[2.0 - 2.0 ** -6]]), np.array([[x]]), np.array([[x]]), out_dtype="bf16")
    assert not ok
    qc = o.check.quant_check(np.array([1.0, 2.0]), np.array([1.0, 2.5]), atol=0.1, rtol=0.1)
    assert qc == {"ok": False, "max_abs": 0.5, "mean_abs": 0.25, "finite": True}


def pin_ternary_dequant_loop(o):
    """The loop tier's dequant: s16 * t for every row of every sign pattern
    (brute force over 3^6 rows of K = 6, scales 0.25, 3 and a subnormal),
    the same values as the numpy tier, and IEEE zeros of the form +0."""
    import itertools
    K = 6
    for s in (0.25, 3.0, 2.0 ** -20):
        rows = np.array(list(itertools.product((-1, 0, 1), repeat=K)), dtype=np.float64)
        rows = rows[np.any(rows != 0, axis=1)]
        W = (rows * s).astype(np.float32)
        codes, sb = o.ternary.ternary_pack(W)
        loop = np.array(o.ternary.ternary_dequant_loop(codes.tolist(), sb.tolist(), K))
        s16 = o.rne.f16_value_exact(int(sb[0]))
        assert np.all(sb == sb[0]) and s16 == float(np.float16(s))
        assert np.array_equal(loop, rows * s16)
        assert np.array_equal(loop, o.ternary.ternary_dequant(codes, sb, K))
        assert not np.any(np.signbit(loop[rows == 0]))


def pin_bf16_values_exhaustive(o):
    """Both bf16 decoders on all 65536 bit patterns against torch's own
    bfloat16 -> float32 conversion (NaNs as NaNs), plus hand values."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    vec = o.rne.bf16_values(bits)
    loop = np.array([o.rne.bf16_value_exact(int(b)) for b in bits])
    for got in (vec, loop):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert o.rne.bf16_value_exact(0x3F80) == 1.0
    assert o.rne.bf16_value_exact(0x0001) == 2.0 ** -133
    assert o.rne.bf16_value_exact(0x7F7F) == (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert o.rne.bf16_value_exact(0xC040) == -3.0


def pin_tolerance_overflow(o):
    """An infinite output passes only with the sign of the reference and only
    when some value within the bound of it rounds to that infinity: binary16
    rounds magnitudes from 65504 + 16 = 65520 up to infinity (65519.99 rounds
    down to 65504), bfloat16 from (2 - 2^-8) 2^127 up (checked against numpy's
    and torch's own conversions)."""
    import torch
    assert np.float16(65519.99) == 65504.0 and np.isinf(np.float16(65520.0))
    assert o.check.F16_OVERFLOW == 65520.0
    x32 = np.float32(o.check.BF16_OVERFLOW)
    assert float(x32) == o.check.BF16_OVERFLOW  # exact in fp32 (9 significant bits)
    bf = torch.tensor([x32, np.nextafter(x32, np.float32(0))], dtype=torch.float32).to(torch.bfloat16).float()
    assert np.isinf(bf[0].item()) and np.isfinite(bf[1].item())
    inf = np.inf
    # reference 70000 (rounds to +inf in binary16): +inf passes, -inf and a finite value do not
    ok, st = o.check.tolerance_ok(np.array([[inf]]), np.array([[70000.0]]), np.array([[70000.0]]))
    assert ok and not st["finite"], st
    assert not o.check.tolerance_ok(np.array([[-inf]]), np.array([[70000.0]]), np.array([[70000.0]]))[0]
    assert not o.check.tolerance_ok(np.array([[65504.0]]), np.array([[70000.0]]), np.array([[70000.0]]))[0]
    # reference 65500 with magnitude sum 65500: bound 131 reaches past 65520, so +inf passes;
    # with magnitude sum 0 (bound 1e-3) it does not
    assert o.check.tolerance_ok(np.array([[inf]]), np.array([[65500.0]]), np.array([[65500.0]]))[0]
    assert not o.check.tolerance_ok(np.array([[inf]]), np.array([[65500.0]]), np.array([[0.0]]))[0]
    # bf16: 1e38 never rounds to infinity; 3.4e38 with a loose bound does
    assert not o.check.tolerance_ok(np.array([[inf]]), np.array([[1e38]]), np.array([[1e38]]), out_dtype="bf16")[0]
    assert o.check.tolerance_ok(np.array([[-inf]]), np.array([[-3.4e38]]), np.array([[3.4e38]]), out_dtype="bf16")[0]


# ------------------------------------------- W4A16, zero points and act-order

def pin_w4a_format_from_pages(o):
    """Bits, group size, per-group zero point and optional g_idx (golden fixture)."""
    kv = dict(_golden_lines("w4a16_asym_format.txt"))
    assert int(kv["bits"]) == o.w4asym.BITS == 4
    assert int(kv["group_size"]) == o.w4asym.GROUP == 128
    assert int(kv["packed_factor"]) == o.w4asym.PER_WORD == 8
    assert kv["zero_point"] == "per_group" and kv["g_idx"] == "optional"


def _w4a_words_from_codes(codes):
    """Words of one row from its codes, nibble i of word j = column 8j + i."""
    words = []
    for j in range(len(codes) // 8):
        w = 0
        for i in range(8):
            w |= codes[8 * j + i] << (4 * i)
        words.append(w)
    return np.array(words, dtype=np.uint32).view(np.int32)


def pin_w4a_hand_example(o):
    """Hand-derived, K = 384 (three groups), every scale exactly 2^-4:
    group 0: -0.25, 0.6875, 0.1, 0.03125, 0.09375, -0.03125, then zeros:
      range [-0.25, 0.6875] -> s = 0.9375/15 = 0.0625, z = 0.25/s = 4;
      codes 0, 15, rint(1.6)+4 = 6, rint(0.5)+4 = 4 (tie to even),
      rint(1.5)+4 = 6, rint(-0.5)+4 = 4, and 4 for each zero;
    group 1: 0.9375, 0.5, then 0.25 x 126 (all positive: the range widens
      to include 0): s = 0.0625, z = 0; codes 15, 8, 4 ...;
    group 2: -0.9375, then -0.25 x 127 (all negative): s = 0.0625, z = 15;
      codes 0, then rint(-4)+15 = 11."""
    w = np.zeros((1, 384), dtype=np.float32)
    w[0, :6] = [-0.25, 0.6875, 0.1, 0.03125, 0.09375, -0.03125]
    w[0, 128:256] = 0.25
    w[0, 128], w[0, 129] = 0.9375, 0.5
    w[0, 256:] = -0.25
    w[0, 256] = -0.9375
    codes = [0, 15, 6, 4, 6, 4] + [4] * 122 + [15, 8] + [4] * 126 + [0] + [11] * 127
    for q, sb, z, perm in (o.w4asym.w4a_pack(w), [np.array(x) for x in o.w4asym.w4a_pack_loop(w.tolist())]):
        assert np.array_equal(np.asarray(sb).reshape(-1), [0x2C00] * 3)
        assert np.array_equal(np.asarray(z).reshape(-1), [4, 0, 15])
        words = np.asarray(q).reshape(-1).astype(np.int64) & 0xFFFFFFFF
        assert np.array_equal(words, _w4a_words_from_codes(codes).view(np.uint32).astype(np.int64))
        assert np.array_equal(np.asarray(perm).reshape(-1), np.arange(384))
    q, sb, z, perm = o.w4asym.w4a_pack(w)
    d = o.w4asym.w4a_dequant(q, sb, z, 384, perm)[0]
    assert d[0] == -0.25 and d[1] == 0.6875 and d[2] == 0.125 and d[3] == 0.0 and d[5] == 0.0
    assert d[128] == 0.9375 and d[129] == 0.5 and d[130] == 0.25 and d[256] == -0.9375 and d[300] == -0.25


def _w4a_expected(cols, group_vals):
    """Exact-rational quantization of one group (independent RNE scan):
    returns (scale bits, zero point, {column: code})."""
    fr = [Fraction(v) for v in group_vals]
    lo = min([Fraction(0)] + fr)
    hi = max([Fraction(0)] + fr)
    sb = _round_to_grid_f16((hi - lo) / 15)
    s = _f16_frac(sb)
    if s == 0:
        return sb, 0, {c: 0 for c in cols}
    z = min(max(round(-lo / s), 0), 15)         # Fraction rounds half to even
    return sb, z, {c: min(max(round(f / s) + z, 0), 15) for c, f in zip(cols, fr)}


def pin_w4a_vs_fraction(o):
    """Scales, zero points and codes equal the exact-rational definition, with
    and without a random g_idx (groups of 8), both tiers; dequant in the input
    column order equals (q - z) * s of each column's own group."""
    rng = random.Random(11)
    for trial in range(40):
        N, group = 3, 8
        K = group * rng.choice([1, 2, 3])
        G = K // group
        scale = rng.choice([1e-3, 0.02, 1.0, 300.0])
        w = np.array([[rng.gauss(0, scale) if rng.random() > 0.1 else 0.0 for _ in range(K)] for _ in range(N)],
                     dtype=np.float32)
        if trial % 5 == 0:
            w[0] = np.abs(w[0])
        if trial % 7 == 0:
            w[1] = 0.0
        g_idx = None
        if trial % 2:
            lab = [k // group for k in range(K)]
            rng.shuffle(lab)
            g_idx = np.array(lab, dtype=np.int32)
        q, sb, z, perm = o.w4asym.w4a_pack(w, g_idx, group=group)
        ql, sbl, zl, perml = o.w4asym.w4a_pack_loop(w.tolist(), None if g_idx is None else g_idx.tolist(), group=group)
        assert np.array_equal(np.array(ql, dtype=np.uint32).view(np.int32), q)
        assert np.array_equal(np.array(sbl, dtype=np.uint16), sb) and np.array_equal(np.array(zl, dtype=np.uint8), z)
        assert np.array_equal(np.array(perml), perm)
        codes = o.w4asym.w4a_unpack(q, K)
        d = o.w4asym.w4a_dequant(q, sb, z, K, perm, group=group)
        dl = o.w4asym.w4a_dequant_loop(ql, sbl, zl, perml, K, group=group)
        labels = [k // group for k in range(K)] if g_idx is None else g_idx.tolist()
        for n in range(N):
            for g in range(G):
                cols = [k for k in range(K) if labels[k] == g]       # membership, not the sort
                esb, ez, ecode = _w4a_expected(cols, [float(w[n, k]) for k in cols])
                s = _f16_frac(esb)
                for k in cols:
                    i = int(np.nonzero(perm == k)[0][0])             # where column k was packed
                    assert i // group == g, "a column left its group"
                    assert codes[n, i] == ecode[k], (trial, n, k)
                    assert sb[n, g] == esb and z[n, g] == ez, (trial, n, g)
                    assert Fraction(d[n, k]) == (ecode[k] - ez) * s
                    assert Fraction(dl[n][k]) == (ecode[k] - ez) * s
        if g_idx is not None:
            assert np.all(np.diff(np.array(labels)[perm]) >= 0)
            for g in range(G):
                ks = perm[g * group:(g + 1) * group]
                assert np.all(np.diff(ks) > 0), "columns of a group not in ascending order"


def pin_w4a_bounds_and_zero(o):
    """Zero dequantizes to exactly 0; the group's minimum gets code 0; every
    error is at most half a step plus the scale's rounding over 15 steps."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    w[:, ::17] = 0.0
    q, sb, z, perm = o.w4asym.w4a_pack(w)
    d = o.w4asym.w4a_dequant(q, sb, z, 1024, perm)
    assert np.all(d[:, ::17] == 0.0)
    g = w.reshape(64, 8, 128).astype(np.float64)
    lo = np.minimum(g.min(axis=2), 0)
    hi = np.maximum(g.max(axis=2), 0)
    s = o.rne.f16_values(sb)
    bound = 0.5 * s + 15 * np.abs(s - (hi - lo) / 15) + 1e-12
    err = np.abs(d - w.astype(np.float64)).reshape(64, 8, 128).max(axis=2)
    assert np.all(err <= bound)
    codes = o.w4asym.w4a_unpack(q, 1024).reshape(64, 8, 128)
    amin = g.argmin(axis=2)
    neg = g.min(axis=2) < 0
    got = np.take_along_axis(codes, amin[:, :, None], axis=2)[:, :, 0]
    assert np.all(got[neg] == 0)


def pin_w4a_errors_and_identity_order(o):
    """g_idx with a group of the wrong size or out of range is a GROUP error;
    g_idx = k // 128 gives the identity order and the results without it."""
    w = (np.random.default_rng(2).standard_normal((4, 256)) * 0.02).astype(np.float32)
    ident = np.arange(256) // 128
    a = o.w4asym.w4a_pack(w)
    b = o.w4asym.w4a_pack(w, ident)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    for bad in (np.zeros(256, dtype=np.int32), np.full(256, 2), np.r_[np.zeros(129), np.ones(127)]):
        for fn in (o.w4asym.w4a_pack, lambda W, g: o.w4asym.w4a_pack_loop(W.tolist(), g.tolist())):
            try:
                fn(w, bad)
            except o.errors.OracleError as e:
                assert e.kind == "GROUP"
            else:
                raise AssertionError("bad g_idx accepted")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
