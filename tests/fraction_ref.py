"""Brute-force exact reference used only to pin the oracle (tiny inputs).

Independent of the C oracle in method, not just in code:
  * value sets are built as SETS of rationals from the formats' closed-form
    descriptions (significand x power of two), not by decoding bit fields;
  * rounding is an argmin of |q - v| over every finite value (ties to the even
    code), not a table walk with midpoint comparisons;
  * log2 floors and fp32 rounding are done in exact rational arithmetic.
"""
from __future__ import annotations

import bisect
from fractions import Fraction as Fr


def _e4m3_values():
    # subnormals m/8 * 2^-6 (m = 0..7), normals (1 + m/8) * 2^(e-7) for e = 1..15,
    # minus the all-ones pattern (e = 15, m = 7), which is NaN in the "fn" variant.
    vals = {Fr(m, 8) * Fr(2) ** -6 for m in range(8)}
    vals |= {Fr(8 + m, 8) * Fr(2) ** (e - 7) for e in range(1, 16) for m in range(8)}
    vals.discard(Fr(15, 8) * Fr(2) ** 8)
    return sorted(vals)


def _e5m2_values():
    vals = {Fr(m, 4) * Fr(2) ** -14 for m in range(4)}
    vals |= {Fr(4 + m, 4) * Fr(2) ** (e - 15) for e in range(1, 31) for m in range(4)}
    return sorted(vals)


def _e2m1_values():
    return sorted({Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)})


E4M3 = _e4m3_values()
E5M2 = _e5m2_values()
E2M1 = _e2m1_values()
TABLES = {0: E4M3, 1: E5M2, 2: E2M1}
SIGN_BIT = {0: 0x80, 1: 0x80, 2: 0x8}


def rne_sat(q: Fr, table) -> int:
    """Index (= magnitude code) of the value nearest to q >= 0; ties -> even code."""
    best = None
    for i, v in enumerate(table):
        d = abs(q - v)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def rne_sat_near(q: Fr, table) -> int:
    """rne_sat for large inputs: the two table values around q found by bisection,
    then the same argmin with ties to the even code over those neighbours only.
    Checked against rne_sat (the full argmin) in the tests."""
    i = bisect.bisect_right(table, q)        # table[i - 1] <= q < table[i]
    cands = [j for j in (i - 1, i) if 0 <= j < len(table)]
    best = None
    for j in cands:
        d = abs(q - table[j])
        if best is None or d < best[0] or (d == best[0] and j % 2 == 0):
            best = (d, j)
    return best[1]


def bf16_value(bits: int) -> Fr:
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF
    if e == 0:
        return s * Fr(m, 128) * Fr(2) ** -126
    return s * Fr(128 + m, 128) * Fr(2) ** (e - 127)


def floor_log2(v: Fr) -> int:
    assert v > 0
    e = 0
    while Fr(2) ** (e + 1) <= v:
        e += 1
    while Fr(2) ** e > v:
        e -= 1
    return e


def rn_fp32(v: Fr) -> Fr:
    """Round a non-negative rational to the nearest fp32 value, ties to even."""
    assert v >= 0
    if v == 0:
        return Fr(0)
    e = max(floor_log2(v), -126)          # below 2^-126 the spacing stays 2^-149
    ulp = Fr(2) ** (e - 23)
    k = v / ulp
    lo = k.numerator // k.denominator
    rem = k - lo
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * ulp
    assert r < Fr(2) ** 128
    return r


def quant_mx(x_bits, rows: int, cols: int, fmt: int, rnd=rne_sat):
    """MXFP8: per 32-block E = floor(log2 amax) - emax (clamped), codes by argmin."""
    table = TABLES[fmt]
    emax = floor_log2(table[-1])
    q = [[0] * cols for _ in range(rows)]
    s = [[0] * (cols // 32) for _ in range(rows)]
    for r in range(rows):
        for b in range(cols // 32):
            blk = [x_bits[r][b * 32 + i] for i in range(32)]
            vals = [bf16_value(v) for v in blk]
            amax = max(abs(v) for v in vals)
            E = -127 if amax == 0 else min(127, max(-127, floor_log2(amax) - emax))
            s[r][b] = E + 127
            for i in range(32):
                code = rnd(abs(vals[i]) / Fr(2) ** E, table)
                q[r][b * 32 + i] = code | (SIGN_BIT[fmt] if blk[i] & 0x8000 else 0)
    return q, s


def quant_nv(x_bits, rows: int, cols: int, global_in=None, rnd=rne_sat):
    """NVFP4: s_g = RN_fp32(amax_t / 2688), S_b = RN_E4M3(amax_b / (6 s_g)),
    q = RN_E2M1(x / (S_b s_g)); returns unpacked nibbles."""
    allv = [bf16_value(x_bits[r][c]) for r in range(rows) for c in range(cols)]
    if global_in is None:
        amax_t = max(abs(v) for v in allv)
        sg = Fr(1) if amax_t == 0 else rn_fp32(amax_t / 2688)
    else:
        sg = Fr(global_in)
    q = [[0] * cols for _ in range(rows)]
    s = [[0] * (cols // 16) for _ in range(rows)]
    for r in range(rows):
        for b in range(cols // 16):
            blk = [x_bits[r][b * 16 + i] for i in range(16)]
            vals = [bf16_value(v) for v in blk]
            amax = max(abs(v) for v in vals)
            sb = rnd(amax / (6 * sg), E4M3)
            s[r][b] = sb
            S = E4M3[sb]
            for i in range(16):
                mag = 0 if S == 0 else rnd(abs(vals[i]) / (S * sg), E2M1)
                q[r][b * 16 + i] = mag | (0x8 if blk[i] & 0x8000 else 0)
    return q, s, sg


def quant_fp8_tensor(x_bits, rows: int, cols: int, scale=None):
    """Weight-only FP8: s = RN_fp32(amax / 448) (1 for an all-zero tensor) or the
    given scale; q = RN_E4M3,sat(x / s) with the input's sign bit."""
    allv = [bf16_value(x_bits[r][c]) for r in range(rows) for c in range(cols)]
    if scale is None:
        amax = max(abs(v) for v in allv)
        s = Fr(1) if amax == 0 else rn_fp32(amax / 448)
    else:
        s = Fr(scale)
    q = [[0] * cols for _ in range(rows)]
    for r in range(rows):
        for c in range(cols):
            b = x_bits[r][c]
            q[r][c] = rne_sat(abs(bf16_value(b)) / s, E4M3) | (0x80 if b & 0x8000 else 0)
    return q, s
