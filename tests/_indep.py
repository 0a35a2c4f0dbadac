"""Independent re-derivations used to pin the oracle (tests only).

Formulated differently from the oracle on purpose: the oracle's encoders search for
the nearest code; these use exact rationals (fractions.Fraction), the literal value
tables in tests/golden/formats.json, and threshold comparisons.  A mistake in either
formulation shows up as a disagreement.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "formats.json")))
E2M1_MAG = [Fraction(x).limit_denominator(2) for x in GOLDEN["e2m1_magnitudes"]["value"]]
E2M1_VALUES = E2M1_MAG + [-m for m in E2M1_MAG]          # code c -> value (bit 3 = sign)

# Midpoints between adjacent E2M1 magnitudes and which side an exact tie goes to
# (the neighbour whose code is even).
_E2M1_THRESH = []
for c in range(7):
    mid = (E2M1_MAG[c] + E2M1_MAG[c + 1]) / 2
    _E2M1_THRESH.append((mid, c if c % 2 == 0 else c + 1))


def e2m1_code_exact(u: Fraction) -> int:
    """Code of the rational u under round-to-nearest-even with saturation at 6."""
    a = abs(u)
    code = 0
    for c, (mid, tie_code) in enumerate(_E2M1_THRESH):
        if a > mid:
            code = c + 1
        elif a == mid:
            code = tie_code
            break
        else:
            break
    return code


def floor_log2_fraction(a: Fraction) -> int:
    """floor(log2(a)) for a rational a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def mxfp4_block_exact(vals, neg=None):
    """Quantise 32 rationals; `neg` gives the sign bit of each element (defaults to
    v < 0).  Returns (list of 32 codes, scale byte)."""
    amax = max(abs(v) for v in vals)
    if amax == 0:
        X = -127
    else:
        X = max(-127, min(127, floor_log2_fraction(amax) - 2))
    scale = Fraction(2) ** X
    codes = []
    for i, v in enumerate(vals):
        c = e2m1_code_exact(v / scale)
        s = (v < 0) if neg is None else neg[i]
        codes.append(c | (8 if s else 0))
    return codes, X + 127


def pack_nibbles(codes):
    return bytes((codes[2 * j] & 15) | ((codes[2 * j + 1] & 15) << 4) for j in range(len(codes) // 2))


def unpack_nibbles(b: bytes):
    out = []
    for x in b:
        out += [x & 15, x >> 4]
    return out


# ------------------------------------------------------------------------- e4m3
def _e4m3_table():
    pts = {int(c): Fraction(v) for c, v in GOLDEN["e4m3_points"]["value"]}
    # Enumerate from the OFP8 definition's structure: within each binade [2^e, 2^(e+1))
    # there are 8 equally spaced values; subnormals step 2^-9 from 0.
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            v = Fraction(m, 512)
        else:
            v = Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        vals.append(v)
    for c, v in pts.items():
        mag = vals[c & 0x7F]
        assert (mag if c < 128 else -mag) == v, (c, v)
    return vals


E4M3_MAG = _e4m3_table()


def e4m3_code_exact(u: Fraction, negative: bool) -> int:
    a = abs(u)
    if a >= E4M3_MAG[-1]:
        code = 0x7E
    else:
        lo = max(i for i, v in enumerate(E4M3_MAG) if v <= a)
        if E4M3_MAG[lo] == a:
            code = lo
        else:
            hi = lo + 1
            d_lo, d_hi = a - E4M3_MAG[lo], E4M3_MAG[hi] - a
            code = lo if d_lo < d_hi else hi if d_hi < d_lo else (lo if lo % 2 == 0 else hi)
    return code | (0x80 if negative else 0)


def e4m3_value(code: int) -> Fraction:
    mag = E4M3_MAG[code & 0x7F]
    return -mag if code & 0x80 else mag


# ------------------------------------------------------------------------- K store
def f32_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def bf16_fraction(bits: int) -> Fraction:
    return Fraction(float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0]))


def k_row_exact(bits_row, gamma, eps, cs_row, digits=60):
    """Exact-as-possible K row: rationals throughout, the square root in `digits`
    decimal digits.  Returns a list of 128 Decimals (the normed, rotated row)."""
    getcontext().prec = digits
    x = [bf16_fraction(b) for b in bits_row]
    ms = sum(v * v for v in x) / 128 + f32_fraction(eps)
    r = Decimal(ms.numerator) / Decimal(ms.denominator)
    r = r.sqrt()
    def dec(f):
        return Decimal(f.numerator) / Decimal(f.denominator)
    y = [dec(x[i]) / r * dec(f32_fraction(gamma[i])) for i in range(128)]
    z = list(y)
    for i in range(32):
        c, n = dec(f32_fraction(cs_row[i])), dec(f32_fraction(cs_row[32 + i]))
        z[i] = y[i] * c - y[i + 32] * n
        z[i + 32] = y[i + 32] * c + y[i] * n
    return z


def decimal_to_fraction(d: Decimal) -> Fraction:
    return Fraction(d)


def near_boundary_mxfp4(vals, rel=1e-12):
    """Indices (and the scale flag) where a decision of the block quantiser sits
    within `rel` of a boundary: an element near a midpoint, or amax near a power of 2."""
    amax = max(abs(v) for v in vals)
    flags = set()
    if amax == 0:
        return flags, False
    X = max(-127, min(127, floor_log2_fraction(amax) - 2))
    scale_near = False
    lg = math.log2(float(amax))
    if abs(lg - round(lg)) < 1e-12:
        scale_near = True
    s = Fraction(2) ** X
    for i, v in enumerate(vals):
        a = abs(v / s)
        for mid, _ in _E2M1_THRESH:
            if abs(a - mid) <= rel * max(mid, Fraction(1)):
                flags.add(i)
        if a == 0 and v != 0:
            flags.add(i)
    return flags, scale_near
