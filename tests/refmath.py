"""Independent reference arithmetic for pinning the oracle (tests only).

Nothing here is imported by the oracle or by the library.  These are
brute-force and exact-rational formulations of the number formats, written
differently from the oracle on purpose: bf16 values come from reinterpreting
bit patterns with numpy, rounding is decided by exhaustive nearest-neighbour
search or by exact comparisons with Fractions/Decimals, and transcendental
values come from Python's arbitrary-precision Decimal.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

getcontext().prec = 60


# ---------------------------------------------------------------- bf16 ---

def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


_ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
_ALLV = bf16_bits_to_f64(_ALL)
# non-negative finite bf16, sorted ascending by value (bit order == value order)
POS_BF16_BITS = _ALL[(_ALL < 0x7F80)]
POS_BF16_VALS = bf16_bits_to_f64(POS_BF16_BITS)
FINITE_BF16_BITS = _ALL[np.isfinite(_ALLV)]


def nearest_bf16_exact(x):
    """Round an exact number (Fraction, Decimal, int or float) to bf16 bits,
    ties to the even bit pattern, by locating its two bf16 neighbours and
    comparing exactly with their midpoint.  Overflow past the largest finite
    value's rounding range gives Inf."""
    xf = Fraction(x) if not isinstance(x, Fraction) else x
    neg = xf < 0
    a = -xf if neg else xf
    sign = 0x8000 if neg else 0
    if a == 0:
        return sign
    maxv = Fraction(float(POS_BF16_VALS[-1]))
    # rounding boundary above max finite is max + half its quantum (2^127 * 2^-8)
    if a >= maxv + Fraction(2) ** 119:
        return sign | 0x7F80
    idx = int(np.searchsorted(POS_BF16_VALS, float(a), side="right")) - 1
    # float(a) may sit on a neighbour; search a little around it exactly
    lo_i = max(idx - 1, 0)
    while lo_i + 1 < len(POS_BF16_VALS) and Fraction(float(POS_BF16_VALS[lo_i + 1])) <= a:
        lo_i += 1
    while Fraction(float(POS_BF16_VALS[lo_i])) > a:
        lo_i -= 1
    lo = Fraction(float(POS_BF16_VALS[lo_i]))
    if lo == a or lo_i + 1 >= len(POS_BF16_VALS):
        return sign | int(POS_BF16_BITS[lo_i])
    hi = Fraction(float(POS_BF16_VALS[lo_i + 1]))
    mid = (lo + hi) / 2
    if a < mid:
        pick = lo_i
    elif a > mid:
        pick = lo_i + 1
    else:
        pick = lo_i if int(POS_BF16_BITS[lo_i]) % 2 == 0 else lo_i + 1
    return sign | int(POS_BF16_BITS[pick])


def bf16_tie_distance_rel(x):
    """|x - nearest bf16 tie point| / |x| for an exact x (Fraction)."""
    a = abs(Fraction(x))
    if a == 0:
        return Fraction(1)
    idx = int(np.searchsorted(POS_BF16_VALS, float(a), side="right")) - 1
    idx = min(max(idx, 0), len(POS_BF16_VALS) - 2)
    best = None
    for i in range(max(idx - 1, 0), min(idx + 2, len(POS_BF16_VALS) - 1)):
        mid = (Fraction(float(POS_BF16_VALS[i])) + Fraction(float(POS_BF16_VALS[i + 1]))) / 2
        d = abs(a - mid) / a
        best = d if best is None or d < best else best
    return best


# ---------------------------------------------------------------- E4M3 ---

def e4m3_table():
    """Values of all 256 E4M3 ('fn') codes, NaN at 0x7F/0xFF, from the format's
    field layout: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field
    0 is subnormal (m/8 * 2^-6); no infinities."""
    vals = np.zeros(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals[c] = -mag if s else mag
    return vals


E4M3 = e4m3_table()
E4M3_POS = E4M3[:127]           # codes 0x00..0x7E, ascending


def nearest_e4m3_bruteforce(y):
    """RNE-saturating E4M3 encode by exhaustive search over the 127
    non-negative finite magnitudes; ties go to the even code."""
    y = float(y)
    if np.isnan(y):
        return 0xFF if np.signbit(y) else 0x7F
    sign = 0x80 if np.signbit(y) else 0
    a = abs(y)
    if a >= 448.0:
        return sign | 0x7E
    d = np.abs(E4M3_POS - a)
    best = np.flatnonzero(d == d.min())
    if len(best) == 1:
        return sign | int(best[0])
    even = [int(b) for b in best if b % 2 == 0]
    return sign | even[0]


# ---------------------------------------------------------------- E8M0 ---

def e8m0_bruteforce(amax):
    """Smallest E in 0..254 with amax <= 448 * 2^(E-127); NaN/Inf -> 255;
    falls back to 0 when even E = 0 satisfies it (the lower clamp)."""
    if np.isnan(amax) or np.isinf(amax):
        return 255
    a = Fraction(float(amax))
    for E in range(0, 255):
        if a <= 448 * Fraction(2) ** (E - 127):
            return E
    return 254


# ------------------------------------------------------ exact transcendental ---

def dec(x):
    return Decimal(float(x))


def silu_dec(g):
    g = dec(g) if not isinstance(g, Decimal) else g
    if g < -1000:
        # |silu| < 1000 * e^-1000, far below half the smallest bf16 subnormal:
        # an exact tiny negative stands in for it (exp(-g) would overflow)
        return -Decimal(10) ** -500
    return g / (1 + (-g).exp())


def dsilu_dec_fd(g, h=Decimal("1e-25")):
    """silu'(g) by a central finite difference in 60-digit Decimal arithmetic
    (error ~ h^2), independent of any closed form for the derivative."""
    g = dec(g)
    return (silu_dec(g + h) - silu_dec(g - h)) / (2 * h)


def dec_to_fraction(d):
    return Fraction(d)
