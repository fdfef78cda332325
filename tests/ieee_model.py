"""An exact integer model of IEEE-754 binary64 addition (test helper).

Every finite double is an integer multiple of 2^-1074, so the exact sum of two
doubles is an integer N in those units.  Rounding N to binary64 with round to
nearest, ties to even, is done here with Python integers only (bit lengths,
shifts, the parity of the kept quotient), independent of any floating-point
hardware.  It is used to pin the oracle, never to produce the values a test
compares the GPU against.
"""

from __future__ import annotations

import math
from fractions import Fraction

UNIT_EXP = 1074          # value = N * 2^-1074
MAX_BITS = 53
# Largest finite double in units: (2^53 - 1) * 2^971 * 2^1074
OVERFLOW_LIMIT = (2 ** 53) << (971 + 1074)      # rounding to this overflows


def to_units(x: float) -> int:
    if not math.isfinite(x):
        raise ValueError("finite values only")
    p, q = x.as_integer_ratio()        # q is a power of two <= 2^1074
    return (p << UNIT_EXP) // q if q else 0


def round_units(n: int) -> int:
    """Round an integer (units of 2^-1074) to a representable binary64,
    RNE; returns units, or raises OverflowError."""
    a = abs(n)
    if a < (1 << MAX_BITS):
        return n                       # subnormal range or first normal binade: exact
    shift = a.bit_length() - MAX_BITS
    q, rem = divmod(a, 1 << shift)
    half = 1 << (shift - 1)
    if rem > half or (rem == half and (q & 1)):
        q += 1
    r = q << shift
    if r >= OVERFLOW_LIMIT:
        raise OverflowError
    return r if n >= 0 else -r


def from_units(n: int) -> float:
    """Units to float; n must be representable (at most 53 significant bits)."""
    if n == 0:
        return 0.0
    shift = max(0, abs(n).bit_length() - MAX_BITS)
    q = abs(n) >> shift
    assert q << shift == abs(n), "not representable"
    v = math.ldexp(q, shift - UNIT_EXP)
    return v if n > 0 else -v


def add(a: float, b: float) -> float:
    """fl(a + b) for finite a, b."""
    na, nb = to_units(a), to_units(b)
    s = na + nb
    if s == 0:
        neg = math.copysign(1.0, a) < 0 and math.copysign(1.0, b) < 0
        return -0.0 if neg else 0.0
    try:
        return from_units(round_units(s))
    except OverflowError:
        return math.inf if s > 0 else -math.inf


def seq_sum(xs, init: float = 0.0) -> float:
    s = init
    for x in xs:
        s = add(s, x)
    return s


def round_fraction(v: Fraction) -> float:
    """Nearest binary64 to an exact rational, RNE (finite results only)."""
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    # scale to units of 2^-1074 with enough guard: compare remainders exactly
    num, den = a.numerator << UNIT_EXP, a.denominator
    q, rem = divmod(num, den)          # a * 2^1074 = q + rem/den
    # first round to an integer number of units with RNE, then to 53 bits
    if a * (1 << UNIT_EXP) >= (1 << MAX_BITS):
        shift = q.bit_length() - MAX_BITS
        top, low = divmod(q, 1 << shift)
        # exact remainder relative to the kept unit 2^shift
        frac = Fraction(low * den + rem, den << shift)
        if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and (top & 1)):
            top += 1
        r = top << shift
        if r >= OVERFLOW_LIMIT:
            return sign * math.inf
        return sign * from_units(r)
    frac = Fraction(rem, den)
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and (q & 1)):
        q += 1
    return sign * from_units(q)
