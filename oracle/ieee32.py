"""Exact-rational IEEE-754 binary32 arithmetic (the referee).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The DaisyChain-Train page "Verification — why you can trust the numbers",
section "Layer 4: the referee — an IEEE-754 oracle", describes a binary32
oracle built from the IEEE-754 definition in exact arithmetic:
round-to-nearest-even, subnormals and signed zero, with no host float
rounding anywhere.  This module is that referee in Python: every value is a
32-bit pattern (``int``), every operation is done on ``fractions.Fraction``
exactly and rounded once by :func:`round_fraction`.

It is deliberately independent of numpy: the numpy oracle (``ref``) relies on
the host FPU's float32 rounding, this module relies on nothing but integer
arithmetic, so agreement between the two pins both.

binary32 layout: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits.
Normal numbers are (1.f) * 2^(E-127) for E in 1..254; subnormals are
(0.f) * 2^-126; E = 255 encodes inf (f = 0) and NaN (f != 0).
"""
from fractions import Fraction
import struct

SIGN = 0x80000000
POS_INF = 0x7F800000
NEG_INF = 0xFF800000
QNAN = 0x7FC00000
PRECISION = 24          # significand bits including the hidden bit
EMIN = -126             # exponent of the smallest normal number
EMAX = 127              # exponent of the largest finite number


class NaNError(ValueError):
    """Raised when a NaN would have to be decoded as a rational."""


def bits_of(x: float) -> int:
    """Bit pattern of the binary32 value nearest to the Python float ``x``.

    Only for writing test constants; the rounding is the host's.
    """
    return struct.unpack("<I", struct.pack("<f", x))[0]


def float_of(bits: int) -> float:
    """The binary32 value with pattern ``bits`` as a Python float (exact)."""
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


def is_nan(b: int) -> bool:
    return (b & 0x7F800000) == 0x7F800000 and (b & 0x007FFFFF) != 0


def is_inf(b: int) -> bool:
    return (b & 0x7FFFFFFF) == POS_INF


def sign_bit(b: int) -> int:
    return (b >> 31) & 1


def decode(b: int) -> Fraction:
    """Exact rational value of a finite binary32 pattern (-0 decodes to 0)."""
    b &= 0xFFFFFFFF
    e_field = (b >> 23) & 0xFF
    frac = b & 0x7FFFFF
    if e_field == 0xFF:
        raise NaNError("inf or NaN has no rational value")
    if e_field == 0:
        mag = Fraction(frac, 1 << 149)                       # 0.f * 2^-126
    else:
        mag = Fraction(frac | (1 << 23)) * Fraction(2) ** (e_field - 150)
    return -mag if b >> 31 else mag


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a rational a > 0."""
    n, d = a.numerator, a.denominator
    e = n.bit_length() - d.bit_length()
    # 2^e <= a  <=>  n * 2^-e >= d
    if e >= 0:
        if n < (d << e):
            e -= 1
    else:
        if (n << -e) < d:
            e -= 1
    return e


def round_fraction(q: Fraction, zero_sign: int = 0) -> int:
    """Round the exact rational ``q`` to binary32, ties to even.

    Gradual underflow: values below 2^-126 round on the subnormal grid of
    spacing 2^-149.  Overflow: a magnitude that rounds to 2^128 or above
    becomes infinity of the same sign.  A value that is exactly zero returns
    the zero whose sign is ``zero_sign`` (the sign rule of the operation that
    produced it); a non-zero value that rounds to zero keeps its own sign.
    """
    if q == 0:
        return SIGN if zero_sign else 0
    neg = q < 0
    a = -q if neg else q
    e = max(_floor_log2(a), EMIN)
    # a = m * 2^(e-23): m is the significand on the grid of this binade.
    scaled = a * (Fraction(2) ** (PRECISION - 1 - e))
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (m & 1)):
        m += 1
    if m == (1 << PRECISION):           # rounding carried into the next binade
        m >>= 1
        e += 1
    if m >= (1 << (PRECISION - 1)):     # normal
        if e > EMAX:
            out = POS_INF
        else:
            out = ((e + 127) << 23) | (m - (1 << 23))
    else:                               # subnormal (e == EMIN) or zero
        out = m
    return out | (SIGN if neg else 0)


def from_int(n: int) -> int:
    """binary32 nearest to the integer ``n`` (int -> float conversion, RNE)."""
    return round_fraction(Fraction(n))


def mul(a: int, b: int) -> int:
    """a * b correctly rounded (RNE); signed zero by the sign-xor rule."""
    s = sign_bit(a) ^ sign_bit(b)
    if is_nan(a) or is_nan(b):
        return QNAN
    if is_inf(a) or is_inf(b):
        other = b if is_inf(a) else a
        if not is_inf(other) and decode(other) == 0:
            return QNAN
        return POS_INF | (SIGN if s else 0)
    return round_fraction(decode(a) * decode(b), zero_sign=s)


def add(a: int, b: int) -> int:
    """a + b correctly rounded (RNE).

    An exact zero sum is +0 unless both operands are -0 (round-to-nearest
    sign rule); infinities of opposite sign give NaN.
    """
    if is_nan(a) or is_nan(b):
        return QNAN
    if is_inf(a) or is_inf(b):
        if is_inf(a) and is_inf(b) and sign_bit(a) != sign_bit(b):
            return QNAN
        return a if is_inf(a) else b
    zs = 1 if (sign_bit(a) and sign_bit(b)) else 0
    return round_fraction(decode(a) + decode(b), zero_sign=zs)


def sub(a: int, b: int) -> int:
    return add(a, b ^ SIGN)


def div(a: int, b: int) -> int:
    """a / b correctly rounded (RNE); x/0 gives a signed infinity, 0/0 NaN."""
    s = sign_bit(a) ^ sign_bit(b)
    if is_nan(a) or is_nan(b):
        return QNAN
    if is_inf(a):
        return QNAN if is_inf(b) else (POS_INF | (SIGN if s else 0))
    if is_inf(b):
        return SIGN if s else 0
    db = decode(b)
    da = decode(a)
    if db == 0:
        return QNAN if da == 0 else (POS_INF | (SIGN if s else 0))
    return round_fraction(da / db, zero_sign=s)


def fma(a: int, b: int, c: int) -> int:
    """a * b + c with ONE rounding (only used to model a contracted kernel)."""
    exact = decode(a) * decode(b) + decode(c)
    prod_sign = sign_bit(a) ^ sign_bit(b)
    zs = 1 if (prod_sign and sign_bit(c)) else 0
    return round_fraction(exact, zero_sign=zs)


def floor_int(b: int) -> int:
    """floor of a finite binary32 value, as a Python int (exact)."""
    v = decode(b)
    return v.numerator // v.denominator


def gt_zero(b: int) -> bool:
    """b > 0 under IEEE comparison (false for +0, -0 and negatives)."""
    return not is_nan(b) and sign_bit(b) == 0 and (b & 0x7FFFFFFF) != 0


def abs_(b: int) -> int:
    return b & 0x7FFFFFFF


def max_(a: int, b: int) -> int:
    """max of two finite binary32 values; on equal values the first is kept."""
    return b if decode(b) > decode(a) else a


def pred(b: int) -> int:
    """Next binary32 value toward zero for a positive finite non-zero pattern."""
    assert b & SIGN == 0 and b != 0
    return b - 1


def succ(b: int) -> int:
    """Next binary32 value away from zero for a positive finite pattern."""
    assert b & SIGN == 0
    return b + 1
