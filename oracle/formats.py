"""Scale and storage variants of the method: power-of-two scales and int4.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the presk page, section "Integer weights" and the list of solver
rungs that follows it.  A parameter can be stored as int8 or int4 with one
scale per channel, the scale being the symmetric absmax scale
max|w| / (2^(b-1) - 1) rounded to f32; the "pow2" scheme rounds each scale
up to a power of two, at most twice as coarse, so that q*s is exact; int4
values are stored two to a byte.

Readings taken here (each listed in the design doc):
  * the variants keep every other step of the block-scaled method
    ("Verification -- why you can trust the numbers", section "The verified
    INT8 units"): the 1e-8 floor, inv = RN(1/s), q = floor(RN(RN(x*inv)+0.5)),
    the exact integer contraction and the epilogue
    RN(RN(RN(acc)*s_row)*s_col);
  * b = 4 gives qmax = 7: s = max(RN(a/7), RN(1e-8)), q in [-7, 7];
  * pow2: s is the smallest power of two >= max(RN(a/qmax), RN(1e-8)); the
    floor therefore becomes 2^-26;
  * int4 storage (the page fixes no nibble order): element k of a line is
    held in byte 16*(k // 32) + (k % 16), in the low nibble when k % 32 < 16
    and in the high nibble otherwise, as a 4-bit two's complement value; a
    line of length L takes 16*ceil(L/32) bytes and every nibble past L is 0.

Two independent implementations: numpy (``scales``, ``quantize_*``,
``pack_int4``, ``unpack_int4``) and pure Python on exact rationals
(``brute_*``), which the tests compare on small inputs.
"""
from fractions import Fraction

import numpy as np

from . import ieee32 as I
from . import ref

F32 = np.float32
POW2 = 1          # format flag: power-of-two scales
INT4 = 2          # format flag: 4-bit values, two per byte


def qmax_of(fmt):
    """Largest |q| of a format: 2^(b-1) - 1 for b = 8 or 4."""
    return 7 if fmt & INT4 else 127


# ---------------------------------------------------------------------------
# numpy
# ---------------------------------------------------------------------------
def pow2_ceil(s):
    """Smallest power of two >= s, elementwise, for positive normal binary32 s."""
    s = np.asarray(s, dtype=F32)
    m, e = np.frexp(s.astype(np.float64))          # s = m * 2^e, m in [0.5, 1)
    p = np.where(m == 0.5, e - 1, e)
    return np.ldexp(np.ones_like(m), p).astype(F32)


def scales(a, fmt):
    """(s, inv) from the line maxima a for format ``fmt``."""
    a = np.asarray(a, dtype=F32)
    s = np.maximum(a / F32(qmax_of(fmt)), ref.SCALE_FLOOR).astype(F32)
    if fmt & POW2:
        s = pow2_ceil(s)
    inv = (F32(1.0) / s).astype(F32)
    return s, inv


def quantize_rows(X, fmt):
    """Per-row codes (int8 array, R x C) and scales of X in format ``fmt``."""
    X = np.asarray(X, dtype=F32)
    s, inv = scales(ref.absmax_rows(X), fmt)
    t = (X * inv[:, None]).astype(F32)
    u = (t + F32(0.5)).astype(F32)
    q = np.floor(u)
    assert np.all(np.abs(q) <= qmax_of(fmt)), "code outside the format's range"
    return q.astype(np.int8), s


def quantize_cols(X, fmt):
    """Per-column codes, transposed (C x R), and scales of X."""
    X = np.asarray(X, dtype=F32)
    return quantize_rows(np.ascontiguousarray(X.T), fmt)


def int4_row_bytes(length):
    return 16 * ((length + 31) // 32)


def pack_int4(Q):
    """Codes (R x L, each in [-8, 7]) -> packed bytes (R x 16*ceil(L/32), uint8)."""
    Q = np.asarray(Q, dtype=np.int64)
    R, L = Q.shape
    G = (L + 31) // 32
    full = np.zeros((R, G * 32), dtype=np.int64)
    full[:, :L] = Q
    assert np.all((full >= -8) & (full <= 7))
    nib = (full & 0xF).reshape(R, G, 2, 16)         # [row, group, half, position]
    packed = nib[:, :, 0, :] | (nib[:, :, 1, :] << 4)
    return packed.reshape(R, G * 16).astype(np.uint8)


def unpack_int4(P, length):
    """Packed bytes (R x >= 16*ceil(L/32)) -> codes (R x L, int8)."""
    P = np.asarray(P, dtype=np.uint8)
    R = P.shape[0]
    G = (length + 31) // 32
    b = P[:, :G * 16].reshape(R, G, 16).astype(np.int64)
    lo, hi = b & 0xF, b >> 4
    codes = np.stack([lo, hi], axis=2).reshape(R, G * 32)
    codes = np.where(codes >= 8, codes - 16, codes)
    return codes[:, :length].astype(np.int8)


def blockscaled_gemm(A, B, fmt_a, fmt_b, relu=False):
    """The method with A quantized per row in fmt_a and B per column in
    fmt_b.  Returns (C, QA codes, s_row, QBt codes, s_col)."""
    QA, sr = quantize_rows(A, fmt_a)
    QB, sc = quantize_cols(B, fmt_b)
    return ref.gemm_i8_blockscaled(QA, sr, QB, sc, relu), QA, sr, QB, sc


# ---------------------------------------------------------------------------
# pure Python, exact rationals (tiny inputs)
# ---------------------------------------------------------------------------
_FLOOR = I.round_fraction(Fraction(1, 10**8))


def _pow2_ceil_bits(s_bits):
    v = I.decode(s_bits)
    assert v > 0
    e = 0
    while Fraction(2) ** e < v:
        e += 1
    while Fraction(2) ** (e - 1) >= v:
        e -= 1
    return I.round_fraction(Fraction(2) ** e)


def brute_scale_inv(vec_bits, fmt):
    """(s, inv) as binary32 patterns for one line given as patterns."""
    a = 0
    for x in vec_bits:
        a = I.max_(a, I.abs_(x))
    s = I.max_(I.div(a, I.from_int(qmax_of(fmt))), _FLOOR)
    if fmt & POW2:
        s = _pow2_ceil_bits(s)
    return s, I.div(I.from_int(1), s)


def brute_quantize(vec_bits, fmt):
    """(codes, s) of one line by exact-rational rounding of every step."""
    s, inv = brute_scale_inv(vec_bits, fmt)
    half = I.round_fraction(Fraction(1, 2))
    out = []
    for x in vec_bits:
        q = I.floor_int(I.add(I.mul(x, inv), half))
        assert abs(q) <= qmax_of(fmt)
        out.append(q)
    return out, s


def brute_pack_int4(codes):
    """One line of codes -> its packed bytes, element by element."""
    L = len(codes)
    out = [0] * (16 * ((L + 31) // 32))
    for k, q in enumerate(codes):
        byte = 16 * (k // 32) + (k % 16)
        shift = 0 if (k % 32) < 16 else 4
        out[byte] |= (int(q) & 0xF) << shift
    return out
