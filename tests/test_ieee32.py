"""Pins of the exact-rational binary32 referee (oracle/ieee32.py).

The DaisyChain-Train page "Verification — why you can trust the numbers",
section "Layer 4", builds its referee from the IEEE-754 definition and
checks it on 500k+ cases including a tie-to-even ladder around 2^24.  Here
the referee is pinned against things that are not itself:

* the host FPU's IEEE float32 operations through numpy (a library routine),
  on ~500k random and edge operands;
* closed forms: the integer ladder around 2^24 .. 2^31 against Python's
  round() (which rounds a Fraction half to even), subnormal and overflow
  boundaries, and the sign rules of zero.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import ieee32 as I

F32 = np.float32
N_RANDOM = 150_000


def _finite_patterns(rng, n):
    """Random finite binary32 patterns: half uniform bits, half in narrow
    exponent bands (so that additions really round)."""
    bits = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    band = rng.integers(100, 156, n, dtype=np.uint32)        # exponents near 1
    frac = rng.integers(0, 2**23, n, dtype=np.uint32)
    sign = rng.integers(0, 2, n, dtype=np.uint32) << np.uint32(31)
    narrow = sign | (band << np.uint32(23)) | frac
    use = rng.random(n) < 0.5
    out = np.where(use, bits, narrow).astype(np.uint32)
    expo = (out >> np.uint32(23)) & np.uint32(0xFF)
    out[expo == 0xFF] &= np.uint32(0x807FFFFF)                # no inf / NaN
    return out


def _edge_patterns():
    vals = [0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x00800000,
            0x00800001, 0x3F800000, 0xBF800000, 0x3F000000, 0x3EFFFFFF, 0x7F7FFFFF,
            0xFF7FFFFF, 0x4B800000, 0x4B7FFFFF, 0x322BCC77, 0x42FE0000, 0x3C010204]
    return np.array(vals, dtype=np.uint32)


def _check_binop(op_ref, op_np, a, b):
    with np.errstate(all="ignore"):
        got_np = op_np(a.view(F32), b.view(F32)).astype(F32).view(np.uint32)
    bad = []
    for x, y, g in zip(a.tolist(), b.tolist(), got_np.tolist()):
        r = op_ref(x, y)
        if I.is_nan(r) and I.is_nan(g):
            continue
        if r != g:
            bad.append((hex(x), hex(y), hex(r), hex(g)))
            if len(bad) > 5:
                break
    assert not bad, bad


@pytest.mark.parametrize("name,op_ref,op_np", [
    ("mul", I.mul, np.multiply),
    ("add", I.add, np.add),
    ("div", I.div, np.divide),
])
def test_binop_matches_host_ieee(name, op_ref, op_np):
    rng = np.random.default_rng({"mul": 11, "add": 12, "div": 13}[name])
    a = _finite_patterns(rng, N_RANDOM)
    b = _finite_patterns(rng, N_RANDOM)
    e = _edge_patterns()
    a = np.concatenate([a, np.repeat(e, e.size)])
    b = np.concatenate([b, np.tile(e, e.size)])
    _check_binop(op_ref, op_np, a, b)


def test_int_to_f32_matches_host():
    rng = np.random.default_rng(14)
    n = rng.integers(-(2**31), 2**31, 50_000, dtype=np.int64)
    n = np.concatenate([n, np.arange(2**24 - 40, 2**24 + 40), np.arange(-(2**25) - 40, -(2**25) + 40)])
    got = n.astype(np.int32).astype(F32).view(np.uint32)
    for v, g in zip(n.tolist(), got.tolist()):
        assert I.from_int(v) == g, (v, hex(g))


def test_tie_ladder_around_2_pow_24():
    """Integers near powers of two 2^24 .. 2^31: RNE against round() on Fractions."""
    for e in range(24, 32):
        ulp = 1 << (e - 23)
        for j in range(-3 * ulp, 4 * ulp + 1):
            n = (1 << e) + j
            if n >= 2**31:
                continue
            # grid spacing is 2^(e-24) just below 2^e and 2^(e-23) from 2^e on
            step = ulp if n >= (1 << e) else ulp // 2
            expect = round(Fraction(n, step)) * step       # half to even
            assert I.decode(I.from_int(n)) == expect, (e, j)
    # the explicit values the tests are named after
    assert I.decode(I.from_int(2**24 + 1)) == 2**24
    assert I.decode(I.from_int(2**24 + 3)) == 2**24 + 4
    assert I.decode(I.from_int(2**25 + 2)) == 2**25
    assert I.decode(I.from_int(2**25 + 6)) == 2**25 + 8
    assert I.decode(I.from_int(2**31 - 1)) == 2**31


def test_subnormal_overflow_and_zero_signs():
    tiny = 0x00000001                                   # 2^-149
    half = I.round_fraction(Fraction(1, 2))
    three_q = I.round_fraction(Fraction(3, 4))
    assert I.mul(tiny, half) == 0                        # 2^-150: tie -> even (0)
    assert I.mul(tiny | I.SIGN, half) == I.SIGN          # keeps its sign
    assert I.mul(tiny, three_q) == tiny                  # 0.75 ulp -> 1 ulp
    assert I.decode(I.mul(0x00800000, half)) == Fraction(1, 2**127)   # subnormal result
    big = 0x7F7FFFFF
    assert I.mul(big, I.from_int(2)) == I.POS_INF
    assert I.add(big, 0x73000000) == I.POS_INF         # + half an ulp of max -> tie -> inf
    assert I.add(big, 0x72FFFFFF) == big
    neg0 = I.SIGN
    one = I.from_int(1)
    assert I.add(neg0, neg0) == neg0
    assert I.add(neg0, 0) == 0
    assert I.sub(one, one) == 0
    assert I.mul(I.from_int(-1), 0) == neg0
    assert I.mul(neg0, neg0) == 0
    assert I.div(0, I.from_int(-3)) == neg0


def test_scale_floor_constant():
    """RN(1e-8) from the exact decimal 1/10^8 is 0x322BCC77 and equals the
    host's float32(1e-8) (no double-rounding difference at this value)."""
    b = I.round_fraction(Fraction(1, 10**8))
    assert b == 0x322BCC77
    assert int(F32(1e-8).view(np.uint32)) == b
    v = I.decode(b)
    assert abs(v - Fraction(1, 10**8)) <= Fraction(1, 2) * Fraction(2) ** (-27 - 23)


def test_fma_differs_from_two_roundings():
    """The fused form rounds once: x*y+z differs from RN(RN(x*y)+z) somewhere."""
    x = int(F32(1 + 2**-12).view(np.uint32))
    z = int(F32(-1).view(np.uint32))
    two = I.add(I.mul(x, x), z)
    one = I.fma(x, x, z)
    assert I.decode(one) == Fraction(2 * 2**12 + 1, 2**24)
    assert one != two
