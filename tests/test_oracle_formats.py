"""Pins of the scale and storage variants in the oracle (oracle/formats.py):
presk page, section "Integer weights" (absmax or power-of-two scales, int8
or int4 values, two int4 values to a byte) on top of the block-scaled method
of "Verification -- why you can trust the numbers", "The verified INT8 units"."""
import json
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import ieee32 as I
from oracle import ref

FMTS = [0, F.POW2, F.INT4, F.INT4 | F.POW2]
HERE = os.path.dirname(__file__)


def _lines(seed, rows, cols):
    rng = np.random.default_rng(seed)
    X = rng.standard_t(2, (rows, cols)).astype(np.float32)
    X[1] = 0.0                                   # zero line: the floor
    X[2] *= np.float32(1e-12)                    # tiny line: the floor binds
    X[3, :] = np.float32(-0.0)
    return X


@pytest.mark.parametrize("fmt", FMTS)
def test_numpy_equals_exact_rational(fmt):
    """Two independent implementations: numpy float32 ops vs pure Python on
    exact rationals (every rounding by the IEEE-754 definition)."""
    X = _lines(fmt + 10, 8, 37)
    Q, s = F.quantize_rows(X, fmt)
    for i in range(X.shape[0]):
        qb, sb = F.brute_quantize([I.bits_of(float(v)) for v in X[i]], fmt)
        assert qb == [int(q) for q in Q[i]]
        assert sb == I.bits_of(float(s[i]))


@pytest.mark.parametrize("fmt", [F.POW2, F.INT4 | F.POW2])
def test_pow2_scales(fmt):
    """Page: the scale is rounded up to a power of two, at most twice as
    coarse, and q*s is then exact."""
    X = _lines(3, 64, 200)
    Q, s = F.quantize_rows(X, fmt)
    s_abs, _ = F.scales(ref.absmax_rows(X), fmt & ~F.POW2)
    sb = s.view(np.uint32)
    assert np.all(sb & 0x7FFFFF == 0), "not a power of two"
    assert np.all(s >= s_abs) and np.all(s.astype(np.float64) < 2 * s_abs.astype(np.float64))
    # q*s exact: the f32 product equals the exact product
    prod32 = (Q.astype(np.float32) * s[:, None]).astype(np.float32)
    assert np.array_equal(prod32.astype(np.float64), Q.astype(np.float64) * s[:, None].astype(np.float64))
    # the floor of the pow2 scheme is 2^-26 (RN(1e-8) lies between 2^-27 and 2^-26)
    assert s[1] == np.float32(2.0 ** -26) and s[2] == np.float32(2.0 ** -26)


@pytest.mark.parametrize("fmt", FMTS)
def test_error_rule(fmt):
    """Page's error rule: |x - q*s| <= s/2 (plus nothing else: q*s is checked
    in exact arithmetic)."""
    X = _lines(4, 32, 300)
    Q, s = F.quantize_rows(X, fmt)
    err = np.abs(X.astype(np.float64) - Q.astype(np.float64) * s[:, None].astype(np.float64))
    # RN(x*inv) and the +0.5 can each move the value by one rounding: bound
    # s/2 plus a few ulps of |x|
    slack = np.abs(X.astype(np.float64)) * 2.0 ** -22
    assert np.all(err <= s[:, None].astype(np.float64) / 2 + slack)


def test_int4_range_and_max_code():
    """b = 4: codes in [-7, 7], and a line whose scale is above the floor
    reaches |q| = 7 at its max (absmax scheme)."""
    X = _lines(5, 64, 129)
    Q, s = F.quantize_rows(X, F.INT4)
    assert np.abs(Q).max() <= 7
    live = s > ref.SCALE_FLOOR
    assert np.all(np.abs(Q[live]).max(axis=1) == 7)


def test_unit_scale_closed_form():
    """Integer lines with max |x| = qmax give s = 1 and q = x (both schemes)."""
    rng = np.random.default_rng(6)
    for fmt, qm in ((F.INT4, 7), (F.INT4 | F.POW2, 7), (0, 127), (F.POW2, 127)):
        X = rng.integers(-qm, qm + 1, (10, 50)).astype(np.float32)
        X[:, 0] = qm
        Q, s = F.quantize_rows(X, fmt)
        assert np.all(s == 1.0) and np.array_equal(Q.astype(np.float32), X)


def test_pow2_epilogue_closed_form():
    """With power-of-two scales both epilogue multiplies are exact: out is
    RN(acc) * s_row * s_col exactly (no under- or overflow here)."""
    rng = np.random.default_rng(7)
    A = rng.standard_normal((20, 300)).astype(np.float32)
    B = (rng.standard_normal((300, 30)) * 0.02).astype(np.float32)
    for fa, fb in ((F.POW2, F.POW2), (F.INT4 | F.POW2, F.INT4 | F.POW2)):
        C, QA, sr, QB, sc = F.blockscaled_gemm(A, B, fa, fb)
        acc = QA.astype(np.int64) @ QB.astype(np.int64).T
        assert np.abs(acc).max() < 2**24
        want = acc.astype(np.float64) * sr[:, None].astype(np.float64) * sc[None, :].astype(np.float64)
        assert np.array_equal(C.astype(np.float64), want)


def test_int4_layout_golden():
    with open(os.path.join(HERE, "golden", "int4_layout.json")) as f:
        g = json.load(f)
    L = g["length"]
    codes = np.zeros((1, L), dtype=np.int8)
    for k, v in g["codes"].items():
        codes[0, int(k)] = v
    want = np.zeros(g["row_bytes"], dtype=np.uint8)
    for k, v in g["bytes"].items():
        want[int(k)] = v
    assert np.array_equal(F.pack_int4(codes)[0], want)
    assert F.brute_pack_int4(list(codes[0])) == list(want)
    assert np.array_equal(F.unpack_int4(want[None, :], L), codes)


@pytest.mark.parametrize("L", [1, 15, 16, 17, 31, 32, 33, 64, 100])
def test_int4_pack_roundtrip_and_brute(L):
    rng = np.random.default_rng(L)
    codes = rng.integers(-8, 8, (6, L)).astype(np.int8)
    P = F.pack_int4(codes)
    assert P.shape == (6, F.int4_row_bytes(L))
    assert np.array_equal(F.unpack_int4(P, L), codes)
    for i in range(6):
        assert list(P[i]) == F.brute_pack_int4(list(codes[i]))
    # nibbles past the end are zero
    if L % 32:
        full = F.unpack_int4(P, F.int4_row_bytes(L) * 2)
        assert np.all(full[:, L:] == 0)


def test_formats_zero_is_the_method():
    """Format 0 is exactly the int8 absmax method of oracle.ref."""
    X = _lines(9, 16, 77)
    Q, s = F.quantize_rows(X, 0)
    Q2, s2 = ref.quantize_rows(X)
    assert np.array_equal(Q, Q2) and np.array_equal(s, s2)
