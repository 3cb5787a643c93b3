"""Property-based pins of the oracle's quantizer over the whole finite
binary32 range (subnormals, values near FLT_MAX, signed zeros): the numpy
oracle (one float32 operation per step) against the exact-rational version
written from the IEEE-754 definition, in every storage format."""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import formats as F
from oracle import ieee32 as I
from oracle import ref

finite32 = st.floats(width=32, allow_nan=False, allow_infinity=False)
lines = st.lists(finite32, min_size=1, max_size=24)


@settings(max_examples=300, deadline=None)
@given(lines, st.sampled_from([0, F.POW2, F.INT4, F.INT4 | F.POW2]))
def test_quantize_line_any_finite_values(vals, fmt):
    x = np.array(vals, dtype=np.float32)[None, :]
    q, s = F.quantize_rows(x, fmt)
    qb, sb = F.brute_quantize([I.bits_of(float(v)) for v in x[0]], fmt)
    assert I.bits_of(float(s[0])) == sb
    assert [int(v) for v in q[0]] == qb
    if fmt == 0:
        q2, s2 = ref.quantize_rows(x)
        assert np.array_equal(q2, q) and np.array_equal(s2, s)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(min_value=-2.0 ** -100, max_value=2.0 ** -100, width=32, allow_nan=False), min_size=1,
                max_size=16))
def test_tiny_lines_take_the_floor(vals):
    """Lines whose max is below 127 * RN(1e-8) take the floor scale, and
    their codes come from x * RN(1/RN(1e-8)) (subnormal inputs included)."""
    x = np.array(vals, dtype=np.float32)[None, :]
    q, s = ref.quantize_rows(x)
    assert s[0] == ref.SCALE_FLOOR
    qb, sb = F.brute_quantize([I.bits_of(float(v)) for v in x[0]], 0)
    assert [int(v) for v in q[0]] == qb


@settings(max_examples=200, deadline=None)
@given(st.integers(min_value=1, max_value=5), st.integers(min_value=1, max_value=5),
       st.integers(min_value=1, max_value=6), st.integers(min_value=0, max_value=2**32 - 1))
def test_gemm_equals_exact_rational_on_random_tiny_shapes(M, N, K, seed):
    """The whole method (numpy oracle) against the pure-Python exact-rational
    brute force on random tiny shapes with heavy-tailed values."""
    from oracle import brute
    rng = np.random.default_rng(seed)
    A = (rng.standard_t(2, (M, K)) * 10.0 ** rng.integers(-6, 6)).astype(np.float32)
    B = (rng.standard_t(2, (K, N)) * 10.0 ** rng.integers(-6, 6)).astype(np.float32)
    relu = bool(seed & 1)
    C = ref.blockscaled_gemm(A, B, relu)[0]
    bits = lambda X: [[I.bits_of(float(v)) for v in row] for row in X]
    out, _ = brute.gemm(bits(A), bits(B), relu)
    assert [[I.bits_of(float(v)) for v in row] for row in C] == out
