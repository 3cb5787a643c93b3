"""Pins of the oracle's contraction and epilogue (oracle/ref.py, oracle/brute.py).

Page: DaisyChain-Train "Verification — why you can trust the numbers":
section "The verified INT8 units" steps 2-3 (exact int32 accumulation, the
epilogue f32(f32(f32(acc)*a)*b)), section "Layer 4" (the referee rejects a
round-once epilogue on a large share of inputs) and section "Layer 5"
(relations: row permutation, zero rows, batch decomposition, single-cell
sensitivity; absolutes: ReLU output never negative, unit scales give the
exact integer dot product).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute, hashref, ieee32 as I, ref

F32 = np.float32
U32 = np.uint32


def _bits_rows(X):
    return [[int(v) for v in row] for row in np.asarray(X, dtype=F32).view(U32)]


def _tiny_cases():
    rng = np.random.default_rng(31)
    for M in range(1, 5):
        for N in range(1, 5):
            for K in range(1, 6):
                A = rng.standard_t(2, (M, K)).astype(F32)
                B = rng.standard_t(2, (K, N)).astype(F32)
                A[rng.random((M, K)) < 0.1] = F32(-0.0)
                if rng.random() < 0.2:
                    A[0] = 0
                yield A, B, bool(rng.random() < 0.5)


def test_numpy_oracle_equals_exact_rational_brute_force():
    """T5: every rounding of brute.py is exact-rational; ref.py uses the host
    FPU and float64 BLAS.  All M, N <= 4, K <= 5 (with -0 and zero rows)."""
    for A, B, relu in _tiny_cases():
        C, QA, s_row, QBt, s_col = ref.blockscaled_gemm(A, B, relu)
        out, ex = brute.gemm(_bits_rows(A), _bits_rows(B), relu)
        assert np.array_equal(C.view(U32), np.array(out, dtype=np.uint64).astype(U32).reshape(C.shape))
        assert QA.tolist() == ex["QA"] and QBt.tolist() == ex["QBt"]
        assert s_row.view(U32).tolist() == ex["s_row"] and s_col.view(U32).tolist() == ex["s_col"]
        assert hashref.output_hash(C) == brute.output_hash(out)


def test_float64_contraction_is_exact():
    """acc via float64 BLAS equals int64 accumulation, incl. |acc| near 2^31."""
    rng = np.random.default_rng(32)
    QA = rng.integers(-127, 128, (33, 777)).astype(np.int8)
    QB = rng.integers(-127, 128, (45, 777)).astype(np.int8)
    exact = QA.astype(np.int64) @ QB.astype(np.int64).T
    assert np.array_equal(ref.accumulate(QA, QB), exact)
    K = ref.K_MAX
    assert K == 133144 and 127 * 127 * K <= 2**31 - 1 < 127 * 127 * (K + 1)
    a = np.full((2, K), 127, dtype=np.int8)
    a[1, ::2] = -127
    b = np.full((2, K), 127, dtype=np.int8)
    b[1, 1::3] = -127
    got = ref.accumulate(a, b)
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(got, want) and got[0, 0] == 127 * 127 * K


def test_unit_scales_give_exact_integer_dot_product():
    """Absolute of section "Layer 5": integer rows/columns whose absmax is 127
    have scale 1.0, so out = RN(sum a*b) = sum a*b for K <= 1040."""
    rng = np.random.default_rng(33)
    for K in (1, 17, 255, 1040):
        A = rng.integers(-127, 128, (9, K)).astype(F32)
        B = rng.integers(-127, 128, (K, 11)).astype(F32)
        A[:, 0] = 127
        B[0, :] = -127
        C, QA, s_row, QBt, s_col = ref.blockscaled_gemm(A, B)
        assert np.all(s_row == 1) and np.all(s_col == 1)
        exact = [[sum(int(A[i, k]) * int(B[k, j]) for k in range(K)) for j in range(11)]
                 for i in range(9)]
        assert C.astype(np.int64).tolist() == exact
        assert np.all(np.abs(np.array(exact)) < 2**24)


def test_epilogue_conversion_ladder_above_2_pow_24():
    """RN(acc) above 2^24 ties to even, checked through the whole method:
    unit scales and a constructed acc = 2^24 + j."""
    K = 2200
    for target in (2**24 + 1, 2**24 + 2, 2**24 + 3, 2**24 + 5, 2**25 + 2, 2**25 + 6):
        # 127*127*q + r*127 + rest: choose ints with |x| <= 127
        a = np.zeros(K, dtype=np.int64)
        b = np.zeros(K, dtype=np.int64)
        rem = target
        k = 0
        while rem >= 127 * 127:
            a[k] = b[k] = 127
            rem -= 127 * 127
            k += 1
        a[k], b[k] = 127, rem // 127
        a[k + 1], b[k + 1] = rem % 127, 1
        assert int(a @ b) == target
        C, *_ = ref.blockscaled_gemm(a[None, :].astype(F32), b[:, None].astype(F32))
        step = 2 if target < 2**25 else 4
        assert Fraction(float(C[0, 0])) == round(Fraction(target, step)) * step


def test_epilogue_power_of_two_scales_closed_form():
    """s_row = 2^e1, s_col = 2^e2 exactly: out = RN(acc) * 2^(e1+e2)."""
    rng = np.random.default_rng(34)
    K = 300
    A = rng.integers(-127, 128, (5, K)).astype(F32)
    B = rng.integers(-127, 128, (K, 6)).astype(F32)
    A[:, 0] = 127
    B[0, :] = 127
    e1 = np.array([-3, 0, 4, -20, 9])
    e2 = np.array([2, -7, 0, 11, -1, 5])
    As = (A * (2.0 ** e1)[:, None]).astype(F32)
    Bs = (B * (2.0 ** e2)[None, :]).astype(F32)
    C, QA, s_row, QBt, s_col = ref.blockscaled_gemm(As, Bs)
    assert np.array_equal(s_row, 2.0 ** e1) and np.array_equal(s_col, 2.0 ** e2)
    acc = A.astype(np.int64) @ B.astype(np.int64)
    want = acc.astype(np.float64) * (2.0 ** e1)[:, None] * (2.0 ** e2)[None, :]
    assert np.array_equal(C.astype(np.float64), want)


def test_round_once_epilogue_is_rejected_often():
    """Section "Layer 4": the referee rejects the older round-once epilogue
    RN(acc*a*b) on ~34% of inputs.  The share depends on the distribution;
    it must be large (> 20%) here and the pinned epilogue must differ from it."""
    rng = np.random.default_rng(35)
    n = 20_000
    acc = rng.integers(-(2**27), 2**27, n)
    sa = (np.abs(rng.standard_normal(n)) * 0.03 + 1e-3).astype(F32)
    sb = (np.abs(rng.standard_normal(n)) * 1e-3 + 1e-5).astype(F32)
    y3 = ((acc.astype(F32) * sa).astype(F32) * sb).astype(F32)
    once = np.array([I.round_fraction(Fraction(int(a)) * I.decode(x) * I.decode(y))
                     for a, x, y in zip(acc[:4000].tolist(), sa[:4000].view(U32).tolist(),
                                        sb[:4000].view(U32).tolist())], dtype=np.uint64)
    once = once.astype(U32).view(F32)
    share = np.mean(once != y3[:4000])
    assert share > 0.20, share
    # the referee agrees with the pinned schedule everywhere it checks
    for a, x, y, got in zip(acc[:2000].tolist(), sa[:2000].view(U32).tolist(),
                            sb[:2000].view(U32).tolist(), y3[:2000].view(U32).tolist()):
        assert I.mul(I.mul(I.from_int(a), x), y) == got


def test_scale_order_matters():
    """Row scale first, then column scale: the swapped order changes bytes."""
    rng = np.random.default_rng(36)
    A = rng.standard_normal((128, 256)).astype(F32)
    B = rng.standard_normal((256, 128)).astype(F32)
    C, QA, s_row, QBt, s_col = ref.blockscaled_gemm(A, B)
    acc = ref.accumulate(QA, QBt).astype(np.int32).astype(F32)
    swapped = ((acc * s_col[None, :]).astype(F32) * s_row[:, None]).astype(F32)
    share = np.mean(swapped.view(U32) != C.view(U32))
    assert share > 0.2, share


def test_relu_never_negative_and_zero_is_positive():
    rng = np.random.default_rng(37)
    A = rng.standard_normal((64, 100)).astype(F32)
    B = rng.standard_normal((100, 50)).astype(F32)
    A[3] = 0
    B[:, 7] = 0
    C, QA, s_row, QBt, s_col = ref.blockscaled_gemm(A, B, relu=True)
    assert np.all(C.view(U32) >> 31 == 0)             # no negative, no -0
    assert np.all(C[3].view(U32) == 0) and np.all(C[:, 7].view(U32) == 0)
    plain, *_ = ref.blockscaled_gemm(A, B, relu=False)
    assert np.array_equal(C, np.where(plain > 0, plain, 0))
    # a multiplicative ReLU y * (y > 0) produces -0 and is caught bitwise
    mult = (plain * (plain > 0)).astype(F32)
    assert np.any(mult.view(U32) != C.view(U32))
    assert np.all(mult == C)                            # while float == is blind


def test_metamorphic_relations():
    """Section "Layer 5" relations on the oracle."""
    rng = np.random.default_rng(38)
    A = rng.standard_t(2, (70, 90)).astype(F32)
    B = rng.standard_t(2, (90, 60)).astype(F32)
    C, *_ = ref.blockscaled_gemm(A, B)
    # permuting rows permutes outputs
    p = rng.permutation(70)
    Cp, *_ = ref.blockscaled_gemm(A[p], B)
    assert np.array_equal(Cp.view(U32), C[p].view(U32))
    # a zero row of A / column of B yields +0 across it
    A0 = A.copy(); A0[5] = 0
    B0 = B.copy(); B0[:, 9] = 0
    C0, *_ = ref.blockscaled_gemm(A0, B0)
    assert np.all(C0[5].view(U32) == 0) and np.all(C0[:, 9].view(U32) == 0)
    # batches decompose: row blocks and column blocks give identical pieces
    top, *_ = ref.blockscaled_gemm(A[:31], B)
    right, *_ = ref.blockscaled_gemm(A, B[:, 17:])
    assert np.array_equal(top.view(U32), C[:31].view(U32))
    assert np.array_equal(right.view(U32), C[:, 17:].view(U32))
    # single-cell sensitivity: changing A[i,k] changes only row i
    A1 = A.copy(); A1[11, 4] += F32(3.0)
    C1, *_ = ref.blockscaled_gemm(A1, B)
    changed = np.any(C1.view(U32) != C.view(U32), axis=1)
    assert changed[11] and changed.sum() == 1
    B1 = B.copy(); B1[4, 13] += F32(3.0)
    C2, *_ = ref.blockscaled_gemm(A, B1)
    changed = np.any(C2.view(U32) != C.view(U32), axis=0)
    assert changed[13] and changed.sum() == 1


def test_output_cell_agrees_with_full_oracle():
    rng = np.random.default_rng(39)
    A = rng.standard_normal((20, 40)).astype(F32)
    B = rng.standard_normal((40, 30)).astype(F32)
    for relu in (False, True):
        C, QA, s_row, QBt, s_col = ref.blockscaled_gemm(A, B, relu)
        for i, j in [(0, 0), (19, 29), (7, 3)]:
            v = ref.output_cell(QA[i], s_row[i], QBt[j], s_col[j], relu)
            assert v.view(U32) == C[i, j].view(U32)
