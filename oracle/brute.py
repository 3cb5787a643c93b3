"""The block-scaled int8 GEMM in pure Python, every rounding exact-rational.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Same method and readings as ``oracle.ref`` (DaisyChain-Train page
"Verification — why you can trust the numbers", section "The verified INT8
units", steps 1-3), but written with Python loops over 32-bit patterns and
``oracle.ieee32`` for each binary32 operation, so it shares neither code nor
host rounding with ``ref``.  Meant for tiny shapes (M, N, K <= ~8).

Inputs and outputs are lists of lists of binary32 bit patterns (ints);
quantized values are Python ints.
"""
from . import ieee32 as I
from . import hashref

_127 = I.from_int(127)
_ONE = I.from_int(1)
_HALF = I.round_fraction(__import__("fractions").Fraction(1, 2))
SCALE_FLOOR = I.round_fraction(__import__("fractions").Fraction(1, 10**8))


def scale_and_inv(vec):
    """(s, inv) for one row or column given as binary32 patterns."""
    a = 0                                   # +0
    for x in vec:
        a = I.max_(a, I.abs_(x))
    s = I.max_(I.div(a, _127), SCALE_FLOOR)
    return s, I.div(_ONE, s)


def quantize_vec(vec, inv):
    out = []
    for x in vec:
        t = I.mul(x, inv)
        u = I.add(t, _HALF)
        q = I.floor_int(u)
        assert -127 <= q <= 127
        out.append(q)
    return out


def gemm(A_bits, B_bits, relu=False):
    """A: M x K patterns, B: K x N patterns -> (out M x N patterns, extras).

    extras = dict(QA, s_row, QBt, s_col, acc).
    """
    M = len(A_bits)
    K = len(A_bits[0]) if M else 0
    N = len(B_bits[0]) if K else 0
    s_row, QA = [], []
    for i in range(M):
        s, inv = scale_and_inv(A_bits[i])
        s_row.append(s)
        QA.append(quantize_vec(A_bits[i], inv))
    s_col, QBt = [], []
    for j in range(N):
        col = [B_bits[k][j] for k in range(K)]
        s, inv = scale_and_inv(col)
        s_col.append(s)
        QBt.append(quantize_vec(col, inv))
    out, acc_all = [], []
    for i in range(M):
        row, arow = [], []
        for j in range(N):
            acc = 0
            for k in range(K):
                acc += QA[i][k] * QBt[j][k]
            arow.append(acc)
            y = I.from_int(acc)
            y = I.mul(y, s_row[i])
            y = I.mul(y, s_col[j])
            if relu and not I.gt_zero(y):
                y = 0
            row.append(y)
        out.append(row)
        acc_all.append(arow)
    return out, dict(QA=QA, s_row=s_row, QBt=QBt, s_col=s_col, acc=acc_all)


def output_hash(out_bits):
    M = len(out_bits)
    N = len(out_bits[0]) if M else 0
    return hashref.output_hash_py(out_bits, M, N)
