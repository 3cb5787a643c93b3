"""Pins of the requantizing epilogue in the oracle (oracle/requant.py)."""
import numpy as np

from oracle import brute, ieee32 as I, ref, requant


def test_requant_equals_exact_rational_chain():
    """Tiny shapes: the numpy composition against the pure-Python exact-
    rational GEMM followed by its own per-row quantizer."""
    rng = np.random.default_rng(1)
    for M, N, K in ((1, 1, 1), (3, 4, 5), (4, 3, 2), (2, 5, 4)):
        for relu in (False, True):
            A = rng.standard_t(3, (M, K)).astype(np.float32)
            B = rng.standard_normal((K, N)).astype(np.float32)
            bits = lambda X: [[I.bits_of(float(v)) for v in row] for row in X]
            out, _ = brute.gemm(bits(A), bits(B), relu)
            QA, sA = ref.quantize_rows(A)
            QB, sB = ref.quantize_cols(B)
            Q, s, C = requant.gemm_requant(QA, sA, QB, sB, relu)
            for i in range(M):
                sc, inv = brute.scale_and_inv(out[i])
                assert I.bits_of(float(s[i])) == sc
                assert brute.quantize_vec(out[i], inv) == [int(q) for q in Q[i]]


def test_requant_properties():
    """Rows above the floor reach |q| = 127 at their max; a row that ReLU
    empties gets the floor scale and zero codes."""
    rng = np.random.default_rng(2)
    A = rng.standard_normal((40, 64)).astype(np.float32)
    A[5] = -np.abs(A[5])
    B = np.abs(rng.standard_normal((64, 30))).astype(np.float32)   # row 5: every output <= 0
    QA, sA = ref.quantize_rows(A)
    QB, sB = ref.quantize_cols(B)
    Q, s, C = requant.gemm_requant(QA, sA, QB, sB, relu=True)
    assert np.all(C[5] == 0) and s[5] == ref.SCALE_FLOOR and np.all(Q[5] == 0)
    live = s > ref.SCALE_FLOOR
    assert np.all(np.abs(Q[live]).max(axis=1) == 127)
    assert np.all(Q >= 0)                                           # ReLU output
