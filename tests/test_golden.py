"""Hand-derived worked examples (tests/golden/*.json) against the oracle.

Each fixture cites the passage it follows and carries its derivation; the
values in it were worked out by hand, not produced by any code here.
"""
import json
import os

import numpy as np

from oracle import brute, ref

F32 = np.float32
U32 = np.uint32


def _load(repo_root, name):
    with open(os.path.join(repo_root, "tests", "golden", name)) as f:
        return json.load(f)


def _hexes(rows):
    return np.array([[int(b, 16) for b in row] for row in rows], dtype=np.uint64).astype(U32)


def test_worked_example_numpy_oracle(repo_root):
    g = _load(repo_root, "worked_example_pow2.json")
    A = np.array(g["A"], dtype=F32)
    B = np.array(g["B"], dtype=F32)
    A[1, 1] = F32(-0.0)
    C, QA, s_row, QBt, s_col = ref.blockscaled_gemm(A, B)
    assert QA.tolist() == g["QA"] and QBt.tolist() == g["QBt"]
    assert [hex(int(v)) for v in s_row.view(U32)] == g["s_row_bits"]
    assert [hex(int(v)) for v in s_col.view(U32)] == g["s_col_bits"]
    assert ref.accumulate(QA, QBt).tolist() == g["acc"]
    assert np.array_equal(C.view(U32), _hexes(g["out_bits"]))
    assert C.tolist() == g["out"]
    Cr, *_ = ref.blockscaled_gemm(A, B, relu=True)
    assert np.array_equal(Cr.view(U32), _hexes(g["out_relu_bits"]))


def test_worked_example_brute_force(repo_root):
    g = _load(repo_root, "worked_example_pow2.json")
    A = np.array(g["A"], dtype=F32)
    A[1, 1] = F32(-0.0)
    B = np.array(g["B"], dtype=F32)
    rows = lambda X: [[int(v) for v in r] for r in X.view(U32)]
    out, ex = brute.gemm(rows(A), rows(B))
    assert ex["acc"] == g["acc"] and ex["QA"] == g["QA"]
    assert np.array_equal(np.array(out, dtype=np.uint64).astype(U32), _hexes(g["out_bits"]))
