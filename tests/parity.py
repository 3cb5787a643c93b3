"""The comparison the GPU parity tests apply to every stage of the method,
shared with the CPU mutation scoring (tests/test_mutation_scores.py) so that
the checker scored there is exactly the one the GPU runs face.

Bit-exact: int8 bytes, scale bit patterns, output bit patterns (-0 and +0
differ) and the 64-bit output hash, against the oracle run on the same f32
inputs (DaisyChain-Train page "Verification -- why you can trust the
numbers", section "Layer 1: exact init gates": comparisons at the bit level).
"""
import numpy as np

from oracle import hashref, ref

U32 = np.uint32


def assert_bits(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        bad = got.view(U32) != want.view(U32)
    else:
        bad = got != want
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(i), got[tuple(i)], want[tuple(i)]) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ, e.g. {detail}")


def check_against_oracle(got, A, B, relu):
    """got: dict of the stages QA, s_row, QBt, s_col, C (numpy) and hash (int)."""
    C, QA, s_row, QBt, s_col = ref.blockscaled_gemm(A, B, relu)
    assert_bits(got["QA"], QA, "QA")
    assert_bits(got["s_row"], s_row, "s_row")
    assert_bits(got["QBt"], QBt, "QBt")
    assert_bits(got["s_col"], s_col, "s_col")
    assert_bits(got["C"], C, "C")
    assert got["hash"] == hashref.output_hash(C), "hash"
    return C
