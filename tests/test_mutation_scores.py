"""Mutation scores of the GPU parity checker, on the CPU.

The DaisyChain-Train page "Verification -- why you can trust the numbers",
section "Layer 5: properties and mutation scores", scores its checks by
planting known mistakes and counting how many the checks catch.  Here each
mutant is the method with one mistake a GEMM kernel could plausibly make,
built from the oracle's own steps; it is run on inputs of the kinds the GPU
tests use (the 256^3 GEMM, ragged adversarial cases with ReLU on odd cases,
a forced K split) and judged by tests/parity.check_against_oracle, the
comparison the GPU parity tests apply.  Every mutant must be caught by some
case, and the unmutated control by none.  Nothing here runs on a GPU.
"""
import numpy as np
import pytest

from oracle import hashref, ref
from synth import inputs as S
from tests.parity import check_against_oracle

F32 = np.float32
MASK64 = (1 << 64) - 1
BK = 64                                    # bytes of K per stage of the kernels


def stages(A, B, relu, acc_fn=ref.accumulate, epi_fn=ref.epilogue, hash_fn=hashref.output_hash):
    """The method on f32 inputs with replaceable steps; returns what the GPU
    tests read back (quantized operands, scales, output, hash)."""
    QA, s_row = ref.quantize_rows(A)
    QBt, s_col = ref.quantize_cols(B)
    C = epi_fn(acc_fn(QA, QBt), s_row, s_col, relu)
    return dict(QA=QA, s_row=s_row, QBt=QBt, s_col=s_col, C=C, hash=hash_fn(C))


# ---- the mutants: one plausible kernel mistake each ----
def acc_drop_split(QA, QBt, splits=5):
    """Split K as the kernels do (whole 64-byte stages per split) and lose the
    last split's partial sums."""
    K = QA.shape[1]
    kst = -(-K // BK)
    per = -(-kst // splits) * BK
    last = (min(splits, -(-kst * BK // per)) - 1) * per
    return ref.accumulate(QA, QBt) - ref.accumulate(QA[:, last:], QBt[:, last:])


def acc_int16_saturating(QA, QBt):
    """A 16-bit accumulator that saturates instead of holding the exact sum."""
    a = QA.astype(np.int64)
    b = QBt.astype(np.int64)
    acc = np.zeros((a.shape[0], b.shape[0]), dtype=np.int64)
    for k in range(a.shape[1]):
        acc = np.clip(acc + np.outer(a[:, k], b[:, k]), -32768, 32767)
    return acc


def acc_k_tail_off_by_one(QA, QBt):
    """The mask of a ragged K tail drops its last valid byte."""
    K = QA.shape[1]
    if K % BK == 0:
        return ref.accumulate(QA, QBt)
    return ref.accumulate(QA[:, :K - 1], QBt[:, :K - 1])


def acc_n_edge_off_by_one(QA, QBt):
    """A ragged last column tile clamps its column index one short: the last
    column repeats its neighbour's sums."""
    acc = ref.accumulate(QA, QBt)
    if acc.shape[1] % 16 != 0 and acc.shape[1] > 1:
        acc[:, -1] = acc[:, -2]
    return acc


def epi_scales_swapped(acc, s_row, s_col, relu=False):
    """Column scale applied before the row scale."""
    y = np.asarray(acc, dtype=np.int64).astype(np.int32).astype(F32)
    y = (y * s_col[None, :]).astype(F32)
    y = (y * s_row[:, None]).astype(F32)
    return np.where(y > 0, y, F32(0)).astype(F32) if relu else y


def epi_relu_negative_zero(acc, s_row, s_col, relu=False):
    """ReLU as a multiplication by (y > 0): negative outputs become -0."""
    y = ref.epilogue(acc, s_row, s_col, relu=False)
    return (y * (y > 0).astype(F32)).astype(F32) if relu else y


def hash_row_index_shifted(C):
    """Hash terms taken with the row key of the next row."""
    m, n = C.shape
    return hashref.finalize(hashref.partial_sum(C, 1) & MASK64, m, n)


MUTANTS = {
    "dropped split-K chunk": dict(acc_fn=acc_drop_split),
    "int16 saturating accumulator": dict(acc_fn=acc_int16_saturating),
    "K tail off by one": dict(acc_fn=acc_k_tail_off_by_one),
    "ragged N edge off by one": dict(acc_fn=acc_n_edge_off_by_one),
    "swapped scale order": dict(epi_fn=epi_scales_swapped),
    "-0 from ReLU": dict(epi_fn=epi_relu_negative_zero),
    "wrong hash row index": dict(hash_fn=hash_row_index_shifted),
}


def cases():
    """Inputs of the GPU tests' kinds: the 256^3 GEMM, ragged adversarial
    cases (ReLU on odd ones), and a long K that the kernels split."""
    A, B = S.w1_inputs()
    out = [("w1 256^3", A, B, False)]
    for c in range(6):
        case = S.adversarial_case(c)
        if max(case.shape) <= 700:        # bound the int16 mutant's K loop
            out.append((f"adversarial {c}", case.A, case.B, case.relu))
    rng = np.random.default_rng(77)
    out.append(("split K 60x70x3000", rng.standard_t(3, (60, 3000)).astype(F32),
                rng.standard_normal((3000, 70)).astype(F32), True))
    return out


CASES = cases()


def caught(kw, A, B, relu):
    try:
        check_against_oracle(stages(A, B, relu, **kw), A, B, relu)
    except AssertionError:
        return True
    return False


def test_cases_cover_what_the_mutants_need():
    assert any(r for *_, r in CASES), "a ReLU case"
    assert any(A.shape[1] % BK for _, A, _, _ in CASES), "a ragged K"
    assert any(B.shape[1] % 16 for _, _, B, _ in CASES), "a ragged N"
    assert len(CASES) >= 4


@pytest.mark.parametrize("name", list(CASES and [c[0] for c in CASES]))
def test_control_is_clean(name):
    _, A, B, relu = next(c for c in CASES if c[0] == name)
    assert not caught({}, A, B, relu), "the unmutated method failed the checker"


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_mutant_is_caught(mutant):
    kills = [name for name, A, B, relu in CASES if caught(MUTANTS[mutant], A, B, relu)]
    assert kills, f"mutant '{mutant}' survived every case"


def test_mutation_score():
    """Score = mutants caught / mutants (the page's "Layer 5" reports its
    score the same way); every mutant here must be caught."""
    killed = sum(any(caught(kw, A, B, relu) for _, A, B, relu in CASES) for kw in MUTANTS.values())
    assert killed == len(MUTANTS), f"mutation score {killed}/{len(MUTANTS)}"
