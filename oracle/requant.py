"""The requantizing epilogue: a GEMM whose output leaves as int8 codes and
per-row scales, ready to be the A operand of the next GEMM.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: the presk page, section "What is left open" (quantisation of
activations, W8A8, with int32 accumulation and requantisation), and the
DaisyChain-Train page "Verification -- why you can trust the numbers",
section "Layer 1: exact init gates" (a gate over a back-to-back chain of
quantized GEMMs).

Reading: the requantized output is exactly what the method gives when the
f32 output is formed (steps 2-3 of "The verified INT8 units") and then
quantized per row (step 1): codes and scales are quantize_rows(C).  So the
oracle is that composition of two pinned functions; the tests pin the
composition once more against the exact-rational brute force.
"""
from . import ref


def gemm_requant(QA, s_row, QBt, s_col, relu=False):
    """(Q, s, C): Q, s = quantize_rows(C) with C the method's f32 output."""
    C = ref.gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu)
    Q, s = ref.quantize_rows(C)
    return Q, s, C
