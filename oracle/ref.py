"""The block-scaled int8 GEMM in plain numpy, one IEEE binary32 op per step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: DaisyChain-Train page "Verification — why you can trust the numbers",
section "The verified INT8 units":

  step 1  inputs are quantized per row (of A) and per column (of B) with
          scale = max(|row|)/127 floored at 1e-8, values to int8;
  step 2  products of int8 values, accumulated exactly in int32;
  step 3  the epilogue f32(f32(f32(acc)*a)*b): round to binary32 after the
          int->float conversion and after each multiply.

Readings taken where the page leaves a step open (all listed in the design doc):
  * the scale is rounded to binary32: s = max(RN(a/127), RN(1e-8)), with a
    correctly rounded binary32 division (the page derives it in f64 and
    stores f32; for a division, one correctly rounded f32 division gives the
    same value as the f64 division rounded to f32);
  * values go to int8 through the reciprocal of the stored scale:
    inv = RN(1/s), t = RN(x*inv), u = RN(t + 0.5), q = floor(u)  -- two
    roundings, never fused (section "Hardware ground truth (RDNA2 ISA
    audit)" discusses the fused form; it is NOT equivalent near |x*inv| =
    0.5);
  * the epilogue multiplies by the row scale of A first, then by the column
    scale of B: out = RN(RN(RN(acc)*s_row[i])*s_col[j]);
  * the fused ReLU (section "Layer 5: properties and mutation scores":
    output never negative) is out = (y > 0) ? y : +0.

numpy float32 ufuncs round each operation to nearest-even on the host FPU
with no contraction; the int8 contraction is done in float64, which is exact
here (products are integers below 2^14, every partial sum an integer below
127^2 * K <= 2^31 < 2^53, so no rounding occurs in any summation order) and
is cross-checked against int64 on small shapes by the tests.
"""
import numpy as np

F32 = np.float32
SCALE_FLOOR = F32(1e-8)       # RN(1e-8) = 0x322BCC77
QMAX = F32(127.0)
HALF = F32(0.5)
ONE = F32(1.0)
K_MAX = (2**31 - 1) // (127 * 127)   # 133144: largest K with |acc| < 2^31


def absmax_rows(X):
    """a_i = max_k |X[i, k]| (|-0| = 0); a row of length 0 has a_i = 0."""
    X = np.asarray(X, dtype=F32)
    if X.shape[1] == 0:
        return np.zeros(X.shape[0], dtype=F32)
    return np.max(np.abs(X), axis=1)


def scales_from_absmax(a):
    """s = max(RN(a/127), RN(1e-8)) and inv = RN(1/s), both binary32."""
    a = np.asarray(a, dtype=F32)
    s = np.maximum(a / QMAX, SCALE_FLOOR)
    inv = ONE / s
    return s.astype(F32), inv.astype(F32)


def quantize_values(X, inv_b):
    """q = floor(RN(RN(x*inv) + 0.5)) as int8; ``inv_b`` broadcasts over X."""
    t = (np.asarray(X, dtype=F32) * inv_b).astype(F32)     # RN(x*inv)
    u = (t + HALF).astype(F32)                              # RN(t + 0.5)
    q = np.floor(u)                                         # exact
    assert np.all(np.abs(q) <= 127), "quantized value outside [-127, 127]"
    return q.astype(np.int8)


def quantize_rows(X):
    """Per-row quantization of X (R x C) -> (Q int8 R x C, scale f32 R)."""
    X = np.asarray(X, dtype=F32)
    s, inv = scales_from_absmax(absmax_rows(X))
    return quantize_values(X, inv[:, None]), s


def quantize_cols(X):
    """Per-column quantization of X (R x C) -> (Qt int8 C x R, scale f32 C).

    The int8 output is the transpose, so that both GEMM operands are
    contiguous along the contraction index.
    """
    X = np.asarray(X, dtype=F32)
    Q, s = quantize_rows(np.ascontiguousarray(X.T))
    return Q, s


def accumulate(QA, QBt):
    """acc[i, j] = sum_k QA[i, k] * QBt[j, k], exact, returned as int64."""
    QA = np.asarray(QA, dtype=np.int8)
    QBt = np.asarray(QBt, dtype=np.int8)
    K = QA.shape[1]
    assert QBt.shape[1] == K
    assert K <= K_MAX, "K beyond the exact int32 range"
    acc = QA.astype(np.float64) @ QBt.astype(np.float64).T
    return acc.astype(np.int64)


def epilogue(acc, s_row, s_col, relu=False):
    """out = RN(RN(RN(acc) * s_row[i]) * s_col[j]); ReLU gives +0 for y <= 0."""
    acc = np.asarray(acc, dtype=np.int64)
    assert np.all(np.abs(acc) <= 2**31 - 1)
    y = acc.astype(np.int32).astype(F32)                       # RN(acc)
    y = (y * np.asarray(s_row, dtype=F32)[:, None]).astype(F32)
    y = (y * np.asarray(s_col, dtype=F32)[None, :]).astype(F32)
    if relu:
        y = np.where(y > F32(0), y, F32(0)).astype(F32)
    return y


def gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu=False):
    """C (M x N f32) from int8 QA (M x K), QBt (N x K) and their scales."""
    return epilogue(accumulate(QA, QBt), s_row, s_col, relu)


def blockscaled_gemm(A, B, relu=False):
    """The whole method on f32 inputs: A (M x K) per-row, B (K x N) per-column.

    Returns (C, QA, s_row, QBt, s_col).
    """
    QA, s_row = quantize_rows(A)
    QBt, s_col = quantize_cols(B)
    return gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu), QA, s_row, QBt, s_col


def output_cell(QA_row, s_row_i, QBt_row, s_col_j, relu=False):
    """One output element, computed on its own (for sampled checks)."""
    acc = int(np.dot(np.asarray(QA_row, dtype=np.int64),
                     np.asarray(QBt_row, dtype=np.int64)))
    return epilogue(np.array([[acc]]), np.array([s_row_i], dtype=F32),
                    np.array([s_col_j], dtype=F32), relu)[0, 0]
