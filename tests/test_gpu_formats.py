"""GPU parity of the storage formats (presk page, section "Integer weights":
int8 / int4 values, absmax / power-of-two scales) against oracle/formats.py,
bit for bit: quantize outputs (int4: the packed bytes), GEMM outputs and
hashes with int4 operands."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import hashref, ref

pytestmark = pytest.mark.gpu

FMTS = [F.POW2, F.INT4, F.INT4 | F.POW2]


def say(*a):
    print("[formats]", *a, flush=True)


@pytest.fixture(scope="module")
def g():
    import int8_gemm_amd as g
    g.load()
    assert g.FMT_POW2 == F.POW2 and g.FMT_INT4 == F.INT4
    return g


def _data(seed, rows, cols):
    rng = np.random.default_rng(seed)
    X = rng.standard_t(2, (rows, cols)).astype(np.float32)
    if rows > 3:
        X[1] = 0.0
        X[3] *= np.float32(1e-12)
    if cols > 3:
        X[:, 2] = 0.0
    return X


def _bytes(t):
    return t.cpu().numpy().view(np.uint8)


QSHAPES = [(1, 1), (5, 31), (7, 32), (33, 33), (100, 70), (300, 1000), (64, 4097), (1500, 96)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", QSHAPES)
def test_quantize_formats(g, fmt, shape):
    rows, cols = shape
    say("quantize fmt", fmt, rows, cols)
    X = _data(rows * 7 + cols, rows, cols)
    Xd = torch.from_numpy(X).cuda()
    Q, s = g.quantize_rows_fmt(Xd, fmt)
    Qt, st = g.quantize_cols_fmt(Xd, fmt)
    torch.cuda.synchronize()
    qr, sr = F.quantize_rows(X, fmt)
    qc, sc = F.quantize_cols(X, fmt)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(st.cpu().numpy().view(np.uint32), sc.view(np.uint32))
    if fmt & F.INT4:
        assert np.array_equal(_bytes(Q), F.pack_int4(qr))
        assert np.array_equal(_bytes(Qt), F.pack_int4(qc))
    else:
        assert np.array_equal(Q.cpu().numpy(), qr)
        assert np.array_equal(Qt.cpu().numpy(), qc)


def _upload_int4(codes):
    P = F.pack_int4(codes)
    return torch.from_numpy(P.view(np.int8)).cuda()


def _upload_int8(codes):
    M, K = codes.shape
    ld = max(16, (K + 15) // 16 * 16)
    buf = np.zeros((M, ld), dtype=np.int8)
    buf[:, :K] = codes
    return torch.from_numpy(buf).cuda()[:, :K]


GSHAPES = [(1, 1, 1), (17, 33, 15), (130, 190, 70), (300, 520, 192), (256, 256, 1000), (129, 65, 4097)]


@pytest.fixture(params=["widened", "direct"])
def int4_path(request, g):
    """int4 operands widened to int8 for the int8 kernels (the default), or
    read packed by gemm_i4_kernel (the int4_direct plan override)."""
    with g.plan_overrides(int4_direct=request.param == "direct"):
        yield request.param


@pytest.mark.parametrize("combo", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("shape", GSHAPES)
def test_gemm_int4_operands(g, combo, shape, int4_path):
    a4, b4 = combo
    M, N, K = shape
    relu = (M + N) % 2 == 1
    say("gemm int4", int4_path, a4, b4, M, N, K, relu)
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    A = rng.standard_t(3, (M, K)).astype(np.float32)
    B = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    fa = F.INT4 if a4 else 0
    fb = (F.INT4 | F.POW2) if b4 else F.POW2
    C_ref, QA, sr, QB, sc = F.blockscaled_gemm(A, B, fa, fb, relu)
    dA = _upload_int4(QA) if a4 else _upload_int8(QA)
    dB = _upload_int4(QB) if b4 else _upload_int8(QB)
    C, h = g.gemm_i8_blockscaled(dA, torch.from_numpy(sr).cuda(), dB, torch.from_numpy(sc).cuda(),
                                 relu=relu, want_hash=True, K=K, a_int4=a4, b_int4=b4)
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), C_ref.view(np.uint32))
    assert g.hash_value(h) == hashref.output_hash(C_ref)


def test_gemm_int4_forced_splits(g, int4_path):
    """Split K with int4 operands (the partial sums are shifted back before
    they are stored, so the combine is the int8 one)."""
    M, N, K = 96, 200, 4160
    rng = np.random.default_rng(5)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    C_ref, QA, sr, QB, sc = F.blockscaled_gemm(A, B, F.INT4, F.INT4)
    with g.plan_overrides(force_splits=5):
        assert g.plan_query(M, N, K, flags=g.I8G_B_INT4)[1] == 5
        for a4 in (True, False):
            say("gemm int4 split", a4)
            QA_use = QA if a4 else ref.quantize_rows(A)[0]
            sr_use = sr if a4 else ref.quantize_rows(A)[1]
            want = ref.gemm_i8_blockscaled(QA_use, sr_use, QB, sc)
            dA = _upload_int4(QA_use) if a4 else _upload_int8(QA_use)
            C = g.gemm_i8_blockscaled(dA, torch.from_numpy(sr_use).cuda(), _upload_int4(QB),
                                      torch.from_numpy(sc).cuda(), K=K, a_int4=a4, b_int4=True)
            torch.cuda.synchronize()
            assert np.array_equal(C.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_whole_method_int4_weights_mlp_down(g, int4_path):
    """GPT-2-small MLP down-projection shape (2048 tokens) with int4 / pow2
    weights quantized on the device, activations int8: every step on the
    GPU, compared with the oracle bit for bit."""
    M, K, N = 2048, 3072, 768
    rng = np.random.default_rng(11)
    A = np.maximum(rng.standard_normal((M, K)), 0).astype(np.float32)
    B = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    for fb in (F.INT4, F.INT4 | F.POW2):
        say("mlp down int4 weights fmt", fb)
        C_ref, QA, sr, QB, sc = F.blockscaled_gemm(A, B, 0, fb)
        dA, dsr = g.quantize_rows(torch.from_numpy(A).cuda())
        dB, dsc = g.quantize_cols_fmt(torch.from_numpy(B).cuda(), fb)
        C, h = g.gemm_i8_blockscaled(dA, dsr, dB, dsc, want_hash=True, K=K, b_int4=True)
        torch.cuda.synchronize()
        assert np.array_equal(_bytes(dB), F.pack_int4(QB))
        assert np.array_equal(C.cpu().numpy().view(np.uint32), C_ref.view(np.uint32))
        assert g.hash_value(h) == hashref.output_hash(C_ref)


@pytest.mark.parametrize("tile", [6, 7])
def test_int4_weights_on_persistent_tiles(g, tile):
    """int4 weights widened to int8 codes and multiplied by each 128-byte-stage
    persistent tile (forced), up-projection shape with 1024 tokens, ragged N
    and ReLU: bit for bit against the oracle."""
    M, K, N = 1024, 768, 1000
    rng = np.random.default_rng(40 + tile)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    C_ref, QA, sr, QB, sc = F.blockscaled_gemm(A, B, 0, F.INT4, relu=True)
    dA, dsr = g.quantize_rows(torch.from_numpy(A).cuda())
    dB, dsc = g.quantize_cols_fmt(torch.from_numpy(B).cuda(), F.INT4)
    say("int4 weights tile", tile)
    with g.plan_overrides(force_tile=tile):
        assert g.plan_query(M, N, K, flags=g.I8G_B_INT4)[0] == tile, "the forced plan did not run"
        C, h = g.gemm_i8_blockscaled(dA, dsr, dB, dsc, relu=True, want_hash=True, K=K, b_int4=True)
        torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().view(np.uint32), C_ref.view(np.uint32))
    assert g.hash_value(h) == hashref.output_hash(C_ref)


def test_format_argument_errors(g):
    lib = g.load()
    X = torch.zeros((4, 40), dtype=torch.float32, device="cuda")
    s = torch.empty(4, dtype=torch.float32, device="cuda")
    Q = torch.empty((4, 32), dtype=torch.int8, device="cuda")
    # unknown format bit
    assert lib.quantize_rows_fmt(X.data_ptr(), 4, 40, 40, Q.data_ptr(), 32, s.data_ptr(), 4, None) == 1
    # int4 line of 40 values needs 32 bytes: ldq 16 is too small
    assert lib.quantize_rows_fmt(X.data_ptr(), 4, 40, 40, Q.data_ptr(), 16, s.data_ptr(), 2, None) == 1
    # misaligned int4 output
    assert lib.quantize_rows_fmt(X.data_ptr(), 2, 40, 40, Q.data_ptr() + 1, 32, s.data_ptr(), 2, None) == 3


@pytest.mark.parametrize("fmt", [F.INT4, F.INT4 | F.POW2])
@pytest.mark.parametrize("two_pass", [False, True])
@pytest.mark.parametrize("shape", [(300, 1000), (8192, 40), (9000, 40), (31, 5)])
def test_int4_columns_both_paths(g, fmt, two_pass, shape):
    """int4 column passes on the one-kernel band path (up to 8192 rows,
    packed as they are stored) and on the multi-kernel path (forced here;
    taken by itself above 8192 rows)."""
    rows, cols = shape
    say("int4 cols", fmt, "two_pass", two_pass, rows, cols)
    X = _data(rows + cols + fmt, rows, cols)
    with g.plan_overrides(qcols_path=1 if two_pass else 0):
        Qt, st = g.quantize_cols_fmt(torch.from_numpy(X).cuda(), fmt)
        torch.cuda.synchronize()
    qc, sc = F.quantize_cols(X, fmt)
    assert np.array_equal(st.cpu().numpy().view(np.uint32), sc.view(np.uint32))
    assert np.array_equal(_bytes(Qt), F.pack_int4(qc))
