"""GPU parity of the requantizing epilogue (gemm_i8_requant) against the
oracle (oracle/requant.py: quantize_rows of the method's output) and against
the library's own two-call path, bit for bit, with the hash of the f32 output
that the call never stores."""

import numpy as np
import pytest
import torch

from oracle import hashref, ref, requant

pytestmark = pytest.mark.gpu


def say(*a):
    print("[requant]", *a, flush=True)


@pytest.fixture(scope="module")
def g():
    import int8_gemm_amd as g
    g.load()
    return g


def _operands(g, M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_t(3, (M, K)).astype(np.float32)
    B = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    if M > 4:
        A[3] = 0.0                     # zero row: floor scale downstream
    QA, sA = ref.quantize_rows(A)
    QB, sB = ref.quantize_cols(B)
    dQA, dsA = g.quantize_rows(torch.from_numpy(A).cuda())
    dQB, dsB = g.quantize_cols(torch.from_numpy(B).cuda())
    return (QA, sA, QB, sB), (dQA, dsA, dQB, dsB)


SHAPES = [(1, 1, 1), (17, 33, 15), (130, 190, 70), (300, 520, 192), (256, 200, 768), (64, 64, 4096),
          (129, 1000, 33)]


@pytest.mark.parametrize("relu", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_requant_matches_oracle(g, shape, relu):
    M, N, K = shape
    say("requant", M, N, K, relu)
    (QA, sA, QB, sB), dev = _operands(g, M, N, K, M + N + K)
    Qw, sw, Cw = requant.gemm_requant(QA, sA, QB, sB, relu)
    Q, s, h = g.gemm_i8_requant(*dev, relu=relu, want_hash=True)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(Q.cpu().numpy(), Qw)
    assert g.hash_value(h) == hashref.output_hash(Cw)


@pytest.mark.parametrize("tile", [0, 1, 2])
def test_requant_every_tile(g, tile):
    M, N, K = 300, 700, 200
    say("requant tile", tile)
    (QA, sA, QB, sB), dev = _operands(g, M, N, K, 77)
    Qw, sw, Cw = requant.gemm_requant(QA, sA, QB, sB, True)
    with g.plan_overrides(force_tile=tile):
        Q, s, h = g.gemm_i8_requant(*dev, relu=True, want_hash=True)
        torch.cuda.synchronize()
    assert np.array_equal(Q.cpu().numpy(), Qw) and np.array_equal(s.cpu().numpy(), sw)
    assert g.hash_value(h) == hashref.output_hash(Cw)


# shapes the persistent 128x192 passes take (K % 128 == 0, K >= 768, M % 128
# == 0): ragged last column tile, N below one tile, more tiles than
# workgroups (the drained epilogue of the previous tile carries the row
# maxima and the codes), a long K
PERSIST_SHAPES = [(256, 200, 768, False), (512, 50, 1536, True), (4096, 1600, 768, True),
                  (1280, 1000, 896, False), (384, 640, 3072, True)]


@pytest.mark.parametrize("M,N,K,relu", PERSIST_SHAPES)
def test_requant_persistent(g, M, N, K, relu):
    """The persistent passes (partial row maxima per wave and tile, the
    scale kernel, codes from the reciprocals in the scale slot) against the
    oracle, with the hash of the never-stored f32 output."""
    say("requant persistent", M, N, K, relu)
    (QA, sA, QB, sB), dev = _operands(g, M, N, K, M * 3 + N + K)
    Qw, sw, Cw = requant.gemm_requant(QA, sA, QB, sB, relu)
    lib = g.load()
    with g.plan_overrides(force_tile=6):
        # the persistent plan's workspace holds a partial maximum per row for
        # each wave column of each tile column (two per 192 columns)
        assert lib.gemm_i8_requant_workspace_bytes(M, N, K) >= M * 4 * 2 * -(-N // 192)
        Q, s, h = g.gemm_i8_requant(*dev, relu=relu, want_hash=True)
        torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(Q.cpu().numpy(), Qw)
    assert g.hash_value(h) == hashref.output_hash(Cw)
    # the non-persistent passes give the same bytes
    with g.plan_overrides(force_tile=2):
        Q2, s2, h2 = g.gemm_i8_requant(*dev, relu=relu, want_hash=True)
        torch.cuda.synchronize()
    assert torch.equal(Q, Q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    assert g.hash_value(h) == g.hash_value(h2)


# shapes with K <= 1024, which the 128x128 passes with two workgroups per CU
# take by default: ragged last column tile, more tiles than workgroups, K of
# 7 and 8 stages
T7_SHAPES = [s for s in PERSIST_SHAPES if s[2] <= 1024] + [(512, 384, 1024, True), (4096, 2100, 768, False)]


@pytest.mark.parametrize("M,N,K,relu", T7_SHAPES)
def test_requant_persistent_two_per_cu(g, M, N, K, relu):
    """The 128x128 passes (two workgroups per CU; pass 1 reduces each tile's
    row maxima right after the tile's last k-step) against the oracle and
    against the 128x192 passes, bit for bit."""
    say("requant persistent 128x128", M, N, K, relu)
    (QA, sA, QB, sB), dev = _operands(g, M, N, K, M * 5 + N + K)
    Qw, sw, Cw = requant.gemm_requant(QA, sA, QB, sB, relu)
    lib = g.load()
    # the planner's choice for these shapes: one partial maximum per row for
    # each wave column of each 128-column tile
    assert lib.gemm_i8_requant_workspace_bytes(M, N, K) >= M * 4 * 2 * -(-N // 128)
    with g.plan_overrides(force_tile=7):
        assert lib.gemm_i8_requant_workspace_bytes(M, N, K) >= M * 4 * 2 * -(-N // 128)
        Q, s, h = g.gemm_i8_requant(*dev, relu=relu, want_hash=True)
        torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sw.view(np.uint32))
    assert np.array_equal(Q.cpu().numpy(), Qw)
    assert g.hash_value(h) == hashref.output_hash(Cw)
    with g.plan_overrides(force_tile=6):
        Q6, s6, h6 = g.gemm_i8_requant(*dev, relu=relu, want_hash=True)
        torch.cuda.synchronize()
    assert torch.equal(Q, Q6) and torch.equal(s.view(torch.int32), s6.view(torch.int32))
    assert g.hash_value(h) == g.hash_value(h6)


@pytest.mark.parametrize("pad", [52, 53])
def test_requant_persistent_padded_ldq(g, pad):
    """Codes written with a leading dimension larger than N: the padding
    bytes between rows are left as they were (an even and an odd leading
    dimension)."""
    M, N, K = 512, 300, 768
    say("requant persistent ldq", M, N, K, pad)
    (QA, sA, QB, sB), (dQA, dsA, dQB, dsB) = _operands(g, M, N, K, 515)
    Qw, sw, Cw = requant.gemm_requant(QA, sA, QB, sB, True)
    lib = g.load()
    ldq = N + pad
    Qp = torch.full((M, ldq), 77, dtype=torch.int8, device="cuda")
    s = torch.empty(M, dtype=torch.float32, device="cuda")
    h = torch.zeros(1, dtype=torch.int64, device="cuda")
    wsb = int(lib.gemm_i8_requant_workspace_bytes(M, N, K))
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.gemm_i8_requant(dQA.data_ptr(), dQA.stride(0), dsA.data_ptr(), dQB.data_ptr(), dQB.stride(0),
                             dsB.data_ptr(), M, N, K, Qp.data_ptr(), ldq, s.data_ptr(), 3, h.data_ptr(),
                             ws.data_ptr(), wsb, st)
    torch.cuda.synchronize()
    assert rc == 0
    Qh = Qp.cpu().numpy()
    assert np.array_equal(Qh[:, :N], Qw)
    assert np.all(Qh[:, N:] == 77)
    assert np.array_equal(s.cpu().numpy(), sw)
    assert g.hash_value(h) == hashref.output_hash(Cw)


def test_requant_mlp_up_full_size(g):
    """GPT-2-small MLP up-projection 8192x3072x768 with ReLU: the codes and
    scales equal quantize_rows of the library's own f32 output and the
    oracle's; the hash equals the oracle's hash of the f32 output."""
    from synth import inputs as S
    X, Wu, _ = S.w2_inputs()
    say("requant mlp up full size")
    dQA, dsA = g.quantize_rows(torch.from_numpy(X).cuda())
    dQB, dsB = g.quantize_cols(torch.from_numpy(Wu).cuda())
    Q, s, h = g.gemm_i8_requant(dQA, dsA, dQB, dsB, relu=True, want_hash=True)
    C, h2 = g.gemm_i8_blockscaled(dQA, dsA, dQB, dsB, relu=True, want_hash=True)
    Q2, s2 = g.quantize_rows(C)
    torch.cuda.synchronize()
    assert torch.equal(Q, Q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    assert g.hash_value(h) == g.hash_value(h2)
    QA, sA = ref.quantize_rows(X)
    QB, sB = ref.quantize_cols(Wu)
    Qw, sw, Cw = requant.gemm_requant(QA, sA, QB, sB, True)
    assert np.array_equal(Q.cpu().numpy(), Qw) and np.array_equal(s.cpu().numpy(), sw)
    assert g.hash_value(h) == hashref.output_hash(Cw)


def test_requant_empty(g):
    lib = g.load()
    dev = torch.device("cuda")
    s = torch.full((5,), -1.0, device=dev)
    h = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = torch.zeros(256, dtype=torch.uint8, device=dev)
    Q = torch.empty((5, 16), dtype=torch.int8, device=dev)
    A = torch.zeros((5, 16), dtype=torch.int8, device=dev)
    sa = torch.ones(5, device=dev)
    rc = lib.gemm_i8_requant(A.data_ptr(), 16, sa.data_ptr(), None, 16, None, 5, 0, 7, Q.data_ptr(), 16,
                             s.data_ptr(), 2, h.data_ptr(), ws.data_ptr(), 256, None)
    torch.cuda.synchronize()
    assert rc == 0
    assert np.all(s.cpu().numpy() == ref.SCALE_FLOOR)
    assert g.hash_value(h) == hashref.output_hash(np.zeros((5, 0), dtype=np.float32))
    # argument errors
    assert lib.gemm_i8_requant(A.data_ptr(), 16, sa.data_ptr(), A.data_ptr(), 16, sa.data_ptr(), 5, 5, 7,
                               Q.data_ptr(), 4, s.data_ptr(), 0, None, ws.data_ptr(), 256, None) == 1
    assert lib.gemm_i8_requant(A.data_ptr(), 16, sa.data_ptr(), A.data_ptr(), 16, sa.data_ptr(), 5, 5, 7,
                               Q.data_ptr(), 16, s.data_ptr(), 4, None, ws.data_ptr(), 256, None) == 1
