"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

The bar is bit-exact: int8 bytes, scale bit patterns, output bit patterns
(so -0 and +0 differ) and the 64-bit output hash.  The DaisyChain-Train page
"Verification — why you can trust the numbers" compares "at the bit level"
in its init gates ("Layer 1: exact init gates") for exactly this reason.

Every case prints its name before it touches the GPU.
"""

import numpy as np
import pytest
import torch

from oracle import adversarial, hashref, ref
from oracle import formats as F
from synth import inputs as S
from tests.parity import assert_bits, check_against_oracle

pytestmark = pytest.mark.gpu
F32 = np.float32
U32 = np.uint32


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_gemm_amd as lib
    lib.load()
    return lib


def say(*a):
    print("[case]", *a, flush=True)


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_method(g, A, B, relu, want_hash=True):
    """The whole method on the GPU; returns numpy copies of every stage."""
    QA, sr = g.quantize_rows(to_dev(A))
    QBt, sc = g.quantize_cols(to_dev(B))
    C, h = g.gemm_i8_blockscaled(QA, sr, QBt, sc, relu=relu, want_hash=True)
    torch.cuda.synchronize()
    return dict(QA=QA.cpu().numpy(), s_row=sr.cpu().numpy(), QBt=QBt.cpu().numpy(),
                s_col=sc.cpu().numpy(), C=C.cpu().numpy(), hash=g.hash_value(h))


def adversarial_inputs(c):
    case = S.adversarial_case(c)
    rng = np.random.default_rng([7, c])
    A, _ = adversarial.plant_ties(case.A, "rows", rng, frac=0.02)
    A, _ = adversarial.plant_fma_splits(A, "rows", rng, per_line=1)
    B, _ = adversarial.plant_ties(case.B, "cols", rng, frac=0.02)
    B, _ = adversarial.plant_fma_splits(B, "cols", rng, per_line=1)
    return A, B, case.relu


# ---------------------------------------------------------------------------
# quantize
# ---------------------------------------------------------------------------
QR_SHAPES = [(1, 1), (3, 5), (17, 300), (64, 768), (100, 1000), (6, 2044), (9, 3072), (5, 4000),
             (7, 4097), (3, 5000), (2, 33000), (2, 70000)]


def _quant_input(rows, cols, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_t(2, (rows, cols)).astype(F32)
    X[rng.random((rows, cols)) < 0.01] = F32(-0.0)
    if rows > 2:
        X[1] = 0
    X, _ = adversarial.plant_ties(X, "rows", rng, frac=0.02)
    X, _ = adversarial.plant_fma_splits(X, "rows", rng, per_line=2)
    return X


@pytest.mark.parametrize("rows,cols", QR_SHAPES)
def test_quantize_rows_parity(g, rows, cols):
    say("quantize_rows", rows, cols)
    X = _quant_input(rows, cols, rows * 100003 + cols)
    Q, s = g.quantize_rows(to_dev(X))
    Qo, so = ref.quantize_rows(X)
    assert_bits(Q.cpu().numpy(), Qo, "Q")
    assert_bits(s.cpu().numpy(), so, "scale")


def test_quantize_rows_unaligned(g):
    say("quantize_rows unaligned view")
    base = _quant_input(33, 771, 5)
    dev = to_dev(base)[:, 1:]            # pointer and ld not multiples of 4 floats
    Q, s = g.quantize_rows(dev)
    Qo, so = ref.quantize_rows(base[:, 1:])
    assert_bits(Q.cpu().numpy(), Qo, "Q")
    assert_bits(s.cpu().numpy(), so, "scale")


# includes the GPT-2 weights' bands (768 rows: 32 columns, 3072 rows: 8) and
# the same widths with a ragged last band
QC_SHAPES = [(1, 1), (5, 3), (300, 17), (768, 64), (1000, 100), (130, 257), (3072, 40), (65, 1030),
             (512, 300), (8192, 70), (8193, 33), (2, 5000), (768, 3072), (3072, 768), (1000, 2100),
             (3000, 700)]


@pytest.mark.parametrize("rows,cols", QC_SHAPES)
def test_quantize_cols_parity(g, rows, cols):
    say("quantize_cols", rows, cols)
    X = np.ascontiguousarray(_quant_input(cols, rows, rows * 7919 + cols).T)
    Qt, s = g.quantize_cols(to_dev(X))
    Qo, so = ref.quantize_cols(X)
    assert_bits(Qt.cpu().numpy(), Qo, "Qt")
    assert_bits(s.cpu().numpy(), so, "scale")


@pytest.mark.parametrize("rows,cols", QC_SHAPES)
def test_quantize_cols_two_pass(g, rows, cols):
    """The two-pass column kernels (scale pass with atomicMax on partial
    scales, then quantize-transpose) on every shape, forced."""
    say("quantize_cols two-pass", rows, cols)
    X = np.ascontiguousarray(_quant_input(cols, rows, rows * 7919 + cols + 1).T)
    with g.plan_overrides(qcols_path=1):
        Qt, s = g.quantize_cols(to_dev(X))
        torch.cuda.synchronize()
    Qo, so = ref.quantize_cols(X)
    assert_bits(Qt.cpu().numpy(), Qo, "Qt")
    assert_bits(s.cpu().numpy(), so, "scale")


# shapes the cooperative one-read column kernel takes (rows a multiple of
# 256, at least 1024; columns a multiple of 32): one member per band, several
# members with a partial last chunk, more bands than resident groups
COOP_SHAPES = [(1024, 32), (1280, 96), (3072, 768), (2048, 4096), (8192, 800), (4352, 6400)]


@pytest.mark.parametrize("path", [2, 3])
@pytest.mark.parametrize("rows,cols", COOP_SHAPES)
def test_quantize_cols_cooperative(g, rows, cols, path):
    """The whole-line column kernels, forced on their shapes: the cooperative
    one-read kernel (path 2: partial maxima exchanged between the workgroups
    of a band, counter in the band's first Qt bytes) and the two whole-line
    passes (path 3), against the oracle; also with power-of-two scales."""
    say("quantize_cols whole-line path", path, rows, cols)
    X = np.ascontiguousarray(_quant_input(cols, rows, rows * 31 + cols).T)
    X[:, 3] = 0
    dX = to_dev(X)
    with g.plan_overrides(qcols_path=path):
        Qt, s = g.quantize_cols(dX)
        Qp, sp = g.quantize_cols_fmt(dX, g.FMT_POW2)
        torch.cuda.synchronize()
    Qo, so = ref.quantize_cols(X)
    assert_bits(Qt.cpu().numpy(), Qo, "Qt")
    assert_bits(s.cpu().numpy(), so, "scale")
    Qpo, spo = F.quantize_cols(X, F.POW2)
    assert_bits(Qp.cpu().numpy(), Qpo, "Qt pow2")
    assert_bits(sp.cpu().numpy(), spo, "scale pow2")


def test_quantize_cols_cooperative_graph_replays(g):
    """The cooperative launch captured in a HIP graph: every replay, with
    eager work between replays, writes the oracle's bytes."""
    rows, cols = 4096, 1024
    X = np.ascontiguousarray(_quant_input(cols, rows, 4242).T)
    Qo, so = ref.quantize_cols(X)
    dX = to_dev(X)
    Qt = torch.empty((cols, rows), dtype=torch.int8, device="cuda")
    s = torch.empty(cols, dtype=torch.float32, device="cuda")
    lib = g.load()

    def call():
        st = torch.cuda.current_stream().cuda_stream
        assert lib.quantize_cols(dX.data_ptr(), rows, cols, cols, Qt.data_ptr(), rows, s.data_ptr(), st) == 0

    say("quantize_cols cooperative in a graph")
    with g.plan_overrides(qcols_path=2):
        call()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        for it in range(3):
            Qt.fill_(5)
            s.fill_(-1.0)
            graph.replay()
            torch.cuda.synchronize()
            assert_bits(Qt.cpu().numpy(), Qo, f"Qt replay {it}")
            assert_bits(s.cpu().numpy(), so, f"scale replay {it}")
            call()
            torch.cuda.synchronize()


def test_quantize_cols_cooperative_wait_timeout(g):
    """The cooperative kernel with every wait cut to one spin (test override
    4), so that members give up on each other: the launch still ends, every
    band is either exact or marked failed as a whole (NaN scales, which no
    valid call produces), never silently wrong, and the next call on the
    same buffers is exact again."""
    rows, cols = 4096, 1024                      # four members per band, 32 bands
    X = np.ascontiguousarray(_quant_input(cols, rows, 9090).T)
    Qo, so = ref.quantize_cols(X)
    dX = to_dev(X)
    say("quantize_cols cooperative, waits cut to one spin")
    with g.plan_overrides(qcols_path=4):
        Qt, s = g.quantize_cols(dX)
        torch.cuda.synchronize()
    sh, qh = s.cpu().numpy(), Qt.cpu().numpy()
    failed = np.isnan(sh).reshape(-1, 32)
    assert np.all(failed.all(axis=1) | ~failed.any(axis=1)), "a band failed in part"
    good = ~np.isnan(sh)
    say("bands marked failed:", int(failed.all(axis=1).sum()), "of", failed.shape[0])
    assert_bits(sh[good], so[good], "scale of completed bands")
    assert_bits(qh[good], Qo[good], "Qt of completed bands")
    with g.plan_overrides(qcols_path=2):
        Qt2, s2 = g.quantize_cols(dX)
        torch.cuda.synchronize()
    assert_bits(Qt2.cpu().numpy(), Qo, "Qt after")
    assert_bits(s2.cpu().numpy(), so, "scale after")


def test_quantize_cols_unaligned(g):
    say("quantize_cols unaligned view")
    base = np.ascontiguousarray(_quant_input(130, 67, 6).T)      # 67 x 130
    dev = to_dev(base)[:, 3:]
    Qt, s = g.quantize_cols(dev)
    Qo, so = ref.quantize_cols(base[:, 3:])
    assert_bits(Qt.cpu().numpy(), Qo, "Qt")
    assert_bits(s.cpu().numpy(), so, "scale")


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
def test_w1_single_gemm_256(g):
    say("w1 256x256x256")
    A, B = S.w1_inputs()
    got = run_method(g, A, B, relu=False)
    check_against_oracle(got, A, B, relu=False)


@pytest.mark.parametrize("chunk", range(4))
def test_w4_adversarial_sweep(g, chunk):
    for c in range(chunk * 50, (chunk + 1) * 50):
        A, B, relu = adversarial_inputs(c)
        say("w4 case", c, "MNK", A.shape[0], B.shape[1], A.shape[1], "relu", relu)
        got = run_method(g, A, B, relu)
        C = check_against_oracle(got, A, B, relu)
        if relu:
            assert np.all(got["C"].view(U32) >> 31 == 0)


@pytest.mark.parametrize("tile", list(range(4)))
def test_tile_and_split_invariance(g, tile):
    """Different tile shapes and K splits give byte-identical outputs (integer
    accumulation is associative), all equal to the oracle."""
    rng = np.random.default_rng(77)
    A = rng.standard_t(3, (300, 3000)).astype(F32)
    B = rng.standard_normal((3000, 520)).astype(F32)
    C, *_ = ref.blockscaled_gemm(A, B, True)
    h = hashref.output_hash(C)
    for splits in (1, 2, 5, 16):
        with g.plan_overrides(force_tile=tile, force_splits=splits):
            assert g.plan_query(300, 520, 3000) == (tile, splits), "the forced plan did not run"
            say("invariance tile", tile, "splits", splits)
            got = run_method(g, A, B, relu=True)
        assert_bits(got["C"], C, f"C tile {tile} splits {splits}")
        assert got["hash"] == h


@pytest.mark.parametrize("N", [517, 518, 519])
def test_split_reduction_ragged_columns(g, N):
    """Split K with a column count that is not a multiple of 4 (the combine
    reads and writes the last column group one word at a time), on three
    tile configurations, and a second call with another shape on the same
    workspace after each."""
    rng = np.random.default_rng(N)
    A = rng.standard_t(3, (700, 2048)).astype(F32)
    B = rng.standard_normal((2048, N)).astype(F32)
    C, *_ = ref.blockscaled_gemm(A, B, False)
    h = hashref.output_hash(C)
    A2 = rng.standard_t(3, (2304, 1024)).astype(F32)
    B2 = rng.standard_normal((1024, 3000)).astype(F32)
    C2, *_ = ref.blockscaled_gemm(A2, B2, True)
    for tile, splits in ((2, 3), (1, 4), (0, 2)):
        with g.plan_overrides(force_tile=tile, force_splits=splits):
            assert g.plan_query(700, N, 2048) == (tile, splits)
            say("split ragged N", N, "tile", tile, "splits", splits)
            got = run_method(g, A, B, relu=False)
            assert_bits(got["C"], C, f"C N {N} tile {tile} splits {splits}")
            assert got["hash"] == h
            got2 = run_method(g, A2, B2, relu=True)
            assert_bits(got2["C"], C2, f"C2 tile {tile} splits {splits}")
            assert got2["hash"] == hashref.output_hash(C2)


# (M, N, K, relu): ragged edges; more tiles than CUs so that workgroups walk
# several tiles (and some one fewer); K with fewer 64-byte stages than a
# wave has output blocks, and with more
PERSIST_CASES = [(300, 520, 3008, True), (4100, 2500, 192, False), (4100, 2500, 640, True),
                 (1000, 1000, 1024, False), (2056, 6000, 256, True)]


@pytest.mark.parametrize("tile", [4, 5])
def test_persistent_kernel(g, tile):
    """The persistent kernel (epilogue of one tile drained under the next
    tile's MFMAs) against the oracle, every byte and the hash."""
    rng = np.random.default_rng(90 + tile)
    with g.plan_overrides(force_tile=tile):
        for (m, n, k, relu) in PERSIST_CASES:
            A = rng.standard_t(3, (m, k)).astype(F32)
            B = rng.standard_normal((k, n)).astype(F32)
            A[rng.random(m) < 0.02] = 0
            say("persistent tile", tile, "MNK", m, n, k, "relu", relu)
            assert g.plan_query(m, n, k) == (tile, 1), "the forced plan did not run"
            got = run_method(g, A, B, relu=relu)
            check_against_oracle(got, A, B, relu)


# 128-byte-stage persistent kernel: M % 128 == 0, K % 128 == 0, K / 128 at
# least the 32x32 blocks of a wave (tile 6, 128x192: K >= 768; tile 7,
# 128x128 with two workgroups per CU: K >= 512; shapes below the bound fall
# back to another tile).  Ragged N (masked through the buffer range check),
# one and several tiles per workgroup, K with more stages than epilogue blocks
# (runtime stage loop), and for tile 7 K at its bound (four stages, two ring
# slots) and more tiles than two per CU.
PERSIST128_CASES = [(1024, 1000, 768, True), (4096, 1552, 768, False), (2048, 2000, 1536, True),
                    (8192, 520, 896, False), (4224, 3000, 1280, True), (2048, 1000, 512, True),
                    (8192, 3000, 640, False)]


@pytest.mark.parametrize("tile", [6, 7])
def test_persistent128_kernel(g, tile):
    """The persistent kernels with 128-byte K stages against the oracle, every
    byte and the hash."""
    rng = np.random.default_rng(96 + tile)
    with g.plan_overrides(force_tile=tile):
        for (m, n, k, relu) in PERSIST128_CASES:
            if tile == 6 and k < 768:
                continue                  # below tile 6's bound: another tile would run
            A = rng.standard_t(3, (m, k)).astype(F32)
            B = rng.standard_normal((k, n)).astype(F32)
            A[rng.random(m) < 0.02] = 0
            B[:, rng.random(n) < 0.02] = 0
            say("persistent128 tile", tile, "MNK", m, n, k, "relu", relu)
            assert g.plan_query(m, n, k) == (tile, 1), "the forced plan did not run"
            got = run_method(g, A, B, relu=relu)
            check_against_oracle(got, A, B, relu)


@pytest.mark.parametrize("tile", [5, 6, 7])
def test_persistent_nontemporal_stores(g, tile):
    """An output above 128 MB is written with nontemporal stores by the
    persistent kernels: ragged N, ReLU, several tiles per workgroup, every
    byte and the hash against the oracle."""
    M, N, K = 4096, 8200, 768                   # 134 MB of f32 output
    rng = np.random.default_rng(700 + tile)
    A = rng.standard_t(3, (M, K)).astype(F32)
    B = rng.standard_normal((K, N)).astype(F32)
    A[rng.random(M) < 0.02] = 0
    with g.plan_overrides(force_tile=tile):
        assert g.plan_query(M, N, K) == (tile, 1), "the forced plan did not run"
        say("nontemporal persistent tile", tile, "MNK", M, N, K)
        got = run_method(g, A, B, relu=True)
    check_against_oracle(got, A, B, True)


def test_w2_mlp_full_size(g):
    """MLP up-projection (ReLU) and the down-projection on its output, full
    size, every output byte."""
    X, W_up, W_down = S.w2_inputs()
    say("w2 up 8192x3072x768 relu")
    got = run_method(g, X, W_up, relu=True)
    H = check_against_oracle(got, X, W_up, relu=True)
    say("w2 down 8192x768x3072")
    got2 = run_method(g, got["C"], W_down, relu=False)
    check_against_oracle(got2, H, W_down, relu=False)


def test_long_k_split(g):
    """A long-K shape that the planner splits (the LM-head dgrad's K=50304,
    at reduced M and N), every byte."""
    rng = np.random.default_rng(78)
    A = (rng.standard_normal((512, 50304)) * 1e-4).astype(F32)
    B = (rng.standard_normal((50304, 256)) * 0.02).astype(F32)
    say("long K 512x256x50304")
    got = run_method(g, A, B, relu=False)
    check_against_oracle(got, A, B, relu=False)


@pytest.mark.parametrize("splits", [0, 7])
def test_max_k_int32_limit(g, splits):
    """K = 133144, the largest K whose sums of +-127 * +-127 products stay in
    int32: codes all +-127 put |acc| within 127^2 of 2^31 - 1 (and above
    2^24, so RN(acc) rounds), unsplit and over forced K splits whose partial
    sums are combined exactly."""
    M, N, K = 48, 40, ref.K_MAX
    rng = np.random.default_rng(133144)
    QA = np.where(rng.random((M, K)) < 0.5, 127, -127).astype(np.int8)
    QB = np.where(rng.random((N, K)) < 0.5, 127, -127).astype(np.int8)
    QA[0] = 127
    QB[0] = 127                           # acc[0, 0] = 127^2 K = 2147479576
    QB[1] = -127                          # acc[0, 1] = -2147479576
    sr = (rng.random(M) + 0.5).astype(F32)
    sc = (rng.random(N) * 1e-9 + 1e-10).astype(F32)
    want = ref.gemm_i8_blockscaled(QA, sr, QB, sc)
    acc = ref.accumulate(QA, QB)
    assert acc[0, 0] == 127 * 127 * K and acc[0, 1] == -127 * 127 * K
    ld = (K + 15) // 16 * 16
    dA = torch.zeros((M, ld), dtype=torch.int8, device="cuda")
    dB = torch.zeros((N, ld), dtype=torch.int8, device="cuda")
    dA[:, :K] = torch.from_numpy(QA).cuda()
    dB[:, :K] = torch.from_numpy(QB).cuda()
    say("max K", M, N, K, "splits", splits)
    with g.plan_overrides(force_splits=splits):
        if splits:
            assert g.plan_query(M, N, K)[1] == splits
        C, h = g.gemm_i8_blockscaled(dA[:, :K], torch.from_numpy(sr).cuda(), dB[:, :K],
                                     torch.from_numpy(sc).cuda(), want_hash=True)
        torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert g.hash_value(h) == hashref.output_hash(want)


@pytest.mark.parametrize("case", [(256, 200, 768, 333, None), (256, 200, 768, 333, 6),
                                  (256, 200, 768, 333, 7), (300, 70, 200, 80, None),
                                  (3, 64, 128, (1 << 23) + 64, None)])
def test_output_leading_dimension(g, case):
    """C written through a row stride larger than N: the cells of C match
    the oracle, the columns between N and ldc keep their contents, and the
    hash covers C only.  A stride above 2^23 floats takes the non-persistent
    kernels (the persistent ones address C with 32-bit offsets); the 256-row
    case also runs on both 128-byte-stage persistent tiles (6 and 7)."""
    M, N, K, ldc, tile = case
    rng = np.random.default_rng(M + N + K)
    A = rng.standard_normal((M, K)).astype(F32)
    B = rng.standard_normal((K, N)).astype(F32)
    want, QA, sA, QB, sB = ref.blockscaled_gemm(A, B, relu=True)
    say("ldc", M, N, K, ldc, "tile", tile)
    dQA, dsA = g.quantize_rows(torch.from_numpy(A).cuda())
    dQB, dsB = g.quantize_cols(torch.from_numpy(B).cuda())
    buf = torch.full((M, ldc), -7.25, dtype=torch.float32, device="cuda")
    with g.plan_overrides(force_tile=-1 if tile is None else tile):
        if tile is not None:
            assert g.plan_query(M, N, K, ldc=ldc)[0] == tile, "the forced plan did not run"
        C, h = g.gemm_i8_blockscaled(dQA, dsA, dQB, dsB, relu=True, want_hash=True, out=buf[:, :N])
        torch.cuda.synchronize()
    got = buf[:, :N].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    pad = buf[:, N:min(ldc, N + 4096)]
    assert torch.all(pad == -7.25)
    assert g.hash_value(h) == hashref.output_hash(want)
    del buf


# ---------------------------------------------------------------------------
# hash, errors, workspace
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,pad", [(1, 1, 0), (3, 5, 0), (37, 1029, 3), (513, 64, 0), (5, 4, 0)])
def test_output_hash_parity(g, m, n, pad):
    say("output_hash", m, n, pad)
    rng = np.random.default_rng(m * 31 + n)
    base = rng.standard_normal((m, n + pad)).astype(F32)
    base[rng.random(base.shape) < 0.1] = F32(-0.0)
    dev = to_dev(base)[:, :n]
    h = g.hash_value(g.output_hash(dev))
    assert h == hashref.output_hash(np.ascontiguousarray(base[:, :n]))


def test_empty_shapes(g):
    say("empty shapes")
    z = torch.zeros((0, 5), dtype=torch.float32, device="cuda")
    assert g.hash_value(g.output_hash(z)) == hashref.output_hash(np.zeros((0, 5), F32))
    Q, s = g.quantize_rows(z)
    assert Q.shape == (0, 5) and s.shape == (0,)
    A = torch.zeros((4, 0), dtype=torch.float32, device="cuda")
    QA, sr = g.quantize_rows(A)
    assert np.all(sr.cpu().numpy().view(U32) == 0x322BCC77)
    QB, sc = g.quantize_cols(torch.zeros((0, 3), dtype=torch.float32, device="cuda"))
    C, h = g.gemm_i8_blockscaled(QA, sr, QB, sc, want_hash=True)
    torch.cuda.synchronize()
    assert np.all(C.cpu().numpy().view(U32) == 0)
    assert g.hash_value(h) == hashref.output_hash(np.zeros((4, 3), F32))


def test_error_statuses(g):
    say("error statuses")
    QA = torch.zeros((2, ref.K_MAX + 1), dtype=torch.int8, device="cuda")
    s = torch.ones(2, dtype=torch.float32, device="cuda")
    with pytest.raises(g.I8GError) as e:
        g.gemm_i8_blockscaled(QA, s, QA, s)
    assert e.value.status == 2
    QA = torch.zeros((2, 48), dtype=torch.int8, device="cuda")[:, 1:33]   # misaligned
    with pytest.raises(g.I8GError) as e:
        g.gemm_i8_blockscaled(QA, s, QA, s)
    assert e.value.status == 3
    lib = g.load()
    rc = lib.gemm_i8_blockscaled(None, 16, None, None, 16, None, 2, 2, 16, None, 2, 0, None,
                                 None, 0, None)
    assert rc == 4                                   # no workspace
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    rc = lib.gemm_i8_blockscaled(None, 16, None, None, 16, None, 2, 2, 16, None, 2, 0, None,
                                 ws.data_ptr(), 256, None)
    assert rc == 1                                   # null operands
    rc = lib.quantize_rows(None, -1, 2, 2, None, 2, None, None)
    assert rc == 1


def test_workspace_scratch_contents_do_not_matter(g):
    """Beyond its 256-byte header the workspace is scratch: garbage there
    changes no byte; the header is zero after every call; repeated split-K
    calls give identical bytes and hashes."""
    say("workspace garbage")
    rng = np.random.default_rng(79)
    A = rng.standard_normal((700, 9000)).astype(F32)
    B = rng.standard_normal((9000, 300)).astype(F32)
    C, *_ = ref.blockscaled_gemm(A, B, False)
    for it in range(3):
        for ws in g._ws.values():
            ws[256:].random_(0, 256)
        with g.plan_overrides(force_splits=3):
            assert g.plan_query(700, 300, 9000)[1] == 3
            got = run_method(g, A, B, relu=False)
        assert_bits(got["C"], C, f"C call {it}")
        assert got["hash"] == hashref.output_hash(C)
        for ws in g._ws.values():
            assert int(torch.count_nonzero(ws[:256]).item()) == 0


def test_metamorphic_on_gpu(g):
    """Section "Layer 5" relations and absolutes, checked on the GPU output."""
    rng = np.random.default_rng(80)
    A = rng.standard_t(2, (333, 555)).astype(F32)
    B = rng.standard_t(2, (555, 444)).astype(F32)
    say("metamorphic base")
    C = run_method(g, A, B, relu=False)["C"]
    p = rng.permutation(333)
    say("metamorphic permuted rows")
    Cp = run_method(g, A[p], B, relu=False)["C"]
    assert_bits(Cp, C[p], "row permutation")
    A0 = A.copy(); A0[10] = 0
    say("metamorphic zero row")
    C0 = run_method(g, A0, B, relu=False)["C"]
    assert np.all(C0[10].view(U32) == 0)
    say("metamorphic blocks")
    top = run_method(g, A[:100], B, relu=False)["C"]
    assert_bits(top, C[:100], "row block")
    right = run_method(g, A, B[:, 200:], relu=False)["C"]
    assert_bits(right, C[:, 200:], "column block")
    say("metamorphic relu")
    Cr = run_method(g, A, B, relu=True)["C"]
    assert np.all(Cr.view(U32) >> 31 == 0)
    assert np.array_equal(Cr, np.where(C > 0, C, 0))
    # unit scales: integer inputs whose lines contain +-127 give the exact dot product
    Ai = rng.integers(-127, 128, (64, 1000)).astype(F32); Ai[:, 0] = 127
    Bi = rng.integers(-127, 128, (1000, 48)).astype(F32); Bi[0, :] = -127
    say("unit scales")
    Ci = run_method(g, Ai, Bi, relu=False)["C"]
    exact = Ai.astype(np.int64) @ Bi.astype(np.int64)
    assert np.array_equal(Ci.astype(np.int64), exact)
