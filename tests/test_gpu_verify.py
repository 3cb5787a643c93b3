"""The library's self-checks on the GPU: the init gate (page section
"Layer 1: exact init gates"), the live audits ("Layer 2: continuous audit")
and the kernel probe ("Layer 3: the kernel probe") against the oracle."""
import numpy as np
import pytest
import torch

from oracle import probe, ref

pytestmark = pytest.mark.gpu


def say(*a):
    print("[verify]", *a, flush=True)


@pytest.fixture(scope="module")
def g():
    import int8_gemm_amd as g
    g.load()
    return g


def test_gate_passes(g):
    say("i8g_gate")
    rc, rep = g.gate()
    assert rc == 0, (g.load().i8g_status_string(rc), rep)
    assert rep["check"] == 0
    # quantize cases (16) + GEMM cases x configurations (5 x 8) + int4 GEMMs x 2 paths (3 x 2)
    # + requant (1)
    assert rep["cases"] >= 16 + 5 * 8 + 3 * 2 + 1


def _live_gemm(g, M, N, K, relu, seed):
    rng = np.random.default_rng(seed)
    A = torch.from_numpy(rng.standard_t(3, (M, K)).astype(np.float32)).cuda()
    B = torch.from_numpy(rng.standard_normal((K, N)).astype(np.float32)).cuda()
    QA, sr = g.quantize_rows(A)
    QB, sc = g.quantize_cols(B)
    C = g.gemm_i8_blockscaled(QA, sr, QB, sc, relu=relu)
    return A, B, QA, sr, QB, sc, C


@pytest.mark.parametrize("shape", [(300, 520, 192, True), (2048, 2000, 1536, False)])
def test_audit_gemm_clean_and_corrupted(g, shape):
    M, N, K, relu = shape
    say("audit gemm", M, N, K, relu)
    A, B, QA, sr, QB, sc, C = _live_gemm(g, M, N, K, relu, 5)
    r = g.audit_gemm(QA, sr, QB, sc, C, relu=relu, seed=11, samples=4096)
    torch.cuda.synchronize()
    assert r[0].item() == 0 and r[1].item() == -1
    # one ulp added to every cell of row 7: every sample in that row differs
    # (65536 samples put about 32 in row 7 of the larger shape)
    C2 = C.clone()
    C2[7] = torch.nextafter(C2[7], torch.full_like(C2[7], float("inf")))
    r = g.audit_gemm(QA, sr, QB, sc, C2, relu=relu, seed=11, samples=65536)
    torch.cuda.synchronize()
    assert r[0].item() > 0 and r[1].item() // N == 7
    # every cell one ulp off: every sample differs
    C3 = torch.nextafter(C, torch.full_like(C, float("inf")))
    r = g.audit_gemm(QA, sr, QB, sc, C3, relu=relu, seed=12, samples=1000)
    torch.cuda.synchronize()
    assert r[0].item() == 1000


def test_audit_quantize_clean_and_corrupted(g):
    rng = np.random.default_rng(8)
    X = torch.from_numpy(rng.standard_t(3, (777, 1500)).astype(np.float32)).cuda()
    Q, s = g.quantize_rows(X)
    Qt, st = g.quantize_cols(X)
    for (QQ, ss, by_col) in ((Q, s, False), (Qt, st, True)):
        say("audit quantize by_col", by_col)
        r = g.audit_quantize(X, QQ, ss, by_col, seed=3, samples=256)
        torch.cuda.synchronize()
        assert r[0].item() == 0 and r[1].item() == -1
        bad = QQ.clone()
        bad[5:, :] = 0                       # every line but 0..4 wrong (the rows there hold no zeros)
        lines = ss.numel()
        r = g.audit_quantize(X, bad, ss, by_col, seed=3, samples=256)
        torch.cuda.synchronize()
        # lines >= 5 that were sampled are reported; the smallest is >= 5
        assert r[0].item() > 0 and 5 <= r[1].item() < lines


@pytest.mark.parametrize("case", [(20261202, 256, 320, 768), (7, 77, 130, 200), (1, 1, 1, 1)])
def test_probe_hash_matches_oracle(g, case):
    seed, M, N, K = case
    say("probe", seed, M, N, K)
    h = g.hash_value(g.probe_hash(seed, M, N, K))
    assert h == probe.probe_hash(seed, M, N, K)


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_audit_quantize_formats(g, fmt):
    """The live quantize audit on pow2 / int4 outputs: clean, then with one
    packed byte (int4) or code changed in line 9."""
    rng = np.random.default_rng(30 + fmt)
    X = torch.from_numpy(rng.standard_t(3, (200, 333)).astype(np.float32)).cuda()
    for by_col in (False, True):
        say("audit quantize fmt", fmt, "by_col", by_col)
        Q, s = (g.quantize_cols_fmt if by_col else g.quantize_rows_fmt)(X, fmt)
        lines = s.numel()
        r = g.audit_quantize(X, Q, s, by_col, seed=5, samples=16 * lines, fmt=fmt)
        torch.cuda.synchronize()
        assert r[0].item() == 0 and r[1].item() == -1
        bad = Q.clone()
        bad[9, 3] = bad[9, 3] ^ 0x11          # one code (int4: two nibbles) changed
        r = g.audit_quantize(X, bad, s, by_col, seed=5, samples=16 * lines, fmt=fmt)
        torch.cuda.synchronize()
        assert r[0].item() > 0 and r[1].item() == 9


@pytest.mark.parametrize("combo", [(False, True), (True, True)])
def test_audit_gemm_int4_operands(g, combo):
    a4, b4 = combo
    M, N, K = 130, 190, 333
    rng = np.random.default_rng(44)
    A = torch.from_numpy(rng.standard_t(3, (M, K)).astype(np.float32)).cuda()
    B = torch.from_numpy((rng.standard_normal((K, N)) * 0.02).astype(np.float32)).cuda()
    QA, sr = g.quantize_rows_fmt(A, 2 if a4 else 0)
    QB, sc = g.quantize_cols_fmt(B, 2 if b4 else 0)
    C = g.gemm_i8_blockscaled(QA, sr, QB, sc, relu=True, K=K, a_int4=a4, b_int4=b4)
    say("audit gemm int4", a4, b4)
    r = g.audit_gemm(QA, sr, QB, sc, C, relu=True, seed=2, samples=20000, K=K, a_int4=a4, b_int4=b4)
    torch.cuda.synchronize()
    assert r[0].item() == 0
    C2 = torch.nextafter(C, torch.full_like(C, float("inf")))
    r = g.audit_gemm(QA, sr, QB, sc, C2, relu=True, seed=2, samples=1000, K=K, a_int4=a4, b_int4=b4)
    torch.cuda.synchronize()
    assert r[0].item() == 1000
