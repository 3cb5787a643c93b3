"""gemm_i8_blockscaled_noalloc (the entry point that allocates nothing: its
scratch is the library's static device array) against gemm_i8_blockscaled
with a workspace, through the C ABI: every output bit and the hash, on two
calls in a row with the second one smaller (the array keeps the previous
call's contents), with ReLU and ragged edges, through a persistent plan and
through a forced K split whose int32 partial planes live in the array.  A
shape that needs more scratch than the array holds is refused with
I8G_ESCRATCH and leaves the output untouched.

Every case prints its name before it touches the GPU.
"""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
U32 = np.uint32


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_gemm_amd as lib
    lib.load()
    return lib


def operands(g, M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_t(3, (M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    QA, sr = g.quantize_rows(torch.from_numpy(A).cuda())
    QB, sc = g.quantize_cols(torch.from_numpy(B).cuda())
    return QA, sr, QB, sc


def noalloc(g, QA, sr, QB, sc, relu, C, h):
    """The entry point called directly through ctypes."""
    M, K = QA.shape
    N = QB.shape[0]
    flags = (g.I8G_RELU if relu else 0) | g.I8G_HASH
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return g.load().gemm_i8_blockscaled_noalloc(
        ctypes.c_void_p(QA.data_ptr()), QA.stride(0), ctypes.c_void_p(sr.data_ptr()),
        ctypes.c_void_p(QB.data_ptr()), QB.stride(0), ctypes.c_void_p(sc.data_ptr()), M, N, K,
        ctypes.c_void_p(C.data_ptr()), C.stride(0), flags, ctypes.c_void_p(h.data_ptr()), stream)


def compare(g, M, N, K, relu, seed):
    QA, sr, QB, sc = operands(g, M, N, K, seed)
    C_ws, h_ws = g.gemm_i8_blockscaled(QA, sr, QB, sc, relu=relu, want_hash=True)
    C = torch.full((M, N), -3.5, dtype=torch.float32, device="cuda")
    h = torch.zeros(1, dtype=torch.int64, device="cuda")
    assert noalloc(g, QA, sr, QB, sc, relu, C, h) == 0
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().view(U32), C_ws.cpu().numpy().view(U32)), "output bits"
    assert g.hash_value(h) == g.hash_value(h_ws), "hash"


@pytest.mark.parametrize("seq", ["persistent", "split"])
def test_noalloc_matches_workspace_call(g, seq):
    """Two calls in a row, the second smaller, against the workspace call."""
    if seq == "persistent":
        shapes = [(1024, 1000, 768, True), (256, 200, 768, False)]
        for M, N, K, relu in shapes:
            say("noalloc", seq, M, N, K, relu)
            compare(g, M, N, K, relu, M + N + K)
    else:
        shapes = [(300, 520, 3000, True), (130, 190, 1000, False)]
        with g.plan_overrides(force_tile=2, force_splits=5):
            for M, N, K, relu in shapes:
                assert g.plan_query(M, N, K)[1] > 1      # 5, clamped to whole stages
                say("noalloc", seq, M, N, K, relu)
                compare(g, M, N, K, relu, M + N + K)


def test_noalloc_refuses_beyond_its_scratch(g):
    M, N, K = 4096, 4096, 1024
    QA = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    QB = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    sr = torch.ones(M, dtype=torch.float32, device="cuda")
    sc = torch.ones(N, dtype=torch.float32, device="cuda")
    C = torch.full((M, N), -3.5, dtype=torch.float32, device="cuda")
    h = torch.zeros(1, dtype=torch.int64, device="cuda")
    say("noalloc refused", M, N, K)
    with g.plan_overrides(force_tile=2, force_splits=2):     # two 64 MiB partial planes
        assert noalloc(g, QA, sr, QB, sc, False, C, h) == 7
    torch.cuda.synchronize()
    assert bool(torch.all(C == -3.5)) and int(h.item()) == 0
