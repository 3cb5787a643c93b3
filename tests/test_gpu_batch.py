"""quantize_batch on the GPU: every job's output equals the single call's
(which the other GPU tests hold to the oracle) byte for byte, and a sample
of jobs is compared with the oracle directly."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import ref

pytestmark = pytest.mark.gpu


def say(*a):
    print("[batch]", *a, flush=True)


@pytest.fixture(scope="module")
def g():
    import int8_gemm_amd as g
    g.load()
    return g


def _x(seed, rows, cols):
    rng = np.random.default_rng(seed)
    X = rng.standard_t(3, (rows, cols)).astype(np.float32)
    if rows > 2 and cols > 2:
        X[1] = 0.0
        X[:, 2] = 0.0
    return torch.from_numpy(X).cuda()


# (rows, cols, by_col, fmt): rows passes of every length class (wave path,
# block path, long rows), column passes on the register path and on the tall
# multi-kernel path, int4 and pow2 formats, empty lines.  Aligned rows of
# 1025-3072 values run inside the batch (8 and 12 float4 per lane); a length
# that is not a multiple of 4 runs its own kernel.  Column jobs of the GPT-2
# weights' shapes take wider bands in the batch than in a call of their own
# (32 and 8 columns against 16 and 4), in every format.
JOBS = [(8192, 768, False, 0), (768, 3072, True, 0), (3072, 768, True, 0), (100, 1, False, 0),
        (37, 4000, False, 0), (5, 5000, False, 0), (3, 40000, False, 0), (100, 70, True, 0),
        (9000, 33, True, 0), (64, 300, False, F.POW2), (300, 64, True, F.POW2), (50, 77, False, F.INT4),
        (77, 50, True, F.INT4), (0, 10, False, 0), (10, 0, False, 0), (0, 10, True, 0), (1, 1, True, 0),
        (8192, 3072, False, 0), (300, 2044, False, 0), (40, 1030, False, 0), (64, 2048, False, F.POW2),
        (33, 3072, False, F.POW2), (768, 3072, True, F.INT4), (3072, 768, True, F.POW2)]


def test_batch_equals_single_calls(g):
    specs = [(_x(i, r, c), bc, f) for i, (r, c, bc, f) in enumerate(JOBS)]
    say("batch of", len(specs))
    outs = g.quantize_batch(specs)
    torch.cuda.synchronize()
    for (X, bc, f), (Q, s), job in zip(specs, outs, JOBS):
        Q1, s1 = (g.quantize_cols_fmt if bc else g.quantize_rows_fmt)(X, f)
        torch.cuda.synchronize()
        assert torch.equal(Q, Q1), job
        assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), job
    # oracle on a few jobs directly
    for k in (0, 1, 2, 4, 9, 17, 18, 20, 22, 23):
        X, bc, f = specs[k]
        Q, s = outs[k]
        qo, so = (F.quantize_cols if bc else F.quantize_rows)(X.cpu().numpy(), f)
        Qn = Q.cpu().numpy()
        if f & F.INT4:                     # packed lines, two codes per byte
            Qn, qo = Qn.view(np.uint8), F.pack_int4(qo)
        assert np.array_equal(Qn, qo) and np.array_equal(s.cpu().numpy(), so), JOBS[k]


def test_batch_many_jobs_several_launches(g):
    """More jobs than one launch holds (24): the batch is split."""
    specs = [(_x(100 + i, 17 + 13 * i, 31 + 7 * i), i % 2 == 1, 0) for i in range(53)]
    # aligned long rows (the batch's long-row body) in the later launches too
    specs += [(_x(200 + i, 3 + i, 1024 + 512 * i), False, 0) for i in range(1, 5)]
    say("batch of", len(specs))
    outs = g.quantize_batch(specs)
    torch.cuda.synchronize()
    for (X, bc, f), (Q, s) in zip(specs, outs):
        qo, so = (ref.quantize_cols if bc else ref.quantize_rows)(X.cpu().numpy())
        assert np.array_equal(Q.cpu().numpy(), qo) and np.array_equal(s.cpu().numpy(), so)


def test_batch_rejects_before_enqueueing(g):
    """An invalid job fails the call and nothing runs, not even the valid jobs."""
    X = _x(7, 64, 64)
    arr, outs = g.quantize_jobs([(X, False, 0), (X, True, 0)])
    for Q, s in outs:
        Q.fill_(5)
        s.fill_(-1.0)
    arr[1].ldq = 3                      # below the line length
    lib = g.load()
    assert lib.quantize_batch(arr, 2, torch.cuda.current_stream().cuda_stream) == 1
    assert lib.quantize_batch(None, 1, None) == 1
    assert lib.quantize_batch(None, 0, None) == 0
    torch.cuda.synchronize()
    for Q, s in outs:
        assert torch.all(Q == 5) and torch.all(s == -1.0)
