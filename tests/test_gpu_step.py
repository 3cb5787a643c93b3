"""Full-size parity of the GPT-2-small LM-head GEMMs and of all 147 GEMMs of
one training step (the synthetic workloads of synth/inputs.py).

The expected hashes come from tests/golden/step_golden.json, written by
tests/golden/make_step_golden.py with the CPU oracle (the oracle is too slow
to rerun at this size on every GPU run).  Equal hashes mean equal output
bytes up to the hash's collision probability; the LM-head test also
recomputes sampled output cells with the oracle from the f32 inputs, one by
one, and compares their bits.  Input generation is checked against the
digests stored with the hashes before any GPU work.

Every case prints its name before it touches the GPU.
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

from oracle import hashref, ref
from synth import inputs as S

pytestmark = pytest.mark.gpu
U32 = np.uint32
HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN_PATH = os.path.join(HERE, "golden", "step_golden.json")


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_gemm_amd as lib
    lib.load()
    return lib


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN_PATH) as f:
        return json.load(f)


def sample_digest(x):
    return hashlib.sha256(np.ascontiguousarray(x.reshape(-1)[::4099]).tobytes()).hexdigest()


def gpu_gemm(g, dev, a_src, a_mode, b_src, b_mode, relu=False):
    qa = g.quantize_rows if a_mode == "rows" else g.quantize_cols
    qb = g.quantize_rows if b_mode == "rows" else g.quantize_cols
    QA, s_row = qa(dev[a_src])
    QBt, s_col = qb(dev[b_src])
    C, h = g.gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu=relu, want_hash=True)
    torch.cuda.synchronize()
    return C, g.hash_value(h)


def oracle_cells(A, B, rows, cols):
    """Output cells (i, j) of C = A B from the f32 inputs, one by one: row i
    of A quantized per row, column j of B per column, then the epilogue."""
    QA, s_row = ref.quantize_rows(A[rows])
    QBt, s_col = ref.quantize_cols(np.ascontiguousarray(B[:, cols]))
    return np.array([ref.output_cell(QA[t], s_row[t], QBt[t], s_col[t]) for t in range(len(rows))],
                    dtype=np.float32)


def test_w3_lm_head(g, golden):
    gh = golden["head"]
    X, W = S.w3_fwd_inputs()
    _, dY = S.w3_wgrad_inputs()
    host = {"X": X, "W": W, "dY": dY}
    for name, x in host.items():
        assert sample_digest(x) == gh["digests"][name], f"input generator changed ({name})"
    dev = {k: torch.from_numpy(v).cuda() for k, v in host.items()}
    rng = np.random.default_rng(91)

    say("w3 LM-head forward 8192x50304x768")
    C, h = gpu_gemm(g, dev, "X", "rows", "W", "cols")
    assert list(C.shape) == gh["fwd"]["shape"]
    assert hex(h) == gh["fwd"]["hash"], "forward hash"
    i = rng.integers(0, 8192, 256); j = rng.integers(0, 50304, 256)
    got = C[torch.from_numpy(i).cuda(), torch.from_numpy(j).cuda()].cpu().numpy()
    want = oracle_cells(X, W, i, j)
    assert np.array_equal(got.view(U32), want.view(U32)), "sampled forward cells"
    del C

    say("w3 LM-head weight gradient 768x50304x8192")
    C, h = gpu_gemm(g, dev, "X", "cols", "dY", "cols")
    assert list(C.shape) == gh["wgrad"]["shape"]
    assert hex(h) == gh["wgrad"]["hash"], "weight-gradient hash"
    i = rng.integers(0, 768, 256); j = rng.integers(0, 50304, 256)
    got = C[torch.from_numpy(i).cuda(), torch.from_numpy(j).cuda()].cpu().numpy()
    want = oracle_cells(np.ascontiguousarray(X.T), dY, i, j)
    assert np.array_equal(got.view(U32), want.view(U32)), "sampled weight-gradient cells"


@pytest.mark.timeout(900)
def test_w5_training_step(g, golden):
    """The 147 GEMMs of one step in order: every GEMM's hash, then the step
    hash that folds them."""
    rows = golden["step"]["gemms"]
    gemms = S.step_gemms()
    assert len(rows) == len(gemms) == 147
    host = {}
    hashes = []
    for gm, want in zip(gemms, rows):
        a, am, b, bm = gm.operands
        for name in (a, b):
            key = (gm.linear, name)
            if key not in host:
                host[key] = S.step_tensor(gm.linear, name, gm.d_in, gm.d_out)
                assert sample_digest(host[key]) == want["digests"][name], \
                    f"input generator changed ({gm.linear} {name})"
        say("w5", gm.index, gm.linear, gm.kind, "MNK", *gm.mnk)
        dev = {name: torch.from_numpy(host[(gm.linear, name)]).cuda() for name in (a, b)}
        C, h = gpu_gemm(g, dev, a, am, b, bm)
        assert list(C.shape) == want["shape"]
        assert hex(h) == want["hash"], f"GEMM {gm.index} ({gm.linear} {gm.kind})"
        hashes.append(h)
        del C, dev
    assert hex(hashref.step_hash(hashes)) == golden["step"]["step_hash"]
