"""Full-size parity of the GPT-2-small LM-head GEMMs and of all 147 GEMMs of
one training step (the synthetic workloads of synth/inputs.py).

The expected values come from tests/golden/step_golden.json, written by
tests/golden/make_step_golden.py with the CPU oracle (the oracle is too slow
to rerun the whole step on every GPU run).  Every GEMM is checked four ways:
  * the hash the GEMM kernel fuses into its epilogue (summed from registers);
  * output_hash of the stored output, which reads the bytes back from device
    memory (a store to a wrong address, a wrong mask or a lost nontemporal
    store changes it even when the fused hash is right);
  * SHA-256 of the stored output's bytes, copied to the host, against the
    oracle's: a bit-for-bit comparison that does not rest on this library's
    own hash definition;
  * SHA-256 of the quantized operands and scales the GPU wrote.
The LM-head GEMMs (outputs above 128 MB, written with nontemporal stores)
are also recomputed by the oracle from the f32 inputs and compared element
by element, in row chunks.  Input generation is checked against the sample
digests stored with the expected values before any GPU work.

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


def full_digest(t):
    """SHA-256 of a device tensor's logical bytes (row-major), read back."""
    a = t.contiguous().cpu().numpy()
    return hashlib.sha256(np.ascontiguousarray(a).reshape(-1).view(np.uint8)).hexdigest()


def gpu_gemm(g, dev, a_src, a_mode, b_src, b_mode, relu=False):
    qa = g.quantize_rows if a_mode == "rows" else g.quantize_cols
    qb = g.quantize_rows if b_mode == "rows" else g.quantize_cols
    QA, s_row = qa(dev[a_src])
    QBt, s_col = qb(dev[b_src])
    C, h = g.gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu=relu, want_hash=True)
    h_stored = g.output_hash(C)
    torch.cuda.synchronize()
    return C, g.hash_value(h), g.hash_value(h_stored), (QA, s_row, QBt, s_col)


def check_gemm(g, C, h, h_stored, ops, want, what):
    """Fused hash, hash of the stored bytes, SHA-256 of the stored bytes and
    of the quantized operands, against the oracle's record."""
    assert list(C.shape) == want["shape"], what
    assert hex(h) == want["hash"], f"{what}: fused hash"
    assert hex(h_stored) == want["hash"], f"{what}: output_hash of the stored output"
    QA, s_row, QBt, s_col = ops
    assert full_digest(QA) == want["qa_sha256"], f"{what}: quantized A"
    assert full_digest(s_row) == want["sa_sha256"], f"{what}: row scales"
    assert full_digest(QBt) == want["qb_sha256"], f"{what}: quantized B"
    assert full_digest(s_col) == want["sb_sha256"], f"{what}: column scales"
    assert full_digest(C) == want["c_sha256"], f"{what}: stored output bytes"


def compare_rows(C_dev, A, B, a_mode, b_mode, chunk, what):
    """Every element of C against the oracle computed from the f32 inputs,
    `chunk` output rows at a time (first differing element reported)."""
    QA, s_row = ref.quantize_rows(A) if a_mode == "rows" else ref.quantize_cols(A)
    QBt, s_col = ref.quantize_rows(B) if b_mode == "rows" else ref.quantize_cols(B)
    M = QA.shape[0]
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        want = ref.gemm_i8_blockscaled(QA[r0:r1], s_row[r0:r1], QBt, s_col)
        got = C_dev[r0:r1].cpu().numpy()
        diff = got.view(U32) != want.view(U32)
        if diff.any():
            i, j = np.argwhere(diff)[0]
            raise AssertionError(f"{what}: {int(diff.sum())} elements differ in rows {r0}..{r1 - 1}; "
                                 f"first ({r0 + i}, {j}): got {got[i, j].view(U32):#010x} "
                                 f"want {want[i, j].view(U32):#010x}")


def test_w3_lm_head(g, golden):
    gh = golden["head"]
    X, W = S.w3_fwd_inputs()
    _, dY = S.w3_wgrad_inputs()
    host = {"X": X, "W": W, "dY": dY}
    for name, x in host.items():
        assert sample_digest(x) == gh["digests"][name], f"input generator changed ({name})"
    dev = {k: torch.from_numpy(v).cuda() for k, v in host.items()}

    say("w3 LM-head forward 8192x50304x768")
    C, h, hs, ops = gpu_gemm(g, dev, "X", "rows", "W", "cols")
    check_gemm(g, C, h, hs, ops, gh["fwd"], "LM-head forward")
    del ops
    say("w3 LM-head forward, every element against the oracle")
    compare_rows(C, X, W, "rows", "cols", 2048, "LM-head forward")
    del C

    say("w3 LM-head weight gradient 768x50304x8192")
    C, h, hs, ops = gpu_gemm(g, dev, "X", "cols", "dY", "cols")
    check_gemm(g, C, h, hs, ops, gh["wgrad"], "LM-head weight gradient")
    del ops
    say("w3 LM-head weight gradient, every element against the oracle")
    compare_rows(C, X, dY, "cols", "cols", 768, "LM-head weight gradient")


@pytest.mark.timeout(900)
def test_w5_training_step(g, golden):
    """The 147 GEMMs of one step in order: every GEMM's fused hash, the hash
    and SHA-256 of its stored output, the SHA-256 of its quantized operands,
    then the step hash that folds the GEMM hashes."""
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
        C, h, hs, ops = gpu_gemm(g, dev, a, am, b, bm)
        check_gemm(g, C, h, hs, ops, want, f"GEMM {gm.index} ({gm.linear} {gm.kind})")
        hashes.append(hs)
        del C, dev, ops
    assert hex(hashref.step_hash(hashes)) == golden["step"]["step_hash"]
