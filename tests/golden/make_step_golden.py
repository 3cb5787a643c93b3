"""Writes step_golden.json: what the CPU oracle computes for the GPT-2-small
LM-head GEMMs and for all 147 GEMMs of one training step (the synthetic
workloads of synth/inputs.py), plus the step hash.

Calls only oracle/ and the seeded generators of synth/ (no GPU code).  The
GPU tests regenerate the same inputs, run them through the library and
compare, so this file is what lets a full-size step be checked byte for byte
without re-running the slow CPU oracle on the GPU host.  Per GEMM it stores:
  hash       the output hash (oracle/hashref) of the f32 output;
  c_sha256   SHA-256 of the output's bytes (row-major f32, M x N): the GPU
             test digests the bytes it reads back from device memory, so a
             wrong store address, mask or cache hint cannot hide behind a hash
             accumulated from registers;
  qa_sha256, sa_sha256, qb_sha256, sb_sha256
             SHA-256 of the quantized operands (int8 M x K and N x K, both
             K-contiguous) and of their f32 scales;
  digests    a sample digest of each f32 input tensor (SHA-256 of every 4099th
             element): a mismatch there means the input generator changed,
             not the library.

    python tests/golden/make_step_golden.py          # ~5 minutes, ~14 GB RAM
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import hashref, ref  # noqa: E402
from synth import inputs as S  # noqa: E402


def sample_digest(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x.reshape(-1)[::4099]).tobytes()).hexdigest()


def full_digest(x: np.ndarray) -> str:
    """SHA-256 of an array's bytes in row-major order."""
    return hashlib.sha256(np.ascontiguousarray(x).reshape(-1).view(np.uint8)).hexdigest()


def quantize(x, mode):
    return ref.quantize_rows(x) if mode == "rows" else ref.quantize_cols(x)


def run_gemm(tensors, a_src, a_mode, b_src, b_mode, relu=False):
    """C = A B with A quantized per row, B per column, where A or B may be
    given transposed (the mode says which way the source tensor is quantized).
    Returns the record of one GEMM (without the input digests)."""
    QA, s_row = quantize(tensors[a_src], a_mode)
    QBt, s_col = quantize(tensors[b_src], b_mode)
    C = ref.gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu)
    h = hashref.output_hash(C)
    return h, {"shape": list(C.shape), "hash": hex(h), "c_sha256": full_digest(C),
               "qa_sha256": full_digest(QA), "sa_sha256": full_digest(s_row),
               "qb_sha256": full_digest(QBt), "sb_sha256": full_digest(s_col)}


def head_cases():
    X, W = S.w3_fwd_inputs()
    _, dY = S.w3_wgrad_inputs()
    t = {"X": X, "W": W, "dY": dY}
    out = {"digests": {k: sample_digest(v) for k, v in t.items()}}
    _, out["fwd"] = run_gemm(t, "X", "rows", "W", "cols")
    _, out["wgrad"] = run_gemm(t, "X", "cols", "dY", "cols")
    return out


def step_cases():
    gemms = S.step_gemms()
    cache = {}
    rows = []
    hashes = []
    for g in gemms:
        a, am, b, bm = g.operands
        t = {}
        for name in (a, b):
            key = (g.linear, name)
            if key not in cache:      # every tensor is kept (about 7 GB in all)
                cache[key] = S.step_tensor(g.linear, name, g.d_in, g.d_out)
            t[name] = cache[key]
        t0 = time.time()
        h, rec = run_gemm(t, a, am, b, bm)
        hashes.append(h)
        rows.append({"index": g.index, "linear": g.linear, "kind": g.kind, **rec,
                     "digests": {n: sample_digest(t[n]) for n in (a, b)}})
        print(f"[golden] {g.index:3d} {g.linear:10s} {g.kind:5s} {rec['shape']} {time.time() - t0:.1f}s",
              flush=True)
    return {"gemms": rows, "step_hash": hex(hashref.step_hash(hashes))}


def main():
    out = {"note": "written by tests/golden/make_step_golden.py from oracle/ (ref, hashref) "
                   "on the inputs of synth/inputs.py",
           "digest": "sha256 of every 4099th element of the f32 tensor",
           "full_digests": "sha256 of the whole array's bytes, row-major: c = f32 output, "
                           "qa / qb = int8 operands (M x K, N x K), sa / sb = f32 scales",
           "head": head_cases(),
           "step": step_cases()}
    with open(os.path.join(HERE, "step_golden.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
