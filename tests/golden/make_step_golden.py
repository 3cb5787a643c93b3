"""Writes step_golden.json: the oracle's output hashes of the GPT-2-small
LM-head GEMMs and of all 147 GEMMs of one training step (the synthetic
workloads of synth/inputs.py), plus the step hash.

Calls only oracle/ and the seeded generators of synth/ (no GPU code).  The
GPU tests regenerate the same inputs, run them through the library and
compare hashes, so this file is what lets a full-size step be checked
without re-running the slow CPU oracle on the GPU host.  Each tensor's
sample digest (SHA-256 of every 4099th element) is stored too: a mismatch
there means the input generator changed, not the library.

    python tests/golden/make_step_golden.py          # a few minutes, ~12 GB RAM
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


def quantize(x, mode):
    return ref.quantize_rows(x) if mode == "rows" else ref.quantize_cols(x)


def run_gemm(tensors, a_src, a_mode, b_src, b_mode, relu=False):
    """C = A B with A quantized per row, B per column, where A or B may be
    given transposed (the mode says which way the source tensor is quantized)."""
    QA, s_row = quantize(tensors[a_src], a_mode)
    QBt, s_col = quantize(tensors[b_src], b_mode)
    C = ref.gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu)
    return hashref.output_hash(C), C.shape


def head_cases():
    X, W = S.w3_fwd_inputs()
    _, dY = S.w3_wgrad_inputs()
    t = {"X": X, "W": W, "dY": dY}
    out = {"digests": {k: sample_digest(v) for k, v in t.items()}}
    h, shp = run_gemm(t, "X", "rows", "W", "cols")
    out["fwd"] = {"shape": list(shp), "hash": hex(h)}
    h, shp = run_gemm(t, "X", "cols", "dY", "cols")
    out["wgrad"] = {"shape": list(shp), "hash": hex(h)}
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
        h, shp = run_gemm(t, a, am, b, bm)
        hashes.append(h)
        rows.append({"index": g.index, "linear": g.linear, "kind": g.kind, "shape": list(shp),
                     "hash": hex(h), "digests": {n: sample_digest(t[n]) for n in (a, b)}})
        print(f"[golden] {g.index:3d} {g.linear:10s} {g.kind:5s} {shp} {time.time() - t0:.1f}s",
              flush=True)
    return {"gemms": rows, "step_hash": hex(hashref.step_hash(hashes))}


def main():
    out = {"note": "written by tests/golden/make_step_golden.py from oracle/ (ref, hashref) "
                   "on the inputs of synth/inputs.py",
           "digest": "sha256 of every 4099th element of the f32 tensor",
           "head": head_cases(),
           "step": step_cases()}
    with open(os.path.join(HERE, "step_golden.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
