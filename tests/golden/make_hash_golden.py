"""Writes hash_vectors.json: output hashes of small fixed matrices.

Calls only oracle/ (the hash is this library's own definition; the pages
name no hash function, so these vectors pin the definition against
accidental change, not against the pages).  Run from the repo root:
    python tests/golden/make_hash_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import hashref  # noqa: E402


def cases():
    yield "zeros_3x5", np.zeros((3, 5), dtype=np.float32)
    yield "negzero_1x1", np.array([[-0.0]], dtype=np.float32)
    yield "posone_1x1", np.array([[1.0]], dtype=np.float32)
    yield "ramp_4x7", (np.arange(28, dtype=np.float32).reshape(4, 7) - 13.5) / 4
    yield "ramp_7x4", (np.arange(28, dtype=np.float32).reshape(7, 4) - 13.5) / 4


def main():
    out = {"note": "written by tests/golden/make_hash_golden.py from oracle/hashref.py",
           "vectors": []}
    for name, C in cases():
        out["vectors"].append({"name": name, "shape": list(C.shape),
                               "bits": [hex(int(v)) for v in C.view(np.uint32).reshape(-1)],
                               "hash": hex(hashref.output_hash(C))})
    with open(os.path.join(HERE, "hash_vectors.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
