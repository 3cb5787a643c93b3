"""Build libint8_gemm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m int8_gemm_amd.build            # build the library
    python -m int8_gemm_amd.build --asm DIR  # also write the gfx950 assembly

Compile flags that the method's bit-exactness depends on:
  -ffp-contract=off                          no multiply-add fusion anywhere
  -fhip-fp32-correctly-rounded-divide-sqrt   '/' is the IEEE division
and, for every HIP source on this target, packed-FP32 instruction
selection is switched off (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libint8_gemm.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "quantize.hip", "gemm.hip", "hash.hip", "verify.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libint8_gemm.so)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False, asm_dir: str = None) -> str:
    cc = hipcc()
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, *common_flags(), "-shared", "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    # A kernel template whose host-side instantiation fails leaves its launch
    # stub undefined: the link succeeds, but loading the library would not.
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
        stubs = [l.split()[-1] for l in und.splitlines() if "__device_stub__" in l]
        if stubs:
            raise RuntimeError("undefined kernel launch stubs in the built library: " + ", ".join(stubs))
    os.replace(tmp, LIB_PATH)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for s in srcs:
            out = os.path.join(asm_dir, os.path.basename(s) + f".{ARCH}.s")
            cmd = [cc, *common_flags(), "--cuda-device-only", "-S", "-o", out, s]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError("hipcc -S failed")
    return LIB_PATH


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for gfx950 assembly listings")
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.v, asm_dir=a.asm))


if __name__ == "__main__":
    main()
