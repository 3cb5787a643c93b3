"""Structural guard on the built gfx950 code: every floating-point step of
the method stays a separately rounded IEEE operation.

The DaisyChain-Train page "Verification -- why you can trust the numbers",
section "Hardware ground truth (RDNA2 ISA audit)", checks the instructions a
shader compiler actually emitted, because a fused multiply-add or an
approximate reciprocal changes output bytes while every behavioural test on
ordinary inputs may still pass.  This test does the same for the gfx950
assembly of the library's device code (built with the library's own flags):

  * no packed FP32 instruction (v_pk_*_f32) anywhere;
  * no mixed-precision FMA (v_fma_mix*, v_mad_mix*), no legacy mad/mac, no
    FMA with a literal addend (v_fmaak_f32), no approximate transcendental
    (v_rsq, v_sqrt, v_exp, v_log, v_rcp_legacy);
  * v_fma_f32, v_fmac_f32 and v_rcp_f32 occur only inside the two expansions
    that are exact by construction, and exactly as often as those need:
      - the correctly rounded binary32 division (scales s = a/127 and
        reciprocals 1/s): v_div_scale x2, v_rcp_f32, v_fma_f32 x3,
        v_fmac_f32 x2, v_div_fmas, v_div_fixup per division;
      - the 64-bit unsigned integer division the compiler expands through
        float (a v_fmamk_f32 with the literal 2^32, v_rcp_f32, a v_fmamk_f32
        with -2^32, then integer corrections): one v_rcp_f32 per expansion;
    and v_rcp_iflag_f32 only as the 32-bit integer division's estimate (at
    most one per int->float conversion).
So a contraction of x*inv + 0.5, of the epilogue's multiplies, or an
approximate reciprocal anywhere in the quantize, epilogue or drain code adds
an instruction the counts do not allow.  The last tests show that the rules
catch exactly those mistakes in a small kernel compiled with contraction on.
"""
import collections
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from int8_gemm_amd import build as B  # noqa: E402

SOURCES = ["quantize.hip", "gemm.hip", "hash.hip", "verify.hip", "api.hip"]
# kernels that must be present in the scanned code (the scan is not vacuous)
EXPECTED = ["qrows_wave_kernel", "qrows_block_kernel", "qcols_reg_kernel", "qcols_scale_kernel",
            "qcols_quant_kernel", "quantize_batch_kernel", "q4rows_kernel", "gemm_i8_dma_kernel",
            "gemm_i8_persist_kernel", "gemm_i8_persist128_kernel", "splitk_combine_kernel",
            "gemm_i4_kernel", "output_hash_kernel", "audit_gemm_kernel"]

FORBIDDEN = re.compile(r"^v_(pk_\w*f32|fma_mix\w*|mad_mix\w*|mad_f32|mac_f32|fmaak_f32|"
                       r"rsq\w*|sqrt\w*|exp\w*|log\w*|rcp_legacy\w*)$")


def have_hipcc():
    try:
        B.hipcc()
        return True
    except RuntimeError:
        return False


pytestmark = pytest.mark.skipif(not have_hipcc(), reason="hipcc (ROCm) is needed to build the code")


def compile_asm(src_path, out_path, extra=()):
    cmd = [B.hipcc(), *B.common_flags(), *extra, "--cuda-device-only", "-S", "-o", out_path, src_path]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def scan(path):
    """Per function: a Counter of instruction mnemonics (encoding suffixes
    dropped), with v_fmamk_f32 split by its literal."""
    funcs = {}
    fn, counts = None, None
    with open(path) as f:
        for line in f:
            m = re.match(r"^([A-Za-z_][\w.$]*):", line)
            if m and not line.startswith((".L", "$")):
                fn, counts = m.group(1), collections.Counter()
                continue
            if fn is None:
                continue
            s = line.strip()
            if not s or s.startswith((";", ".")):
                continue
            op = s.split()[0]
            op = re.sub(r"_e(32|64)$", "", op)
            if op == "v_fmamk_f32":
                lit = s.split(",")[2].strip()
                op = f"v_fmamk_f32[{lit}]"
            counts[op] += 1
            if op == "s_endpgm":
                funcs[fn] = counts
                fn = None
    return funcs


def violations(c):
    """Rule violations of one function's instruction counts."""
    bad = [f"{op} x{n}" for op, n in c.items() if FORBIDDEN.match(op)]
    n_div = c["v_div_fixup_f32"]
    n_u64 = c["v_fmamk_f32[0x4f800000]"]
    fmamk_other = sum(n for op, n in c.items()
                      if op.startswith("v_fmamk_f32") and op not in ("v_fmamk_f32[0x4f800000]",
                                                                     "v_fmamk_f32[0xcf800000]"))
    want = {"v_div_fmas_f32": n_div, "v_div_scale_f32": 2 * n_div, "v_fma_f32": 3 * n_div,
            "v_fmac_f32": 2 * n_div, "v_rcp_f32": n_div + n_u64,
            "v_fmamk_f32[0xcf800000]": n_u64}
    for op, n in want.items():
        if c[op] != n:
            bad.append(f"{op} x{c[op]} (allowed {n}: {n_div} divisions, {n_u64} 64-bit integer divisions)")
    if fmamk_other:
        bad.append(f"v_fmamk_f32 with another literal x{fmamk_other}")
    if c["v_rcp_iflag_f32"] > c["v_cvt_f32_u32"]:
        bad.append(f"v_rcp_iflag_f32 x{c['v_rcp_iflag_f32']} beyond the int->float conversions "
                   f"x{c['v_cvt_f32_u32']}")
    return bad


@pytest.fixture(scope="module")
def library_asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    procs = []
    for s in SOURCES:
        out = str(d / (s + ".s"))
        procs.append((s, out, compile_asm(os.path.join(B.CSRC, s), out)))
    funcs = {}
    for s, out, p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, f"hipcc -S {s} failed:\n{err[-2000:]}"
        for fn, c in scan(out).items():
            funcs[f"{s}:{fn}"] = c
    return funcs


@pytest.mark.timeout(600)
def test_scan_sees_every_kernel(library_asm):
    names = " ".join(library_asm)
    missing = [k for k in EXPECTED if k not in names]
    assert not missing, f"kernels not found in the assembly: {missing}"
    assert sum(c["v_div_fixup_f32"] for c in library_asm.values()) > 0, "no division found at all"
    assert sum(c["v_mfma_i32_32x32x32_i8"] for c in library_asm.values()) > 0, "no int8 MFMA found"


@pytest.mark.timeout(600)
def test_float_ops_separately_rounded(library_asm):
    report = {fn: v for fn, c in library_asm.items() if (v := violations(c))}
    assert not report, "fused, packed or approximate float instructions:\n" + "\n".join(
        f"{fn}: {', '.join(v)}" for fn, v in sorted(report.items()))


# ---- the rules have teeth: a small kernel with the quantizer and the
# ---- epilogue, compiled with and without contraction ----
PROBE = r"""
#include <hip/hip_runtime.h>
extern "C" __global__ void probe(const float* x, const int* acc, float a, float sr, float sc,
                                 int* q, float* y) {
  const int i = threadIdx.x;
  const float s = a / 127.0f;            // correctly rounded division
  const float inv = 1.0f / s;
  q[i] = (int)floorf(x[i] * inv + 0.5f);  // the quantizer
  y[i] = (float)acc[i] * sr * sc;         // the epilogue
}
"""
APPROX = r"""
#include <hip/hip_runtime.h>
extern "C" __global__ void probe(const float* x, float s, int* q) {
  const int i = threadIdx.x;
  const float inv = __builtin_amdgcn_rcpf(s);   // approximate reciprocal
  q[i] = (int)floorf(x[i] * inv + 0.5f);
}
"""


def probe_counts(tmp_path, text, extra):
    src = tmp_path / "probe.hip"
    src.write_text(text)
    out = str(tmp_path / "probe.s")
    p = compile_asm(str(src), out, extra)
    _, err = p.communicate()
    assert p.returncode == 0, err[-2000:]
    funcs = scan(out)
    assert "probe" in funcs
    return funcs["probe"]


@pytest.mark.timeout(300)
def test_rules_pass_the_separately_rounded_probe(tmp_path):
    c = probe_counts(tmp_path, PROBE, [])
    assert c["v_div_fixup_f32"] == 2
    assert violations(c) == []


@pytest.mark.timeout(300)
def test_rules_catch_contraction(tmp_path):
    # the library's flags end with -ffp-contract=off; a later flag overrides it
    c = probe_counts(tmp_path, PROBE, ["-ffp-contract=fast"])
    assert violations(c), "a contracted quantizer / epilogue was not caught"


@pytest.mark.timeout(300)
def test_rules_catch_approximate_reciprocal(tmp_path):
    c = probe_counts(tmp_path, APPROX, [])
    assert violations(c), "an approximate reciprocal was not caught"
