"""Host-side logic of bench.py (no GPU): the kernel-code digest that decides
whether the stored HBM traffic counters still describe the kernels."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_digest_ignores_comments_and_layout():
    a = "int f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n"
    b = "int f(int x) { return x + 1; }  // another comment\n"
    assert bench.code_digest_text(a) == bench.code_digest_text(b)


def test_digest_sees_code_changes():
    a = "int f(int x) { return x + 1; }"
    for b in ("int f(int x) { return x + 2; }", "int f(int x) { return x+1; }",
              "int f(int x) { return x + 1; } int g;"):
        assert bench.code_digest_text(a) != bench.code_digest_text(b), b


def test_digest_keeps_code_between_comments():
    text = "a /* x */ b // y\nc"
    assert bench.code_digest_text(text) == "a b c"


def test_kernel_source_sha_is_stable():
    s1, s2 = bench.kernel_source_sha(), bench.kernel_source_sha()
    assert s1 == s2 and len(s1) == 16

