"""The C-ABI library loads on a host without a GPU and exports every symbol
that include/int8_gemm.h declares (no compute calls here)."""
import ctypes
import os
import re

import pytest


def _declared(repo_root):
    text = open(os.path.join(repo_root, "include", "int8_gemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^#.*$", "", text, flags=re.M)
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{]*\)\s*;", text)
    return sorted(set(n for n in names if n not in ("if", "while", "sizeof")))


def test_header_declares_the_four_entry_points(repo_root):
    names = _declared(repo_root)
    for n in ("quantize_rows", "quantize_cols", "gemm_i8_blockscaled", "output_hash"):
        assert n in names


def test_library_exports_every_declared_symbol(repo_root):
    import int8_gemm_amd as g
    if not os.path.exists(g.library_path()):
        pytest.fail("libint8_gemm.so is not built (python -m int8_gemm_amd.build)")
    lib = g.load()
    for n in _declared(repo_root):
        assert hasattr(lib, n), n
        assert isinstance(getattr(lib, n), ctypes._CFuncPtr)
    assert set(g.EXPORTED) == set(_declared(repo_root))


def test_host_only_calls(repo_root):
    """Calls that touch no device: status strings, version, workspace sizing."""
    import int8_gemm_amd as g
    lib = g.load()
    assert lib.i8g_version().startswith(b"int8_gemm")
    for st in range(8):
        assert lib.i8g_status_string(st)
    assert lib.i8g_status_string(99) == b"unknown status"
    assert g.workspace_bytes(256, 256, 256) >= 256
    assert g.workspace_bytes(0, 5, 5) == 256
    # argument errors are reported before anything is enqueued
    assert lib.quantize_rows(None, -1, 2, 2, None, 2, None, None) == 1
    assert lib.output_hash(None, 1, 1, 1, None, None, 0, None) == 1


def test_argument_checks_of_the_extended_entry_points():
    """Validation happens on the host before anything is enqueued, so these
    calls return their status without a device."""
    import int8_gemm_amd as g
    lib = g.load()
    P = ctypes.c_void_p
    fake = P(1 << 20)                      # never dereferenced: every call below fails validation
    # quantize_*_fmt: unknown format bit, negative size, ld below the (int4) line length
    assert lib.quantize_rows_fmt(fake, 4, 40, 40, fake, 40, fake, 4, None) == 1
    assert lib.quantize_cols_fmt(fake, -1, 4, 4, fake, 4, fake, 0, None) == 1
    assert lib.quantize_rows_fmt(fake, 4, 40, 40, fake, 16, fake, 2, None) == 1    # needs 32 bytes
    assert lib.quantize_cols_fmt(fake, 40, 4, 4, fake, 16, fake, 2, None) == 1     # needs 32 bytes
    assert lib.quantize_rows_fmt(fake, 4, 40, 40, P((1 << 20) + 1), 32, fake, 2, None) == 3
    assert lib.quantize_rows_fmt(fake, 4, 40, 40, fake, 40, None, 0, None) == 1    # null scale
    assert lib.quantize_rows_fmt(None, 0, 40, 40, None, 40, None, 0, None) == 0    # nothing to do
    # quantize_batch: bad count, null array, a bad job stops the whole batch
    assert lib.quantize_batch(None, -1, None) == 1
    assert lib.quantize_batch(None, 2, None) == 1
    assert lib.quantize_batch(None, 0, None) == 0
    jobs = (g.QuantizeJob * 2)(g.QuantizeJob(fake.value, 4, 40, 40, fake.value, 40, fake.value, 0, 0),
                               g.QuantizeJob(fake.value, 4, 40, 40, fake.value, 3, fake.value, 1, 0))
    assert lib.quantize_batch(jobs, 2, None) == 1          # job 1: its lines (columns) hold 4 values, ldq 3
    # gemm: unknown flag, K beyond the int32 range, int4 operand ld below 16*ceil(K/32)
    ws = P(1 << 24)
    assert lib.gemm_i8_blockscaled(fake, 16, fake, fake, 16, fake, 4, 4, 4, fake, 4, 16, None, ws, 1 << 20, None) == 1
    assert lib.gemm_i8_blockscaled(fake, 16, fake, fake, 16, fake, 4, 4, 133145, fake, 4, 0, None, ws, 1 << 20, None) == 2
    assert lib.gemm_i8_blockscaled(fake, 16, fake, fake, 16, fake, 4, 4, 64, fake, 4, 4, None, ws, 1 << 20, None) == 3
    # requant: unknown flag, null outputs, ldq < N, misaligned workspace
    assert lib.gemm_i8_requant(fake, 16, fake, fake, 16, fake, 4, 4, 4, fake, 4, fake, 4, None, ws, 1 << 20, None) == 1
    assert lib.gemm_i8_requant(fake, 16, fake, fake, 16, fake, 4, 4, 4, None, 4, fake, 0, None, ws, 1 << 20, None) == 1
    assert lib.gemm_i8_requant(fake, 16, fake, fake, 16, fake, 4, 5, 4, fake, 4, fake, 0, None, ws, 1 << 20, None) == 1
    assert lib.gemm_i8_requant(fake, 16, fake, fake, 16, fake, 4, 4, 4, fake, 4, fake, 0, None, P(1 << 20 | 8), 1 << 20, None) == 4
    # workspace sizes: int4 operands need room for their widened copies
    M, N, K = 512, 768, 3072
    base = lib.gemm_i8_workspace_bytes(M, N, K)
    assert lib.gemm_i8_workspace_bytes_flags(M, N, K, 0) == base
    assert lib.gemm_i8_workspace_bytes_flags(M, N, K, 8) >= N * K
    assert lib.gemm_i8_workspace_bytes_flags(M, N, K, 12) >= (M + N) * K
    assert lib.gemm_i8_requant_workspace_bytes(M, N, K) >= 256 + 4 * M
    assert lib.gemm_i8_requant_workspace_bytes(0, N, K) == 256
    assert lib.i8g_status_string(6).startswith(b"self-check failed")


def test_test_overrides_and_plan_query():
    """The test hooks are explicit calls (no environment variable is read on
    the plan path): the override entry point validates its arguments and the
    plan query reports what the planner picks under it (host-only logic)."""
    import int8_gemm_amd as g
    lib = g.load()
    assert lib.i8g_set_test_overrides(8, 0, 0, 0) == 1        # no tile configuration 8
    assert lib.i8g_set_test_overrides(-2, 0, 0, 0) == 1
    assert lib.i8g_set_test_overrides(-1, -1, 0, 0) == 1
    assert lib.i8g_set_test_overrides(-1, 0, 5, 0) == 1        # column paths 0..4
    assert lib.i8g_set_test_overrides(-1, 0, 4, 0) == 0
    assert lib.i8g_set_test_overrides(-1, 0, 0, 0) == 0
    with pytest.raises(g.I8GError):
        g.plan_query(0, 5, 5)
    free_cfg, free_splits = g.plan_query(1000, 1000, 1024)
    with g.plan_overrides(force_tile=2, force_splits=4):
        assert g.plan_query(1000, 1000, 1024) == (2, 4)
        with g.plan_overrides(force_splits=0):                 # nested: the tile stays forced
            assert g.plan_query(1000, 1000, 1024) == (2, 1)
        assert g.plan_query(1000, 1000, 1024) == (2, 4)
    assert g.plan_query(1000, 1000, 1024) == (free_cfg, free_splits)
    # a forced two-workgroups-per-CU tile runs beyond the K the cost model
    # keeps it to (it is still correct there, only slower)
    with g.plan_overrides(force_tile=7):
        assert g.plan_query(2048, 2000, 1536) == (7, 1)
    with g.plan_overrides(int4_direct=True):
        assert g.plan_query(96, 200, 4160, flags=g.I8G_B_INT4)[0] == 8


def test_noalloc_argument_checks():
    """gemm_i8_blockscaled_noalloc validates and plans on the host before
    anything is enqueued (no device is touched by these calls): argument
    errors as gemm_i8_blockscaled, and a plan needing more than the static
    64 MiB scratch is refused with I8G_ESCRATCH."""
    import int8_gemm_amd as g
    lib = g.load()
    P = ctypes.c_void_p
    fake = P(1 << 20)                      # 16-byte aligned, never dereferenced
    f = lib.gemm_i8_blockscaled_noalloc
    assert f(fake, 64, fake, fake, 64, fake, -1, 8, 64, fake, 8, 0, None, None) == 1      # negative M
    assert f(fake, 64, fake, fake, 64, fake, 8, 8, 64, fake, 8, 2, None, None) == 1       # hash without pointer
    assert f(fake, 64, fake, fake, 64, fake, 8, 8, 200000, fake, 8, 0, None, None) == 2   # K beyond int32
    assert f(P((1 << 20) + 1), 64, fake, fake, 64, fake, 8, 8, 64, fake, 8, 0, None, None) == 3
    assert f(fake, 64, fake, fake, 64, fake, 8, 8, 64, fake, 8, 1 << 7, None, None) == 1  # unknown flag
    with g.plan_overrides(force_tile=2, force_splits=2):
        # two int32 partial planes of 4096 x 4096: 128 MiB > 64 MiB
        assert f(fake, 8192, fake, fake, 8192, fake, 4096, 4096, 8192, fake, 4096, 0, None, None) == 7
    assert lib.i8g_status_string(7).startswith(b"the shape needs more scratch")
