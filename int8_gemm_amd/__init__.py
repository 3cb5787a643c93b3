"""Python binding of libint8_gemm.so (bit-reproducible block-scaled int8 GEMM).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  The
entry points have the names of the C ABI in ``include/int8_gemm.h``:

    quantize_rows(X)                 -> (Q, scale)      per-row, Q is rows x cols
    quantize_cols(X)                 -> (Qt, scale)     per-column, Qt is cols x rows
    gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu=False, want_hash=False)
                                     -> C  or  (C, hash_tensor)
    output_hash(C)                   -> hash_tensor     (1 element, device)
    blockscaled_gemm(A, B, relu=False, want_hash=False)  A @ B, all steps
    quantize_rows_fmt(X, fmt) / quantize_cols_fmt(X, fmt)   FMT_POW2 / FMT_INT4
                                     storage formats (int4: 16*ceil(len/32) bytes per line)
    gemm_i8_blockscaled(..., K=K, a_int4=True / b_int4=True)  int4 operands

Hash tensors hold the 64-bit hash in an int64 element; ``hash_value``
returns it as a Python int in [0, 2^64).  If the library is not built, or
cannot be loaded, every entry point raises: there is no fallback.
"""
import contextlib
import ctypes
import os

import torch

__all__ = ["quantize_rows", "quantize_cols", "gemm_i8_blockscaled", "output_hash",
           "blockscaled_gemm", "hash_value", "workspace_bytes", "library_path", "load",
           "I8G_RELU", "I8G_HASH", "K_MAX", "I8GError", "quantize_rows_fmt", "quantize_cols_fmt",
           "FMT_POW2", "FMT_INT4", "int4_line_bytes", "gemm_i8_requant", "quantize_batch"]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libint8_gemm.so")
I8G_RELU = 1
I8G_HASH = 2
I8G_A_INT4 = 4
I8G_B_INT4 = 8
FMT_POW2 = 1
FMT_INT4 = 2
K_MAX = 133144
EXPORTED = ("quantize_rows", "quantize_cols", "gemm_i8_blockscaled", "gemm_i8_workspace_bytes",
            "output_hash", "output_hash_workspace_bytes", "i8g_status_string", "i8g_version",
            "i8g_gate", "i8g_gate_workspace_bytes", "i8g_audit_gemm", "i8g_audit_quantize",
            "i8g_probe_hash", "i8g_probe_workspace_bytes", "quantize_rows_fmt", "quantize_cols_fmt",
            "gemm_i8_requant", "gemm_i8_requant_workspace_bytes", "quantize_batch",
            "gemm_i8_workspace_bytes_flags", "i8g_audit_quantize_fmt", "i8g_set_test_overrides",
            "i8g_plan_query", "gemm_i8_blockscaled_noalloc")

_lib = None
_ws = {}


class I8GError(RuntimeError):
    def __init__(self, status, text):
        super().__init__(f"int8_gemm status {status}: {text}")
        self.status = status


def library_path() -> str:
    return LIB_PATH


def load():
    """Load libint8_gemm.so (once).  torch is imported first so that the
    library binds to the HIP runtime torch already loaded."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m int8_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_LOCAL)
    c_i64, c_vp, c_u32, c_sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_size_t
    lib.quantize_rows.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp]
    lib.quantize_rows.restype = ctypes.c_int
    lib.quantize_cols.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp]
    lib.quantize_cols.restype = ctypes.c_int
    lib.quantize_rows_fmt.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_u32, c_vp]
    lib.quantize_rows_fmt.restype = ctypes.c_int
    lib.quantize_cols_fmt.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_u32, c_vp]
    lib.quantize_cols_fmt.restype = ctypes.c_int
    lib.gemm_i8_blockscaled.argtypes = [c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64,
                                        c_vp, c_i64, c_u32, c_vp, c_vp, c_sz, c_vp]
    lib.gemm_i8_blockscaled.restype = ctypes.c_int
    lib.quantize_batch.argtypes = [ctypes.POINTER(QuantizeJob), ctypes.c_int32, c_vp]
    lib.quantize_batch.restype = ctypes.c_int
    lib.gemm_i8_requant.argtypes = [c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64,
                                    c_vp, c_i64, c_vp, c_u32, c_vp, c_vp, c_sz, c_vp]
    lib.gemm_i8_requant.restype = ctypes.c_int
    lib.gemm_i8_requant_workspace_bytes.argtypes = [c_i64, c_i64, c_i64]
    lib.gemm_i8_requant_workspace_bytes.restype = c_sz
    lib.gemm_i8_workspace_bytes_flags.argtypes = [c_i64, c_i64, c_i64, c_u32]
    lib.gemm_i8_workspace_bytes_flags.restype = c_sz
    lib.gemm_i8_workspace_bytes.argtypes = [c_i64, c_i64, c_i64]
    lib.gemm_i8_workspace_bytes.restype = c_sz
    lib.output_hash.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]
    lib.output_hash.restype = ctypes.c_int
    lib.output_hash_workspace_bytes.argtypes = []
    lib.output_hash_workspace_bytes.restype = c_sz
    lib.i8g_status_string.argtypes = [ctypes.c_int]
    lib.i8g_status_string.restype = ctypes.c_char_p
    lib.i8g_version.argtypes = []
    lib.i8g_version.restype = ctypes.c_char_p
    lib.i8g_gate_workspace_bytes.argtypes = []
    lib.i8g_gate_workspace_bytes.restype = c_sz
    lib.i8g_gate.argtypes = [c_vp, c_sz, c_vp, ctypes.POINTER(GateReport)]
    lib.i8g_gate.restype = ctypes.c_int
    lib.i8g_audit_gemm.argtypes = [c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_vp,
                                   c_i64, c_u32, ctypes.c_uint64, ctypes.c_int32, c_vp, c_vp]
    lib.i8g_audit_gemm.restype = ctypes.c_int
    lib.i8g_audit_quantize.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, ctypes.c_int32,
                                       ctypes.c_uint64, ctypes.c_int32, c_vp, c_vp]
    lib.i8g_audit_quantize.restype = ctypes.c_int
    lib.i8g_audit_quantize_fmt.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, ctypes.c_int32, c_u32,
                                           ctypes.c_uint64, ctypes.c_int32, c_vp, c_vp]
    lib.i8g_audit_quantize_fmt.restype = ctypes.c_int
    lib.i8g_probe_workspace_bytes.argtypes = [c_i64, c_i64, c_i64]
    lib.i8g_probe_workspace_bytes.restype = c_sz
    lib.i8g_probe_hash.argtypes = [ctypes.c_uint64, c_i64, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]
    lib.i8g_probe_hash.restype = ctypes.c_int
    c_i32 = ctypes.c_int32
    lib.gemm_i8_blockscaled_noalloc.argtypes = [c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i64, c_i64,
                                                c_i64, c_vp, c_i64, c_u32, c_vp, c_vp]
    lib.gemm_i8_blockscaled_noalloc.restype = ctypes.c_int
    lib.i8g_set_test_overrides.argtypes = [c_i32, c_i32, c_i32, c_i32]
    lib.i8g_set_test_overrides.restype = ctypes.c_int
    lib.i8g_plan_query.argtypes = [c_i64, c_i64, c_i64, c_i64, c_u32, ctypes.POINTER(c_i32),
                                   ctypes.POINTER(c_i32)]
    lib.i8g_plan_query.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        raise I8GError(rc, load().i8g_status_string(rc).decode())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _req_matrix(x, dtype, name):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    if x.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if x.numel() > 0 and x.size(1) > 1 and x.stride(1) != 1:   # (empty tensors may carry stride 0)
        raise ValueError(f"{name} must be row-major (unit column stride)")


def _ld(x):
    return max(x.stride(0), x.size(1), 1)


def _round16(n):
    return (n + 15) // 16 * 16


def _int8_padded(rows, cols, device):
    """rows x cols int8 view of a buffer whose rows are padded to 16 bytes."""
    ld = max(_round16(cols), 16)
    return torch.empty((rows, ld), dtype=torch.int8, device=device)[:, :cols]


def quantize_rows(X):
    _req_matrix(X, torch.float32, "X")
    rows, cols = X.shape
    Q = _int8_padded(rows, cols, X.device)
    s = torch.empty(rows, dtype=torch.float32, device=X.device)
    _check(load().quantize_rows(_ptr(X), rows, cols, _ld(X), _ptr(Q), Q.stride(0), _ptr(s),
                                _stream(X)))
    return Q, s


def quantize_cols(X):
    _req_matrix(X, torch.float32, "X")
    rows, cols = X.shape
    Qt = _int8_padded(cols, rows, X.device)
    s = torch.empty(cols, dtype=torch.float32, device=X.device)
    _check(load().quantize_cols(_ptr(X), rows, cols, _ld(X), _ptr(Qt), Qt.stride(0), _ptr(s),
                                _stream(X)))
    return Qt, s


def int4_line_bytes(n):
    """Bytes of one int4 line of n values (whole 16-byte groups of 32)."""
    return 16 * ((n + 31) // 32)


def _line_buffer(lines, n, fmt, device):
    if fmt & FMT_INT4:
        return torch.empty((lines, max(int4_line_bytes(n), 16)), dtype=torch.int8,
                           device=device)[:, :int4_line_bytes(n)]
    return _int8_padded(lines, n, device)


def quantize_rows_fmt(X, fmt):
    """quantize_rows in storage format ``fmt`` (FMT_POW2 | FMT_INT4 bits).
    int4: Q is rows x int4_line_bytes(cols) int8 (the packed bytes)."""
    _req_matrix(X, torch.float32, "X")
    rows, cols = X.shape
    Q = _line_buffer(rows, cols, fmt, X.device)
    s = torch.empty(rows, dtype=torch.float32, device=X.device)
    _check(load().quantize_rows_fmt(_ptr(X), rows, cols, _ld(X), _ptr(Q), Q.stride(0), _ptr(s),
                                    fmt, _stream(X)))
    return Q, s


def quantize_cols_fmt(X, fmt):
    """quantize_cols in storage format ``fmt``; int4: Qt is cols x
    int4_line_bytes(rows)."""
    _req_matrix(X, torch.float32, "X")
    rows, cols = X.shape
    Qt = _line_buffer(cols, rows, fmt, X.device)
    s = torch.empty(cols, dtype=torch.float32, device=X.device)
    _check(load().quantize_cols_fmt(_ptr(X), rows, cols, _ld(X), _ptr(Qt), Qt.stride(0), _ptr(s),
                                    fmt, _stream(X)))
    return Qt, s


class QuantizeJob(ctypes.Structure):
    """i8g_quantize_job (include/int8_gemm.h)."""
    _fields_ = [("X", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ldx", ctypes.c_int64), ("Q", ctypes.c_void_p), ("ldq", ctypes.c_int64),
                ("scale", ctypes.c_void_p), ("by_col", ctypes.c_uint32), ("format", ctypes.c_uint32)]


def quantize_jobs(specs):
    """ctypes job array and outputs for specs = [(X, by_col, fmt), ...]:
    returns (array, [(Q, scale), ...]) with outputs laid out as the single
    calls lay them out."""
    arr = (QuantizeJob * len(specs))()
    outs = []
    for i, (X, by_col, fmt) in enumerate(specs):
        _req_matrix(X, torch.float32, "X")
        rows, cols = X.shape
        lines, n = (cols, rows) if by_col else (rows, cols)
        Q = _line_buffer(lines, n, fmt, X.device)
        s = torch.empty(lines, dtype=torch.float32, device=X.device)
        arr[i] = QuantizeJob(X.data_ptr(), rows, cols, _ld(X), Q.data_ptr(), Q.stride(0), s.data_ptr(),
                             1 if by_col else 0, fmt)
        outs.append((Q, s))
    return arr, outs


def quantize_batch(specs):
    """Several quantize passes in one call: specs = [(X, by_col, fmt), ...];
    returns [(Q, scale), ...], each equal to quantize_{rows,cols}_fmt(X, fmt)."""
    if not specs:
        return []
    arr, outs = quantize_jobs(specs)
    _check(load().quantize_batch(arr, len(specs), _stream(specs[0][0])))
    return outs


def workspace_bytes(M, N, K, flags=0):
    return int(load().gemm_i8_workspace_bytes_flags(M, N, K, flags))


def _workspace(device, nbytes):
    """Scratch buffer per (device, stream), grown on demand.  It is zeroed
    when allocated: the library needs its 256-byte header zero and leaves
    it zero after every call."""
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           torch.cuda.current_stream(device).cuda_stream)
    ws = _ws.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws[key] = ws
    return ws


def gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu=False, want_hash=False, out=None, K=None,
                        a_int4=False, b_int4=False):
    """C = epilogue(QA . QBt^T).  With a_int4 / b_int4 the operand holds
    packed int4 lines (quantize_*_fmt with FMT_INT4) and K must be given."""
    _req_matrix(QA, torch.int8, "QA")
    _req_matrix(QBt, torch.int8, "QBt")
    M, ka = QA.shape
    N, kb = QBt.shape
    if K is None:
        if a_int4 or b_int4:
            raise ValueError("K is required with int4 operands")
        K = ka
    if ka != (int4_line_bytes(K) if a_int4 else K) or kb != (int4_line_bytes(K) if b_int4 else K):
        raise ValueError(f"operand widths {ka}, {kb} do not match K = {K}")
    if s_row.dtype != torch.float32 or s_col.dtype != torch.float32:
        raise ValueError("scales must be float32")
    if s_row.numel() != M or s_col.numel() != N:
        raise ValueError("scale lengths must be M and N")
    if not (s_row.is_contiguous() and s_col.is_contiguous()):
        raise ValueError("scales must be contiguous")
    dev = QA.device
    C = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _req_matrix(C, torch.float32, "out")
    h = torch.zeros(1, dtype=torch.int64, device=dev) if want_hash else None
    flags = ((I8G_RELU if relu else 0) | (I8G_HASH if want_hash else 0) |
             (I8G_A_INT4 if a_int4 else 0) | (I8G_B_INT4 if b_int4 else 0))
    ws = _workspace(dev, workspace_bytes(M, N, K, flags))
    lda = QA.stride(0) if M > 0 else _round16(K)
    ldb = QBt.stride(0) if N > 0 else _round16(K)
    _check(load().gemm_i8_blockscaled(
        _ptr(QA), lda, _ptr(s_row), _ptr(QBt), ldb, _ptr(s_col), M, N, K,
        _ptr(C), max(C.stride(0), N, 1), flags, _ptr(h), ctypes.c_void_p(ws.data_ptr()),
        ws.numel(), _stream(QA)))
    return (C, h) if want_hash else C


def gemm_i8_blockscaled_noalloc(QA, s_row, QBt, s_col, relu=False, want_hash=False, out=None):
    """gemm_i8_blockscaled through the entry point that allocates nothing (its
    scratch is the library's static device array): int8 operands only.  The
    output (and hash tensor) are allocated here unless `out` is given."""
    _req_matrix(QA, torch.int8, "QA")
    _req_matrix(QBt, torch.int8, "QBt")
    M, K = QA.shape
    N, K2 = QBt.shape
    if K2 != K:
        raise ValueError(f"K mismatch: QA has {K}, QBt has {K2}")
    if s_row.numel() != M or s_col.numel() != N or s_row.dtype != torch.float32 or \
            s_col.dtype != torch.float32 or not (s_row.is_contiguous() and s_col.is_contiguous()):
        raise ValueError("scales must be contiguous float32 of lengths M and N")
    dev = QA.device
    C = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    _req_matrix(C, torch.float32, "out")
    h = torch.zeros(1, dtype=torch.int64, device=dev) if want_hash else None
    flags = (I8G_RELU if relu else 0) | (I8G_HASH if want_hash else 0)
    _check(load().gemm_i8_blockscaled_noalloc(
        _ptr(QA), QA.stride(0) if M > 0 else _round16(K), _ptr(s_row), _ptr(QBt),
        QBt.stride(0) if N > 0 else _round16(K), _ptr(s_col), M, N, K, _ptr(C), max(C.stride(0), N, 1),
        flags, _ptr(h), _stream(QA)))
    return (C, h) if want_hash else C


def gemm_i8_requant(QA, s_row, QBt, s_col, relu=False, want_hash=False):
    """The requantizing epilogue: (Q, scale) = quantize_rows of the GEMM's
    f32 output, which is never stored; with want_hash also the output's
    hash tensor."""
    _req_matrix(QA, torch.int8, "QA")
    _req_matrix(QBt, torch.int8, "QBt")
    M, K = QA.shape
    N, K2 = QBt.shape
    if K2 != K:
        raise ValueError(f"K mismatch: QA has {K}, QBt has {K2}")
    dev = QA.device
    Q = _int8_padded(M, N, dev)
    s = torch.empty(M, dtype=torch.float32, device=dev)
    h = torch.zeros(1, dtype=torch.int64, device=dev) if want_hash else None
    ws = _workspace(dev, int(load().gemm_i8_requant_workspace_bytes(M, N, K)))
    flags = (I8G_RELU if relu else 0) | (I8G_HASH if want_hash else 0)
    _check(load().gemm_i8_requant(
        _ptr(QA), QA.stride(0) if M > 0 else _round16(K), _ptr(s_row), _ptr(QBt),
        QBt.stride(0) if N > 0 else _round16(K), _ptr(s_col), M, N, K, _ptr(Q), max(Q.stride(0), N, 1),
        _ptr(s), flags, _ptr(h), ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(QA)))
    return (Q, s, h) if want_hash else (Q, s)


def output_hash(C):
    _req_matrix(C, torch.float32, "C")
    M, N = C.shape
    h = torch.zeros(1, dtype=torch.int64, device=C.device)
    ws = _workspace(C.device, int(load().output_hash_workspace_bytes()))
    _check(load().output_hash(_ptr(C), M, N, max(C.stride(0), N, 1), _ptr(h),
                              ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(C)))
    return h


class GateReport(ctypes.Structure):
    """i8g_gate_report (include/int8_gemm.h)."""
    _fields_ = [("check", ctypes.c_int32), ("config", ctypes.c_int32), ("m", ctypes.c_int64),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("index", ctypes.c_int64),
                ("got", ctypes.c_uint32), ("want", ctypes.c_uint32), ("cases", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


def gate(device=None):
    """Runs the init gate (i8g_gate) on `device` (default: the current one).
    Returns (status, report dict); status 0 means every check passed."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    lib = load()
    nbytes = int(lib.i8g_gate_workspace_bytes())
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rep = GateReport()
    with torch.cuda.device(dev):
        rc = lib.i8g_gate(ctypes.c_void_p(ws.data_ptr()), nbytes,
                          ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream), ctypes.byref(rep))
    return rc, rep.as_dict()


def audit_gemm(QA, s_row, QBt, s_col, C, relu=False, seed=0, samples=1024, K=None, a_int4=False,
               b_int4=False):
    """i8g_audit_gemm on a GEMM output: returns a 2-element int64 device
    tensor (number of differing sampled cells, smallest i*N + j of them or -1).
    With int4 operands (packed lines) K must be given."""
    M, ka = QA.shape
    N = QBt.shape[0]
    if K is None:
        if a_int4 or b_int4:
            raise ValueError("K is required with int4 operands")
        K = ka
    flags = (I8G_RELU if relu else 0) | (I8G_A_INT4 if a_int4 else 0) | (I8G_B_INT4 if b_int4 else 0)
    r = torch.empty(2, dtype=torch.int64, device=C.device)
    _check(load().i8g_audit_gemm(
        _ptr(QA), QA.stride(0) if M > 0 else _round16(K), _ptr(s_row), _ptr(QBt),
        QBt.stride(0) if N > 0 else _round16(K), _ptr(s_col), M, N, K, _ptr(C), max(C.stride(0), N, 1),
        flags, seed & ((1 << 64) - 1), samples, _ptr(r), _stream(C)))
    return r


def audit_quantize(X, Q, scale, by_col, seed=0, samples=64, fmt=0):
    """i8g_audit_quantize_fmt: X with its quantize_rows_fmt (by_col=False) or
    quantize_cols_fmt (by_col=True) output in format ``fmt``; returns as
    audit_gemm (lines)."""
    rows, cols = X.shape
    r = torch.empty(2, dtype=torch.int64, device=X.device)
    _check(load().i8g_audit_quantize_fmt(
        _ptr(X), rows, cols, max(X.stride(0), cols, 1), _ptr(Q), max(Q.stride(0), 1), _ptr(scale),
        1 if by_col else 0, fmt, seed & ((1 << 64) - 1), samples, _ptr(r), _stream(X)))
    return r


def probe_hash(seed, M, N, K, device=None):
    """i8g_probe_hash: the output hash of the seeded probe GEMM (int64 tensor)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    lib = load()
    nbytes = int(lib.i8g_probe_workspace_bytes(M, N, K))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    h = torch.zeros(1, dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        _check(lib.i8g_probe_hash(seed & ((1 << 64) - 1), M, N, K, _ptr(h), ctypes.c_void_p(ws.data_ptr()),
                                  nbytes, ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)))
    return h


_overrides = {"force_tile": -1, "force_splits": 0, "qcols_path": 0, "int4_direct": 0}


@contextlib.contextmanager
def plan_overrides(**kw):
    """Plan overrides for tests (i8g_set_test_overrides) inside a with-block:
    force_tile (-1: the planner's choice), force_splits (0: the planner's),
    qcols_path (0: the planner's, 1: two-pass kernels, 2: cooperative
    one-read kernel, 3: two whole-line passes, 4: the cooperative kernel
    with its waits cut to one spin; 2 to 4 where the shape allows them),
    int4_direct.  Blocks nest: settings not given are kept
    from the enclosing block, and each block restores the previous ones."""
    unknown = set(kw) - set(_overrides)
    if unknown:
        raise TypeError(f"unknown plan overrides {sorted(unknown)}")
    prev = dict(_overrides)
    new = dict(prev)
    new.update({k: int(v) for k, v in kw.items()})

    def apply(o):
        _check(load().i8g_set_test_overrides(o["force_tile"], o["force_splits"], o["qcols_path"],
                                             o["int4_direct"]))
        _overrides.update(o)

    apply(new)
    try:
        yield
    finally:
        apply(prev)


def plan_query(M, N, K, ldc=None, flags=0):
    """(tile configuration, K splits) that gemm_i8_blockscaled would use now."""
    cfg, splits = ctypes.c_int32(), ctypes.c_int32()
    _check(load().i8g_plan_query(M, N, K, N if ldc is None else ldc, flags, ctypes.byref(cfg),
                                 ctypes.byref(splits)))
    return cfg.value, splits.value


def hash_value(h) -> int:
    """The 64-bit hash held by a 1-element int64 tensor, as an unsigned int."""
    return int(h.item()) & ((1 << 64) - 1)


def blockscaled_gemm(A, B, relu=False, want_hash=False):
    """C = A @ B through the whole method: quantize_rows(A), quantize_cols(B),
    then the int8 GEMM with its epilogue."""
    QA, s_row = quantize_rows(A)
    QBt, s_col = quantize_cols(B)
    return gemm_i8_blockscaled(QA, s_row, QBt, s_col, relu=relu, want_hash=want_hash)
