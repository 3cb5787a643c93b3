// api.hip -- the C ABI of libint8_gemm.so (declared in include/int8_gemm.h):
// argument validation, status codes, workspace layout and kernel launches
// on the caller's stream.  No device memory is allocated here.
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/int8_gemm.h"
#include "i8g_device.h"
#include "i8g_launch.h"

using namespace i8g;

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int hip_status(hipError_t e) { return e == hipSuccess ? I8G_OK : I8G_EHIP; }

// ---------------------------------------------------------------------------
// Scratch of gemm_i8_blockscaled_noalloc: a file-scope device array (one copy
// per GPU, from the code object's load until the process ends).  In host
// code its name is only a stand-in for the device symbol: the device address
// comes from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
constexpr size_t kNoallocScratchBytes = I8G_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Zeroes the workspace control header (64 words); a kernel rather than a
// memset, so that a caller capturing the stream into a HIP graph records a
// kernel node.
__global__ void zero_header_kernel(unsigned int* h) { h[threadIdx.x] = 0u; }

// The scratch array's device address on the current device; at the first
// call on a device also enqueues the zeroing of its header on `stream`.
int scratch_for_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return I8G_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return I8G_EHIP;
    hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(kWsHeader / 4), 0, stream,
                       reinterpret_cast<unsigned int*>(p));
    if (hipGetLastError() != hipSuccess) return I8G_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return I8G_OK;
}

}  // namespace

namespace i8g {

int enqueue_gemm(const int8_t* QA, int64_t lda, const float* s_row, const int8_t* QBt, int64_t ldb,
                 const float* s_col, int64_t M, int64_t N, int64_t K, float* C, int64_t ldc,
                 uint32_t flags, uint64_t* hash, void* workspace, size_t workspace_bytes,
                 hipStream_t stream, int force_tile, int force_splits) {
  // force_tile == -4: validate and plan only (the workspace pointer is not
  // needed, its size is checked), enqueue nothing
  const bool dry = force_tile == -4;
  if (dry) force_tile = -2;
  if (M < 0 || N < 0 || K < 0) return I8G_EINVAL;
  if (M > INT32_MAX || N > INT32_MAX) return I8G_EINVAL;
  if (flags & ~(I8G_RELU | I8G_HASH | I8G_A_INT4 | I8G_B_INT4)) return I8G_EINVAL;
  const bool a4 = (flags & I8G_A_INT4) != 0, b4 = (flags & I8G_B_INT4) != 0;
  const bool want_hash = (flags & I8G_HASH) != 0;
  if (want_hash && !hash) return I8G_EINVAL;
  if (K > I8G_K_MAX) return I8G_EKRANGE;
  if (!dry && (!workspace || ((uintptr_t)workspace % 256) != 0)) return I8G_EWORKSPACE;
  if (M == 0 || N == 0) {
    if (workspace_bytes < kWsHeader) return I8G_EWORKSPACE;
    if (dry) return I8G_OK;
    if (want_hash) return hip_status(launch_output_hash(C, M, N, ldc, hash, workspace, stream));
    return I8G_OK;
  }
  if (!C || !s_row || !s_col || ldc < N) return I8G_EINVAL;
  if (K > 0 && (!QA || !QBt)) return I8G_EINVAL;
  const int64_t k16 = (K + 15) / 16 * 16, k4 = (K + 31) / 32 * 16;   // row bytes: int8, int4
  if (K > 0) {
    if (((uintptr_t)QA % 16) || ((uintptr_t)QBt % 16) || (lda % 16) || (ldb % 16) ||
        lda < (a4 ? k4 : k16) || ldb < (b4 ? k4 : k16))
      return I8G_EALIGN;
  }
  // force_tile == -2: the library's own choice (plan_gemm, which honours the
  // test overrides); -3: the direct int4 kernel; otherwise exactly the forced
  // configuration
  const bool direct4 = (a4 || b4) && (force_tile == -3 || (force_tile == -2 && int4_direct_requested()));
  GemmPlan plan = direct4 ? plan_gemm_int4(M, N, K > 0 ? K : 1, force_tile < 0 ? -1 : force_splits)
                  : force_tile < 0
                      ? plan_gemm(M, N, K > 0 ? K : 1, ldc <= kPersistMaxLdc)
                      : plan_gemm_forced(M, N, K > 0 ? K : 1, ldc <= kPersistMaxLdc, force_tile, force_splits);
  if (workspace_bytes < plan.workspace_bytes) return I8G_EWORKSPACE;
  const bool widen = (a4 || b4) && !direct4 && K > 0;   // int4 operands widened into the workspace
  const int64_t ldw = widen ? int4_widened_ld(K) : 0;
  const size_t wa_off = (plan.workspace_bytes + 255) / 256 * 256;
  const size_t wa_bytes = (widen && a4) ? ((size_t)M * ldw + 255) / 256 * 256 : 0;
  const size_t wb_bytes = (widen && b4) ? ((size_t)N * ldw + 255) / 256 * 256 : 0;
  if (widen && workspace_bytes < wa_off + wa_bytes + wb_bytes) return I8G_EWORKSPACE;
  if (dry) return I8G_OK;
  bool wa = false, wb = false;   // operands widened into the workspace
  if (widen) {
    char* ws = reinterpret_cast<char*>(workspace);
    if (a4) {
      int8_t* w = reinterpret_cast<int8_t*>(ws + wa_off);
      if (launch_widen_int4(QA, lda, M, K, w, stream) != hipSuccess) return I8G_EHIP;
      QA = w;
      lda = ldw;
      wa = true;
    }
    if (b4) {
      int8_t* w = reinterpret_cast<int8_t*>(ws + wa_off + wa_bytes);
      if (launch_widen_int4(QBt, ldb, N, K, w, stream) != hipSuccess) return I8G_EHIP;
      QBt = w;
      ldb = ldw;
      wb = true;
    }
  }
  GemmParams p;
  p.A = QA;
  p.B = QBt;
  p.s_row = s_row;
  p.s_col = s_col;
  p.C = C;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = plan.tiles_m;
  p.tiles_n = plan.tiles_n;
  p.splits = plan.splits;
  p.k_per_split = plan.k_per_split;
  p.relu = (flags & I8G_RELU) ? 1 : 0;
  p.do_hash = want_hash ? 1 : 0;
  p.stream_out = ((double)M * (double)N * 4.0 > kStreamOutBytes) ? 1 : 0;
  char* ws = reinterpret_cast<char*>(workspace);
  p.ticket = reinterpret_cast<unsigned int*>(ws);
  p.hash_parts = reinterpret_cast<unsigned long long*>(ws + kWsHeader);
  p.n_shares = plan.hash_parts;
  p.partials = reinterpret_cast<int*>(ws + plan.partials_offset);
  p.comb_rows = plan.comb_rows;
  p.hash_out = hash;
  p.a4 = (a4 && !wa) ? 1 : 0;
  p.b4 = (b4 && !wb) ? 1 : 0;
  return hip_status(launch_gemm(p, plan, stream));
}

}  // namespace i8g

extern "C" {

const char* i8g_status_string(int status) {
  switch (status) {
    case I8G_OK: return "ok";
    case I8G_EINVAL: return "invalid argument (null pointer, negative size or leading dimension too small)";
    case I8G_EKRANGE: return "K exceeds 133144: exact int32 accumulation is not guaranteed";
    case I8G_EALIGN: return "operand not 16-byte aligned, or its leading dimension not a multiple of 16 covering a whole row (K rounded up to 16 bytes; int4: 16 bytes per 32 values)";
    case I8G_EWORKSPACE: return "workspace missing, misaligned or smaller than gemm_i8_workspace_bytes()";
    case I8G_EHIP: return "HIP runtime error while enqueueing a kernel";
    case I8G_EGATE: return "self-check failed: a device output differs from the exact host mirror";
    case I8G_ESCRATCH: return "the shape needs more scratch than the 64 MiB static buffer of gemm_i8_blockscaled_noalloc holds (a split K of a large output): use gemm_i8_blockscaled with a workspace";
    default: return "unknown status";
  }
}

const char* i8g_version(void) { return "int8_gemm 0.1.0 gfx950"; }

// Validates one quantize pass (quantize_rows_fmt when by_col == 0, else
// quantize_cols_fmt); *work is set when there is something to enqueue.  A
// pass over lines of length 0 still writes the floor scale of each line.
static int check_fmt_args(const float* X, int64_t rows, int64_t cols, int64_t ldx, const int8_t* Q,
                          int64_t ldq, const float* scale, bool by_col, uint32_t format, bool* work) {
  *work = false;
  if (format & ~(I8G_FMT_POW2 | I8G_FMT_INT4)) return I8G_EINVAL;
  if (rows < 0 || cols < 0 || rows > INT32_MAX || cols > INT32_MAX) return I8G_EINVAL;
  const bool int4 = (format & I8G_FMT_INT4) != 0;
  const int64_t lines = by_col ? cols : rows, len = by_col ? rows : cols;
  const int64_t line_bytes = int4 ? (len + 31) / 32 * 16 : len;
  if (lines == 0) return I8G_OK;
  if (!scale) return I8G_EINVAL;
  if (len > 0) {
    if (!X || !Q) return I8G_EINVAL;
    if (ldx < cols || ldq < line_bytes) return I8G_EINVAL;
    if (int4 && (((uintptr_t)Q % 16) || (ldq % 16))) return I8G_EALIGN;
  }
  *work = true;
  return I8G_OK;
}

int quantize_rows_fmt(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Q,
                      int64_t ldq, float* scale, uint32_t format, void* stream) {
  bool work = false;
  const int st = check_fmt_args(X, rows, cols, ldx, Q, ldq, scale, false, format, &work);
  if (st != I8G_OK || !work) return st;
  return hip_status(launch_quantize_rows(X, rows, cols, ldx, Q, ldq, scale, (int)format, as_stream(stream)));
}

int quantize_cols_fmt(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Qt,
                      int64_t ldqt, float* scale, uint32_t format, void* stream) {
  bool work = false;
  const int st = check_fmt_args(X, rows, cols, ldx, Qt, ldqt, scale, true, format, &work);
  if (st != I8G_OK || !work) return st;
  return hip_status(launch_quantize_cols(X, rows, cols, ldx, Qt, ldqt, scale, (int)format, as_stream(stream)));
}

int quantize_batch(const i8g_quantize_job* jobs, int32_t n, void* stream) {
  if (n < 0 || (n > 0 && !jobs)) return I8G_EINVAL;
  const hipStream_t st = as_stream(stream);
  // validate everything before enqueueing anything
  std::vector<char> work((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const i8g_quantize_job& j = jobs[i];
    bool w = false;
    const int s = check_fmt_args(j.X, j.rows, j.cols, j.ldx, j.Q, j.ldq, j.scale, j.by_col != 0, j.format, &w);
    if (s != I8G_OK) return s;
    work[i] = w ? 1 : 0;
  }
  std::vector<QJob> batch;
  for (int32_t i = 0; i < n; ++i) {
    if (!work[i]) continue;
    const i8g_quantize_job& j = jobs[i];
    QJob q{};
    if (plan_qjob(j.X, j.rows, j.cols, j.ldx, j.Q, j.ldq, j.scale, j.by_col != 0, (int)j.format, q)) {
      batch.push_back(q);
      continue;
    }
    const hipError_t e = j.by_col
        ? launch_quantize_cols(j.X, j.rows, j.cols, j.ldx, j.Q, j.ldq, j.scale, (int)j.format, st)
        : launch_quantize_rows(j.X, j.rows, j.cols, j.ldx, j.Q, j.ldq, j.scale, (int)j.format, st);
    if (e != hipSuccess) return I8G_EHIP;
  }
  if (batch.empty()) return I8G_OK;
  // workgroups start in id order: the column passes, whose workgroups each
  // hold a whole band and run longest, go first
  std::stable_partition(batch.begin(), batch.end(), [](const QJob& q) { return q.kind == QK_COLS_REG; });
  return hip_status(launch_quantize_batch(batch.data(), (int)batch.size(), st));
}

int quantize_rows(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Q, int64_t ldq,
                  float* scale, void* stream) {
  return quantize_rows_fmt(X, rows, cols, ldx, Q, ldq, scale, 0u, stream);
}

int quantize_cols(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Qt,
                  int64_t ldqt, float* scale, void* stream) {
  return quantize_cols_fmt(X, rows, cols, ldx, Qt, ldqt, scale, 0u, stream);
}

size_t gemm_i8_workspace_bytes_flags(int64_t M, int64_t N, int64_t K, uint32_t flags) {
  if (M <= 0 || N <= 0) return 256;
  // the plan may depend on ldc (very wide rows exclude the persistent
  // kernel): size for either
  const GemmPlan a = plan_gemm(M, N, K > 0 ? K : 1, true);
  const GemmPlan b = plan_gemm(M, N, K > 0 ? K : 1, false);
  size_t bytes = a.workspace_bytes > b.workspace_bytes ? a.workspace_bytes : b.workspace_bytes;
  if (flags & (I8G_A_INT4 | I8G_B_INT4)) {
    const GemmPlan c = plan_gemm_int4(M, N, K > 0 ? K : 1, -1);   // the direct int4 kernel
    const int64_t ldw = int4_widened_ld(K > 0 ? K : 1);
    const size_t widened = (bytes + 255) / 256 * 256 +
                           ((flags & I8G_A_INT4) ? ((size_t)M * ldw + 255) / 256 * 256 : 0) +
                           ((flags & I8G_B_INT4) ? ((size_t)N * ldw + 255) / 256 * 256 : 0);
    bytes = widened > c.workspace_bytes ? widened : c.workspace_bytes;
  }
  return bytes > 256 ? bytes : 256;
}

size_t gemm_i8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return gemm_i8_workspace_bytes_flags(M, N, K, 0u);
}

size_t output_hash_workspace_bytes(void) { return kWsHeader + (size_t)kHashMaxParts * 8; }

size_t gemm_i8_requant_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0) return 256;
  const GemmPlan plan = plan_gemm_requant(M, N, K > 0 ? K : 1, N);
  return requant_layout(plan, M).bytes;
}

int gemm_i8_requant(const int8_t* QA, int64_t lda, const float* s_row, const int8_t* QBt, int64_t ldb,
                    const float* s_col, int64_t M, int64_t N, int64_t K, int8_t* Q, int64_t ldq,
                    float* s_out, uint32_t flags, uint64_t* hash, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const hipStream_t st = as_stream(stream);
  if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX) return I8G_EINVAL;
  if (flags & ~(I8G_RELU | I8G_HASH)) return I8G_EINVAL;
  const bool want_hash = (flags & I8G_HASH) != 0;
  if (want_hash && !hash) return I8G_EINVAL;
  if (K > I8G_K_MAX) return I8G_EKRANGE;
  if (!workspace || ((uintptr_t)workspace % 256) != 0 || workspace_bytes < kWsHeader) return I8G_EWORKSPACE;
  if (M > 0 && !s_out) return I8G_EINVAL;
  if (M == 0 || N == 0) {
    // an M x 0 output: every row scale is the floor, no codes
    if (M > 0) {
      const int q = hip_status(launch_quantize_rows(nullptr, M, 0, 0, Q, ldq, s_out, 0, st));
      if (q) return q;
    }
    if (want_hash) return hip_status(launch_output_hash(nullptr, M, N, N > 0 ? N : 1, hash, workspace, st));
    return I8G_OK;
  }
  if (!Q || ldq < N || !s_row || !s_col) return I8G_EINVAL;
  if (K > 0 && (!QA || !QBt)) return I8G_EINVAL;
  const int64_t k16 = (K + 15) / 16 * 16;
  if (K > 0 && (((uintptr_t)QA % 16) || ((uintptr_t)QBt % 16) || (lda % 16) || (ldb % 16) || lda < k16 ||
                ldb < k16))
    return I8G_EALIGN;
  const GemmPlan plan = plan_gemm_requant(M, N, K > 0 ? K : 1, ldq);
  const RequantLayout lay = requant_layout(plan, M);
  if (workspace_bytes < lay.bytes) return I8G_EWORKSPACE;
  char* ws = reinterpret_cast<char*>(workspace);
  GemmParams p{};
  p.A = QA;
  p.B = QBt;
  p.s_row = s_row;
  p.s_col = s_col;
  p.C = nullptr;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = N;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_m = plan.tiles_m;
  p.tiles_n = plan.tiles_n;
  p.splits = plan.splits;
  p.k_per_split = plan.k_per_split;
  p.relu = (flags & I8G_RELU) ? 1 : 0;
  p.do_hash = want_hash ? 1 : 0;
  p.stream_out = 0;
  p.ticket = reinterpret_cast<unsigned int*>(ws);
  p.hash_parts = reinterpret_cast<unsigned long long*>(ws + kWsHeader);
  p.n_shares = plan.hash_parts;
  p.partials = nullptr;
  p.comb_rows = plan.comb_rows;
  p.hash_out = hash;
  p.rowmax = reinterpret_cast<unsigned int*>(ws + lay.max_offset);
  p.inv_row = plan.persistent ? reinterpret_cast<const float*>(ws + lay.inv_offset) : nullptr;
  p.Q = Q;
  p.ldq = ldq;
  p.s_out = s_out;
  return hip_status(launch_gemm_requant(p, plan, lay, st));
}

int gemm_i8_blockscaled(const int8_t* QA, int64_t lda, const float* s_row, const int8_t* QBt,
                        int64_t ldb, const float* s_col, int64_t M, int64_t N, int64_t K, float* C,
                        int64_t ldc, uint32_t flags, uint64_t* hash, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return enqueue_gemm(QA, lda, s_row, QBt, ldb, s_col, M, N, K, C, ldc, flags, hash, workspace,
                      workspace_bytes, as_stream(stream), -2, 0);
}

int i8g_set_test_overrides(int32_t force_tile, int32_t force_splits, int32_t qcols_path,
                           int32_t int4_direct) {
  if (force_tile < -1 || force_tile >= kNumGemmCfgs || force_splits < 0 || force_splits > 64 ||
      qcols_path < 0 || qcols_path > 4)
    return I8G_EINVAL;
  set_test_overrides(force_tile, force_splits, qcols_path, int4_direct ? 1 : 0);
  return I8G_OK;
}

int i8g_plan_query(int64_t M, int64_t N, int64_t K, int64_t ldc, uint32_t flags, int32_t* config,
                   int32_t* splits) {
  if (M < 1 || N < 1 || K < 0 || M > INT32_MAX || N > INT32_MAX || ldc < N || !config || !splits)
    return I8G_EINVAL;
  if (flags & ~(I8G_RELU | I8G_HASH | I8G_A_INT4 | I8G_B_INT4)) return I8G_EINVAL;
  const bool int4 = (flags & (I8G_A_INT4 | I8G_B_INT4)) != 0;
  const GemmPlan plan = (int4 && int4_direct_requested())
                            ? plan_gemm_int4(M, N, K > 0 ? K : 1, -1)
                            : plan_gemm(M, N, K > 0 ? K : 1, ldc <= kPersistMaxLdc);
  *config = plan.cfg;
  *splits = plan.splits;
  return I8G_OK;
}

int gemm_i8_blockscaled_noalloc(const int8_t* QA, int64_t lda, const float* s_row, const int8_t* QBt,
                                int64_t ldb, const float* s_col, int64_t M, int64_t N, int64_t K,
                                float* C, int64_t ldc, uint32_t flags, uint64_t* hash, void* stream) {
  const hipStream_t st = as_stream(stream);
  // the same checks as gemm_i8_blockscaled, run on a stand-in workspace
  // first, so that an invalid call or a shape whose plan needs more than the
  // array holds returns before anything (even the header zeroing) is enqueued
  const int pre = enqueue_gemm(QA, lda, s_row, QBt, ldb, s_col, M, N, K, C, ldc, flags, hash,
                               nullptr, kNoallocScratchBytes, st, -4, 0);
  if (pre == I8G_EWORKSPACE) return I8G_ESCRATCH;
  if (pre != I8G_OK) return pre;
  void* ws = nullptr;
  const int s = scratch_for_device(st, &ws);
  if (s != I8G_OK) return s;
  return enqueue_gemm(QA, lda, s_row, QBt, ldb, s_col, M, N, K, C, ldc, flags, hash, ws,
                      kNoallocScratchBytes, st, -2, 0);
}

int output_hash(const float* C, int64_t M, int64_t N, int64_t ldc, uint64_t* hash, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0 || M > INT32_MAX || N > INT32_MAX || !hash) return I8G_EINVAL;
  if (M > 0 && N > 0 && (!C || ldc < N)) return I8G_EINVAL;
  if (!workspace || ((uintptr_t)workspace % 256) != 0 ||
      workspace_bytes < output_hash_workspace_bytes())
    return I8G_EWORKSPACE;
  return hip_status(launch_output_hash(C, M, N, ldc, hash, workspace, as_stream(stream)));
}

}  // extern "C"
