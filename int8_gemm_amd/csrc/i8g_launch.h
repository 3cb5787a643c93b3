// i8g_launch.h -- host-side interface between the C ABI (api.hip) and the
// kernels (quantize.hip, gemm.hip, hash.hip).  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace i8g {

struct GemmParams {
  const int8_t* A;          // QA, M x K, K contiguous
  const int8_t* B;          // QBt, N x K, K contiguous
  const float* s_row;
  const float* s_col;
  float* C;
  int64_t lda, ldb, ldc;
  int M, N, K;
  int tiles_m, tiles_n, splits, k_per_split;
  int relu, do_hash;
  int stream_out;                   // store C with nontemporal hints (large outputs)
  unsigned long long* hash_parts;   // per-tile (or per-combine-group) shares of S
  unsigned int* ticket;             // workspace word counting finished shares (zero between calls)
  int n_shares;                     // shares of S written by the kernel that ends the call
  int* partials;                    // split-K int32 partial sums, [split][M][N]
  int comb_rows;                    // rows per split-K combine workgroup
  uint64_t* hash_out;
  int a4, b4;                       // operand stored as int4, two per byte (gemm_i4_kernel only)
  // requantizing epilogue (gemm_i8_requant): pass 1 only reduces |y| to row
  // maxima (bit patterns); pass 2 writes the int8 codes of y with the row
  // scales those maxima give
  unsigned int* rowmax;             // non-persistent: M words, zero before pass 1;
                                    // persistent: [tiles_n * 2][M] partial maxima
  const float* inv_row;             // persistent pass 2: RN(1/s) of every output row scale s
  int8_t* Q;                        // pass 2: codes, row-major, leading dimension ldq
  int64_t ldq;
  float* s_out;                     // pass 2: the M row scales of the codes
};

struct GemmPlan {
  int cfg;                  // index of the tile configuration
  int bm, bn;
  int tiles_m, tiles_n;
  int splits;
  int k_per_split;          // bytes of K per split (multiple of 64)
  int comb_x, comb_y;       // split-K combine grid
  int comb_rows;            // rows per combine workgroup
  int hash_parts;           // number of shares of S written before the finalize
  size_t partials_offset;   // hash shares at offset 0, split partials here
  size_t workspace_bytes;
  int grid;                 // workgroups of the GEMM kernel
  bool persistent;          // gemm_i8_persist_kernel (one workgroup per CU)
};

// Largest ldc (floats) the persistent kernel addresses with 32-bit buffer
// offsets; larger leading dimensions are planned without it.
constexpr int64_t kPersistMaxLdc = int64_t(1) << 23;

// Outputs larger than this (half of the 256 MB last-level cache) are stored
// with nontemporal hints (GemmParams::stream_out); smaller ones stay in the
// cache for the kernel that reads them next.
constexpr double kStreamOutBytes = 128.0 * 1024 * 1024;

// Number of tile configurations of the planner (indices 0 .. kNumGemmCfgs-1;
// kNumGemmCfgs itself denotes the direct int4 kernel).
constexpr int kNumGemmCfgs = 8;

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool allow_persistent);
// The same with the tile configuration and split count forced (-1 / 0: the
// cost model's choice); a configuration that cannot run the shape falls back
// to the 128x128 tile (i8g_plan_query shows which plan a shape gets).
// plan_gemm takes them from the test overrides (set_test_overrides).
GemmPlan plan_gemm_forced(int64_t M, int64_t N, int64_t K, bool allow_persistent, int force_tile,
                          int force_splits);
// Validates, plans and enqueues one GEMM exactly as gemm_i8_blockscaled does
// (force_tile / force_splits as in plan_gemm_forced; force_tile == -2 is the
// library's own choice, -3 the direct int4 kernel for int4 operands, -4 the
// library's choice validated and planned only: every status check, including
// the workspace size, but nothing enqueued and the workspace pointer unused).
int enqueue_gemm(const int8_t* QA, int64_t lda, const float* s_row, const int8_t* QBt, int64_t ldb,
                 const float* s_col, int64_t M, int64_t N, int64_t K, float* C, int64_t ldc,
                 uint32_t flags, uint64_t* hash, void* workspace, size_t workspace_bytes,
                 hipStream_t stream, int force_tile, int force_splits);
// Plan for int4 operands: the register-staged kernel, 128x128 tiles, split
// K as the cost model of that tile chooses (force_splits as above; < 0 takes
// the test override).
GemmPlan plan_gemm_int4(int64_t M, int64_t N, int64_t K, int force_splits);
hipError_t launch_gemm(const GemmParams& p, const GemmPlan& plan, hipStream_t stream);
// int4 operands are by default widened to int8 codes in the workspace (rows
// of int4_widened_ld(K) bytes) and multiplied by the int8 kernels;
// the int4_direct test override selects gemm_i4_kernel, which reads the
// packed bytes itself.
int64_t int4_widened_ld(int64_t K);
hipError_t launch_widen_int4(const int8_t* P, int64_t ldp, int64_t rows, int64_t K, int8_t* Q,
                             hipStream_t stream);
bool int4_direct_requested();
// Test overrides (i8g_set_test_overrides): forced tile configuration (-1:
// none) and split count (0: none), column quantize path (0: the planner's,
// 1: the two-pass kernels, 2: the cooperative one-read kernel, 3: the two
// whole-line passes, where the shape allows them), int4 operands through
// gemm_i4_kernel.  Process-wide.
void set_test_overrides(int force_tile, int force_splits, int qcols_path, int int4_direct);
int qcols_path_requested();
// The requantizing epilogue's plan: one K split; a persistent tile where the
// shape allows it (K % 128 == 0, K >= 768, M % 128 == 0, ldq <= 2^24: the
// 128x128 tile with two workgroups per CU for K <= 1024, else 128x192), else
// a non-persistent tile (a forced tile 0..2, 6 or 7 is honoured for tests).
// Its workspace after the GEMM's own: the row maxima (non-persistent: M
// words; persistent: `partials` x M words, then the M reciprocals at
// inv_offset).
GemmPlan plan_gemm_requant(int64_t M, int64_t N, int64_t K, int64_t ldq);
struct RequantLayout {
  size_t max_offset, inv_offset, bytes;
  int partials;
};
RequantLayout requant_layout(const GemmPlan& plan, int64_t M);
hipError_t launch_gemm_requant(GemmParams p, const GemmPlan& plan, const RequantLayout& l, hipStream_t stream);

// fmt: FMT_POW2 / FMT_INT4 bits (i8g_device.h); int4 outputs take
// 16*ceil(len/32) bytes per line, 16-byte aligned.
hipError_t launch_quantize_rows(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                                int8_t* Q, int64_t ldq, float* scale, int fmt, hipStream_t stream);
hipError_t launch_quantize_cols(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                                int8_t* Qt, int64_t ldqt, float* scale, int fmt, hipStream_t stream);
// One quantize pass of quantize_batch (planned by plan_qjob): a row pass
// with a wave per row, a row pass with a workgroup per row, a column pass
// with a workgroup per band of columns, or a pass over aligned rows of
// 1025-3072 values with a wave per row (the vector body only).
enum QKind : int { QK_ROWS_WAVE = 0, QK_ROWS_BLOCK = 1, QK_COLS_REG = 2, QK_ROWS_VEC = 3 };
struct QJob {
  const float* X;
  int8_t* Q;
  float* scale;
  int64_t rows, cols, ldx, ldq;
  int kind, param, fmt, vec_in, vec_out;
  int blocks;   // workgroups of 1024 threads the pass takes
  int first;    // first workgroup id of its range in the launch
};
constexpr int kQBatchMax = 24;   // jobs per launch (kernel argument space)
struct QBatch {
  QJob job[kQBatchMax];
  int n;
};
// Fills q for a pass the batch kernel can run (false: int4 row passes,
// empty shapes, and tall column passes that need several kernels).
bool plan_qjob(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Q, int64_t ldq,
               float* scale, bool by_col, int fmt, QJob& q);
hipError_t launch_quantize_batch(QJob* jobs, int n, hipStream_t stream);
hipError_t launch_output_hash(const float* C, int64_t M, int64_t N, int64_t ldc,
                              uint64_t* hash, void* workspace, hipStream_t stream);
// H from n shares of S that an earlier launch on `stream` stored at parts
// (a one-workgroup kernel).
hipError_t launch_hash_parts_finalize(const unsigned long long* parts, int n, int64_t M, int64_t N,
                                      uint64_t* hash_out, hipStream_t stream);

// Workspace layout shared by every call: a 256-byte header (word 0 is the
// share ticket, zero between calls), then 8-byte hash shares, then (GEMM
// split-K only) int32 partial sums.
constexpr size_t kWsHeader = 256;
// output_hash uses at most this many shares
constexpr int kHashMaxParts = 2048;

}  // namespace i8g
