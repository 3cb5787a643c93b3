/*
 * int8_gemm.h -- bit-reproducible block-scaled int8 GEMM for AMD Instinct
 * MI355X (gfx950).  C ABI of libint8_gemm.so.
 *
 * The method is the one of the DaisyChain-Train page "Verification -- why
 * you can trust the numbers", section "The verified INT8 units":
 *   1. A (M x K) is quantized per row and B (K x N) per column with
 *      scale = max(|line|)/127 floored at 1e-8, values to int8;
 *   2. int8 products are accumulated exactly in int32;
 *   3. the f32 epilogue rounds after the int->float conversion and after
 *      each multiply: out = f32(f32(f32(acc) * s_row[i]) * s_col[j]).
 * Every device that follows these steps, and a plain CPU, produce the same
 * output bytes, so outputs can be compared by hashing them (the page's
 * opening paragraph and "Layer 3: the kernel probe").
 *
 * Rounding is binary32 round-to-nearest-even throughout.  The readings this
 * library takes where the page leaves a step open:
 *   s   = max(RN(a / 127), RN(1e-8))      a = max |x| over the line,
 *                                         RN(1e-8) = 0x322BCC77, division
 *                                         correctly rounded
 *   inv = RN(1 / s)                       correctly rounded
 *   q   = floor(RN(RN(x * inv) + 0.5))    two roundings, never fused;
 *                                         q is in [-127, 127]
 *   out = RN(RN(RN(acc) * s_row[i]) * s_col[j]), row scale first;
 *   ReLU (optional, fused): out = out > 0 ? out : +0.0.
 *
 * Conventions for every entry point
 *   - All array pointers are DEVICE pointers (memory from hipMalloc or a
 *     PyTorch tensor on the current device), owned by the caller; the
 *     library keeps no reference to them after the call is enqueued.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream) and runs asynchronously; nothing is synchronized.
 *   - Sizes are int64_t element counts; leading dimensions (ld*) are in
 *     elements of the array they describe, row-major.
 *   - The return value is a status code (I8G_OK = 0).  On a non-zero
 *     status nothing has been enqueued, except for I8G_EHIP, which reports
 *     a launch failure from the HIP runtime.  Nothing is printed and no
 *     C++ exception crosses the ABI.
 *   - Inputs must be finite (no NaN or infinity); other inputs give
 *     unspecified bytes.
 *   - Empty shapes (a zero dimension) are valid and enqueue nothing except
 *     the hash of an empty output where one is requested.
 *   - The library allocates no device memory at run time.  Calls that
 *     share a workspace must be ordered (same stream, or synchronized).
 *     gemm_i8_blockscaled_noalloc uses a static device buffer instead of a
 *     workspace (see there).
 *   - No kernel waits on another workgroup and no call synchronizes with
 *     the host: grid-wide sums end in the workgroup that finishes last.
 */
#ifndef INT8_GEMM_H
#define INT8_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define I8G_OK          0  /* success                                        */
#define I8G_EINVAL      1  /* null pointer, negative size, ld < row length   */
#define I8G_EKRANGE     2  /* K > 133144: int32 accumulation could overflow  */
#define I8G_EALIGN      3  /* a GEMM operand's pointer or ld not 16-byte     */
                           /* aligned, or ld below K rounded up to 16        */
#define I8G_EWORKSPACE  4  /* workspace missing, misaligned or too small     */
#define I8G_EHIP        5  /* the HIP runtime reported a launch error        */
#define I8G_EGATE       6  /* i8g_gate: a device output differs from the     */
                           /* exact host mirror (see i8g_gate_report)        */
#define I8G_ESCRATCH    7  /* gemm_i8_blockscaled_noalloc: the shape needs   */
                           /* more scratch than its static buffer holds      */

/* flags of gemm_i8_blockscaled */
#define I8G_RELU 1u        /* fused ReLU: out = out > 0 ? out : +0          */
#define I8G_HASH 2u        /* also write the output hash to *hash            */
#define I8G_A_INT4 4u      /* QA holds int4 values, two per byte (see below) */
#define I8G_B_INT4 8u      /* QBt holds int4 values, two per byte            */

/* Storage formats of quantize_rows_fmt / quantize_cols_fmt (the presk page,
 * section "Integer weights": int8 or int4 values, absmax or power-of-two
 * scales). */
#define I8G_FMT_POW2 1u    /* scale rounded up to a power of two: q*s exact  */
#define I8G_FMT_INT4 2u    /* qmax 7 instead of 127, two values per byte     */

/* Largest K for which |acc| <= 127*127*K stays below 2^31. */
#define I8G_K_MAX 133144

/*
 * quantize_rows -- per-row quantization (step 1 of "The verified INT8
 * units", applied to the rows of an operand).
 *   X      rows x cols f32, row-major, leading dimension ldx >= cols.
 *   Q      rows x cols int8 output, leading dimension ldq >= cols; bytes in
 *          columns [cols, ldq) are not written.
 *   scale  rows f32 output: scale[i] = max(RN(max_k |X[i,k]|/127), RN(1e-8)).
 * Q[i,k] = floor(RN(RN(X[i,k] * RN(1/scale[i])) + 0.5)).
 * With cols == 0 only the scales are written (each is RN(1e-8)).
 * Any alignment of X and Q is accepted (16-byte aligned rows are faster).
 * Errors: I8G_EINVAL (null pointer with rows*cols > 0, null scale with
 * rows > 0, negative size, ldx < cols, ldq < cols), I8G_EHIP.
 */
int quantize_rows(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                  int8_t* Q, int64_t ldq, float* scale, void* stream);

/*
 * quantize_cols -- per-column quantization with a transposed int8 output,
 * so that both GEMM operands are contiguous along K.
 *   X      rows x cols f32, row-major, leading dimension ldx >= cols.
 *   Qt     cols x rows int8 output (the transpose), leading dimension
 *          ldqt >= rows; bytes in columns [rows, ldqt) are not written.
 *   scale  cols f32 output: scale[j] = max(RN(max_k |X[k,j]|/127), RN(1e-8)).
 *          It is also used as scratch while the call runs.
 * Qt[j,k] = floor(RN(RN(X[k,j] * RN(1/scale[j])) + 0.5)).
 * With rows == 0 only the scales are written (each is RN(1e-8)).
 * Large inputs (at least 256 MiB of X, rows a multiple of 256 and at least
 * 1024, cols a multiple of 32, X and Qt 16-byte aligned, ldx a multiple of 4
 * and ldqt of 16) are quantized by a cooperative launch that reads X once:
 * the workgroups sharing a band of columns exchange partial maxima through
 * `scale` and a counter kept in the first four bytes of the band's first Qt
 * row (written with the codes last), waiting for each other with a bounded
 * wait.  The runtime keeps a cooperative grid resident (or the launch fails
 * and the call takes the other path), so the wait ends; if it ever timed
 * out, the band's scales are left NaN, which no valid call produces.
 * Errors: as quantize_rows (with the roles of rows and cols exchanged).
 */
int quantize_cols(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                  int8_t* Qt, int64_t ldqt, float* scale, void* stream);

/*
 * quantize_rows_fmt / quantize_cols_fmt -- quantize_rows / quantize_cols in
 * one of the storage formats of the presk page, section "Integer weights"
 * (b-bit values with qmax = 2^(b-1) - 1; scales absmax or rounded up to a
 * power of two, "at most twice as coarse" so that q*s is exact; int4 values
 * two to a byte).  format = 0 is exactly quantize_rows / quantize_cols.
 *   scale  s = max(RN(a/qmax), RN(1e-8)) with qmax = 127, or 7 with
 *          I8G_FMT_INT4; with I8G_FMT_POW2, s is then replaced by the
 *          smallest power of two >= s (so the floor becomes 2^-26).
 *   values q = floor(RN(RN(x * RN(1/s)) + 0.5)), |q| <= qmax.
 *   int4 layout (I8G_FMT_INT4): a line of L values (a row of Q, a row of
 *          Qt) takes 16*ceil(L/32) bytes; value k sits in byte
 *          16*(k/32) + k%16, in the low nibble when k%32 < 16 and in the
 *          high nibble otherwise, as a 4-bit two's complement number;
 *          nibbles past L are written 0.  Q (Qt) must be 16-byte aligned and
 *          ldq (ldqt) a multiple of 16 of at least 16*ceil(L/32) bytes.
 * Errors: as quantize_rows / quantize_cols, plus I8G_EINVAL for unknown
 * format bits and I8G_EALIGN for a misaligned int4 output.
 */
int quantize_rows_fmt(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                      int8_t* Q, int64_t ldq, float* scale, uint32_t format, void* stream);
int quantize_cols_fmt(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                      int8_t* Qt, int64_t ldqt, float* scale, uint32_t format, void* stream);

/*
 * quantize_batch -- n independent quantize passes enqueued together: the
 * passes that fit one kernel run in a single launch (24 at most per launch)
 * and share the chip, which matters for the many small passes of a step
 * (weights, skinny activations) whose time is mostly latency; the others
 * (int4 row passes, rows of more than 3072 values, rows of more than 1024
 * values that are not 16-byte aligned with a length that is a multiple of 4,
 * column passes over more than 8192 rows or of at least 256 MiB) are
 * enqueued one by one on the same stream.  Every output is byte for byte
 * that of the single call.
 *   jobs  host array of n descriptions; by_col = 0 is quantize_rows_fmt,
 *         by_col = 1 quantize_cols_fmt, with the same arguments and rules.
 *         No job may write memory another job reads or writes.
 * Errors: the first failing job's status from validating all of them;
 * nothing is enqueued unless every job is valid.  I8G_EINVAL for n < 0 or a
 * null array with n > 0; I8G_EHIP.
 */
typedef struct i8g_quantize_job {
  const float* X;
  int64_t rows, cols, ldx;
  int8_t* Q;
  int64_t ldq;
  float* scale;
  uint32_t by_col;
  uint32_t format;
} i8g_quantize_job;

int quantize_batch(const i8g_quantize_job* jobs, int32_t n, void* stream);

/*
 * gemm_i8_blockscaled -- C = epilogue(QA . QBt^T) (steps 2 and 3 of "The
 * verified INT8 units").
 *   QA     M x K int8, row-major (K contiguous), leading dimension lda.
 *   s_row  M f32 row scales of A.
 *   QBt    N x K int8, row-major (K contiguous): B's quantized columns as
 *          rows, leading dimension ldb.
 *   s_col  N f32 column scales of B.
 *   C      M x N f32 output, row-major, leading dimension ldc >= N.
 *   flags  I8G_RELU and/or I8G_HASH; I8G_A_INT4 / I8G_B_INT4 when QA / QBt
 *          hold int4 values in the layout of quantize_rows_fmt (then that
 *          operand's ld need only cover 16*ceil(K/32) bytes; the
 *          workspace must then be gemm_i8_workspace_bytes_flags(M, N, K,
 *          flags) bytes).  Scales of either scheme are taken as they are.
 *   hash   device pointer to one uint64_t, required with I8G_HASH (else
 *          ignored): receives output_hash(C) for this output.
 *   workspace, workspace_bytes
 *          device scratch of at least gemm_i8_workspace_bytes(M, N, K)
 *          bytes, 256-byte aligned.  Its first 256 bytes (a control
 *          header: the hash's share counter) must be zero before the first
 *          call that uses it; every call leaves them zero again, so one
 *          zeroed buffer serves any sequence of ordered calls.  The rest is
 *          scratch with any contents (per-tile shares of the hash, and with
 *          a split K the int32 partial sums).
 * acc[i,j] = sum_k QA[i,k]*QBt[j,k] is exact (int32); the K range may be
 * split across workgroups, which cannot change a byte since integer
 * addition is associative.
 * out[i,j] = RN(RN(RN(acc[i,j]) * s_row[i]) * s_col[j]) (then ReLU).
 * Requirements: QA and QBt 16-byte aligned, lda and ldb multiples of 16 and
 * >= K rounded up to 16 (bytes k >= K of each row are read but ignored);
 * every QA row is readable for lda bytes and every QBt row for ldb bytes.
 * Errors: I8G_EINVAL, I8G_EKRANGE (K > I8G_K_MAX), I8G_EALIGN,
 * I8G_EWORKSPACE, I8G_EHIP.
 */
int gemm_i8_blockscaled(const int8_t* QA, int64_t lda, const float* s_row,
                        const int8_t* QBt, int64_t ldb, const float* s_col,
                        int64_t M, int64_t N, int64_t K,
                        float* C, int64_t ldc, uint32_t flags, uint64_t* hash,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * gemm_i8_blockscaled_noalloc -- gemm_i8_blockscaled without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *   Arguments, outputs, layouts and rules as gemm_i8_blockscaled.
 *   Scratch: the call's workspace is a static device array of the library
 *   (I8G_NOALLOC_SCRATCH_BYTES = 64 MiB, one per GPU the library runs on,
 *   held until the process ends).  Its address is looked up, and its
 *   control header zeroed by a small kernel on `stream`, at the first call
 *   on each device; every call leaves the header zero again.  Nothing is
 *   allocated by any call (no hipMalloc, no allocating library routine).
 *   A shape whose plan needs more scratch than the array holds (gemm_i8_
 *   workspace_bytes_flags of the plan taken: int32 partial sums of a split
 *   K, int4 operands widened to int8) returns I8G_ESCRATCH before anything
 *   is enqueued; without a split K every GPT-2-small shape fits.
 *   Calls on one GPU share its array: calls that overlap in time on one GPU
 *   (different streams not ordered by the caller, or different threads)
 *   race and give unspecified bytes; calls ordered on one stream are safe.
 * Errors: as gemm_i8_blockscaled, plus I8G_ESCRATCH; I8G_EHIP also when the
 * array's device address cannot be obtained.
 */
#define I8G_NOALLOC_SCRATCH_BYTES 67108864u   /* 64 MiB */
int gemm_i8_blockscaled_noalloc(const int8_t* QA, int64_t lda, const float* s_row,
                                const int8_t* QBt, int64_t ldb, const float* s_col,
                                int64_t M, int64_t N, int64_t K,
                                float* C, int64_t ldc, uint32_t flags, uint64_t* hash,
                                void* stream);

/* Bytes of workspace gemm_i8_blockscaled needs for this shape (>= 256),
 * for int8 operands. */
size_t gemm_i8_workspace_bytes(int64_t M, int64_t N, int64_t K);
/* The same for the given flags: with I8G_A_INT4 / I8G_B_INT4 the workspace
 * also holds the int4 operands widened to int8 (the int8 kernels then run
 * the product), 32*ceil(K/32) bytes per row of each such operand. */
size_t gemm_i8_workspace_bytes_flags(int64_t M, int64_t N, int64_t K, uint32_t flags);

/*
 * gemm_i8_requant -- the requantizing epilogue: the GEMM's output leaves as
 * int8 codes and per-row scales, ready to be the A operand of the next GEMM
 * (the presk page, section "What is left open": activations quantized with
 * int32 accumulation and requantization; the DaisyChain-Train page, section
 * "Layer 1: exact init gates", gates such a back-to-back chain).
 *   QA, lda, s_row, QBt, ldb, s_col, M, N, K   as gemm_i8_blockscaled.
 *   Q      M x N int8 output, row-major, leading dimension ldq >= N.
 *   s_out  M f32 output scales.
 *   flags  I8G_RELU and/or I8G_HASH (hash = output_hash of the f32 output
 *          y, which is never stored).
 *   workspace  at least gemm_i8_requant_workspace_bytes(M, N, K) bytes,
 *          256-byte aligned, first 256 bytes zero as for gemm_i8_blockscaled.
 * Q and s_out equal quantize_rows(y) byte for byte, y being the output
 * gemm_i8_blockscaled would write.  The row scale needs the row's maximum
 * over every column tile, so the call runs the contraction twice: a first
 * pass raises one integer maximum per row (atomicMax on the bit patterns of
 * |y|), the second quantizes with the final scales.  It saves the f32
 * output's memory and bytes, not MACs.
 * Errors: as gemm_i8_blockscaled (I8G_EINVAL also for a null Q or s_out or
 * ldq < N).
 */
int gemm_i8_requant(const int8_t* QA, int64_t lda, const float* s_row,
                    const int8_t* QBt, int64_t ldb, const float* s_col,
                    int64_t M, int64_t N, int64_t K, int8_t* Q, int64_t ldq,
                    float* s_out, uint32_t flags, uint64_t* hash,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace gemm_i8_requant needs for this shape (>= 256). */
size_t gemm_i8_requant_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Bytes of workspace output_hash needs (a constant, 256 + 16 KiB). */
size_t output_hash_workspace_bytes(void);

/*
 * output_hash -- the probe hash of an M x N f32 matrix (the page's "Layer
 * 3: the kernel probe"; the page names no function, this library defines):
 *   bits(i,j) = 32-bit pattern of C[i,j]           (-0 and +0 differ)
 *   r(i)      = 2*mix31(i mod 2^31) + 1            (mix31: a bijection of
 *               [0,2^31): x ^= x>>16; x *= 0x3B9C5A1D; x ^= x>>13;
 *               x *= 0x2F6E8B35; x ^= x>>16, products mod 2^31)
 *   c(j)      = fmix64(j + 0x9E3779B97F4A7C15) | 1  (MurmurHash3 finalizer)
 *   S         = sum_{i,j} c(j) * r(i) * bits(i,j)   mod 2^64
 *   H         = fmix64(S ^ fmix64(M * 2^32 + N))
 *   C      M x N f32, leading dimension ldc >= N; M, N < 2^31.
 *   hash   device pointer to one uint64_t that receives H.
 *   workspace  device scratch of output_hash_workspace_bytes() bytes,
 *          256-byte aligned, with the same 256-byte zero header as the
 *          GEMM's workspace (one zeroed buffer may serve both calls).
 * The sum is taken modulo 2^64, so it is reduced in any order: each
 * workgroup writes its share, and the last one to finish adds them up.
 * Errors: I8G_EINVAL, I8G_EWORKSPACE, I8G_EHIP.
 */
int output_hash(const float* C, int64_t M, int64_t N, int64_t ldc,
                uint64_t* hash, void* workspace, size_t workspace_bytes,
                void* stream);

/* ------------------------------------------------------------------------
 * Self-checks, after the defence layers of the page "Verification -- why
 * you can trust the numbers" ("Layer 1: exact init gates", "Layer 2:
 * continuous audit", "Layer 3: the kernel probe").  Where that page falls
 * back to a CPU mirror on a failed gate, this library refuses (I8G_EGATE):
 * no entry point ever computes its outputs on the CPU.
 * ------------------------------------------------------------------------ */

/* Result of i8g_gate (host memory, filled by the call). */
typedef struct i8g_gate_report {
  int32_t check;     /* 0 = passed; 1 quantize_rows, 2 quantize_cols,
                        3 GEMM output, 4 output hash (fused or standalone),
                        5 the gate's inputs separate no wrong specification
                        (index = which one: 0 round-half-even quantize,
                        1 fused multiply-add quantize, 2 column scale first,
                        3 scales multiplied first, 4 ReLU's +0),
                        6 GEMM output with int4 operands,
                        7 gemm_i8_requant codes or scales                  */
  int32_t config;    /* GEMM tile configuration that failed (for checks 1
                        and 2 the storage format), or -1                    */
  int64_t m, n, k;   /* shape of the failing case (rows, cols for quantize) */
  int64_t index;     /* first differing element (row-major), line, or -1   */
  uint32_t got, want;/* bit patterns at that element (low 32 bits of a hash) */
  int32_t cases;     /* number of cases that passed                         */
} i8g_gate_report;

/* Bytes of workspace i8g_gate needs (a constant, 16 MiB). */
size_t i8g_gate_workspace_bytes(void);

/*
 * i8g_gate -- init gate: runs quantize_rows and quantize_cols (row and
 * column passes, a long row, a tall column pass, the pow2 and int4 formats,
 * quantize_batch), the GEMM in every tile configuration of the planner
 * (ReLU on and off, a split K), the GEMM with int4 operands,
 * gemm_i8_requant, and the fused and standalone output hash on ragged
 * shapes, and compares every output bit with an exact host mirror of the
 * method built into the library.  The
 * inputs hold exact ties x*inv = k + 0.5 and products just below 0.5 (where
 * round-half-even and a fused multiply-add quantize differ from the method),
 * and the gate checks that its GEMM outputs also separate the method from a
 * column-scale-first or combined-scale epilogue and ReLU's +0 from -0; a
 * pass therefore means the device follows the method where wrong
 * specifications differ.  Floating-point behaviour is runtime state on a
 * GPU, so run it at every start.
 *   workspace  device scratch of i8g_gate_workspace_bytes(), 256-byte
 *              aligned, any contents.
 *   report     host pointer (may be NULL): which check failed and where.
 * Unlike the other calls it copies data between host and device and
 * synchronizes `stream`; it takes ~0.1-0.3 s of host time.
 * Returns I8G_OK, I8G_EGATE (mismatch), I8G_EWORKSPACE or I8G_EHIP.
 */
int i8g_gate(void* workspace, size_t workspace_bytes, void* stream, i8g_gate_report* report);

/*
 * i8g_audit_gemm -- live audit of one GEMM output: `samples` cells (i, j),
 * drawn from SplitMix64(seed), are recomputed on the device with a scalar
 * dot product (not the MFMA path) and the epilogue, and compared bit for bit
 * with C.  Arguments as gemm_i8_blockscaled (I8G_HASH in flags is ignored;
 * I8G_A_INT4 / I8G_B_INT4 read int4 operands in their packed layout).
 *   result  device pointer to two uint64_t: result[0] = number of sampled
 *           cells that differ, result[1] = smallest i*N + j among them
 *           (UINT64_MAX if none).  Written by the call's own kernels.
 * Errors: I8G_EINVAL, I8G_EALIGN, I8G_EHIP.
 */
int i8g_audit_gemm(const int8_t* QA, int64_t lda, const float* s_row, const int8_t* QBt,
                   int64_t ldb, const float* s_col, int64_t M, int64_t N, int64_t K,
                   const float* C, int64_t ldc, uint32_t flags, uint64_t seed,
                   int32_t samples, uint64_t* result, void* stream);

/*
 * i8g_audit_quantize -- live audit of a quantize pass: `samples` lines
 * (rows of X for by_col == 0, checked against quantize_rows' Q and scale;
 * columns for by_col == 1, against quantize_cols' Qt and scale), drawn from
 * SplitMix64(seed), have their scale and every code recomputed.
 *   result  as i8g_audit_gemm, with result[1] = smallest differing line.
 * Errors: I8G_EINVAL, I8G_EHIP.
 */
int i8g_audit_quantize(const float* X, int64_t rows, int64_t cols, int64_t ldx, const int8_t* Q,
                       int64_t ldq, const float* scale, int32_t by_col, uint64_t seed,
                       int32_t samples, uint64_t* result, void* stream);
/* The same for an output of quantize_rows_fmt / quantize_cols_fmt in
 * `format` (int4 lines: every value and the zero nibbles after the last one
 * in its 16-byte group are checked). */
int i8g_audit_quantize_fmt(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                           const int8_t* Q, int64_t ldq, const float* scale, int32_t by_col,
                           uint32_t format, uint64_t seed, int32_t samples, uint64_t* result,
                           void* stream);

/* Bytes of workspace i8g_probe_hash needs for this shape. */
size_t i8g_probe_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * i8g_probe_hash -- the kernel probe: a seeded GEMM through the live kernels.
 * A (M x K) and B (K x N), both row-major, take the outputs of SplitMix64
 * seeded with `seed` in order, A first: output z becomes the binary32 value
 * ((z >> 40) - 2^23) / 2^21, in [-4, 4).  SplitMix64 (Steele, Lea and Flood,
 * 2014): output k is mix(seed + (k+1) * 0x9E3779B97F4A7C15) with
 * mix(z) = z ^= z >> 30, z *= 0xBF58476D1CE4E5B9, z ^= z >> 27,
 * z *= 0x94D049BB133111EB, z ^= z >> 31.  Then quantize_rows(A),
 * quantize_cols(B) and gemm_i8_blockscaled (no ReLU) with its hash, which is
 * written to *hash: every device that follows the method writes the same
 * value.  M, N <= 2^20, K <= I8G_K_MAX.
 *   workspace  device scratch of i8g_probe_workspace_bytes(M, N, K),
 *              256-byte aligned, any contents.
 * Errors: I8G_EINVAL, I8G_EWORKSPACE, I8G_EHIP.
 */
int i8g_probe_hash(uint64_t seed, int64_t M, int64_t N, int64_t K, uint64_t* hash,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Test hooks.  The bytes a call writes never depend on the kernel plan (the
 * contraction is exact in any blocking and K split); these two calls let a
 * test run every kernel path on shapes the planner would not give it and
 * check which plan ran.  Not for production use.
 * ------------------------------------------------------------------------ */

/*
 * i8g_set_test_overrides -- process-wide plan overrides for the calls that
 * follow (all devices, all threads; a call racing with it sees either
 * setting).  force_tile: -1 = the planner's choice, else a tile
 * configuration index 0..7 (a configuration that cannot run a shape falls
 * back to the 128x128 tile, index 2); force_splits: 0 = the planner's
 * choice, else the number of K splits (clamped so that no split is empty;
 * the persistent configurations never split); qcols_path: 0 = the
 * planner's column quantize path, 1 = the two-pass kernels, 2 = the
 * cooperative one-read kernel wherever the shape allows it (see
 * quantize_cols), 3 = the two whole-line passes wherever the shape allows
 * them (the cooperative path's shapes), 4 = the cooperative kernel with
 * every wait cut to one spin (its timeout paths: a band whose exchange
 * does not complete at once is left with NaN scales); int4_direct: 1 = int4 GEMM operands read packed by the
 * direct int4 kernel.  All zero / -1 restores the default.  Errors:
 * I8G_EINVAL for out-of-range values.
 */
int i8g_set_test_overrides(int32_t force_tile, int32_t force_splits, int32_t qcols_path,
                           int32_t int4_direct);

/*
 * i8g_plan_query -- the plan gemm_i8_blockscaled would use for this shape on
 * the current device under the current overrides: *config = tile
 * configuration index (8 = the direct int4 kernel), *splits = K splits.
 * Host only; enqueues nothing.  Errors: I8G_EINVAL (M or N < 1, K < 0,
 * ldc < N, null outputs, unknown flags).
 */
int i8g_plan_query(int64_t M, int64_t N, int64_t K, int64_t ldc, uint32_t flags, int32_t* config,
                   int32_t* splits);

/* Static English text for a status code (never NULL). */
const char* i8g_status_string(int status);

/* Library version, e.g. "int8_gemm 0.1.0 gfx950". */
const char* i8g_version(void);

#ifdef __cplusplus
}
#endif
#endif /* INT8_GEMM_H */
