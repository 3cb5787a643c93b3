// quantize.hip -- per-row and per-column absmax quantization to int8.
//
// Step 1 of the DaisyChain-Train page "Verification -- why you can trust
// the numbers", section "The verified INT8 units": scale = max(|line|)/127
// floored at 1e-8, values to int8; with the readings of this library
// (include/int8_gemm.h): s = max(RN(a/127), RN(1e-8)), inv = RN(1/s),
// q = floor(RN(RN(x*inv) + 0.5)).
//
// Both passes are HBM-bound (4 bytes read + 1 byte written per element).
//  * rows: one wavefront per row for rows up to 4096 elements, the row held
//    in registers between the absmax and the quantize (one HBM read); a
//    1024-thread workgroup per row beyond that (registers up to 65536
//    elements, a second read from cache above).  The row max is a wave
//    butterfly reduction (plus LDS across waves).
//  * cols, short columns: one kernel, a workgroup per column band holding
//    the band in registers (see qcols_reg_kernel);
//  * cols, tall columns (bands of at most 8 columns would not read whole
//    cache lines): two passes over X, a column-scale pass and a
//    quantize-transpose pass (see qcols_scale_kernel).
#include "i8g_device.h"
#include "i8g_launch.h"

namespace i8g {

// Four consecutive elements of a row starting at column c (c % 4 == 0),
// zero beyond `cols`.  `vec` selects one 16-byte load (row base aligned).
__device__ __forceinline__ float4 load4(const float* row, int64_t c, int64_t cols, bool vec) {
  if (vec && c + 4 <= cols) return *reinterpret_cast<const float4*>(row + c);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < cols) v.x = row[c];
  if (c + 1 < cols) v.y = row[c + 1];
  if (c + 2 < cols) v.z = row[c + 2];
  if (c + 3 < cols) v.w = row[c + 3];
  return v;
}

__device__ __forceinline__ float absmax4(float m, float4 v) {
  m = fmaxf(m, fabsf(v.x));
  m = fmaxf(m, fabsf(v.y));
  m = fmaxf(m, fabsf(v.z));
  return fmaxf(m, fabsf(v.w));
}

__device__ __forceinline__ unsigned int pack4(float4 v, float inv) {
  unsigned int b0 = (unsigned int)(quantize1(v.x, inv) & 0xFF);
  unsigned int b1 = (unsigned int)(quantize1(v.y, inv) & 0xFF);
  unsigned int b2 = (unsigned int)(quantize1(v.z, inv) & 0xFF);
  unsigned int b3 = (unsigned int)(quantize1(v.w, inv) & 0xFF);
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

__device__ __forceinline__ void store4(int8_t* row, int64_t c, int64_t cols, unsigned int q,
                                       bool vec) {
  if (vec && c + 4 <= cols) {
    *reinterpret_cast<unsigned int*>(row + c) = q;
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (c + e < cols) row[c + e] = (int8_t)((q >> (8 * e)) & 0xFF);
}

// ---------------------------------------------------------------------------
// rows: one wavefront per row, VPL groups of 4 elements per lane in registers
// ---------------------------------------------------------------------------
// The kernel bodies take the workgroup's index within their own grid (`bid`)
// and their LDS from the caller, so that quantize_batch_kernel can run
// several of them in one launch.
// A row of `cols` values (cols % 4 == 0, X rows 16-byte aligned, Q rows
// 4-byte aligned) by one wave, through buffer loads and stores from the
// row's base (uniform in the wave): a lane keeps only the row's data and its
// offset live, no 64-bit addresses; groups past the row's end read as zeros
// and store nothing.
template <int VPL, int FMT>
__device__ __forceinline__ void qrows_wave_vec_body(const float* __restrict__ X, int64_t cols, int64_t ldx,
                                                    int8_t* __restrict__ Q, int64_t ldq,
                                                    float* __restrict__ scale, int64_t r) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(uniform_ptr(X + r * ldx)), 0, (int)(cols * 4), 0x00020000);
  float4 v[VPL];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const v4f x = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rx, lane * 16 + i * 1024, 0, 0));
    v[i] = make_float4(x[0], x[1], x[2], x[3]);
    m = absmax4(m, v[i]);
  }
  m = wave_max_f32(m);
  const float s = scale_of_absmax_fmt<FMT>(m);
  const float inv = recip_rn(s);
  if (lane == 0) scale[r] = s;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(Q + r * ldq), 0, (int)cols, 0x00020000);
#pragma unroll
  for (int i = 0; i < VPL; ++i) __builtin_amdgcn_raw_buffer_store_b32(pack4(v[i], inv), rq, lane * 4 + i * 256, 0, 0);
}

template <int VPL, int FMT>
__device__ __forceinline__ void qrows_wave_body(const float* __restrict__ X, int64_t rows, int64_t cols,
                                                int64_t ldx, int8_t* __restrict__ Q, int64_t ldq,
                                                float* __restrict__ scale, int vec_in, int vec_out,
                                                int64_t bid) {
  const int lane = threadIdx.x & 63;
  const int64_t r = bid * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6);   // a wave per row
  if (r >= rows) return;
  const float* xr = X + r * ldx;
  float4 v[VPL];
  float m = 0.0f;
  if (vec_in && vec_out && (cols & 3) == 0) {
    qrows_wave_vec_body<VPL, FMT>(X, cols, ldx, Q, ldq, scale, r);
    return;
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    v[i] = load4(xr, (int64_t)(lane + 64 * i) * 4, cols, vec_in);
    m = absmax4(m, v[i]);
  }
  m = wave_max_f32(m);
  const float s = scale_of_absmax_fmt<FMT>(m);
  const float inv = recip_rn(s);
  if (lane == 0) scale[r] = s;
  int8_t* qr = Q + r * ldq;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int64_t c = (int64_t)(lane + 64 * i) * 4;
    if (c < cols) store4(qr, c, cols, pack4(v[i], inv), vec_out);
  }
}

template <int VPL, int FMT>
__global__ void __launch_bounds__(256)
qrows_wave_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                  int8_t* __restrict__ Q, int64_t ldq, float* __restrict__ scale, int vec_in,
                  int vec_out) {
  qrows_wave_body<VPL, FMT>(X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out, blockIdx.x);
}

// The same for aligned rows only: no per-element path in the kernel, so it
// keeps fewer registers and more waves resident.
template <int VPL, int FMT>
__global__ void __launch_bounds__(256)
qrows_wave_vec_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                      int8_t* __restrict__ Q, int64_t ldq, float* __restrict__ scale) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // a wave per row
  if (r >= rows) return;
  qrows_wave_vec_body<VPL, FMT>(X, cols, ldx, Q, ldq, scale, r);
}

template <int VPL, int FMT>
static void launch_qrows_wave(dim3 grid, hipStream_t stream, const float* X, int64_t rows, int64_t cols,
                              int64_t ldx, int8_t* Q, int64_t ldq, float* scale, int vec_in, int vec_out) {
  if (vec_in && vec_out && (cols & 3) == 0)
    hipLaunchKernelGGL((qrows_wave_vec_kernel<VPL, FMT>), grid, dim3(256), 0, stream, X, rows, cols, ldx, Q, ldq,
                       scale);
  else
    hipLaunchKernelGGL((qrows_wave_kernel<VPL, FMT>), grid, dim3(256), 0, stream, X, rows, cols, ldx, Q, ldq,
                       scale, vec_in, vec_out);
}

// ---------------------------------------------------------------------------
// rows: one 1024-thread workgroup per row (long rows)
// ---------------------------------------------------------------------------
template <int VPT, int FMT>
__device__ __forceinline__ void qrows_block_body(const float* __restrict__ X, int64_t rows, int64_t cols,
                                                 int64_t ldx, int8_t* __restrict__ Q, int64_t ldq,
                                                 float* __restrict__ scale, int vec_in, int vec_out,
                                                 int64_t bid, float* red /* LDS, 16 floats */) {
  constexpr int NT = 1024;
  constexpr int64_t CHUNK = (int64_t)NT * VPT * 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = bid;
  const float* xr = X + r * ldx;
  int8_t* qr = Q + r * ldq;
  float4 v[VPT];
  float m = 0.0f;
  for (int64_t base = 0; base < cols; base += CHUNK) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      v[i] = load4(xr, base + (int64_t)(tid + NT * i) * 4, cols, vec_in);
      m = absmax4(m, v[i]);
    }
  }
  m = wave_max_f32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (wave == 0) {
    float w = lane < NT / 64 ? red[lane] : 0.0f;
    w = wave_max_f32(w);
    if (lane == 0) red[0] = w;
  }
  __syncthreads();
  const float s = scale_of_absmax_fmt<FMT>(red[0]);
  const float inv = recip_rn(s);
  if (tid == 0) scale[r] = s;
  if (cols <= CHUNK) {   // the row is still in registers
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t c = (int64_t)(tid + NT * i) * 4;
      if (c < cols) store4(qr, c, cols, pack4(v[i], inv), vec_out);
    }
  } else {               // reread (from L2 / MALL)
    for (int64_t base = 0; base < cols; base += CHUNK) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int64_t c = base + (int64_t)(tid + NT * i) * 4;
        if (c < cols) store4(qr, c, cols, pack4(load4(xr, c, cols, vec_in), inv), vec_out);
      }
    }
  }
}

template <int VPT, int FMT>
__global__ void __launch_bounds__(1024)
qrows_block_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                   int8_t* __restrict__ Q, int64_t ldq, float* __restrict__ scale, int vec_in,
                   int vec_out) {
  __shared__ float red[16];
  qrows_block_body<VPT, FMT>(X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out, blockIdx.x, red);
}

// Row path by row length: a wave per row with VPL float4 per lane up to 4096
// values, else a 1024-thread workgroup per row (VPT float4 per thread).
static int rows_wave_vpl(int64_t cols) {
  if (cols <= 256) return 1;
  if (cols <= 512) return 2;
  if (cols <= 768) return 3;
  if (cols <= 1024) return 4;
  if (cols <= 2048) return 8;
  if (cols <= 3072) return 12;
  if (cols <= 4096) return 16;
  return 0;
}
static int rows_block_vpt(int64_t cols) { return cols <= 1024 * 8 * 4 ? 8 : 16; }

template <int FMT>
hipError_t quantize_rows_int8(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                              int8_t* Q, int64_t ldq, float* scale, hipStream_t stream) {
  const int vec_in = ((uintptr_t)X % 16 == 0) && (ldx % 4 == 0);
  const int vec_out = ((uintptr_t)Q % 4 == 0) && (ldq % 4 == 0);
  if (rows_wave_vpl(cols) > 0) {
    const dim3 grid((unsigned int)((rows + 3) / 4));
    if (cols <= 256)
      launch_qrows_wave<1, FMT>(grid, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 512)
      launch_qrows_wave<2, FMT>(grid, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 768)
      launch_qrows_wave<3, FMT>(grid, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 1024)
      launch_qrows_wave<4, FMT>(grid, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 2048)
      launch_qrows_wave<8, FMT>(grid, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 3072)
      launch_qrows_wave<12, FMT>(grid, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else
      launch_qrows_wave<16, FMT>(grid, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
  } else {
    const dim3 grid((unsigned int)rows), block(1024);
    if (rows_block_vpt(cols) == 8)
      hipLaunchKernelGGL((qrows_block_kernel<8, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else
      hipLaunchKernelGGL((qrows_block_kernel<16, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// cols, two passes (tall columns): the column scale needs every row first.
//  1. qcols_init_kernel writes the scale floor RN(1e-8) to every scale;
//  2. qcols_scale_kernel reads X in full, coalesced rows, keeps a per-thread
//     max of |x| per column over its rows, turns it into a partial scale
//     max(RN(a/127), RN(1e-8)) and combines partial scales with atomicMax on
//     their bit patterns.  RN and the floor are monotone, so the largest
//     partial scale is the scale of the column max, exactly and in any order,
//     and positive floats order like their bit patterns;
//  3. qcols_quant_kernel reads X again (it is usually still in the last-level
//     cache), quantizes 64x64 tiles with inv = RN(1/s), transposes them
//     through LDS and writes K-contiguous rows of Qt.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void qcols_init_kernel(float* scale, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) scale[i] = scale_of_absmax_fmt<FMT>(0.0f);   // the (rounded) floor
}

constexpr int QS_ROWS = 64;     // rows per workgroup of qcols_scale_kernel
constexpr int QS_COLS = 256;    // columns per workgroup (64 lanes x 4)

template <int FMT>
__global__ void __launch_bounds__(256)
qcols_scale_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                   float* __restrict__ scale, int vec_in) {
  __shared__ float red[4][QS_COLS];
  const int tid = threadIdx.x;
  const int cg = tid & 63, ph = tid >> 6;          // column group of 4, row phase
  const int64_t c = (int64_t)blockIdx.x * QS_COLS + cg * 4;
  const int64_t r0 = (int64_t)blockIdx.y * QS_ROWS;
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < cols) {
    if (r0 + QS_ROWS <= rows) {
      float4 v[QS_ROWS / 4];
#pragma unroll
      for (int i = 0; i < QS_ROWS / 4; ++i) v[i] = load4(X + (r0 + ph + 4 * i) * ldx, c, cols, vec_in);
#pragma unroll
      for (int i = 0; i < QS_ROWS / 4; ++i) {
        m.x = fmaxf(m.x, fabsf(v[i].x));
        m.y = fmaxf(m.y, fabsf(v[i].y));
        m.z = fmaxf(m.z, fabsf(v[i].z));
        m.w = fmaxf(m.w, fabsf(v[i].w));
      }
    } else {
      for (int64_t r = r0 + ph; r < rows; r += 4) {
        const float4 v = load4(X + r * ldx, c, cols, vec_in);
        m.x = fmaxf(m.x, fabsf(v.x));
        m.y = fmaxf(m.y, fabsf(v.y));
        m.z = fmaxf(m.z, fabsf(v.z));
        m.w = fmaxf(m.w, fabsf(v.w));
      }
    }
  }
  red[ph][cg * 4 + 0] = m.x;
  red[ph][cg * 4 + 1] = m.y;
  red[ph][cg * 4 + 2] = m.z;
  red[ph][cg * 4 + 3] = m.w;
  __syncthreads();
  const float a = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
  const int64_t col = (int64_t)blockIdx.x * QS_COLS + tid;
  if (col < cols)
    atomicMax(reinterpret_cast<unsigned int*>(scale) + col, __float_as_uint(scale_of_absmax_fmt<FMT>(a)));
}

// Quantize a 64 (rows of X = k) x 64 (columns of X = j) tile with the column
// scales, transpose through LDS, write 64 rows of Qt (64 bytes each).
__global__ void __launch_bounds__(256)
qcols_quant_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                   int8_t* __restrict__ Qt, int64_t ldqt, const float* __restrict__ scale,
                   int vec_in, int vec_out) {
  __shared__ float s_inv[64];
  __shared__ unsigned int tq[64][17];              // [j][k/4], padded
  const int tid = threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
  if (tid < 64) {
    const int64_t j = j0 + tid;
    s_inv[tid] = j < cols ? recip_rn(scale[j]) : 0.0f;
  }
  __syncthreads();
  const int cg = tid & 15, rr = tid >> 4;          // 16 groups of 4 columns, 16 rows
  const float i0 = s_inv[cg * 4], i1 = s_inv[cg * 4 + 1], i2 = s_inv[cg * 4 + 2], i3 = s_inv[cg * 4 + 3];
  // each thread quantizes rows k = 4*rr .. 4*rr+3 of its 4 columns, so it can
  // pack 4 consecutive k of one column into one 32-bit word of tq.
  float4 v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t k = k0 + rr * 4 + e;
    v[e] = k < rows ? load4(X + k * ldx, j0 + cg * 4, cols, vec_in) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  unsigned int w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0 |= (unsigned int)(quantize1(v[e].x, i0) & 0xFF) << (8 * e);
    w1 |= (unsigned int)(quantize1(v[e].y, i1) & 0xFF) << (8 * e);
    w2 |= (unsigned int)(quantize1(v[e].z, i2) & 0xFF) << (8 * e);
    w3 |= (unsigned int)(quantize1(v[e].w, i3) & 0xFF) << (8 * e);
  }
  tq[cg * 4 + 0][rr] = w0;
  tq[cg * 4 + 1][rr] = w1;
  tq[cg * 4 + 2][rr] = w2;
  tq[cg * 4 + 3][rr] = w3;
  __syncthreads();
  // write: thread -> (row jl = tid/4 of Qt, 16-byte chunk tid%4)
  const int jl = tid >> 2, ch = tid & 3;
  const int64_t j = j0 + jl;
  if (j >= cols) return;
  int8_t* dst = Qt + j * ldqt;
  const int64_t k = k0 + ch * 16;
  if (k >= rows) return;
  const unsigned int a = tq[jl][ch * 4], b = tq[jl][ch * 4 + 1], c = tq[jl][ch * 4 + 2],
                     d = tq[jl][ch * 4 + 3];
  if (vec_out && k + 16 <= rows) {
    *reinterpret_cast<uint4*>(dst + k) = make_uint4(a, b, c, d);
  } else {
    const unsigned int w[4] = {a, b, c, d};
    for (int e = 0; e < 16 && k + e < rows; ++e) dst[k + e] = (int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFF);
  }
}

// ---------------------------------------------------------------------------
// cols, one read of X for large inputs (cooperative launch).  A band is 32
// columns: one 128-byte line of every row.  The band's rows are split into
// chunks of 1024 rows, one per member of a group of P workgroups (512
// threads each, a lane holding 16 rows x 4 columns in registers); the
// members of a group sit on one XCD (workgroup ids are dealt to the 8 XCDs
// round-robin) and walk the same bands.  Per band a member
//  1. reads its chunk with whole-line loads and reduces its 32 column maxima;
//  2. raises scale[j] to its partial scale max(RN(a/127), RN(1e-8)) with an
//     agent-scope atomicMax on the bit pattern (RN and the floor are
//     monotone and positive floats order like their bits, so the largest
//     partial scale is the scale of the column max, in any order); it waits
//     for the atomics' returned values, so they have been performed;
//  3. adds 1 to the band's counter (agent scope) and waits, with a bounded
//     spin, until all P members have added theirs: every partial maximum is
//     then in place, and the final scales are read with agent-scope atomic
//     loads;
//  4. quantizes its chunk, transposes it through LDS and stores 32 segments
//     of 1024 bytes of Qt.
// The counter lives in the first four bytes of the band's first Qt row,
// zeroed by qcols_coop_init_kernel: those bytes belong to member 0, which
// writes their codes (an atomic exchange) only after the other members have
// left the wait (each adds 1 more, so the count reaches 2P-1).  All waits
// are bounded; a member whose wait times out (the grid was not resident)
// stops waiting for the rest of the launch and leaves the band's scales NaN;
// so does member 0 when its wait for the other members to leave (before it
// writes the counter word's codes) times out.  The spin limit is a kernel
// argument: kQkWaitLimit, or 0 under the test override that exercises these
// paths.
// Requires rows % 256 == 0, rows >= 1024, cols % 32 == 0, X and Qt 16-byte
// aligned, ldx % 4 == 0, ldqt % 16 == 0 and 1024 rows of X addressable with
// 32-bit offsets.
// ---------------------------------------------------------------------------
constexpr int QK_THREADS = 512;            // 8 waves
constexpr int QK_ROWS = 1024;              // rows of X per member and band
constexpr int QK_COLS = 32;                // columns per band (128 bytes of a row)
constexpr int QK_TS = QK_ROWS / 4 + 4;     // words per LDS tile row (padded)
constexpr unsigned int kQkWaitLimit = 1u << 20;   // spins of ~64 cycles: tens of ms
constexpr double kQkMinBytes = 256.0 * 1024 * 1024;   // X bytes from which the path is used

template <int FMT>
__global__ void qcols_coop_init_kernel(float* scale, int64_t cols, int8_t* Qt, int64_t ldqt,
                                       int64_t nbands) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < cols) scale[i] = scale_of_absmax_fmt<FMT>(0.0f);   // the (rounded) floor
  if (i < nbands) *reinterpret_cast<unsigned int*>(Qt + i * QK_COLS * ldqt) = 0u;
}

template <int FMT>
__global__ void __launch_bounds__(QK_THREADS, 4)
qcols_coop_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                  int8_t* __restrict__ Qt, int64_t ldqt, float* __restrict__ scale, int P, int NG,
                  int64_t nbands, unsigned int wait_limit) {
  __shared__ float red[8][QK_COLS];
  __shared__ float s_inv[QK_COLS];
  __shared__ int s_ok;
  __shared__ __attribute__((aligned(16))) unsigned int tile[QK_COLS][QK_TS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int slot = t & 7, rg = t >> 3;                 // 16-byte slot of the line, row group
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int m = q % P, g = xcd + 8 * (q / P);          // member m of group g
  if (g >= NG) return;
  const int64_t r0 = (int64_t)m * QK_ROWS;
  // 256-row blocks of this chunk inside X (workgroup-uniform)
  const int nblk = __builtin_amdgcn_readfirstlane((int)((rows - r0) / 256 < 4 ? (rows - r0) / 256 : 4));
  const int ld4 = (int)(ldx * 4);
  const int vo = (4 * rg) * ld4 + slot * 16;           // rows 4*rg + e + 256*i of the chunk
  bool timed_out = false;
  unsigned int* pend_addr = nullptr;                   // member 0's counter word, codes pending
  unsigned int* pend_sbits = nullptr;                  // ... and that band's scales
  unsigned int pend_codes = 0;
  auto settle = [&](bool block) __attribute__((always_inline)) {
    if (t != 0 || pend_addr == nullptr) return;
    unsigned int n = 0;
    bool left = true;
    while (__hip_atomic_load(pend_addr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           (unsigned int)(2 * P - 1)) {
      if (!block && n >= 64) return;                   // again after the next band
      __builtin_amdgcn_s_sleep(2);
      if (++n > wait_limit) {
        left = false;
        break;
      }
    }
    __hip_atomic_exchange(pend_addr, pend_codes, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // a member still to leave may add to the word after the codes: the band
    // is marked as failed
    if (!left)
      for (int k = 0; k < QK_COLS; ++k)
        __hip_atomic_exchange(pend_sbits + k, 0x7FC00000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pend_addr = nullptr;
  };
  for (int64_t b = g; b < nbands; b += NG) {
    // 1. the chunk in registers: buffer loads from a uniform base, one 32-bit
    // offset per lane, uniform row offsets; blocks past the end of X skipped
    float4 v[16];
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(uniform_ptr(X + r0 * ldx + b * QK_COLS)), 0, 0x7FFFFFF0, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        typedef float v4f __attribute__((ext_vector_type(4)));
        if (i < nblk) {
          const v4f x = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, (e + 256 * i) * ld4, 0));
          v[i * 4 + e] = make_float4(x[0], x[1], x[2], x[3]);
        } else {
          v[i * 4 + e] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      m0 = fmaxf(m0, fabsf(v[i].x));
      m1 = fmaxf(m1, fabsf(v[i].y));
      m2 = fmaxf(m2, fabsf(v[i].z));
      m3 = fmaxf(m3, fabsf(v[i].w));
    }
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {            // lanes with the same slot
      m0 = fmaxf(m0, __shfl_xor(m0, off, 64));
      m1 = fmaxf(m1, __shfl_xor(m1, off, 64));
      m2 = fmaxf(m2, __shfl_xor(m2, off, 64));
      m3 = fmaxf(m3, __shfl_xor(m3, off, 64));
    }
    if (lane < 8) {
      red[wave][slot * 4 + 0] = m0;
      red[wave][slot * 4 + 1] = m1;
      red[wave][slot * 4 + 2] = m2;
      red[wave][slot * 4 + 3] = m3;
    }
    __syncthreads();
    unsigned int* const counter = reinterpret_cast<unsigned int*>(Qt + b * QK_COLS * ldqt);
    unsigned int* const sbits = reinterpret_cast<unsigned int*>(scale) + b * QK_COLS;
    if (t < QK_COLS) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) a = fmaxf(a, red[w][t]);
      // 2. the partial scale into scale[j]; the returned value is consumed
      const unsigned int old = __hip_atomic_fetch_max(sbits + t, __float_as_uint(scale_of_absmax_fmt<FMT>(a)),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("" ::"v"(old));
    }
    __builtin_amdgcn_s_waitcnt(0);                      // this lane's maximum has returned
    __syncthreads();                                    // ... and every lane's
    // 3. arrive, wait for the group, leave
    if (t == 0) {
      const unsigned int mine = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("" ::"v"(mine));
      bool ok;
      if (!timed_out) {
        unsigned int n = 0;
        ok = true;
        while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned int)P) {
          __builtin_amdgcn_s_sleep(1);
          if (++n > wait_limit) {
            ok = false;
            break;
          }
        }
      } else {
        ok = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (unsigned int)P;
      }
      timed_out = timed_out || !ok;
      s_ok = ok ? 1 : 0;
      if (m != 0) __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (t < QK_COLS) {
      const float s = __uint_as_float(__hip_atomic_load(sbits + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (!s_ok) __hip_atomic_exchange(sbits + t, 0x7FC00000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_inv[t] = recip_rn(s);
    }
    __syncthreads();
    // 4. quantize, transpose through LDS (4 consecutive rows per word), store
    const float i0 = s_inv[slot * 4], i1 = s_inv[slot * 4 + 1], i2 = s_inv[slot * 4 + 2], i3 = s_inv[slot * 4 + 3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      unsigned int w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 x = v[i * 4 + e];
        w0 |= ((unsigned int)quantize1(x.x, i0) & 0xFFu) << (8 * e);
        w1 |= ((unsigned int)quantize1(x.y, i1) & 0xFFu) << (8 * e);
        w2 |= ((unsigned int)quantize1(x.z, i2) & 0xFFu) << (8 * e);
        w3 |= ((unsigned int)quantize1(x.w, i3) & 0xFFu) << (8 * e);
      }
      tile[slot * 4 + 0][rg + 64 * i] = w0;
      tile[slot * 4 + 1][rg + 64 * i] = w1;
      tile[slot * 4 + 2][rg + 64 * i] = w2;
      tile[slot * 4 + 3][rg + 64 * i] = w3;
    }
    __syncthreads();
    {
      // Qt row b*32+jj, bytes qq*256 + part*16 .. +16: the 16 lanes of a row
      // store 256 contiguous bytes per instruction
      const int jj = t >> 4, part = t & 15;
      int8_t* dst = Qt + (b * QK_COLS + jj) * ldqt + r0 + part * 16;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int w = qq * 64 + part * 4;
        if (r0 + qq * 256 + part * 16 < rows) {          // rows % 256 == 0: whole 16-byte groups
          const unsigned int a0 = tile[jj][w], a1 = tile[jj][w + 1], a2 = tile[jj][w + 2], a3 = tile[jj][w + 3];
          if (m == 0 && jj == 0 && part == 0 && qq == 0) {
            settle(true);                                // the previous band's word first
            unsigned int* d = reinterpret_cast<unsigned int*>(dst);
            d[1] = a1;
            d[2] = a2;
            d[3] = a3;
            pend_addr = d;                               // d[0] is the counter
            pend_sbits = sbits;
            pend_codes = a0;
          } else {
            *reinterpret_cast<uint4*>(dst + qq * 256) = make_uint4(a0, a1, a2, a3);
          }
        }
      }
    }
    settle(false);
    __syncthreads();                                    // LDS is reused by the next band
  }
  settle(true);
}

// ---------------------------------------------------------------------------
// cols, two passes over whole lines (medium inputs, no cross-workgroup wait).
// The same bands and chunks as qcols_coop_kernel, as two launches after
// qcols_init_kernel has set every scale to the floor:
//  1. qcols_lines_max_kernel: each workgroup (band, chunk) reads its chunk
//     with whole-line loads and raises the band's 32 scales to its partial
//     scales (atomicMax on the bit patterns; the largest partial scale is the
//     scale of the column max);
//  2. qcols_lines_quant_kernel: each workgroup reads its chunk again (an
//     input of up to a few hundred MB is still in the 256 MB last-level
//     cache), reads the final scales, quantizes and stores the transposed
//     chunk.
// Same requirements as the cooperative path.
// ---------------------------------------------------------------------------
// The chunk of (band b, rows r0 .. r0+1023) in registers: lane (slot, rg)
// holds rows 4*rg + e + 256*i, columns 4*slot .. 4*slot+3 of the band
// (v[4*i + e]); 256-row blocks past the end of X are zeros.
__device__ __forceinline__ void qk_load_chunk(const float* X, int64_t ldx, int64_t r0, int64_t b, int nblk,
                                              int vo, int ld4, float4 (&v)[16]) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(uniform_ptr(X + r0 * ldx + b * QK_COLS)), 0, 0x7FFFFFF0, 0x00020000);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      typedef float v4f __attribute__((ext_vector_type(4)));
      if (i < nblk) {
        const v4f x = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, (e + 256 * i) * ld4, 0));
        v[i * 4 + e] = make_float4(x[0], x[1], x[2], x[3]);
      } else {
        v[i * 4 + e] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
}

template <int FMT>
__global__ void __launch_bounds__(QK_THREADS, 4)
qcols_lines_max_kernel(const float* __restrict__ X, int64_t rows, int64_t ldx, float* __restrict__ scale, int P) {
  __shared__ float red[8][QK_COLS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int slot = t & 7, rg = t >> 3;
  const int64_t b = blockIdx.x / P, r0 = (int64_t)(blockIdx.x % P) * QK_ROWS;
  const int nblk = __builtin_amdgcn_readfirstlane((int)((rows - r0) / 256 < 4 ? (rows - r0) / 256 : 4));
  const int ld4 = (int)(ldx * 4);
  float4 v[16];
  qk_load_chunk(X, ldx, r0, b, nblk, (4 * rg) * ld4 + slot * 16, ld4, v);
  float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m0 = fmaxf(m0, fabsf(v[i].x));
    m1 = fmaxf(m1, fabsf(v[i].y));
    m2 = fmaxf(m2, fabsf(v[i].z));
    m3 = fmaxf(m3, fabsf(v[i].w));
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, off, 64));
    m1 = fmaxf(m1, __shfl_xor(m1, off, 64));
    m2 = fmaxf(m2, __shfl_xor(m2, off, 64));
    m3 = fmaxf(m3, __shfl_xor(m3, off, 64));
  }
  if (lane < 8) {
    red[wave][slot * 4 + 0] = m0;
    red[wave][slot * 4 + 1] = m1;
    red[wave][slot * 4 + 2] = m2;
    red[wave][slot * 4 + 3] = m3;
  }
  __syncthreads();
  if (t < QK_COLS) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) a = fmaxf(a, red[w][t]);
    atomicMax(reinterpret_cast<unsigned int*>(scale) + b * QK_COLS + t, __float_as_uint(scale_of_absmax_fmt<FMT>(a)));
  }
}

__global__ void __launch_bounds__(QK_THREADS, 4)
qcols_lines_quant_kernel(const float* __restrict__ X, int64_t rows, int64_t ldx, int8_t* __restrict__ Qt,
                         int64_t ldqt, const float* __restrict__ scale, int P) {
  __shared__ float s_inv[QK_COLS];
  __shared__ __attribute__((aligned(16))) unsigned int tile[QK_COLS][QK_TS];
  const int t = threadIdx.x;
  const int slot = t & 7, rg = t >> 3;
  const int64_t b = blockIdx.x / P, r0 = (int64_t)(blockIdx.x % P) * QK_ROWS;
  const int nblk = __builtin_amdgcn_readfirstlane((int)((rows - r0) / 256 < 4 ? (rows - r0) / 256 : 4));
  const int ld4 = (int)(ldx * 4);
  float4 v[16];
  qk_load_chunk(X, ldx, r0, b, nblk, (4 * rg) * ld4 + slot * 16, ld4, v);
  if (t < QK_COLS) s_inv[t] = recip_rn(scale[b * QK_COLS + t]);
  __syncthreads();
  const float i0 = s_inv[slot * 4], i1 = s_inv[slot * 4 + 1], i2 = s_inv[slot * 4 + 2], i3 = s_inv[slot * 4 + 3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned int w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 x = v[i * 4 + e];
      w0 |= ((unsigned int)quantize1(x.x, i0) & 0xFFu) << (8 * e);
      w1 |= ((unsigned int)quantize1(x.y, i1) & 0xFFu) << (8 * e);
      w2 |= ((unsigned int)quantize1(x.z, i2) & 0xFFu) << (8 * e);
      w3 |= ((unsigned int)quantize1(x.w, i3) & 0xFFu) << (8 * e);
    }
    tile[slot * 4 + 0][rg + 64 * i] = w0;
    tile[slot * 4 + 1][rg + 64 * i] = w1;
    tile[slot * 4 + 2][rg + 64 * i] = w2;
    tile[slot * 4 + 3][rg + 64 * i] = w3;
  }
  __syncthreads();
  // Qt row b*32+jj, bytes qq*256 + part*16 .. +16 (256 contiguous bytes per
  // row and instruction)
  const int jj = t >> 4, part = t & 15;
  int8_t* dst = Qt + (b * QK_COLS + jj) * ldqt + r0 + part * 16;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int w = qq * 64 + part * 4;
    if (r0 + qq * 256 + part * 16 < rows)                // rows % 256 == 0: whole 16-byte groups
      *reinterpret_cast<uint4*>(dst + qq * 256) = make_uint4(tile[jj][w], tile[jj][w + 1], tile[jj][w + 2], tile[jj][w + 3]);
  }
}

// Eligibility of the cooperative path for a column pass (see above).
static bool qcols_coop_shape_ok(const float* X, int64_t rows, int64_t cols, int64_t ldx, const int8_t* Qt,
                                int64_t ldqt, int fmt) {
  return (fmt & FMT_INT4) == 0 && rows >= QK_ROWS && rows % 256 == 0 && cols % QK_COLS == 0 && cols > 0 &&
         ldx % 4 == 0 && ((uintptr_t)X % 16) == 0 && ((uintptr_t)Qt % 16) == 0 && ldqt % 16 == 0 &&
         ldx * 4 * QK_ROWS < 0x7FFFFFF0LL;
}

static bool qcols_takes_coop(const float* X, int64_t rows, int64_t cols, int64_t ldx, const int8_t* Qt,
                             int64_t ldqt, int fmt) {
  const int path = qcols_path_requested();
  if (path == 1 || path == 3 || !qcols_coop_shape_ok(X, rows, cols, ldx, Qt, ldqt, fmt)) return false;
  return path == 2 || path == 4 || (double)rows * (double)cols * 4.0 >= kQkMinBytes;
}

// The two whole-line passes (qcols_lines_*), for tall and narrow inputs:
// measured on MI355X (launch by launch / replayed from a graph), 8192x768
// 11.6 / 12.1 us against 14.6 / 16.5 for the band kernel; 8192x2304 35.5
// against 31.8 and 8192x3072 42.8 against 38.8, where the band kernel's
// wider grid wins; 3072x768 10.2 against 6.5.
static bool qcols_takes_lines(const float* X, int64_t rows, int64_t cols, int64_t ldx, const int8_t* Qt,
                              int64_t ldqt, int fmt) {
  const int path = qcols_path_requested();
  if (path == 1 || path == 2 || path == 4 || !qcols_coop_shape_ok(X, rows, cols, ldx, Qt, ldqt, fmt)) return false;
  return path == 3 || (rows >= 4096 && cols <= 1024);
}

// Workgroups of qcols_coop_kernel<FMT> resident per CU on the current device
// (cached per device).
template <int FMT>
static int qcols_coop_occupancy() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, qcols_coop_kernel<FMT>, QK_THREADS, 0) != hipSuccess)
      n = 0;
    cache[dev] = n > 0 ? n : -1;
  }
  return cache[dev] > 0 ? cache[dev] : 0;
}

// Enqueues the cooperative path; an error means nothing but the (harmless)
// init kernel ran, and the caller takes another path.
template <int FMT>
static hipError_t launch_qcols_coop(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Qt,
                                    int64_t ldqt, float* scale, hipStream_t stream) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return hipErrorInvalidDevice;
  const int occ = qcols_coop_occupancy<FMT>();
  const int P = (int)((rows + QK_ROWS - 1) / QK_ROWS);
  const int64_t nbands = cols / QK_COLS;
  const int64_t cap_groups = ((int64_t)cus * occ / P) / 8 * 8;   // resident groups, a multiple of 8
  if (occ <= 0 || cap_groups < 8) return hipErrorCooperativeLaunchTooLarge;
  const int64_t NG = nbands < cap_groups ? (nbands + 7) / 8 * 8 : cap_groups;
  hipLaunchKernelGGL(qcols_coop_init_kernel<FMT>, dim3((unsigned int)((cols + 255) / 256)), dim3(256), 0,
                     stream, scale, cols, Qt, ldqt, nbands);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int p = P, ng = (int)NG;
  // the test override 4 cuts every wait to one spin (the timeout paths)
  unsigned int wait_limit = qcols_path_requested() == 4 ? 0u : kQkWaitLimit;
  void* args[] = {&X, &rows, &cols, &ldx, &Qt, &ldqt, &scale, &p, &ng, const_cast<int64_t*>(&nbands), &wait_limit};
  e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(qcols_coop_kernel<FMT>), dim3((unsigned int)(NG * P)),
                                 dim3(QK_THREADS), args, 0, stream);
  return e;
}

// ---------------------------------------------------------------------------
// cols, one kernel (rows <= 8192): a 1024-thread workgroup owns a band of BC
// columns and every row, holding the band in registers (at most 32 floats
// per thread), so X is read from HBM once.  The column maxima are reduced
// inside the workgroup (lane shuffles, then LDS across the 16 waves), the
// int8 values are written transposed into an LDS tile [BC][rows] and stored
// as K-contiguous rows of Qt.  Bands that share a 128-byte line of X are
// given to workgroups on the same XCD (ids are dealt to the 8 XCDs
// round-robin), so the line is fetched into one L2 only.
// ---------------------------------------------------------------------------
constexpr int QCR_THREADS = 1024;
constexpr int QCR_VPT = 8;            // float4 groups per thread
constexpr int QCR_MAX_ELEMS = QCR_THREADS * QCR_VPT * 4;   // 32768 per band

__device__ __forceinline__ int xcd_grouped(int wg, int total) {
  const int xcd = wg & 7, idx = wg >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// LDS of qcols_reg_body: the transposed tile, then the column maxima of the
// 16 waves, then the reciprocals.
constexpr int QCR_SMEM_BYTES = QCR_MAX_ELEMS + (QCR_THREADS / 64) * 64 * 4 + 64 * 4;

template <int BC, int FMT>
__device__ __forceinline__ void qcols_reg_body(const float* __restrict__ X, int64_t rows, int64_t cols,
                                               int64_t ldx, int8_t* __restrict__ Qt, int64_t ldqt,
                                               float* __restrict__ scale, int vec_in, int vec_out,
                                               int bid, int nbands, char* smem) {
  constexpr int C4 = BC / 4;                 // threads per row
  constexpr int RPP = QCR_THREADS / C4;      // rows per pass
  int8_t* tile = reinterpret_cast<int8_t*>(smem);
  float (*red)[BC] = reinterpret_cast<float (*)[BC]>(smem + QCR_MAX_ELEMS);
  float* s_inv = reinterpret_cast<float*>(smem + QCR_MAX_ELEMS + (QCR_THREADS / 64) * BC * 4);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t j0 = (int64_t)xcd_grouped(bid, nbands) * BC;
  const int cg = tid % C4, r_off = tid / C4;
  const int rp = (int)((rows + 15) / 16 * 16);     // tile row pitch (bytes per column)

  float4 v[QCR_VPT];
  float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
  if (vec_in && (cols & 3) == 0 && (double)rows * (double)ldx * 4.0 < 2147483648.0) {
    // buffer loads from the band's first column (uniform): 32-bit offsets
    // instead of 64-bit addresses; a row at or past `rows`, or a column group
    // past `cols`, gets an offset beyond the resource and reads as zeros
    typedef float v4f __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(uniform_ptr(X + j0)), 0, (int)((rows - 1) * ldx * 4 + (cols - j0) * 4), 0x00020000);
    const bool col_ok = j0 + cg * 4 < cols;
#pragma unroll
    for (int p = 0; p < QCR_VPT; ++p) {
      const int64_t r = r_off + (int64_t)p * RPP;
      const int vo = col_ok && r < rows ? (int)((r * ldx + cg * 4) * 4) : 0x7FFFFFFF;
      const v4f x = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0));
      v[p] = make_float4(x[0], x[1], x[2], x[3]);
      m0 = fmaxf(m0, fabsf(v[p].x));
      m1 = fmaxf(m1, fabsf(v[p].y));
      m2 = fmaxf(m2, fabsf(v[p].z));
      m3 = fmaxf(m3, fabsf(v[p].w));
    }
  } else {
#pragma unroll
    for (int p = 0; p < QCR_VPT; ++p) {
      const int64_t r = r_off + (int64_t)p * RPP;
      v[p] = r < rows ? load4(X + r * ldx, j0 + cg * 4, cols, vec_in) : make_float4(0.f, 0.f, 0.f, 0.f);
      m0 = fmaxf(m0, fabsf(v[p].x));
      m1 = fmaxf(m1, fabsf(v[p].y));
      m2 = fmaxf(m2, fabsf(v[p].z));
      m3 = fmaxf(m3, fabsf(v[p].w));
    }
  }
  // lanes l, l+C4, l+2*C4, ... of a wave hold the same columns
#pragma unroll
  for (int off = C4; off < 64; off <<= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, off, 64));
    m1 = fmaxf(m1, __shfl_xor(m1, off, 64));
    m2 = fmaxf(m2, __shfl_xor(m2, off, 64));
    m3 = fmaxf(m3, __shfl_xor(m3, off, 64));
  }
  if (lane < C4) {
    red[wave][cg * 4 + 0] = m0;
    red[wave][cg * 4 + 1] = m1;
    red[wave][cg * 4 + 2] = m2;
    red[wave][cg * 4 + 3] = m3;
  }
  __syncthreads();
  if (tid < BC) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < QCR_THREADS / 64; ++w) a = fmaxf(a, red[w][tid]);
    const float s = scale_of_absmax_fmt<FMT>(a);
    s_inv[tid] = recip_rn(s);
    if (j0 + tid < cols) scale[j0 + tid] = s;
  }
  __syncthreads();
  const float i0 = s_inv[cg * 4], i1 = s_inv[cg * 4 + 1], i2 = s_inv[cg * 4 + 2], i3 = s_inv[cg * 4 + 3];
#pragma unroll
  for (int p = 0; p < QCR_VPT; ++p) {
    const int r = r_off + p * RPP;
    if (r < rows) {
      tile[(cg * 4 + 0) * rp + r] = (int8_t)quantize1(v[p].x, i0);
      tile[(cg * 4 + 1) * rp + r] = (int8_t)quantize1(v[p].y, i1);
      tile[(cg * 4 + 2) * rp + r] = (int8_t)quantize1(v[p].z, i2);
      tile[(cg * 4 + 3) * rp + r] = (int8_t)quantize1(v[p].w, i3);
    }
  }
  __syncthreads();
  if constexpr ((FMT & FMT_INT4) != 0) {
    // int4 lines: a thread per 16-byte group of 32 values (low nibbles values
    // 0-15, high nibbles 16-31; zero past the line's end); Qt is 16-byte
    // aligned with ldqt a multiple of 16 for this format
    const int g4 = (int)((rows + 31) / 32);
    for (int q = tid; q < BC * g4; q += QCR_THREADS) {
      const int c = q / g4, gi = q % g4;
      const int64_t j = j0 + c;
      if (j >= cols) continue;
      const int8_t* src = tile + c * rp;
      unsigned int w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        unsigned int v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int k0 = gi * 32 + 4 * i + b, k1 = k0 + 16;
          const unsigned int lo = k0 < rows ? ((unsigned int)src[k0] & 0xFu) : 0u;
          const unsigned int hi = k1 < rows ? ((unsigned int)src[k1] & 0xFu) : 0u;
          v |= (lo | (hi << 4)) << (8 * b);
        }
        w[i] = v;
      }
      *reinterpret_cast<uint4*>(Qt + j * ldqt + gi * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    // store: BC rows of Qt, rows bytes each, 16 bytes per thread
    const int r16 = rp / 16;
    for (int q = tid; q < BC * r16; q += QCR_THREADS) {
      const int c = q / r16, off = (q % r16) * 16;
      const int64_t j = j0 + c;
      if (j >= cols) continue;
      int8_t* dst = Qt + j * ldqt + off;
      const int8_t* src = tile + c * rp + off;
      if (vec_out && off + 16 <= rows) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int e = 0; e < 16 && off + e < rows; ++e) dst[e] = src[e];
      }
    }
  }
}

template <int BC, int FMT>
__global__ void __launch_bounds__(QCR_THREADS)
qcols_reg_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                 int8_t* __restrict__ Qt, int64_t ldqt, float* __restrict__ scale, int vec_in,
                 int vec_out) {
  __shared__ __attribute__((aligned(16))) char smem[QCR_SMEM_BYTES];
  qcols_reg_body<BC, FMT>(X, rows, cols, ldx, Qt, ldqt, scale, vec_in, vec_out, blockIdx.x, gridDim.x,
                          smem);
}

// Band width for the one-kernel path: as wide as the registers allow (BC *
// rows <= 32768) while leaving at least min_wgs workgroups; 0 = use the
// multi-kernel path (more than 8192 rows).  Wider bands read longer pieces
// of each row (fewer L2 requests per byte) with fewer workgroups.  A launch
// of its own keeps at least 128 (768x3072: 16 columns per band, 5.0 us
// against 6.7 with 32); a job of quantize_batch, which shares the launch,
// at least 64 (the GPT-2 weights take 32 and 8 columns instead of 16 and 4:
// MLP step 0.4%, transformer layer 0.9%, LM head 0.6% faster, measured back
// to back on one box).
static int qcols_band(int64_t rows, int64_t cols, int min_wgs = 128) {
  if (rows > QCR_MAX_ELEMS / 4) return 0;
  int bc = 4;
  for (int c = 64; c >= 4; c >>= 1) {
    if ((int64_t)c * rows > QCR_MAX_ELEMS) continue;
    bc = c;
    if ((cols + c - 1) / c >= min_wgs) break;
  }
  return bc;
}

template <int FMT>
hipError_t quantize_cols_int8(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                              int8_t* Qt, int64_t ldqt, float* scale, hipStream_t stream) {
  const int vec_in = ((uintptr_t)X % 16 == 0) && (ldx % 4 == 0);
  const int vec_out = ((uintptr_t)Qt % 16 == 0) && (ldqt % 16 == 0);
  if (qcols_takes_coop(X, rows, cols, ldx, Qt, ldqt, FMT)) {
    if (launch_qcols_coop<FMT>(X, rows, cols, ldx, Qt, ldqt, scale, stream) == hipSuccess) return hipSuccess;
    (void)hipGetLastError();   // the cooperative launch was refused: the paths below
  }
  if (qcols_takes_lines(X, rows, cols, ldx, Qt, ldqt, FMT)) {
    const int P = (int)((rows + QK_ROWS - 1) / QK_ROWS);
    const unsigned int grid = (unsigned int)(cols / QK_COLS * P);
    hipLaunchKernelGGL(qcols_init_kernel<FMT>, dim3((unsigned int)((cols + 255) / 256)), dim3(256), 0, stream,
                       scale, cols);
    hipLaunchKernelGGL(qcols_lines_max_kernel<FMT>, dim3(grid), dim3(QK_THREADS), 0, stream, X, rows, ldx, scale, P);
    hipLaunchKernelGGL(qcols_lines_quant_kernel, dim3(grid), dim3(QK_THREADS), 0, stream, X, rows, ldx, Qt, ldqt,
                       scale, P);
    return hipGetLastError();
  }
  int bc = rows > 0 ? qcols_band(rows, cols) : 0;
  // the test override can force the two-pass kernels (the bytes never
  // depend on the path)
  if (qcols_path_requested() == 1) bc = 0;
  if (bc > 0) {
    const dim3 grid((unsigned int)((cols + bc - 1) / bc)), block(QCR_THREADS);
    switch (bc) {
      case 64: hipLaunchKernelGGL((qcols_reg_kernel<64, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, vec_out); break;
      case 32: hipLaunchKernelGGL((qcols_reg_kernel<32, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, vec_out); break;
      case 16: hipLaunchKernelGGL((qcols_reg_kernel<16, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, vec_out); break;
      case 8: hipLaunchKernelGGL((qcols_reg_kernel<8, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, vec_out); break;
      default: hipLaunchKernelGGL((qcols_reg_kernel<4, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, vec_out); break;
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL(qcols_init_kernel<FMT>, dim3((unsigned int)((cols + 255) / 256)), dim3(256), 0,
                     stream, scale, cols);
  if (rows > 0) {
    hipLaunchKernelGGL(qcols_scale_kernel<FMT>,
                       dim3((unsigned int)((cols + QS_COLS - 1) / QS_COLS),
                            (unsigned int)((rows + QS_ROWS - 1) / QS_ROWS)),
                       dim3(256), 0, stream, X, rows, cols, ldx, scale, vec_in);
    hipLaunchKernelGGL(qcols_quant_kernel,
                       dim3((unsigned int)((cols + 63) / 64), (unsigned int)((rows + 63) / 64)),
                       dim3(256), 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, vec_out);
  }
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// int4 storage (FMT_INT4): values in [-7, 7], two per byte.  Element k of a
// line sits in byte 16*(k/32) + k%16 of the line, in the low nibble when
// k%32 < 16 and in the high nibble otherwise (4-bit two's complement); a line
// of length L takes 16*ceil(L/32) bytes, nibbles past L are 0.  The order
// lets the GEMM widen a 16-byte group to two int8 chunks with one AND each.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 pack_int4_group(const int (&q)[32]) {
  unsigned int w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned int v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const unsigned int lo = (unsigned int)q[4 * i + b] & 0xFu;
      const unsigned int hi = (unsigned int)q[16 + 4 * i + b] & 0xFu;
      v |= (lo | (hi << 4)) << (8 * b);
    }
    w[i] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Rows to int4: one wavefront per row; the absmax pass reads the row with
// coalesced loads, the pack pass gives each lane whole 32-element groups
// (a second read, mostly from cache).
template <int FMT>
__global__ void __launch_bounds__(256)
q4rows_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
              int8_t* __restrict__ Q, int64_t ldq, float* __restrict__ scale, int vec_in) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = X + r * ldx;
  float m = 0.0f;
  for (int64_t c = (int64_t)lane * 4; c < cols; c += 256) m = absmax4(m, load4(xr, c, cols, vec_in));
  m = wave_max_f32(m);
  const float s = scale_of_absmax_fmt<FMT>(m);
  const float inv = recip_rn(s);
  if (lane == 0) scale[r] = s;
  const int64_t groups = (cols + 31) / 32;
  for (int64_t g = lane; g < groups; g += 64) {
    int q[32];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 v = load4(xr, g * 32 + t * 4, cols, vec_in);   // zero past cols -> code 0
      q[4 * t + 0] = quantize1(v.x, inv);
      q[4 * t + 1] = quantize1(v.y, inv);
      q[4 * t + 2] = quantize1(v.z, inv);
      q[4 * t + 3] = quantize1(v.w, inv);
    }
    *reinterpret_cast<uint4*>(Q + r * ldq + g * 16) = pack_int4_group(q);
  }
}

// Columns to int4 (after the column scales are final): thread (column j,
// group g) reads its 32 rows (lanes take consecutive columns, so each row
// read is coalesced) and writes the 16 bytes of group g of row j of Qt.
template <int FMT>
__global__ void __launch_bounds__(256)
q4cols_pack_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                   int8_t* __restrict__ Qt, int64_t ldqt, const float* __restrict__ scale) {
  const int64_t j = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t g = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  const int64_t groups = (rows + 31) / 32;
  if (j >= cols || g >= groups) return;
  const float inv = recip_rn(scale[j]);
  int q[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int64_t k = g * 32 + t;
    q[t] = quantize1(k < rows ? X[k * ldx + j] : 0.0f, inv);
  }
  *reinterpret_cast<uint4*>(Qt + j * ldqt + g * 16) = pack_int4_group(q);
}

template <int FMT>
hipError_t quantize_rows_int4(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Q,
                              int64_t ldq, float* scale, hipStream_t stream) {
  const int vec_in = ((uintptr_t)X % 16 == 0) && (ldx % 4 == 0);
  hipLaunchKernelGGL(q4rows_kernel<FMT>, dim3((unsigned int)((rows + 3) / 4)), dim3(256), 0, stream, X,
                     rows, cols, ldx, Q, ldq, scale, vec_in);
  return hipGetLastError();
}

template <int FMT>
hipError_t quantize_cols_int4(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Qt,
                              int64_t ldqt, float* scale, hipStream_t stream) {
  const int vec_in = ((uintptr_t)X % 16 == 0) && (ldx % 4 == 0);
  // up to 8192 rows: the one-kernel band path, packing as it stores
  int bc = rows > 0 ? qcols_band(rows, cols) : 0;
  if (qcols_path_requested() == 1) bc = 0;
  if (bc > 0) {
    const dim3 grid((unsigned int)((cols + bc - 1) / bc)), block(QCR_THREADS);
    switch (bc) {
      case 64: hipLaunchKernelGGL((qcols_reg_kernel<64, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, 1); break;
      case 32: hipLaunchKernelGGL((qcols_reg_kernel<32, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, 1); break;
      case 16: hipLaunchKernelGGL((qcols_reg_kernel<16, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, 1); break;
      case 8: hipLaunchKernelGGL((qcols_reg_kernel<8, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, 1); break;
      default: hipLaunchKernelGGL((qcols_reg_kernel<4, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Qt, ldqt, scale, vec_in, 1); break;
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL(qcols_init_kernel<FMT>, dim3((unsigned int)((cols + 255) / 256)), dim3(256), 0,
                     stream, scale, cols);
  if (rows > 0) {
    hipLaunchKernelGGL(qcols_scale_kernel<FMT>,
                       dim3((unsigned int)((cols + QS_COLS - 1) / QS_COLS),
                            (unsigned int)((rows + QS_ROWS - 1) / QS_ROWS)),
                       dim3(256), 0, stream, X, rows, cols, ldx, scale, vec_in);
    hipLaunchKernelGGL(q4cols_pack_kernel<FMT>,
                       dim3((unsigned int)((cols + 63) / 64), (unsigned int)(((rows + 31) / 32 + 3) / 4)),
                       dim3(256), 0, stream, X, rows, cols, ldx, Qt, ldqt, scale);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Q,
                                int64_t ldq, float* scale, int fmt, hipStream_t stream) {
  switch (fmt) {
    case 0: return quantize_rows_int8<0>(X, rows, cols, ldx, Q, ldq, scale, stream);
    case FMT_POW2: return quantize_rows_int8<FMT_POW2>(X, rows, cols, ldx, Q, ldq, scale, stream);
    case FMT_INT4: return quantize_rows_int4<FMT_INT4>(X, rows, cols, ldx, Q, ldq, scale, stream);
    default: return quantize_rows_int4<FMT_INT4 | FMT_POW2>(X, rows, cols, ldx, Q, ldq, scale, stream);
  }
}

hipError_t launch_quantize_cols(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Qt,
                                int64_t ldqt, float* scale, int fmt, hipStream_t stream) {
  switch (fmt) {
    case 0: return quantize_cols_int8<0>(X, rows, cols, ldx, Qt, ldqt, scale, stream);
    case FMT_POW2: return quantize_cols_int8<FMT_POW2>(X, rows, cols, ldx, Qt, ldqt, scale, stream);
    case FMT_INT4: return quantize_cols_int4<FMT_INT4>(X, rows, cols, ldx, Qt, ldqt, scale, stream);
    default: return quantize_cols_int4<FMT_INT4 | FMT_POW2>(X, rows, cols, ldx, Qt, ldqt, scale, stream);
  }
}


// ---------------------------------------------------------------------------
// quantize_batch: independent int8 row / column passes in one launch of
// 1024-thread workgroups.  Each job owns a range of workgroup ids, rounded up
// to a multiple of 8 so that an id keeps its XCD (ids are dealt to the 8 XCDs
// round-robin) within the range; a workgroup finds its job by scanning the
// range starts (uniform across the workgroup) and runs the job's kernel body
// with its index inside the range.  Small passes, bound by latency alone,
// then share the chip instead of following one another.
// ---------------------------------------------------------------------------

template <int FMT>
__device__ __forceinline__ void run_qjob(const QJob& q, int bid, char* smem) {
  if constexpr ((FMT & FMT_INT4) != 0) {   // int4 jobs are column passes only
    switch (q.param) {
      case 64: qcols_reg_body<64, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
      case 32: qcols_reg_body<32, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
      case 16: qcols_reg_body<16, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
      case 8: qcols_reg_body<8, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
      default: qcols_reg_body<4, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
    }
    return;
  }
  if (q.kind == QK_ROWS_VEC) {
    const int64_t r = (int64_t)bid * (blockDim.x >> 6) + (threadIdx.x >> 6);   // a wave per row
    if (r >= q.rows) return;
    if (q.param == 8)
      qrows_wave_vec_body<8, FMT>(q.X, q.cols, q.ldx, q.Q, q.ldq, q.scale, r);
    else
      qrows_wave_vec_body<12, FMT>(q.X, q.cols, q.ldx, q.Q, q.ldq, q.scale, r);
  } else if (q.kind == QK_ROWS_WAVE) {
    switch (q.param) {
      case 1: qrows_wave_body<1, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid); break;
      case 2: qrows_wave_body<2, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid); break;
      case 3: qrows_wave_body<3, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid); break;
      default: qrows_wave_body<4, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid); break;
    }
  } else {
    switch (q.param) {
      case 64: qcols_reg_body<64, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
      case 32: qcols_reg_body<32, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
      case 16: qcols_reg_body<16, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
      case 8: qcols_reg_body<8, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
      default: qcols_reg_body<4, FMT>(q.X, q.rows, q.cols, q.ldx, q.Q, q.ldq, q.scale, q.vec_in, q.vec_out, bid, q.blocks, smem); break;
    }
  }
}

__global__ void __launch_bounds__(1024) quantize_batch_kernel(const QBatch b) {
  __shared__ __attribute__((aligned(16))) char smem[QCR_SMEM_BYTES];
  const int id = blockIdx.x;
  int j = 0;
  while (j + 1 < b.n && id >= b.job[j + 1].first) ++j;
  const QJob& q = b.job[j];
  const int bid = id - q.first;
  if (bid >= q.blocks) return;   // the padding of the job's range
  switch (q.fmt) {
    case 0: run_qjob<0>(q, bid, smem); break;
    case FMT_POW2: run_qjob<FMT_POW2>(q, bid, smem); break;
    case FMT_INT4: run_qjob<FMT_INT4>(q, bid, smem); break;
    default: run_qjob<FMT_INT4 | FMT_POW2>(q, bid, smem); break;
  }
}

bool plan_qjob(const float* X, int64_t rows, int64_t cols, int64_t ldx, int8_t* Q, int64_t ldq,
               float* scale, bool by_col, int fmt, QJob& q) {
  if (rows <= 0 || cols <= 0) return false;
  if ((fmt & FMT_INT4) && !by_col) return false;   // int4 rows: their own kernel
  q.X = X; q.Q = Q; q.scale = scale;
  q.rows = rows; q.cols = cols; q.ldx = ldx; q.ldq = ldq;
  q.fmt = fmt;
  q.vec_in = ((uintptr_t)X % 16 == 0) && (ldx % 4 == 0);
  if (!by_col) {
    q.vec_out = ((uintptr_t)Q % 4 == 0) && (ldq % 4 == 0);
    // The kernel's registers are the largest of its bodies': rows of up to
    // 1024 values run the general body (4 float4 per lane), longer ones up to
    // 3072 values only the aligned-row body (12 float4 per lane; the launch
    // stays within 64 registers, two workgroups per CU); other rows would cut
    // the workgroups a CU holds for every job of the launch.
    const int vpl = rows_wave_vpl(cols);
    if (vpl == 0) return false;
    if (vpl > 4) {
      if (vpl > 12 || !q.vec_in || !q.vec_out || (cols & 3) != 0) return false;
      q.kind = QK_ROWS_VEC;
    } else {
      q.kind = QK_ROWS_WAVE;
    }
    q.param = vpl;
    q.blocks = (int)((rows + 15) / 16);   // 16 waves per workgroup, a wave per row
    return true;
  }
  q.vec_out = ((uintptr_t)Q % 16 == 0) && (ldq % 16 == 0);
  const int bc = qcols_band(rows, cols, 64);
  if (bc == 0 || qcols_path_requested() == 1) return false;   // the multi-kernel path
  // the cooperative path needs a launch of its own; a pass the whole-line
  // kernels would take alone stays a band job here, where it overlaps the
  // batch's other passes (measured on a transformer layer's 24 input passes:
  // 309 us batched against 337 with five 8192x768 column passes launched
  // apart), unless a test forces the whole-line path
  if (qcols_takes_coop(X, rows, cols, ldx, Q, ldq, fmt) || qcols_path_requested() == 3) return false;
  q.kind = QK_COLS_REG; q.param = bc;
  q.blocks = (int)((cols + bc - 1) / bc);
  return true;
}

hipError_t launch_quantize_batch(QJob* jobs, int n, hipStream_t stream) {
  for (int i0 = 0; i0 < n; i0 += kQBatchMax) {
    QBatch b;
    b.n = n - i0 < kQBatchMax ? n - i0 : kQBatchMax;
    int64_t next = 0;
    for (int j = 0; j < b.n; ++j) {
      b.job[j] = jobs[i0 + j];
      b.job[j].first = (int)next;
      next += (b.job[j].blocks + 7) / 8 * 8;
    }
    if (next > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_batch_kernel, dim3((unsigned int)next), dim3(1024), 0, stream, b);
  }
  return hipGetLastError();
}

}  // namespace i8g
