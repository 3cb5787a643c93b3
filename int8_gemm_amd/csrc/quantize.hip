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
    const dim3 grid((unsigned int)((rows + 3) / 4)), block(256);
    if (cols <= 256)
      hipLaunchKernelGGL((qrows_wave_kernel<1, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 512)
      hipLaunchKernelGGL((qrows_wave_kernel<2, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 768)
      hipLaunchKernelGGL((qrows_wave_kernel<3, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 1024)
      hipLaunchKernelGGL((qrows_wave_kernel<4, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 2048)
      hipLaunchKernelGGL((qrows_wave_kernel<8, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else if (cols <= 3072)
      hipLaunchKernelGGL((qrows_wave_kernel<12, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
    else
      hipLaunchKernelGGL((qrows_wave_kernel<16, FMT>), grid, block, 0, stream, X, rows, cols, ldx, Q, ldq, scale, vec_in, vec_out);
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
#pragma unroll
  for (int p = 0; p < QCR_VPT; ++p) {
    const int64_t r = r_off + (int64_t)p * RPP;
    v[p] = r < rows ? load4(X + r * ldx, j0 + cg * 4, cols, vec_in) : make_float4(0.f, 0.f, 0.f, 0.f);
    m0 = fmaxf(m0, fabsf(v[p].x));
    m1 = fmaxf(m1, fabsf(v[p].y));
    m2 = fmaxf(m2, fabsf(v[p].z));
    m3 = fmaxf(m3, fabsf(v[p].w));
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
// rows <= 32768) while leaving at least 128 workgroups; 0 = use the
// multi-kernel path (more than 8192 rows).
static int qcols_band(int64_t rows, int64_t cols) {
  if (rows > QCR_MAX_ELEMS / 4) return 0;
  int bc = 4;
  for (int c = 64; c >= 4; c >>= 1) {
    if ((int64_t)c * rows > QCR_MAX_ELEMS) continue;
    bc = c;
    if ((cols + c - 1) / c >= 128) break;
  }
  return bc;
}

template <int FMT>
hipError_t quantize_cols_int8(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                              int8_t* Qt, int64_t ldqt, float* scale, hipStream_t stream) {
  const int vec_in = ((uintptr_t)X % 16 == 0) && (ldx % 4 == 0);
  const int vec_out = ((uintptr_t)Qt % 16 == 0) && (ldqt % 16 == 0);
  int bc = rows > 0 ? qcols_band(rows, cols) : 0;
  // the test override forces the two-pass kernels (the bytes never depend
  // on the path)
  if (qcols_two_pass_requested()) bc = 0;
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
  if (qcols_two_pass_requested()) bc = 0;
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
  if (q.kind == QK_ROWS_WAVE) {
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
    // only short rows (at most 1024 values, 4 float4 per lane): the kernel's
    // registers are the largest of its bodies', and longer rows would halve
    // the workgroups a CU holds for every job of the launch
    const int vpl = rows_wave_vpl(cols);
    if (vpl == 0 || vpl > 4) return false;
    q.kind = QK_ROWS_WAVE; q.param = vpl;
    q.blocks = (int)((rows + 15) / 16);   // 16 waves per workgroup, a wave per row
    return true;
  }
  q.vec_out = ((uintptr_t)Q % 16 == 0) && (ldq % 16 == 0);
  const int bc = qcols_band(rows, cols);
  if (bc == 0 || qcols_two_pass_requested()) return false;   // the multi-kernel path
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
