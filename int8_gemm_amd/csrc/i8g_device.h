// i8g_device.h -- device-side arithmetic shared by the library's kernels.
//
// Every float operation of the method is written here once, as a separate
// IEEE binary32 operation rounded to nearest-even.  The library is compiled
// with -ffp-contract=off and the helpers carry `#pragma clang fp
// contract(off)`, so no multiply is ever fused with the following add (the
// DaisyChain-Train page "Verification -- why you can trust the numbers",
// section "The verified INT8 units", step 3 rounds after each multiply; its
// section "Hardware ground truth (RDNA2 ISA audit)" discusses the fused
// quantizer, which gives different int8 next to |x*inv| = 0.5).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8g {

// A pointer the caller knows to be the same in every lane, in scalar
// registers (a buffer resource built from it then needs no per-lane loop).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// RN(1e-8): the scale floor of step 1, bit pattern 0x322BCC77.
__device__ __forceinline__ float scale_floor() { return __uint_as_float(0x322BCC77u); }

__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

__device__ __forceinline__ float add_rn(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// Correctly rounded division: the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt, which makes '/' the IEEE
// division (never the approximate reciprocal instruction).
__device__ __forceinline__ float div_rn(float a, float b) {
#pragma clang fp contract(off)
  return a / b;
}

// Step 1: s = max(RN(a/127), RN(1e-8)).  a >= 0 and finite, so the larger
// of the two is well defined; fmaxf on two non-NaN, non-zero-tie values is
// exact.
__device__ __forceinline__ float scale_of_absmax(float a) {
  float s = div_rn(a, 127.0f);
  float f = scale_floor();
  return s > f ? s : f;
}

__device__ __forceinline__ float recip_rn(float s) { return div_rn(1.0f, s); }

// Storage formats of the quantize passes (the presk page, section "Integer
// weights": int8 or int4 values, absmax or power-of-two scales).
constexpr int FMT_POW2 = 1;   // the scale rounded up to a power of two
constexpr int FMT_INT4 = 2;   // values in [-7, 7] (qmax = 2^(4-1) - 1), two per byte

// Smallest power of two >= s for a positive normal s (the exponent field
// cannot overflow: s <= FLT_MAX / 7 < 2^126).
__device__ __forceinline__ float pow2_ceil(float s) {
  uint32_t b = __float_as_uint(s);
  if (b & 0x007FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;
  return __uint_as_float(b);
}

// s = max(RN(a/qmax), RN(1e-8)), then rounded up to a power of two for
// FMT_POW2; qmax = 127 for int8, 7 for int4.
template <int FMT>
__device__ __forceinline__ float scale_of_absmax_fmt(float a) {
  float s = div_rn(a, (FMT & FMT_INT4) ? 7.0f : 127.0f);
  const float f = scale_floor();
  s = s > f ? s : f;
  if (FMT & FMT_POW2) s = pow2_ceil(s);
  return s;
}

// q = floor(RN(RN(x*inv) + 0.5)), in [-127, 127] for |x| <= the line max.
__device__ __forceinline__ int quantize1(float x, float inv) {
  float t = mul_rn(x, inv);
  float u = add_rn(t, 0.5f);
  return (int)floorf(u);
}

// Step 3: out = RN(RN(RN(acc)*s_row)*s_col); int->float conversion rounds
// to nearest-even (the MODE register's default, which HIP kernels run with).
__device__ __forceinline__ float epilogue1(int acc, float s_row, float s_col) {
  float y = (float)acc;
  y = mul_rn(y, s_row);
  return mul_rn(y, s_col);
}

// ReLU that never produces -0: out > 0 ? out : +0.
__device__ __forceinline__ float relu_pos0(float y) { return y > 0.0f ? y : 0.0f; }

// ---------------------------------------------------------------------------
// Output hash (see include/int8_gemm.h, output_hash):
//   S = sum_{i,j} c(j) * r(i) * bits(i,j) mod 2^64,
//   H = fmix64(S ^ fmix64(M*2^32 + N)).
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ uint64_t fmix64(uint64_t k) {
  k ^= k >> 33;
  k *= 0xFF51AFD7ED558CCDull;
  k ^= k >> 33;
  k *= 0xC4CEB9FE1A85EC53ull;
  k ^= k >> 33;
  return k;
}

__host__ __device__ __forceinline__ uint32_t mix31(uint32_t x) {
  const uint32_t m = 0x7FFFFFFFu;
  x &= m;
  x ^= x >> 16;
  x = (x * 0x3B9C5A1Du) & m;
  x ^= x >> 13;
  x = (x * 0x2F6E8B35u) & m;
  x ^= x >> 16;
  return x;
}

__host__ __device__ __forceinline__ uint32_t hash_row_key(uint32_t i) { return (mix31(i) << 1) | 1u; }

__host__ __device__ __forceinline__ uint64_t hash_col_key(uint64_t j) {
  return fmix64(j + 0x9E3779B97F4A7C15ull) | 1ull;
}

__host__ __device__ __forceinline__ uint64_t hash_finalize(uint64_t s, uint64_t m, uint64_t n) {
  return fmix64(s ^ fmix64((m << 32) | n));
}

// Sum of a 64-bit value over the 64 lanes of a wavefront (mod 2^64).
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Sum of a 64-bit value over a workgroup of NT threads (mod 2^64); the
// result is valid in thread 0.  `red` is LDS scratch of NT/64 words.
template <int NT>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, unsigned long long* red) {
  v = wave_sum_u64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint64_t t = 0;
  if (threadIdx.x == 0)
    for (int w = 0; w < NT / 64; ++w) t += red[w];
  return t;
}

// Ends a grid-wide sum of per-workgroup hash shares without a second kernel
// and without agent-scope release/acquire fences (on this GPU those write
// back / invalidate the whole L2 of the XCD).  Every workgroup stores its
// share with an agent-scope atomic store (written through to the coherence
// point), waits for that store to be acknowledged (s_waitcnt vmcnt(0); a
// workgroup-scope fence alone emits no wait for global stores here), then
// takes a ticket with an agent-scope atomic add.  The workgroup that draws the last ticket knows
// every other share was complete before its ticket was taken; it reads the
// shares with agent-scope atomic loads, writes H, and returns the ticket to
// zero for the next call.  `ticket` must be zero when the grid starts.
// Call from all NT threads of every workgroup; `part` is valid in thread 0.
template <int NT>
__device__ __forceinline__ void hash_share_and_finalize(uint64_t part, unsigned long long* shares,
                                                        unsigned int* ticket, int n_shares,
                                                        int my_share, uint64_t M, uint64_t N,
                                                        uint64_t* hash_out,
                                                        unsigned long long* red, int* flag) {
  if (threadIdx.x == 0) {
    __hip_atomic_store(shares + my_share, (unsigned long long)part, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // keeps the compiler's order
    __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0): the store is acknowledged
    const unsigned int t =
        __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (t == (unsigned int)(n_shares - 1));
  }
  __syncthreads();
  if (*flag) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    uint64_t s = 0;
    for (int i = threadIdx.x; i < n_shares; i += NT)
      s += __hip_atomic_load(shares + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s = block_sum_u64<NT>(s, red);
    if (threadIdx.x == 0) {
      *hash_out = hash_finalize(s, M, N);
      __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace i8g
