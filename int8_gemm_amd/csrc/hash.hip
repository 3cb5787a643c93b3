// hash.hip -- the output hash of an f32 matrix (standalone form).
//
// The DaisyChain-Train page "Verification -- why you can trust the
// numbers" compares outputs by hashing their raw bytes ("Layer 3: the
// kernel probe"); the function is this library's (include/int8_gemm.h):
//   S = sum_{i,j} c(j) * r(i) * bits(i,j) mod 2^64,
//   H = fmix64(S ^ fmix64(M*2^32 + N)).
// HBM-bound: each thread owns 4 consecutive columns and walks bands of rows
// (grid-stride, at most kHashMaxParts workgroups), summing r(i)*bits with
// one 32x32->64 multiply-add per element and multiplying by the column keys
// once; the workgroup that finishes last adds the workgroups' shares of S
// (integer sums: no order dependence) and writes H.
#include "i8g_device.h"
#include "i8g_launch.h"

namespace i8g {

constexpr int HASH_ROWS = 32;     // rows per band

__global__ void __launch_bounds__(256)
output_hash_kernel(const float* __restrict__ C, int64_t M, int64_t N, int64_t ldc, int vec_in,
                   unsigned long long* parts) {
  __shared__ unsigned long long red[4];
  const int tid = threadIdx.x;
  uint64_t part = 0;
  for (int64_t c = ((int64_t)blockIdx.x * 256 + tid) * 4; c < N; c += (int64_t)gridDim.x * 1024) {
    uint64_t t0 = 0, t1 = 0, t2 = 0, t3 = 0;
    for (int64_t r0 = (int64_t)blockIdx.y * HASH_ROWS; r0 < M; r0 += (int64_t)gridDim.y * HASH_ROWS) {
      const int64_t r1 = r0 + HASH_ROWS < M ? r0 + HASH_ROWS : M;
      int64_t r = r0;
      if (vec_in && c + 4 <= N) {
        // eight rows' loads in flight together (the terms are summed mod 2^64:
        // any order)
        for (; r + 8 <= r1; r += 8) {
          uint4 b[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) b[u] = *reinterpret_cast<const uint4*>(C + (r + u) * ldc + c);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint64_t rk = hash_row_key((uint32_t)(r + u));
            t0 += rk * b[u].x;
            t1 += rk * b[u].y;
            t2 += rk * b[u].z;
            t3 += rk * b[u].w;
          }
        }
      }
      for (; r < r1; ++r) {
        const float* row = C + r * ldc;
        const uint64_t rk = hash_row_key((uint32_t)r);
        if (vec_in && c + 4 <= N) {
          const uint4 b = *reinterpret_cast<const uint4*>(row + c);
          t0 += rk * b.x;
          t1 += rk * b.y;
          t2 += rk * b.z;
          t3 += rk * b.w;
        } else {
          t0 += rk * __float_as_uint(row[c]);
          if (c + 1 < N) t1 += rk * __float_as_uint(row[c + 1]);
          if (c + 2 < N) t2 += rk * __float_as_uint(row[c + 2]);
          if (c + 3 < N) t3 += rk * __float_as_uint(row[c + 3]);
        }
      }
    }
    part += hash_col_key((uint64_t)c) * t0;
    if (c + 1 < N) part += hash_col_key((uint64_t)c + 1) * t1;
    if (c + 2 < N) part += hash_col_key((uint64_t)c + 2) * t2;
    if (c + 3 < N) part += hash_col_key((uint64_t)c + 3) * t3;
  }
  // this workgroup's share; launch_hash_parts_finalize's kernel, launched
  // next, sums the shares (the workgroups end together: a last-arriving
  // workgroup would wait for its share's acknowledgement and a ticket)
  part = block_sum_u64<256>(part, red);
  if (tid == 0) parts[blockIdx.y * gridDim.x + blockIdx.x] = part;
}

__global__ void empty_hash_kernel(uint64_t* hash_out, uint64_t M, uint64_t N) {
  if (threadIdx.x == 0) *hash_out = hash_finalize(0, M, N);
}

hipError_t launch_output_hash(const float* C, int64_t M, int64_t N, int64_t ldc, uint64_t* hash,
                              void* workspace, hipStream_t stream) {
  if (M == 0 || N == 0) {
    hipLaunchKernelGGL(empty_hash_kernel, dim3(1), dim3(64), 0, stream, hash, (uint64_t)M, (uint64_t)N);
    return hipGetLastError();
  }
  unsigned long long* parts =
      reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(workspace) + kWsHeader);
  const int vec_in = ((uintptr_t)C % 16 == 0) && (ldc % 4 == 0);
  int64_t gx = (N + 1023) / 1024;
  if (gx > kHashMaxParts) gx = kHashMaxParts;   // columns beyond: grid-stride
  int64_t gy = (M + HASH_ROWS - 1) / HASH_ROWS;
  if (gx * gy > kHashMaxParts) gy = kHashMaxParts / gx;   // rows beyond: grid-stride
  const dim3 grid((unsigned int)gx, (unsigned int)gy);
  hipLaunchKernelGGL(output_hash_kernel, grid, dim3(256), 0, stream, C, M, N, ldc, vec_in, parts);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_hash_parts_finalize(parts, (int)(gx * gy), M, N, hash, stream);
}

}  // namespace i8g
