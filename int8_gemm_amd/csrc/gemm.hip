// gemm.hip -- block-scaled int8 GEMM on gfx950 matrix cores.
//
// C[i,j] = RN(RN(RN(acc)*s_row[i])*s_col[j]),  acc = sum_k QA[i,k]*QBt[j,k]
// (DaisyChain-Train page "Verification -- why you can trust the numbers",
// section "The verified INT8 units", steps 2 and 3).
//
// Design (CDNA4):
//  * v_mfma_i32_32x32x32_i8: one instruction multiplies a 32x32 int8 block
//    of A by a 32x32 int8 block of B^T into 32x32 int32 accumulators; the
//    products and the int32 sums are exact, so the result does not depend
//    on how K is blocked or split.
//  * A workgroup owns a BM x BN output tile; its waves own WTM x WTN
//    sub-tiles made of 32x32 MFMA blocks.  K advances in stages of 64
//    bytes, double-buffered in LDS: global -> registers -> LDS, one barrier
//    per stage.  Rows are 64 bytes in LDS; the 16-byte chunk index is XORed
//    with (row/2)%4 so that a wave's 16-byte reads of 32 rows at the same
//    chunk spread over all banks.
//  * Workgroup ids are remapped so that consecutive tiles of one L2 (one
//    XCD: workgroups are dealt to the 8 XCDs round-robin) are neighbours,
//    grouped GROUP_M tile-rows at a time to share A and B in that L2.
//  * Split-K: when there are too few tiles to fill 256 CUs, K is split; each
//    split writes its int32 partial tile to the workspace and takes a ticket;
//    the last split of a tile adds the others' partials (integer, exact in
//    any order) and runs the epilogue.
//  * The epilogue converts, scales (row scale, then column scale, separate
//    roundings), applies ReLU as a select (so never -0), stores f32, and
//    accumulates the output hash S = sum c(j)*r(i)*bits(i,j) mod 2^64.
#include <cmath>
#include <cstdlib>

#include "i8g_device.h"
#include "i8g_launch.h"

namespace i8g {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BK = 64;        // bytes of K per LDS stage
constexpr int GROUP_M = 8;    // tile-rows per L2 group

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

// Zero the bytes at positions >= nvalid (1..15) of a 16-byte vector.
__device__ __forceinline__ v4i mask_tail(v4i x, int nvalid) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int lo = w * 4;
    unsigned int m;
    if (nvalid >= lo + 4) m = 0xFFFFFFFFu;
    else if (nvalid <= lo) m = 0u;
    else m = (1u << (8 * (nvalid - lo))) - 1u;
    x[w] = (int)((unsigned int)x[w] & m);
  }
  return x;
}

// Load one 16-byte chunk of a K-contiguous int8 row; zero beyond K.
__device__ __forceinline__ v4i load_chunk(const int8_t* rowp, int k, int K) {
  if (k + 16 <= K) return *reinterpret_cast<const v4i*>(rowp + k);
  v4i z = {0, 0, 0, 0};
  if (k >= K) return z;
  return mask_tail(*reinterpret_cast<const v4i*>(rowp + k), K - k);
}

// Map the linear workgroup id to (tile_m, tile_n, split).
__device__ __forceinline__ void map_workgroup(int wg, int total, int tiles_m, int tiles_n,
                                              int splits, int& tm, int& tn, int& split) {
  // Undo the round-robin dealing over 8 XCDs: XCD x receives ids x, x+8, ...
  const int xcd = wg & 7, idx = wg >> 3;
  const int per = total >> 3, rem = total & 7;
  const int w = xcd * per + (xcd < rem ? xcd : rem) + idx;
  split = w % splits;
  const int tile = w / splits;
  const int group_size = GROUP_M * tiles_n;
  const int group = tile / group_size;
  const int first_m = group * GROUP_M;
  const int gm = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
  const int in_group = tile - group * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
gemm_i8_kernel(const GemmParams p) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CPR = BK / 16;                       // 16-byte chunks per row
  constexpr int A_LD = BM * CPR / NT, B_LD = BN * CPR / NT;
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "stage not divisible");
  constexpr int STAGE = (BM + BN) * BK;
  constexpr int EPI_BYTES = (2 * BM + BN) * 4 + 4 * 16;
  constexpr int SMEM = (2 * STAGE > EPI_BYTES) ? 2 * STAGE : EPI_BYTES;
  __shared__ __attribute__((aligned(16))) int8_t smem[SMEM];
  __shared__ int s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  int tm, tn, split;
  map_workgroup(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.splits, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;

  const int k_begin = split * p.k_per_split;
  int k_end = k_begin + p.k_per_split;
  if (k_end > K) k_end = K;
  const int nk = (k_end - k_begin + BK - 1) / BK;

  // Per-thread global load sources (rows clamped into range: rows past M or
  // N are computed on duplicated data and never stored).
  const int8_t* a_src[A_LD];
  const int8_t* b_src[B_LD];
  int a_off[A_LD], b_off[B_LD], a_ck[A_LD], b_ck[B_LD];
#pragma unroll
  for (int q = 0; q < A_LD; ++q) {
    int c = tid + q * NT, row = c / CPR, ck = c % CPR;
    int gr = m0 + row; gr = gr < M ? gr : M - 1;
    a_src[q] = p.A + (int64_t)gr * p.lda;
    a_ck[q] = ck * 16;
    a_off[q] = row * BK + (swz(row, ck) << 4);
  }
#pragma unroll
  for (int q = 0; q < B_LD; ++q) {
    int c = tid + q * NT, row = c / CPR, ck = c % CPR;
    int gr = n0 + row; gr = gr < N ? gr : N - 1;
    b_src[q] = p.B + (int64_t)gr * p.ldb;
    b_ck[q] = ck * 16;
    b_off[q] = BM * BK + row * BK + (swz(row, ck) << 4);
  }

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  v4i ra[A_LD], rb[B_LD];
  if (nk > 0) {
#pragma unroll
    for (int q = 0; q < A_LD; ++q) ra[q] = load_chunk(a_src[q], k_begin + a_ck[q], k_end);
#pragma unroll
    for (int q = 0; q < B_LD; ++q) rb[q] = load_chunk(b_src[q], k_begin + b_ck[q], k_end);
#pragma unroll
    for (int q = 0; q < A_LD; ++q) *reinterpret_cast<v4i*>(smem + a_off[q]) = ra[q];
#pragma unroll
    for (int q = 0; q < B_LD; ++q) *reinterpret_cast<v4i*>(smem + b_off[q]) = rb[q];
  }
  __syncthreads();

  // LDS read offsets of this lane's MFMA operands (stage-relative).
  const int lrow = lane & 31, lhalf = lane >> 5;

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = (kt & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      const int kn = k_begin + (kt + 1) * BK;
#pragma unroll
      for (int q = 0; q < A_LD; ++q) ra[q] = load_chunk(a_src[q], kn + a_ck[q], k_end);
#pragma unroll
      for (int q = 0; q < B_LD; ++q) rb[q] = load_chunk(b_src[q], kn + b_ck[q], k_end);
    }
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      const int ck = s * 2 + lhalf;
      v4i af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        int row = wm * WTM + i * 32 + lrow;
        af[i] = *reinterpret_cast<const v4i*>(smem + cur + row * BK + (swz(row, ck) << 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int row = wn * WTN + j * 32 + lrow;
        bf[j] = *reinterpret_cast<const v4i*>(smem + cur + BM * BK + row * BK + (swz(row, ck) << 4));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      const int nxt = STAGE - cur;
#pragma unroll
      for (int q = 0; q < A_LD; ++q) *reinterpret_cast<v4i*>(smem + nxt + a_off[q]) = ra[q];
#pragma unroll
      for (int q = 0; q < B_LD; ++q) *reinterpret_cast<v4i*>(smem + nxt + b_off[q]) = rb[q];
    }
    __syncthreads();
  }

  // ---- split-K: exchange int32 partial tiles through the workspace ----
  const int tile = tm * p.tiles_n + tn;
  if (p.splits > 1) {
    v4i* mine = reinterpret_cast<v4i*>(p.partials) +
                ((int64_t)tile * p.splits + split) * (BM * BN / 4);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v4i v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          mine[((i * FN + j) * 4 + q) * NT + tid] = v;
        }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      unsigned int t = __hip_atomic_fetch_add(p.tickets + tile, 1u, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
      s_flag = (t == (unsigned int)(p.splits - 1));
      if (s_flag) __hip_atomic_store(p.tickets + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_flag) return;
    __threadfence();
    for (int o = 0; o < p.splits; ++o) {
      if (o == split) continue;
      const v4i* other = reinterpret_cast<const v4i*>(p.partials) +
                         ((int64_t)tile * p.splits + o) * (BM * BN / 4);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v4i v = __builtin_nontemporal_load(other + ((i * FN + j) * 4 + q) * NT + tid);
            acc[i][j][4 * q] += v[0];
            acc[i][j][4 * q + 1] += v[1];
            acc[i][j][4 * q + 2] += v[2];
            acc[i][j][4 * q + 3] += v[3];
          }
    }
  }

  // ---- epilogue: scales, keys and the hash ----
  float* s_sr = reinterpret_cast<float*>(smem);
  unsigned int* s_rk = reinterpret_cast<unsigned int*>(smem + BM * 4);
  float* s_sc = reinterpret_cast<float*>(smem + 2 * BM * 4);
  unsigned long long* s_red = reinterpret_cast<unsigned long long*>(smem + (2 * BM + BN) * 4);
  for (int r = tid; r < BM; r += NT) {
    int gr = m0 + r;
    s_sr[r] = gr < M ? p.s_row[gr] : 0.0f;
    s_rk[r] = hash_row_key((unsigned int)gr);
  }
  for (int c = tid; c < BN; c += NT) {
    int gc = n0 + c;
    s_sc[c] = gc < N ? p.s_col[gc] : 0.0f;
  }
  __syncthreads();

  const bool relu = p.relu != 0;
  const bool do_hash = p.do_hash != 0;
  uint64_t hsum = 0;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int lc = wn * WTN + j * 32 + lrow;
    const int gc = n0 + lc;
    const bool col_ok = gc < N;
    const float sc = s_sc[lc];
    uint64_t tcol = 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = wm * WTM + i * 32 + (v >> 2) * 8 + lhalf * 4 + (v & 3);
        const int gr = m0 + lr;
        if (col_ok && gr < M) {
          float y = epilogue1(acc[i][j][v], s_sr[lr], sc);
          if (relu) y = relu_pos0(y);
          p.C[(int64_t)gr * p.ldc + gc] = y;
          tcol += (uint64_t)s_rk[lr] * (uint64_t)__float_as_uint(y);
        }
      }
    }
    if (do_hash && col_ok) hsum += hash_col_key((uint64_t)gc) * tcol;
  }
  if (do_hash) {
    hsum = wave_sum_u64(hsum);
    if (lane == 0) s_red[wave] = hsum;
    __syncthreads();
    if (tid == 0) {
      uint64_t part = 0;
      for (int w = 0; w < NT / 64; ++w) part += s_red[w];
      hash_commit(p.ws, part, (unsigned int)(p.tiles_m * p.tiles_n), (uint64_t)M, (uint64_t)N,
                  p.hash_out, nullptr);
    }
  }
}

// ---------------------------------------------------------------------------
// host side: plan and launch
// ---------------------------------------------------------------------------
struct TileCfg {
  int bm, bn, nt;
};
static const TileCfg kCfgs[] = {{256, 256, 256}, {256, 128, 256}, {128, 128, 256}};

// Optional overrides for tests (the output never depends on the plan):
// I8G_FORCE_TILE = 0 (256x256), 1 (256x128) or 2 (128x128); I8G_FORCE_SPLITS
// = number of K splits (clamped so that no split is empty).
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan best{};
  if (M <= 0 || N <= 0) return best;
  const int force_tile = env_int("I8G_FORCE_TILE", -1);
  const int force_splits = env_int("I8G_FORCE_SPLITS", 0);
  const double cus = 256.0;
  double best_cost = 1e300;
  for (int c = 0; c < 3; ++c) {
    if (force_tile >= 0 ? c != force_tile : c == 0) continue;   // 256x256 only on request
    const TileCfg& t = kCfgs[c];
    const int64_t tm = (M + t.bm - 1) / t.bm, tn = (N + t.bn - 1) / t.bn;
    const int64_t tiles = tm * tn;
    // slots: workgroups resident per CU (256x256 uses more registers)
    const double slots = cus * (t.bm * t.bn >= 65536 ? 1.0 : 2.0);
    // relative MAC rate of one workgroup of this tile shape
    const double eff = (t.bm * t.bn >= 65536) ? 1.0 : (t.bm * t.bn >= 32768 ? 0.5 : 0.25);
    const int64_t kstages = (K + BK - 1) / BK;
    for (int s = 1; s <= 16; ++s) {
      if (force_splits > 0) {
        if (s != (force_splits < kstages ? force_splits : (int)kstages)) continue;
      } else {
        if (s > 1 && kstages / s < 8) break;         // keep >= 8 stages per split
        if (s > 1 && tiles * s > 4 * (int64_t)slots) break;
      }
      const int64_t kps_st = (kstages + s - 1) / s;
      const int s_eff = (int)((kstages + kps_st - 1) / kps_st);   // no empty split
      const double waves = std::ceil((double)(tiles * s_eff) / slots);
      double cost = waves * (double)kps_st / eff;
      cost += (s_eff > 1 ? 0.05 * cost : 0.0);       // partial exchange
      cost += (double)tiles * t.bm * t.bn * 1e-9;    // prefer less padding
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        best.cfg = c;
        best.bm = t.bm;
        best.bn = t.bn;
        best.tiles_m = (int)tm;
        best.tiles_n = (int)tn;
        best.splits = s_eff;
        best.k_per_split = (int)(kps_st * BK);
      }
    }
  }
  if (best.bm == 0) {   // unreachable: the 128x128, one-split plan is always a candidate
    best.cfg = 2; best.bm = best.bn = 128;
    best.tiles_m = (int)((M + 127) / 128); best.tiles_n = (int)((N + 127) / 128);
    best.splits = 1; best.k_per_split = (int)((K + BK - 1) / BK * BK);
  }
  int64_t tiles = (int64_t)best.tiles_m * best.tiles_n;
  size_t bytes = sizeof(WsHeader);
  bytes += ((size_t)tiles * 4 + 255) / 256 * 256;            // tickets
  best.tickets_offset = sizeof(WsHeader);
  best.partials_offset = bytes;
  if (best.splits > 1) bytes += (size_t)tiles * best.splits * best.bm * best.bn * 4;
  best.workspace_bytes = bytes;
  return best;
}

hipError_t launch_gemm(const GemmParams& p, const GemmPlan& plan, hipStream_t stream) {
  const unsigned int grid = (unsigned int)((int64_t)plan.tiles_m * plan.tiles_n * plan.splits);
  switch (plan.cfg) {
    case 0:
      hipLaunchKernelGGL((gemm_i8_kernel<256, 256, 2, 2>), dim3(grid), dim3(256), 0, stream, p);
      break;
    case 1:
      hipLaunchKernelGGL((gemm_i8_kernel<256, 128, 2, 2>), dim3(grid), dim3(256), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((gemm_i8_kernel<128, 128, 2, 2>), dim3(grid), dim3(256), 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace i8g
