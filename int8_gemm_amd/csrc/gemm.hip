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
//    with (row/4)%4 so that a wave's 16-byte reads of 32 rows at the same
//    chunk spread over all 64 banks.
//  * Workgroup ids are remapped so that consecutive tiles of one L2 (one
//    XCD: workgroups are dealt to the 8 XCDs round-robin) are neighbours,
//    grouped GROUP_M tile-rows at a time to share A and B in that L2.
//  * Split-K: when there are too few tiles to fill 256 CUs, K is split; each
//    split writes its int32 partial tile to the workspace and a second
//    kernel adds the splits (integer, exact in any order) and runs the
//    epilogue.  No kernel synchronizes with another workgroup: agent-scope
//    release/acquire would write back and invalidate the XCD's L2.
//  * The epilogue converts, scales (row scale, then column scale, separate
//    roundings), applies ReLU as a select (so never -0), stores f32, and
//    computes the tile's share of the output hash S = sum c(j)*r(i)*bits(i,j)
//    mod 2^64; the workgroup that finishes last adds the shares (mod 2^64,
//    any order) and writes H (see hash_share_and_finalize).
#include <cmath>
#include <cstdlib>

#include "i8g_device.h"
#include "i8g_launch.h"

namespace i8g {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BK = 64;        // bytes of K per LDS stage
constexpr int GROUP_M = 8;    // tile-rows per L2 group

// LDS rows of a stage are 64 bytes (four 16-byte chunks).  gfx950's LDS has
// 64 banks and serves a 16-byte read for 16 lanes per cycle, so the 16 rows
// a quarter-wave reads at one chunk position must cover all 16 distinct
// 16-byte bank groups: rows r..r+15 sit at groups 4*(r%4) + chunk', and XOR
// with (r/4)%4 makes chunk' distinct among the rows that share r%4.
// (Measured: 214 B/clk per CU conflict-free, 123 with (r/2)%4, 62 without.)
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

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

// ---------------------------------------------------------------------------
// Main loop with direct global->LDS loads (global_load_lds_dwordx4) and a
// ring of STAGES LDS buffers: the loads for stage kt+STAGES-1 are in flight
// while stage kt is multiplied, without staging registers.  Each load
// instruction fills 1 KiB of LDS (64 lanes x 16 bytes, lane l at byte 16*l),
// i.e. 16 rows of 64 bytes; the swizzle is applied on the global side: lane
// l of a block fetches logical chunk swz(row, l%4) of its row, so the
// physical layout is the same XOR-swizzled one the fragment reads expect
// (swz is an involution in the chunk index).
// A K tail shorter than one stage goes through registers (masked).
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
  // vmcnt[3:0] | expcnt[6:4] = 7 | lgkmcnt[11:8] = 15 | vmcnt[5:4] at [15:14]).
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | (((N >> 4) & 3) << 14));
}

// One direct global->LDS load of 16 bytes per lane: lane l's bytes land at
// lds + 16*l (lds must be the same for the whole wave).
__device__ __forceinline__ void dma_load16(const int8_t* g, int8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// Workgroup barrier without a memory fence (the fence of __syncthreads()
// would wait for every outstanding global load, including prefetches).
// Callers make the LDS data visible first: s_waitcnt on the counter that
// tracks it (vmcnt for direct-to-LDS loads, lgkmcnt for ds_write).
__device__ __forceinline__ void barrier_nofence() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Output rows are written once by this kernel.  A large output (more than
// half of the 256 MB last-level cache) is streamed past the caches
// (nontemporal); a smaller one is stored normally so that a following
// kernel (e.g. the next layer's quantize pass) can still find it in cache.
__device__ __forceinline__ void store_out4(float* dst, float a, float b, float c, float d,
                                           bool stream) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f v = {a, b, c, d};
  if (stream) __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(dst));
  else *reinterpret_cast<v4f*>(dst) = v;
}

// Epilogue through LDS.  Each wave parks its raw int32 accumulators 32 rows
// at a time in a private LDS slab (MFMA layout written: lane = one column,
// 16 rows; row stride WTN+8 words, so the two half-waves' rows land on
// disjoint banks), reads the slab back row-major, 4 consecutive columns per
// lane, computes y = RN(RN(RN(acc) * s_row) * s_col), the ReLU select and
// the hash terms r(i)*bits(y) (summed per column), and writes 16 bytes per
// lane per row, so the lanes cover whole row segments.  The workgroup's
// share of S is published last (hash_share_and_finalize).  With split-K the
// raw int32 sums are stored instead, to the split's plane.
template <int BM, int BN, int WAVES_M, int WAVES_N, int FM, int FN>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p, v16i (&acc)[FM][FN], int8_t* smem,
                                             int tm, int tn, int split) {
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int STRIDE = WTN + 8;                    // words per slab row
  constexpr int SLAB = 32 * STRIDE;                  // words per wave
  constexpr int LPR = WTN / 4;                       // lanes per row when reading back
  constexpr int RPI = 64 / LPR;                      // rows per read instruction
  constexpr int NWAVES = WAVES_M * WAVES_N, NT = NWAVES * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int M = p.M, N = p.N;
  const int col0 = tn * BN + wn * WTN;
  const bool raw = p.splits > 1;
  const bool relu = p.relu != 0;
  const bool stream = p.stream_out != 0;

  int* slab = reinterpret_cast<int*>(smem) + wave * SLAB;
  float* s_sr = reinterpret_cast<float*>(smem) + NWAVES * SLAB;
  unsigned int* s_rk = reinterpret_cast<unsigned int*>(s_sr + BM);
  unsigned long long* s_red = reinterpret_cast<unsigned long long*>(s_rk + BM);   // NWAVES + 1 words
  // row scales and row keys of the tile (zero beyond M: such rows add nothing)
  for (int r = tid; r < BM; r += NT) {
    const int gr = tm * BM + r;
    s_sr[r] = gr < M ? p.s_row[gr] : 0.0f;
    s_rk[r] = gr < M ? hash_row_key((unsigned int)gr) : 0u;
  }
  // this lane's four columns in the row-major read-back
  const int rr0 = lane / LPR, cc = (lane % LPR) * 4;
  const int gc0 = col0 + cc;
  float sc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sc[e] = gc0 + e < N ? p.s_col[gc0 + e] : 0.0f;
  __syncthreads();

  // slab i of this wave: park the accumulators, then visit its rows
  // row-major; the slab is private to the wave and LDS operations of a wave
  // complete in order, so no barrier is needed between the two
  auto park = [&](int i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int srow = (v >> 2) * 8 + lhalf * 4 + (v & 3);
#pragma unroll
      for (int j = 0; j < FN; ++j) slab[srow * STRIDE + j * 32 + lrow] = acc[i][j][v];
    }
  };

  uint64_t tcol[4] = {0, 0, 0, 0};
  const int64_t ld = raw ? (int64_t)N : p.ldc;
  const bool vec = raw ? (N % 4 == 0) : ((p.ldc % 4 == 0) && (((uintptr_t)p.C & 15) == 0));
  int* part_base = raw ? p.partials + (int64_t)split * M * N : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    park(i);
#pragma unroll
    for (int t = 0; t < 32 / RPI; ++t) {
      const int srow = t * RPI + rr0;
      const int4 a = *reinterpret_cast<const int4*>(slab + srow * STRIDE + cc);
      const int lr = wm * WTM + i * 32 + srow;
      const int gr = tm * BM + lr;
      const int av[4] = {a.x, a.y, a.z, a.w};
      if (raw) {
        if (gr >= M) continue;
        int* dst = part_base + (int64_t)gr * ld + gc0;
        if (vec && gc0 + 4 <= N) {
          *reinterpret_cast<int4*>(dst) = a;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gc0 + e < N) dst[e] = av[e];
        }
      } else {
        const float sr = s_sr[lr];
        const uint64_t rk = s_rk[lr];
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = epilogue1(av[e], sr, sc[e]);
          if (relu) y[e] = relu_pos0(y[e]);
          tcol[e] += rk * (uint64_t)__float_as_uint(y[e]);
        }
        if (gr >= M) continue;
        float* dst = p.C + (int64_t)gr * ld + gc0;
        if (vec && gc0 + 4 <= N) {
          store_out4(dst, y[0], y[1], y[2], y[3], stream);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gc0 + e < N) dst[e] = y[e];
        }
      }
    }
  }
  if (!raw && p.do_hash) {
    uint64_t hsum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (gc0 + e < N) hsum += hash_col_key((uint64_t)(gc0 + e)) * tcol[e];
    const uint64_t part = block_sum_u64<NT>(hsum, s_red);
    hash_share_and_finalize<NT>(part, p.hash_parts, p.ticket, p.n_shares, tm * p.tiles_n + tn,
                                (uint64_t)M, (uint64_t)N, p.hash_out, s_red,
                                reinterpret_cast<int*>(s_red + NWAVES));
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
gemm_i8_dma_kernel(const GemmParams p) {
  constexpr int NWAVES = WAVES_M * WAVES_N, NT = NWAVES * 64;
  static_assert(NWAVES == 4 || NWAVES == 8, "four or eight waves");
  static_assert(STAGES >= 3, "the ring needs at least three stages");
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * BK, STAGE = (BM + BN) * BK;
  constexpr int A_INS = BM / (16 * NWAVES), B_INS = BN / (16 * NWAVES);   // 16-row blocks per wave
  static_assert(A_INS * 16 * NWAVES == BM && B_INS * 16 * NWAVES == BN, "rows per stage");
  constexpr int LPS = A_INS + B_INS;                   // load instructions per wave per stage
  constexpr int EPI_BYTES = NWAVES * 32 * (WTN + 8) * 4 + 2 * BM * 4 + 128;
  constexpr int SMEM = STAGES * STAGE > EPI_BYTES ? STAGES * STAGE : EPI_BYTES;
  __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  int tm, tn, split;
  map_workgroup(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.splits, tm, tn, split);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int k_begin = split * p.k_per_split;
  int k_end = k_begin + p.k_per_split;
  if (k_end > K) k_end = K;
  const int klen = k_end > k_begin ? k_end - k_begin : 0;
  const int nfull = klen / BK;
  const bool tail = (klen % BK) != 0;

  // global sources of this lane's 16-byte chunks (rows clamped into range)
  const int r_in = lane >> 2, slot = lane & 3;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // wave id in a scalar register
  const int8_t* ga[A_INS];
  const int8_t* gb[B_INS];
#pragma unroll
  for (int q = 0; q < A_INS; ++q) {
    const int row = (q * NWAVES + wave) * 16 + r_in;
    int gr = m0 + row; gr = gr < M ? gr : M - 1;
    ga[q] = p.A + (int64_t)gr * p.lda + k_begin + (swz(row, slot) << 4);
  }
#pragma unroll
  for (int q = 0; q < B_INS; ++q) {
    const int row = (q * NWAVES + wave) * 16 + r_in;
    int gr = n0 + row; gr = gr < N ? gr : N - 1;
    gb[q] = p.B + (int64_t)gr * p.ldb + k_begin + (swz(row, slot) << 4);
  }
  auto issue = [&](int buf, int kt) {
    int8_t* base = smem + buf * STAGE + wave_s * 1024;
#pragma unroll
    for (int q = 0; q < A_INS; ++q) dma_load16(ga[q] + kt * BK, base + q * NWAVES * 1024);
#pragma unroll
    for (int q = 0; q < B_INS; ++q) dma_load16(gb[q] + kt * BK, base + A_BYTES + q * NWAVES * 1024);
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  const int lrow = lane & 31, lhalf = lane >> 5;
  // per-lane LDS offsets (stage-relative) of the fragments of k-steps 0 and 1
  int offa[2][FM], offb[2][FN];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * WTM + i * 32 + lrow;
      offa[s][i] = row * BK + (swz(row, s * 2 + lhalf) << 4);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * WTN + j * 32 + lrow;
      offb[s][j] = A_BYTES + row * BK + (swz(row, s * 2 + lhalf) << 4);
    }
  }
  auto load_frags = [&](int buf, int s, v4i (&fa)[FM], v4i (&fb)[FN]) {
    const int8_t* sb = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const v4i*>(sb + offa[s][i]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const v4i*>(sb + offb[s][j]);
  };
  auto mfmas = [&](const v4i (&fa)[FM], const v4i (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // Ask the scheduler to alternate the FM+FN fragment reads of the next
  // k-step with this k-step's MFMAs (1 MFMA, 1 read, ...), so the reads stay
  // queued behind MFMA work.  Measured against issuing all reads first: the
  // alternation is 7-10% faster.
  auto interleave = [&]() {
#pragma unroll
    for (int t = 0; t < FM + FN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
  };

  v4i fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  if (nfull > 0) {
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < nfull) issue(st, st);
    if (nfull >= STAGES - 1) wait_vmcnt<(STAGES - 2) * LPS>();
    else wait_vmcnt<0>();
    barrier_nofence();
    load_frags(0, 0, fa0, fb0);
    int kt = 0;
    // steady state: every iteration issues a stage and prepares the next one
    for (; kt + STAGES - 1 < nfull; ++kt) {
      const int buf = kt % STAGES;
      load_frags(buf, 1, fa1, fb1);
      mfmas(fa0, fb0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<(STAGES - 3) * LPS>();                   // stage kt+1 landed (this wave)
      barrier_nofence();                                  // ... and for every wave
      issue((kt + STAGES - 1) % STAGES, kt + STAGES - 1); // into the buffer read at kt-1
      load_frags((kt + 1) % STAGES, 0, fa0, fb0);
      mfmas(fa1, fb1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    }
    // drain: the remaining stages are already in flight
    for (; kt < nfull; ++kt) {
      const int buf = kt % STAGES;
      load_frags(buf, 1, fa1, fb1);
      mfmas(fa0, fb0);
      if (kt + 1 < nfull) {
        wait_vmcnt<0>();
        barrier_nofence();
        load_frags((kt + 1) % STAGES, 0, fa0, fb0);
      }
      mfmas(fa1, fb1);
    }
  }
  if (tail) {
    // last partial stage: masked register loads into a free buffer
    __syncthreads();
    const int buf = nfull % STAGES;
    int8_t* base = smem + buf * STAGE;
    const int k0 = k_begin + nfull * BK;
    constexpr int CPR = BK / 16;
#pragma unroll
    for (int q = 0; q < (BM + BN) * CPR / NT; ++q) {
      const int c = tid + q * NT, row = c / CPR, ck = c % CPR;
      const bool is_a = row < BM;
      const int r = is_a ? row : row - BM;
      int gr = (is_a ? m0 : n0) + r;
      const int lim = is_a ? M : N;
      gr = gr < lim ? gr : lim - 1;
      const int8_t* src = is_a ? p.A + (int64_t)gr * p.lda : p.B + (int64_t)gr * p.ldb;
      const v4i v = load_chunk(src, k0 + ck * 16, k_end);
      *reinterpret_cast<v4i*>(base + (is_a ? 0 : A_BYTES) + r * BK + (swz(r, ck) << 4)) = v;
    }
    __syncthreads();
    load_frags(buf, 0, fa0, fb0);
    load_frags(buf, 1, fa1, fb1);
    mfmas(fa0, fb0);
    mfmas(fa1, fb1);
  }
  wait_vmcnt<0>();
  __syncthreads();
  epilogue_lds<BM, BN, WAVES_M, WAVES_N, FM, FN>(p, acc, smem, tm, tn, split);
}

// ---------------------------------------------------------------------------
// split-K combine: acc = sum over splits (exact), then the same epilogue and
// hash shares as the GEMM kernel; each thread owns 4 consecutive columns of a
// band of COMB_ROWS rows.
// ---------------------------------------------------------------------------
constexpr int COMB_ROWS = 32;

__global__ void __launch_bounds__(256)
splitk_combine_kernel(const GemmParams p) {
  __shared__ unsigned long long red[4];
  __shared__ int last_flag;
  const int M = p.M, N = p.N;
  const int tid = threadIdx.x;
  const int c0 = (blockIdx.x * 256 + tid) * 4;
  const int r0 = blockIdx.y * COMB_ROWS;
  const int r1 = r0 + COMB_ROWS < M ? r0 + COMB_ROWS : M;
  const bool relu = p.relu != 0;
  const int64_t plane = (int64_t)M * N;
  uint64_t t[4] = {0, 0, 0, 0};
  float sc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sc[e] = (c0 + e < N) ? p.s_col[c0 + e] : 0.0f;
  const bool vec = (N % 4 == 0) && (p.ldc % 4 == 0) && (((uintptr_t)p.C & 15) == 0);
  if (c0 < N) {
    for (int r = r0; r < r1; ++r) {
      int a[4] = {0, 0, 0, 0};
      const int* src = p.partials + (int64_t)r * N + c0;
      for (int sp = 0; sp < p.splits; ++sp) {
        if (vec) {
          const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + sp * plane));
          a[0] += v[0]; a[1] += v[1]; a[2] += v[2]; a[3] += v[3];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c0 + e < N) a[e] += src[sp * plane + e];
        }
      }
      const float sr = p.s_row[r];
      const uint64_t rk = hash_row_key((uint32_t)r);
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = epilogue1(a[e], sr, sc[e]);
        if (relu) y[e] = relu_pos0(y[e]);
        t[e] += rk * (uint64_t)__float_as_uint(y[e]);
      }
      float* dst = p.C + (int64_t)r * p.ldc + c0;
      if (vec) {
        *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c0 + e < N) dst[e] = y[e];
      }
    }
  }
  uint64_t part = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (c0 + e < N) part += hash_col_key((uint64_t)(c0 + e)) * t[e];
  if (p.do_hash) {
    part = block_sum_u64<256>(part, red);
    hash_share_and_finalize<256>(part, p.hash_parts, p.ticket, p.n_shares,
                                 blockIdx.y * gridDim.x + blockIdx.x, (uint64_t)M, (uint64_t)N,
                                 p.hash_out, red, &last_flag);
  }
}

// ---------------------------------------------------------------------------
// host side: plan and launch
// ---------------------------------------------------------------------------
// Tile configurations: macro tile, LDS stages, workgroups resident per CU,
// and the int8 MAC rate one workgroup sustains in the steady-state loop
// (measured on MI355X with operands streaming through L2: LM-head weight
// gradient 768x50304x8192, down-projection 8192x768x3072).
struct TileCfg {
  int bm, bn, stages, per_cu;
  double wg_macs;   // MAC/s of one resident workgroup
};
static const TileCfg kCfgs[] = {
    {256, 256, 4, 1, 4.5e12},   // eight waves (two per SIMD), 128x64 each
    {256, 128, 4, 1, 3.0e12},   // four waves, 128x64 each
    {128, 128, 4, 2, 1.25e12},  // four waves, 64x64 each
    {256, 256, 4, 1, 4.0e12},   // four waves, 128x128 each (not chosen by default)
};
constexpr int kNumCfgs = 4;

// Optional overrides for tests (the output never depends on the plan):
// I8G_FORCE_TILE = index into kCfgs; I8G_FORCE_SPLITS = number of K splits
// (clamped so that no split is empty).
static int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan best{};
  if (M <= 0 || N <= 0) return best;
  const int force_tile = env_int("I8G_FORCE_TILE", -1);
  const int force_splits = env_int("I8G_FORCE_SPLITS", 0);
  // Estimated seconds: rounds of resident workgroups x (MAC time of one
  // workgroup's share + the time to write its output tile at ~20 GB/s per
  // CU; with two workgroups per CU one's stores overlap the other's MFMAs),
  // plus the split-K partial round trip.
  const double cu_out_bw = 20e9;
  const double mem_bw = 4.0e12;
  double best_cost = 1e300;
  for (int c = 0; c < kNumCfgs; ++c) {
    if (force_tile >= 0 && c != force_tile) continue;
    if (force_tile < 0 && c == 3) continue;        // dominated by config 0; tests only
    const TileCfg& t = kCfgs[c];
    const int64_t tm = (M + t.bm - 1) / t.bm, tn = (N + t.bn - 1) / t.bn;
    const int64_t tiles = tm * tn;
    const double slots = 256.0 * t.per_cu;
    const int64_t kstages = (K + BK - 1) / BK;
    for (int s = 1; s <= 16; ++s) {
      if (force_splits > 0) {
        if (s != (force_splits < kstages ? force_splits : (int)kstages)) continue;
      } else if (s > 1 && kstages / s < 16) {
        break;                                      // keep >= 16 stages per split
      }
      const int64_t kps_st = (kstages + s - 1) / s;
      const int s_eff = (int)((kstages + kps_st - 1) / kps_st);   // no empty split
      const double rounds = std::ceil((double)(tiles * s_eff) / slots);
      const double tile_s = (double)t.bm * t.bn * kps_st * BK / t.wg_macs +
                            (double)t.bm * t.bn * 4 / cu_out_bw;
      double cost = rounds * tile_s;
      if (s_eff > 1) cost += (double)s_eff * M * N * 8 / mem_bw + 5e-6;
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
  if (best.bm == 0) {   // unreachable: every configuration has a one-split plan
    best.cfg = 2; best.bm = best.bn = 128;
    best.tiles_m = (int)((M + 127) / 128); best.tiles_n = (int)((N + 127) / 128);
    best.splits = 1; best.k_per_split = (int)((K + BK - 1) / BK * BK);
  }
  const int64_t tiles = (int64_t)best.tiles_m * best.tiles_n;
  if (best.splits > 1) {
    best.comb_x = (int)((N + 1023) / 1024);
    best.comb_y = (int)((M + COMB_ROWS - 1) / COMB_ROWS);
    best.hash_parts = best.comb_x * best.comb_y;
  } else {
    best.hash_parts = (int)tiles;
  }
  size_t bytes = kWsHeader + ((size_t)best.hash_parts * 8 + 255) / 256 * 256;
  best.partials_offset = bytes;
  if (best.splits > 1) bytes += (size_t)best.splits * M * N * 4;
  best.workspace_bytes = bytes;
  return best;
}

hipError_t launch_gemm(const GemmParams& p, const GemmPlan& plan, hipStream_t stream) {
  const unsigned int grid = (unsigned int)((int64_t)plan.tiles_m * plan.tiles_n * plan.splits);
  switch (plan.cfg) {
    case 0:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<256, 256, 2, 4, 4>), dim3(grid), dim3(512), 0, stream, p);
      break;
    case 1:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<256, 128, 2, 2, 4>), dim3(grid), dim3(256), 0, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<128, 128, 2, 2, 4>), dim3(grid), dim3(256), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<256, 256, 2, 2, 4>), dim3(grid), dim3(256), 0, stream, p);
      break;
  }
  if (plan.splits > 1)
    hipLaunchKernelGGL(splitk_combine_kernel, dim3(plan.comb_x, plan.comb_y), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace i8g
