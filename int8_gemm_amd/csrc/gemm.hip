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
//    mod 2^64; in the GEMM kernels the workgroup that finishes last adds the
//    shares (mod 2^64, any order) and writes H (see hash_share_and_finalize);
//    the split-K combine, whose workgroups all end together, stores its
//    shares and a one-workgroup kernel launched after it adds them.
#include <atomic>
#include <cmath>
#include <type_traits>

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
  // split-major: the workgroups of one XCD work on one K range, tiles in
  // GROUP_M order inside it, so they share A and B slices in their L2
  const int tiles = tiles_m * tiles_n;
  split = w / tiles;
  const int tile = w - split * tiles;
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

// s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | (((N >> 4) & 3) << 14));
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
// MODE 0 writes C (or the split's partial plane); MODE 1 and 2 are the two
// passes of the requantizing epilogue (GemmParams::rowmax): MODE 1 reduces
// max |y| over the LPR lanes that hold a row and raises rowmax[row] with an
// integer atomicMax on the bit pattern (non-negative floats order like their
// bits, so the result is the exact row max in any order); MODE 2 turns the
// final maxima into scales max(RN(a/127), RN(1e-8)) and writes
// q = floor(RN(RN(y*RN(1/s)) + 0.5)) -- quantize_rows of the output, which
// itself is never stored.
template <int BM, int BN, int WAVES_M, int WAVES_N, int FM, int FN, int MODE = 0>
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
  const bool raw = MODE == 0 && p.splits > 1;
  const bool relu = p.relu != 0;
  const bool stream = p.stream_out != 0;

  int* slab = reinterpret_cast<int*>(smem) + wave * SLAB;
  float* s_sr = reinterpret_cast<float*>(smem) + NWAVES * SLAB;
  unsigned int* s_rk = reinterpret_cast<unsigned int*>(s_sr + BM);
  float* s_inv = reinterpret_cast<float*>(s_rk + BM);
  unsigned long long* s_red = reinterpret_cast<unsigned long long*>(s_inv + BM);   // NWAVES + 1 words
  // row scales and row keys of the tile (zero beyond M: such rows add nothing)
  for (int r = tid; r < BM; r += NT) {
    const int gr = tm * BM + r;
    s_sr[r] = gr < M ? p.s_row[gr] : 0.0f;
    s_rk[r] = gr < M ? hash_row_key((unsigned int)gr) : 0u;
    if (MODE == 2) {
      float inv = 0.0f;
      if (gr < M) {
        const float sq = scale_of_absmax(__uint_as_float(p.rowmax[gr]));
        inv = recip_rn(sq);
        if (tn == 0) p.s_out[gr] = sq;
      }
      s_inv[r] = inv;
    }
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
  const bool qvec = MODE == 2 && (p.ldq % 4 == 0) && (((uintptr_t)p.Q & 3) == 0);
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
      } else if (MODE == 1) {
        const float sr = s_sr[lr];
        unsigned int mb = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float y = epilogue1(av[e], sr, sc[e]);   // 0 or -0 beyond N (scale 0)
          if (relu) y = relu_pos0(y);
          const unsigned int b = __float_as_uint(y) & 0x7FFFFFFFu;
          mb = b > mb ? b : mb;
        }
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) {
          const unsigned int o = (unsigned int)__shfl_xor((int)mb, off, 64);
          mb = o > mb ? o : mb;
        }
        if (lane % LPR == 0 && gr < M) atomicMax(p.rowmax + gr, mb);
      } else if (MODE == 2) {
        const float sr = s_sr[lr];
        const uint64_t rk = s_rk[lr];
        const float inv = s_inv[lr];
        unsigned int packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float y = epilogue1(av[e], sr, sc[e]);
          if (relu) y = relu_pos0(y);
          tcol[e] += rk * (uint64_t)__float_as_uint(y);
          packed |= ((unsigned int)quantize1(y, inv) & 0xFFu) << (8 * e);
        }
        if (gr >= M) continue;
        int8_t* dst = p.Q + (int64_t)gr * p.ldq + gc0;
        if (qvec && gc0 + 4 <= N) {
          *reinterpret_cast<unsigned int*>(dst) = packed;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gc0 + e < N) dst[e] = (int8_t)((packed >> (8 * e)) & 0xFFu);
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
  if (MODE != 1 && !raw && p.do_hash) {
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

// LDS bytes of the ring (and, reused after the main loop, of the epilogue).
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
constexpr int dma_smem_bytes() {
  constexpr int NWAVES = WAVES_M * WAVES_N, WTN = BN / WAVES_N;
  constexpr int STAGE = (BM + BN) * BK;
  constexpr int EPI_BYTES = NWAVES * 32 * (WTN + 8) * 4 + 3 * BM * 4 + 128;
  return STAGES * STAGE > EPI_BYTES ? STAGES * STAGE : EPI_BYTES;
}

// The main loop of one tile over K bytes [k_begin, k_end): acc is set to
// the exact int32 sums.  Called by every wave of the workgroup; the caller
// makes sure no wave still reads the LDS ring of a previous call.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES>
__device__ __forceinline__ void dma_mainloop(
    const GemmParams& p, int8_t* smem, int tm, int tn, int k_begin, int k_end,
    v16i (&acc)[BM / WAVES_M / 32][BN / WAVES_N / 32]) {
  constexpr int NWAVES = WAVES_M * WAVES_N, NT = NWAVES * 64;
  static_assert(NWAVES == 4 || NWAVES == 8, "four or eight waves");
  static_assert(STAGES >= 3, "the ring needs at least three stages");
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * BK, STAGE = (BM + BN) * BK;
  constexpr int A_INS = BM / (16 * NWAVES), B_INS = BN / (16 * NWAVES);   // 16-row blocks per wave
  static_assert(A_INS * 16 * NWAVES == BM && B_INS * 16 * NWAVES == BN, "rows per stage");
  constexpr int LPS = A_INS + B_INS;                   // load instructions per wave per stage
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N;
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
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int MODE = 0>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
gemm_i8_dma_kernel(const GemmParams p) {
  constexpr int FM = BM / WAVES_M / 32, FN = BN / WAVES_N / 32;
  __shared__ __attribute__((aligned(1024))) int8_t smem[dma_smem_bytes<BM, BN, WAVES_M, WAVES_N, STAGES>()];
  int tm, tn, split;
  map_workgroup(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.splits, tm, tn, split);
  const int k_begin = split * p.k_per_split;
  int k_end = k_begin + p.k_per_split;
  if (k_end > p.K) k_end = p.K;
  v16i acc[FM][FN];
  dma_mainloop<BM, BN, WAVES_M, WAVES_N, STAGES>(p, smem, tm, tn, k_begin, k_end, acc);
  epilogue_lds<BM, BN, WAVES_M, WAVES_N, FM, FN, MODE>(p, acc, smem, tm, tn, split);
}

// ---------------------------------------------------------------------------
// Operands stored as int4 (I8G_A_INT4 / I8G_B_INT4), register-staged: each
// 16-byte group of packed values (32 values: the low nibbles of its bytes are
// values 0..15, the high nibbles values 16..31) is widened in registers to
// two 16-byte int8 chunks and written to the same swizzled LDS layout as the
// int8 kernels use.  The widening keeps each nibble in the high half of its
// byte: chunk 0 = (w << 4) & 0xF0F0F0F0, chunk 1 = w & 0xF0F0F0F0, i.e. the
// int8 value 16*q, exact for q in [-8, 7].  The MFMAs then sum
// 16^(a4+b4) * qa * qb exactly (|16*7*127| and |16*7*16*7| are below 127^2,
// so the int32 range of the K limit still holds) and the accumulators are
// shifted right by 4*(a4+b4) before the epilogue, which is exact because
// every term is a multiple of that power of two.  Two LDS buffers, one
// barrier per 64-value stage, the next stage's global loads in flight during
// the current stage's MFMAs.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WAVES_M, int WAVES_N, bool A4, bool B4>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
gemm_i4_kernel(const GemmParams p) {
  constexpr int NWAVES = WAVES_M * WAVES_N, NT = NWAVES * 64;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_BYTES = BM * BK, STAGE = (BM + BN) * BK;
  constexpr int A_PER_ROW = A4 ? 2 : 4, B_PER_ROW = B4 ? 2 : 4;   // 16-byte loads per row per stage
  constexpr int A_LD = BM * A_PER_ROW / NT, B_LD = BN * B_PER_ROW / NT;
  static_assert(A_LD * NT == BM * A_PER_ROW && B_LD * NT == BN * B_PER_ROW, "loads per thread");
  __shared__ __attribute__((aligned(1024))) int8_t smem[dma_smem_bytes<BM, BN, WAVES_M, WAVES_N, 2>()];
  int tm, tn, split;
  map_workgroup(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.splits, tm, tn, split);
  const int k_begin = split * p.k_per_split;
  int k_end = k_begin + p.k_per_split;
  if (k_end > p.K) k_end = p.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int m0 = tm * BM, n0 = tn * BN;

  // this thread's loads: (row, 16-byte position within the stage's row)
  const int8_t* pa[A_LD];
  const int8_t* pb[B_LD];
  int ra_row[A_LD], ra_pos[A_LD], rb_row[B_LD], rb_pos[B_LD];
#pragma unroll
  for (int q = 0; q < A_LD; ++q) {
    const int c = tid + q * NT;
    ra_row[q] = c / A_PER_ROW;
    ra_pos[q] = c % A_PER_ROW;
    int gr = m0 + ra_row[q];
    gr = gr < p.M ? gr : p.M - 1;
    pa[q] = p.A + (int64_t)gr * p.lda;
  }
#pragma unroll
  for (int q = 0; q < B_LD; ++q) {
    const int c = tid + q * NT;
    rb_row[q] = c / B_PER_ROW;
    rb_pos[q] = c % B_PER_ROW;
    int gr = n0 + rb_row[q];
    gr = gr < p.N ? gr : p.N - 1;
    pb[q] = p.B + (int64_t)gr * p.ldb;
  }
  v4i ga[A_LD], gb[B_LD];
  const v4i zero = {0, 0, 0, 0};
  // global -> registers for the stage starting at value k0 (k0 % 64 == 0).
  // int8: 16 values at k0 + 16*pos; int4: 32 values at k0 + 32*pos, i.e. 16
  // bytes at byte (k0 + 32*pos) / 2, which lies inside the row whenever its
  // first value does (a row holds whole 16-byte groups).
  auto gload = [&](int k0) {
    const bool full = k0 + BK <= k_end;
#pragma unroll
    for (int q = 0; q < A_LD; ++q) {
      if (A4) {
        const int kk = k0 + 32 * ra_pos[q];
        ga[q] = (full || kk < k_end) ? *reinterpret_cast<const v4i*>(pa[q] + kk / 2) : zero;
      } else {
        const int kk = k0 + 16 * ra_pos[q];
        ga[q] = full ? *reinterpret_cast<const v4i*>(pa[q] + kk) : load_chunk(pa[q], kk, k_end);
      }
    }
#pragma unroll
    for (int q = 0; q < B_LD; ++q) {
      if (B4) {
        const int kk = k0 + 32 * rb_pos[q];
        gb[q] = (full || kk < k_end) ? *reinterpret_cast<const v4i*>(pb[q] + kk / 2) : zero;
      } else {
        const int kk = k0 + 16 * rb_pos[q];
        gb[q] = full ? *reinterpret_cast<const v4i*>(pb[q] + kk) : load_chunk(pb[q], kk, k_end);
      }
    }
  };
  auto widen_lo = [](v4i w) {
    v4i r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (int)(((unsigned int)w[e] << 4) & 0xF0F0F0F0u);
    return r;
  };
  auto widen_hi = [](v4i w) {
    v4i r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (int)((unsigned int)w[e] & 0xF0F0F0F0u);
    return r;
  };
  // registers -> LDS buffer `buf` (int4 widened; values >= k_end zeroed)
  auto sstore = [&](int buf, int k0) {
    const bool full = k0 + BK <= k_end;
    int8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int q = 0; q < A_LD; ++q) {
      int8_t* rowp = base + ra_row[q] * BK;
      if (A4) {
        const int kk = k0 + 32 * ra_pos[q];
        v4i lo = widen_lo(ga[q]), hi = widen_hi(ga[q]);
        if (!full) {
          lo = mask_tail(lo, k_end - kk);
          hi = mask_tail(hi, k_end - kk - 16);
        }
        *reinterpret_cast<v4i*>(rowp + (swz(ra_row[q], 2 * ra_pos[q]) << 4)) = lo;
        *reinterpret_cast<v4i*>(rowp + (swz(ra_row[q], 2 * ra_pos[q] + 1) << 4)) = hi;
      } else {
        *reinterpret_cast<v4i*>(rowp + (swz(ra_row[q], ra_pos[q]) << 4)) = ga[q];
      }
    }
#pragma unroll
    for (int q = 0; q < B_LD; ++q) {
      int8_t* rowp = base + A_BYTES + rb_row[q] * BK;
      if (B4) {
        const int kk = k0 + 32 * rb_pos[q];
        v4i lo = widen_lo(gb[q]), hi = widen_hi(gb[q]);
        if (!full) {
          lo = mask_tail(lo, k_end - kk);
          hi = mask_tail(hi, k_end - kk - 16);
        }
        *reinterpret_cast<v4i*>(rowp + (swz(rb_row[q], 2 * rb_pos[q]) << 4)) = lo;
        *reinterpret_cast<v4i*>(rowp + (swz(rb_row[q], 2 * rb_pos[q] + 1) << 4)) = hi;
      } else {
        *reinterpret_cast<v4i*>(rowp + (swz(rb_row[q], rb_pos[q]) << 4)) = gb[q];
      }
    }
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
  const int lrow = lane & 31, lhalf = lane >> 5;
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
  const int klen = k_end > k_begin ? k_end - k_begin : 0;
  const int nst = (klen + BK - 1) / BK;
  if (nst > 0) gload(k_begin);
  for (int kt = 0; kt < nst; ++kt) {
    const int buf = kt & 1;
    // buffer `buf` was last read in stage kt-2; every wave has passed the
    // barrier of stage kt-1 since, so it is free
    sstore(buf, k_begin + kt * BK);
    __syncthreads();
    if (kt + 1 < nst) gload(k_begin + (kt + 1) * BK);
    const int8_t* sb = smem + buf * STAGE;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const v4i*>(sb + offa[s][i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const v4i*>(sb + offb[s][j]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();   // the epilogue reuses the LDS
  constexpr int SHIFT = 4 * ((A4 ? 1 : 0) + (B4 ? 1 : 0));
  if (SHIFT > 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] >>= SHIFT;
  }
  epilogue_lds<BM, BN, WAVES_M, WAVES_N, FM, FN>(p, acc, smem, tm, tn, split);
}

// Calls f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// Persistent GEMM with a drained epilogue.
//
// One workgroup per CU walks a sequence of output tiles.  Its four waves
// (one per SIMD) keep two sets of accumulators: while the MFMAs of tile t
// accumulate into one set, the epilogue of tile t-1 is computed from the
// other set, one 32x32 block per K stage, and written with buffer stores
// straight from the MFMA register layout (each store covers two 128-byte
// row segments).  The epilogue's VALU work and its stores are thereby hidden
// under matrix-core work instead of following it, which matters when the
// f32 output write bounds the GEMM (K = 768).
//
// The ring of LDS stages runs across tile boundaries: near the end of a
// tile, the stages of the next tile are already being fetched.  Waits on
// the vector-memory counter count the epilogue's stores as well (gfx950
// retires loads and stores in issue order for s_waitcnt vmcnt).
//
// Output masking: the buffer resource of a tile starts at the tile's first
// row and has a large record count; a lane whose element lies outside the
// matrix gets a voffset at or above that count, so the hardware drops the
// store whether or not the scalar offset enters the range check.
// Requires K % 64 == 0, K >= 64 * (STAGES - 1) and ldc <= kPersistMaxLdc (the
// offsets within a 32-row block stay below the record count).
// ---------------------------------------------------------------------------

// LDS byte address of a pointer into __shared__ memory.
template <class T>
__device__ __forceinline__ uint32_t lds_addr(const T* q) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) T*)q;
}

constexpr unsigned int kBufRecords = 0x7FFFFFF0u;   // record count of the output resource
// Cache policy of the output stores for outputs larger than half the
// last-level cache (GemmParams::stream_out): the nontemporal bit.  Measured
// on the LM-head forward (1.65 GB of f32 output written while the operands
// stream through L2): ~700 us with ordinary stores, ~425 us with this bit,
// ~360 us with the stores dropped altogether; ordinary stores keep a smaller
// output in the last-level cache for the kernel that reads it next.
constexpr int kStoreNT = 2;
constexpr int kBufInvalid = 0x7FFFFFF0;             // voffset of a dropped store

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool RELU, bool NTSTORE>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64, 1)
gemm_i8_persist_kernel(const GemmParams p) {
  constexpr int NWAVES = WAVES_M * WAVES_N, NT = NWAVES * 64;
  static_assert(NWAVES == 4, "four waves, one per SIMD");
  static_assert(STAGES >= 3, "the ring needs at least three stages");
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32, NB = FM * FN;
  constexpr int A_BYTES = BM * BK, STAGE = (BM + BN) * BK;
  constexpr int A_INS = BM / (16 * NWAVES), B_INS = BN / (16 * NWAVES);
  static_assert(A_INS * 16 * NWAVES == BM && B_INS * 16 * NWAVES == BN, "rows per stage");
  constexpr int LPS = A_INS + B_INS;
  constexpr int RING = STAGES * STAGE;
  static_assert(LPS + 2 * 16 < 64, "vmcnt counts fit the 6-bit counter");
  constexpr int SCL = BM + BN;                          // floats per scale slot: rows, then columns
  constexpr int NSI = SCL / 64;                         // dword DMA instructions per slot
  static_assert(NSI * 64 == SCL, "tile sides are multiples of 64");
  constexpr int SQ = (NSI + NWAVES - 1) / NWAVES;       // per wave (at most)
  __shared__ __attribute__((aligned(1024))) int8_t smem[RING + 3 * SCL * 4 + 3 * BM * 4 + 64];
  // three slots: tile r's scales and row keys live in slot r % 3 from the
  // time its first stage is fetched until its epilogue is drained
  float* const s_scl = reinterpret_cast<float*>(smem + RING);                              // [3][SCL]
  unsigned int* const s_rk = reinterpret_cast<unsigned int*>(smem + RING + 3 * SCL * 4);  // [3][BM]
  unsigned long long* const s_red =
      reinterpret_cast<unsigned long long*>(smem + RING + 3 * SCL * 4 + 3 * BM * 4);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int M = p.M, N = p.N;
  const int nst = p.K / BK;
  const int tiles = p.tiles_m * p.tiles_n;
  const int G = gridDim.x;
  const int64_t ldc4 = p.ldc * 4;

  // This workgroup's place in the tile sequence: workgroups are dealt to
  // the 8 XCDs round-robin; in each round the XCDs take consecutive chunks
  // of the L2-grouped tile order.
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int per = G >> 3, rem = G & 7;
  const int wpos = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int my_tiles = wpos < tiles ? (tiles - 1 - wpos) / G + 1 : 0;
  auto tile_coords = [&](int r, int& tm, int& tn) __attribute__((always_inline)) {
    const int n = r * G + wpos;
    const int group_size = GROUP_M * p.tiles_n;
    const int group = n / group_size;
    const int first_m = group * GROUP_M;
    const int gm = (p.tiles_m - first_m) < GROUP_M ? (p.tiles_m - first_m) : GROUP_M;
    const int in_group = n - group * group_size;
    tm = __builtin_amdgcn_readfirstlane(first_m + in_group % gm);
    tn = __builtin_amdgcn_readfirstlane(in_group / gm);
  };

  // ---- direct-to-LDS loads of one stage (see gemm_i8_dma_kernel) ----
  const int r_in = lane >> 2, slot = lane & 3;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform copies
  const int wm_s = wave_s / WAVES_N;
  // Per tile: wave-uniform base addresses (scalar registers) and this
  // lane's 32-bit offsets from them (rows clamped into the matrix).
  struct Src {
    const int8_t* abase;   // A at the tile's first row
    const int8_t* bbase;   // B at the tile's first row
    const float* rbase;    // s_row at the tile's first row
    const float* cbase;    // s_col at the tile's first column
    int a[A_INS];
    int b[B_INS];
    int sp[SQ];            // offset (floats) of this lane's scale, rows then columns
    int slot;              // scale slot of the tile
  };
  auto make_src = [&](int r, int tm, int tn, Src& s) __attribute__((always_inline)) {
    s.slot = __builtin_amdgcn_readfirstlane(r % 3);
    const int row0 = tm * BM, col0 = tn * BN;
    s.abase = uniform_ptr(p.A + (int64_t)row0 * p.lda);
    s.bbase = uniform_ptr(p.B + (int64_t)col0 * p.ldb);
    s.rbase = uniform_ptr(p.s_row + row0);
    s.cbase = uniform_ptr(p.s_col + col0);
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
      const int e = (q * NWAVES + wave) * 64 + lane;   // index into [rows | columns]
      if (e < BM) {
        const int lr = e < M - row0 ? e : M - 1 - row0;
        s.sp[q] = lr;
      } else {
        const int lc = (e - BM) < N - col0 ? (e - BM) : N - 1 - col0;
        s.sp[q] = BM + lc;   // marks a column entry; see issue()
      }
    }
#pragma unroll
    for (int q = 0; q < A_INS; ++q) {
      const int row = (q * NWAVES + wave) * 16 + r_in;
      const int lr = row < M - row0 ? row : M - 1 - row0;
      s.a[q] = lr * (int)p.lda + (swz(row, slot) << 4);
    }
#pragma unroll
    for (int q = 0; q < B_INS; ++q) {
      const int row = (q * NWAVES + wave) * 16 + r_in;
      const int lr = row < N - col0 ? row : N - 1 - col0;
      s.b[q] = lr * (int)p.ldb + (swz(row, slot) << 4);
    }
  };
  auto issue = [&](int buf, const Src& s, int kt) __attribute__((always_inline)) {
    int8_t* base = smem + buf * STAGE + wave_s * 1024;
    const int8_t* ab = s.abase + kt * BK;
    const int8_t* bb = s.bbase + kt * BK;
#pragma unroll
    for (int q = 0; q < A_INS; ++q) dma_load16(ab + s.a[q], base + q * NWAVES * 1024);
#pragma unroll
    for (int q = 0; q < B_INS; ++q) dma_load16(bb + s.b[q], base + A_BYTES + q * NWAVES * 1024);
    if (kt == 0) {
      // the tile's row and column scales ride with its first stage; these
      // extra loads only lengthen the queue that later waits count
      float* sbase = s_scl + s.slot * SCL + wave_s * 64;
#pragma unroll
      for (int q = 0; q < SQ; ++q)
        if (q * NWAVES + wave_s < NSI) {
          const float* src = (q * NWAVES + wave_s) * 64 < BM ? s.rbase + s.sp[q] : s.cbase + (s.sp[q] - BM);
          __builtin_amdgcn_global_load_lds(src, sbase + q * NWAVES * 64, 4, 0, 0);
        }
    }
  };

  // ---- fragments and MFMAs ----
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
  v4i fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto load_frags = [&](int buf, int s, v4i (&fa)[FM], v4i (&fb)[FN]) __attribute__((always_inline)) {
    const int8_t* sb = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const v4i*>(sb + offa[s][i]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const v4i*>(sb + offb[s][j]);
  };
  v16i acc0[FM][FN], acc1[FM][FN];

  // ---- epilogue state of the tile being drained ----
  struct Out {
    float* cbase;                  // C at the tile's first row
    int voff[FN];                  // this lane's column (and half-wave row offset), or kBufInvalid
    uint64_t ckey[FN];             // column hash keys (0 beyond N)
    int rows_valid;                // rows of the tile inside the matrix
    int slot;                      // scale / key slot of the tile
  };
  uint64_t tcol[FN];               // per-column hash sums of the tile being drained
  uint64_t lane_hash = 0;          // this lane's share of S over every drained tile
  auto make_out = [&](int r, int tm, int tn, Out& o) __attribute__((always_inline)) {
    const int row0 = tm * BM;
    o.cbase = uniform_ptr(p.C + (int64_t)row0 * p.ldc);
    o.rows_valid = __builtin_amdgcn_readfirstlane((M - row0) < BM ? (M - row0) : BM);
    o.slot = __builtin_amdgcn_readfirstlane(r % 3);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = tn * BN + wn * WTN + j * 32 + lrow;
      const bool ok = col < N;
      o.voff[j] = ok ? (int)(lhalf * 4 * ldc4 + col * 4) : kBufInvalid;
      o.ckey[j] = ok ? hash_col_key((uint64_t)col) : 0ull;
    }
    // row hash keys of the tile (0 beyond M: those rows add nothing)
    for (int rr = tid; rr < BM; rr += NT) {
      const int gr = row0 + rr;
      s_rk[o.slot * BM + rr] = gr < M ? hash_row_key((unsigned int)gr) : 0u;
    }
  };

  // Drain block b = (i, j) of accumulator set `acc`: epilogue, ReLU, hash
  // terms and 16 stores.  Rows of lane l, register v: (v/4)*8 + 4*(l/32) + v%4
  // within the 32x32 block; column l%32.
  auto drain_block = [&](v16i (&acc)[FM][FN], const Out& o, auto IJ) __attribute__((always_inline)) {
    constexpr int b = decltype(IJ)::value;
    constexpr int i = b / FN, j = b % FN;
    const int rb = wm * WTM + i * 32 + lhalf * 4;             // this lane's first row in the tile
    // Scales (landed by direct-to-LDS loads that earlier waits covered) and
    // row keys, read with explicit LDS instructions: the compiler would
    // otherwise wait for every outstanding direct-to-LDS load first.
    v4i srq[4], rkq[4];
    int scb;
    {
      const uint32_t sa = lds_addr(s_scl + o.slot * SCL + rb);
      const uint32_t ka = lds_addr(s_rk + o.slot * BM + rb);
      const uint32_t ca = lds_addr(s_scl + o.slot * SCL + BM + wn * WTN + j * 32 + lrow);
      asm volatile("ds_read_b128 %0, %1" : "=v"(srq[0]) : "v"(sa));
      asm volatile("ds_read_b128 %0, %1 offset:32" : "=v"(srq[1]) : "v"(sa));
      asm volatile("ds_read_b128 %0, %1 offset:64" : "=v"(srq[2]) : "v"(sa));
      asm volatile("ds_read_b128 %0, %1 offset:96" : "=v"(srq[3]) : "v"(sa));
      asm volatile("ds_read_b128 %0, %1" : "=v"(rkq[0]) : "v"(ka));
      asm volatile("ds_read_b128 %0, %1 offset:32" : "=v"(rkq[1]) : "v"(ka));
      asm volatile("ds_read_b128 %0, %1 offset:64" : "=v"(rkq[2]) : "v"(ka));
      asm volatile("ds_read_b128 %0, %1 offset:96" : "=v"(rkq[3]) : "v"(ka));
      asm volatile("ds_read_b32 %0, %1" : "=v"(scb) : "v"(ca));
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(srq[0]), "+v"(srq[1]), "+v"(srq[2]), "+v"(srq[3]), "+v"(rkq[0]),
                     "+v"(rkq[1]), "+v"(rkq[2]), "+v"(rkq[3]), "+v"(scb));
    }
    const float sc = __int_as_float(scb);
    // rows of this 32-row block that lie inside the matrix (wave-uniform)
    const int lim_w = o.rows_valid - (wm_s * WTM + i * 32);
    // resource based at the block's first row: offsets stay below 32 rows
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(o.cbase + (int64_t)(wm_s * WTM + i * 32) * p.ldc), 0, (int)kBufRecords,
        0x00020000);
    auto body = [&](auto RAGGED) __attribute__((always_inline)) {
      constexpr bool R = decltype(RAGGED)::value;
      const int lim = lim_w - lhalf * 4;   // this lane's rows q*8+e below lim are inside
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float srs[4] = {__int_as_float(srq[q][0]), __int_as_float(srq[q][1]),
                              __int_as_float(srq[q][2]), __int_as_float(srq[q][3])};
        const unsigned int rks[4] = {(unsigned int)rkq[q][0], (unsigned int)rkq[q][1],
                                     (unsigned int)rkq[q][2], (unsigned int)rkq[q][3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = q * 4 + e;
          float y = epilogue1(acc[i][j][v], srs[e], sc);
          if (RELU) y = relu_pos0(y);
          tcol[j] += (uint64_t)rks[e] * (uint64_t)__float_as_uint(y);
          const int soff = (q * 8 + e) * (int)ldc4;
          int vo = o.voff[j];
          if (R) vo = (q * 8 + e) < lim ? vo : kBufInvalid;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), rsrc, vo, soff, NTSTORE ? kStoreNT : 0);
        }
      }
    };
    if (lim_w >= 32) body(std::false_type());
    else body(std::true_type());
  };
  auto close_tile_hash = [&](const Out& o) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      lane_hash += o.ckey[j] * tcol[j];
      tcol[j] = 0;
    }
  };

  // ---- one K stage of tile r (s = 0..nst-1) into accumulator set X ----
  // g = global stage index of this workgroup (r*nst + s); gtotal = stages in
  // all its tiles.  Fragments of k-step 0 of this stage are in fa0/fb0.
  const int gtotal = my_tiles * nst;
  Src src_cur, src_nxt;
  // wait for stage g+1: its loads were issued at stage g-STAGES+2; issued
  // after them are the loads of the next STAGES-3 stages (if the sequence
  // has not ended) and at least ST stores.  Counting fewer operations than
  // were issued only makes the wait stricter.
  auto wait_next = [&](int g, auto STORES) __attribute__((always_inline)) {
    constexpr int ST = decltype(STORES)::value;
    if (g + STAGES - 2 < gtotal) wait_vmcnt<(STAGES - 3) * LPS + ST>();
    else wait_vmcnt<ST>();
  };
  auto stage_body = [&](v16i (&X)[FM][FN], int g, int s, bool first, auto STORES_BEFORE,
                        auto drain_fn) __attribute__((always_inline)) {
    const int buf = g % STAGES;
    load_frags(buf, 1, fa1, fb1);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v16i c = first ? v16i{} : X[i][j];
        X[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa0[i], fb0[j], c, 0, 0, 0);
      }
#pragma unroll
    for (int t = 0; t < FM + FN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
    __builtin_amdgcn_sched_barrier(0);
    if (g + 1 < gtotal) {
      wait_next(g, STORES_BEFORE);
      barrier_nofence();
      const int gi = g + STAGES - 1;
      if (gi < gtotal) {
        const int si = s + STAGES - 1;
        if (si < nst) issue(gi % STAGES, src_cur, si);
        else issue(gi % STAGES, src_nxt, si - nst);
      }
      load_frags((g + 1) % STAGES, 0, fa0, fb0);
    }
    // stores of the drain must stay behind this stage's loads (wait counts)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        X[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa1[i], fb1[j], X[i][j], 0, 0, 0);
    drain_fn();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto no_drain = []() __attribute__((always_inline)) {};

  // One tile: X accumulates tile r; Y (if DRAIN) holds tile r-1, drained
  // during stages 0..NB-1 (each stage drains one block: 16 stores).
  auto run_tile = [&](v16i (&X)[FM][FN], v16i (&Y)[FM][FN], int r, const Out& oy, auto DRAIN)
      __attribute__((always_inline)) {
    constexpr bool D = decltype(DRAIN)::value;
    const int g0 = r * nst;
    // stages that drain one block each (compile-time position b)
    auto drain_stage = [&](auto BI) __attribute__((always_inline)) {
      constexpr int b = decltype(BI)::value;
      // stores issued after the loads this stage waits for: those of stages
      // s-2 and s-1 of this tile (none before stage 0)
      constexpr int ST = D ? (b >= 2 ? 32 : (b == 1 ? 16 : 0)) : 0;
      if (b < nst) {
        if (D) stage_body(X, g0 + b, b, b == 0, std::integral_constant<int, ST>(),
                          [&]() __attribute__((always_inline)) { drain_block(Y, oy, BI); });
        else stage_body(X, g0 + b, b, b == 0, std::integral_constant<int, 0>(), no_drain);
      } else if (D) {
        drain_block(Y, oy, BI);   // fewer stages than blocks: drain without MFMAs
      }
    };
    static_for<0, NB>(drain_stage);
    if (D) close_tile_hash(oy);
    int s = NB;
    if (s < nst) {   // first two stages after the drain still see its stores
      stage_body(X, g0 + s, s, false, std::integral_constant<int, D ? 32 : 0>(), no_drain);
      ++s;
    }
    if (s < nst) {
      stage_body(X, g0 + s, s, false, std::integral_constant<int, D ? 16 : 0>(), no_drain);
      ++s;
    }
    for (; s < nst; ++s) stage_body(X, g0 + s, s, false, std::integral_constant<int, 0>(), no_drain);
  };

  // acc0 accumulates the tile being multiplied; acc1 holds the previous
  // tile while it is drained.  At a tile boundary acc0 is copied to acc1
  // (AGPR to AGPR) and the next tile's first MFMAs restart acc0 from zero.
  Out out_cur, out_prev;
  if (my_tiles > 0) {
    int tm, tn;
    tile_coords(0, tm, tn);
    make_src(0, tm, tn, src_cur);
    make_out(0, tm, tn, out_cur);
    if (my_tiles > 1) {
      int tm1, tn1;
      tile_coords(1, tm1, tn1);
      make_src(1, tm1, tn1, src_nxt);
    }
    // prologue: the first STAGES-1 stages of the sequence
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st) {
      if (st < gtotal) {
        if (st < nst) issue(st, src_cur, st);
        else issue(st, src_nxt, st - nst);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();   // also publishes the row keys of tile 0
    load_frags(0, 0, fa0, fb0);
#pragma unroll
    for (int j = 0; j < FN; ++j) tcol[j] = 0;

    run_tile(acc0, acc1, 0, out_prev, std::false_type());
    for (int r = 1; r < my_tiles; ++r) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc1[i][j] = acc0[i][j];
      out_prev = out_cur;
      // tile r starts: its sources become current; prepare tile r+1's
      src_cur = src_nxt;
      int a, b;
      tile_coords(r, a, b);
      make_out(r, a, b, out_cur);
      if (r + 1 < my_tiles) {
        int c, d;
        tile_coords(r + 1, c, d);
        make_src(r + 1, c, d, src_nxt);
      }
      run_tile(acc0, acc1, r, out_prev, std::true_type());
    }
    // the last tile
    static_for<0, NB>([&](auto BI) __attribute__((always_inline)) { drain_block(acc0, out_cur, BI); });
    close_tile_hash(out_cur);
  }
  if (p.do_hash) {
    const uint64_t part = block_sum_u64<NT>(lane_hash, s_red);
    hash_share_and_finalize<NT>(part, p.hash_parts, p.ticket, p.n_shares, blockIdx.x, (uint64_t)M,
                                (uint64_t)N, p.hash_out, s_red, reinterpret_cast<int*>(s_red + NWAVES));
  }
}

// ---------------------------------------------------------------------------
// Persistent GEMM with 128-byte K stages.
//
// The tile walk and the drained epilogue of gemm_i8_persist_kernel, with a
// schedule built around two measured properties of gfx950:
//  * Direct-to-LDS loads cost per request.  Eight lanes fetching one whole
//    128-byte line per row feed a CU about twice as fast as four lanes
//    fetching half a line (about 56 against 29 bytes per clock per CU, all
//    CUs loading).  A stage therefore holds 128 bytes of K per row.
//  * A wave's waits (barrier, loads landing) leave its matrix core idle unless
//    another wave on the SIMD has MFMAs to issue.  A stage is four k-steps of
//    FM x FN MFMAs per wave; the fragment reads of k-step t+1 are issued during
//    k-step t, and four elements per k-step of the previous tile's epilogue
//    block (one 32x32 block per stage) are interleaved with the MFMAs.  The
//    stage's only barrier sits before k-step 3: after it the stage's slot is
//    free, and k-step 3 issues the loads of stage g+STAGES into it.
// Two configurations: a 128x192 tile, one workgroup per CU and a three-slot
// ring (120 KiB; the loads have two stages to land), and a 128x128 tile, two
// workgroups per CU (WPC) and a two-slot ring (64 KiB each; one stage to land,
// the other workgroup's MFMAs covering the waits).
// LDS rows are 128 bytes.  Chunk c of row r is stored at position
// c ^ ((r / 2) % 8), which puts the 16 lanes of each fragment read on
// distinct banks.
// Requires K % 128 == 0, K / 128 >= blocks per wave (FM * FN), M % BM == 0 (no
// ragged tile-row: only columns are masked, through the buffer range check)
// and ldc <= kPersistMaxLdc.
// ---------------------------------------------------------------------------
constexpr int BK2 = 128;   // bytes of K per stage of gemm_i8_persist128_kernel

// The lane index, read so that the compiler can neither hoist it nor values
// derived from it out of loops: per-lane addresses used once per stage are
// then recomputed (two VALU operations) instead of being kept live across the
// whole kernel, where register pressure would spill them to scratch (and a
// scratch reload waits for every outstanding load of the LDS ring).
__device__ __forceinline__ int lane_id_local() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ int swz128(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Buffer loads that write LDS directly: lane l's 16 (or 4) bytes land at
// lds + 16*l (4*l); lds must be the same for the whole wave.  Offsets at or
// beyond the resource's record count are not read.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ int buffer_atomic_add_ret(__amdgpu_buffer_rsrc_t r, int v, int voff) {
  return __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(v, r, voff, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool RELU, int STAGES, int WPC, bool NTSTORE, int MODE = 0>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64, WPC)
gemm_i8_persist128_kernel(const GemmParams p) {
  constexpr int NWAVES = WAVES_M * WAVES_N, NT = NWAVES * 64;
  static_assert(NWAVES == 4, "four waves, one per SIMD");
  static_assert(STAGES >= 2, "a stage's slot is refilled after the barrier of the stage");
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  // wave tiles of whole 32x32 blocks: every fragment row base is then a
  // multiple of 32, which leaves the swizzle phase (row/2)%8 to the lane
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile of 32x32 blocks");
  constexpr int FM = WTM / 32, FN = WTN / 32, NB = FM * FN;
  static_assert(NB % 2 == 0, "epilogue operands alternate between two register sets");
  constexpr int A_BYTES = BM * BK2, STAGE = (BM + BN) * BK2;
  constexpr int A_INS = BM / (8 * NWAVES), B_INS = BN / (8 * NWAVES);   // 8 rows per load
  static_assert(A_INS * 8 * NWAVES == BM && B_INS * 8 * NWAVES == BN, "rows per stage");
  constexpr int LPS = A_INS + B_INS;                    // loads per wave per stage
  constexpr int RING = STAGES * STAGE;
  // floats per scale slot: row scales, column scales, and in MODE 2 the
  // reciprocals of the output row scales
  constexpr int SCL = BM + BN + (MODE == 2 ? BM : 0);
  constexpr int NSI = SCL / 64;                         // dword loads per scale slot
  static_assert(NSI * 64 == SCL, "tile sides are multiples of 64");
  constexpr int SQ = (NSI + NWAVES - 1) / NWAVES;
  __shared__ __attribute__((aligned(1024))) int8_t smem[RING + 3 * SCL * 4 + 3 * BM * 4 + 64];
  float* const s_scl = reinterpret_cast<float*>(smem + RING);                              // [3][SCL]
  unsigned int* const s_rk = reinterpret_cast<unsigned int*>(smem + RING + 3 * SCL * 4);  // [3][BM]
  unsigned long long* const s_red =
      reinterpret_cast<unsigned long long*>(smem + RING + 3 * SCL * 4 + 3 * BM * 4);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int M = p.M, N = p.N;
  const int nst = p.K / BK2;
  const int tiles = p.tiles_m * p.tiles_n;
  const int G = gridDim.x;
  const int64_t ldc4 = p.ldc * 4;

  // this workgroup's tiles (as in gemm_i8_persist_kernel)
  const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int per = G >> 3, rem = G & 7;
  const int wpos = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int my_tiles = wpos < tiles ? (tiles - 1 - wpos) / G + 1 : 0;
  auto tile_coords = [&](int r, int& tm, int& tn) __attribute__((always_inline)) {
    const int n = r * G + wpos;
    const int group_size = GROUP_M * p.tiles_n;
    const int group = n / group_size;
    const int first_m = group * GROUP_M;
    const int gm = (p.tiles_m - first_m) < GROUP_M ? (p.tiles_m - first_m) : GROUP_M;
    const int in_group = n - group * group_size;
    tm = __builtin_amdgcn_readfirstlane(first_m + in_group % gm);
    tn = __builtin_amdgcn_readfirstlane(in_group / gm);
  };

  // ---- direct-to-LDS loads: lane l of a load fills row l/8, position l%8 ----
  const int r_in = lane >> 3, pch = lane & 7;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm_s = wave_s / WAVES_N, wn_s = wave_s % WAVES_N;
  // Loads go through buffer resources: the tile (and stage) base is scalar,
  // and each lane's offset is the same for every tile.  B rows at or beyond N
  // and column scales at or beyond N fall outside the resource's range and
  // read as zeros: their columns' stores are dropped and their hash keys are 0.
  struct Src {
    const int8_t* abase;   // A at the tile's first row
    const int8_t* bbase;   // B at the tile's first row
    const float* rbase;    // s_row at the tile's first row
    const float* cbase;    // s_col at the tile's first column
    const float* ibase;    // MODE 2: the output scale reciprocals at the tile's first row
    int ncol;              // columns of the tile inside the matrix
    int slot;              // scale slot of the tile
  };
  int a_off[A_INS], b_off[B_INS];
#pragma unroll
  for (int q = 0; q < A_INS; ++q) {
    const int row = (q * NWAVES + wave) * 8 + r_in;
    a_off[q] = row * (int)p.lda + (swz128(row, pch) << 4);
  }
#pragma unroll
  for (int q = 0; q < B_INS; ++q) {
    const int row = (q * NWAVES + wave) * 8 + r_in;
    b_off[q] = row * (int)p.ldb + (swz128(row, pch) << 4);
  }
  const int lane4 = lane * 4;
  auto make_src = [&](int r, int tm, int tn, Src& s) __attribute__((always_inline)) {
    s.slot = __builtin_amdgcn_readfirstlane(r % 3);
    const int row0 = tm * BM, col0 = tn * BN;
    s.abase = uniform_ptr(p.A + (int64_t)row0 * p.lda);
    s.bbase = uniform_ptr(p.B + (int64_t)col0 * p.ldb);
    s.rbase = uniform_ptr(p.s_row + row0);
    s.cbase = uniform_ptr(p.s_col + col0);
    if constexpr (MODE == 2) s.ibase = uniform_ptr(p.inv_row + row0);
    s.ncol = __builtin_amdgcn_readfirstlane(N - col0 < BN ? N - col0 : BN);
  };
  // The loads of one stage: LPS per wave, A's row blocks first, then B's.
  struct Dma {
    __amdgpu_buffer_rsrc_t ra, rb;
    int8_t* base;
  };
  auto dma_setup = [&](int buf, const Src& s, int kt) __attribute__((always_inline)) {
    Dma d;
    d.base = smem + buf * STAGE + wave_s * 1024;
    d.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(s.abase + kt * BK2), 0, (int)kBufRecords,
                                             0x00020000);
    d.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(s.bbase + kt * BK2), 0,
                                             s.ncol * (int)p.ldb - kt * BK2, 0x00020000);
    return d;
  };
  auto dma_range = [&](const Dma& d, auto LO, auto HI) __attribute__((always_inline)) {
    static_for<decltype(LO)::value, decltype(HI)::value>([&](auto LI) __attribute__((always_inline)) {
      constexpr int l = decltype(LI)::value;
      if constexpr (l < A_INS)
        buffer_load_lds16(d.ra, d.base + l * NWAVES * 1024, a_off[l]);
      else
        buffer_load_lds16(d.rb, d.base + A_BYTES + (l - A_INS) * NWAVES * 1024, b_off[l - A_INS]);
    });
  };
  auto issue_ops = [&](int buf, const Src& s, int kt) __attribute__((always_inline)) {
    dma_range(dma_setup(buf, s, kt), std::integral_constant<int, 0>(), std::integral_constant<int, LPS>());
  };
  // the tile's row and column scales (and in MODE 2 the output scale
  // reciprocals) into slot s.slot: load k (k = q*4 + wave) covers entries
  // 64k .. 64k+63 of [rows | columns | reciprocals]
  auto issue_scales = [&](const Src& s) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
      const int k = q * NWAVES + wave_s;
      if (k < NSI) {
        __amdgpu_buffer_rsrc_t rs;
        if (k * 64 < BM) {
          rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s.rbase + k * 64), 0, 256, 0x00020000);
        } else if (MODE == 2 && k * 64 >= BM + BN) {
          rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s.ibase + (k * 64 - BM - BN)), 0, 256,
                                                 0x00020000);
        } else {
          const int c0 = k * 64 - BM;
          const int left = s.ncol - c0;
          rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s.cbase + c0), 0,
                                                 (left > 0 ? left : 0) * 4, 0x00020000);
        }
        buffer_load_lds4(rs, s_scl + s.slot * SCL + k * 64, lane4);
      }
    }
  };

  // ---- fragments: k-step t of a stage reads logical chunk 2t + lane/32 ----
  // Row bases are multiples of 32 (A) or of WTN (B), which keep (row/2)%8 equal
  // to (lrow/2)%8, so one per-lane chunk offset serves every fragment.
  int kc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) kc[t] = lrow * BK2 + (swz128(lrow, 2 * t + lhalf) << 4);
  const int a_row0 = wm * WTM * BK2, b_row0 = A_BYTES + wn * WTN * BK2;
  v4i fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto load_frags = [&](int buf, int t, v4i (&fa)[FM], v4i (&fb)[FN]) __attribute__((always_inline)) {
    const int8_t* sb = smem + buf * STAGE + kc[t];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const v4i*>(sb + a_row0 + i * 32 * BK2);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const v4i*>(sb + b_row0 + j * 32 * BK2);
  };
  v16i acc0[FM][FN], acc1[FM][FN];

  // ---- epilogue of the tile being drained ----
  struct Out {
    float* cbase;          // C at the tile's first row
    int voff[FN];          // this lane's column byte offset (+4 rows for lanes 32..63), or kBufInvalid
    uint32_t sr_base;      // LDS address of this lane's first row scale of the wave's rows
    uint32_t rk_base;      // LDS address of this lane's first row key of the wave's rows
    uint32_t sc_base;      // LDS address of this lane's column scale in the wave's first block column
    uint32_t iv_base;      // MODE 2: LDS address of this lane's first output scale reciprocal
    int8_t* qbase;         // MODE 2: the codes at the tile's first row
    unsigned int* pbase;   // MODE 1: this wave's row maxima of the tile (partial p = tn * WAVES_N + wn)
    int col0;              // the tile's first column
    int slot;              // scale / key slot of the tile
  };
  uint64_t tcol[FN];       // per-column hash sums of the tile being drained
  uint64_t lane_hash = 0;  // this lane's share of S over every drained tile
  auto make_out = [&](int r, int tm, int tn, Out& o) __attribute__((always_inline)) {
    const int row0 = tm * BM;
    o.slot = __builtin_amdgcn_readfirstlane(r % 3);
    if constexpr (MODE == 0) o.cbase = uniform_ptr(p.C + (int64_t)row0 * p.ldc);
    if constexpr (MODE == 1)
      o.pbase = uniform_ptr(p.rowmax + (int64_t)(tn * WAVES_N + wn_s) * M + row0 + wm_s * WTM);
    if constexpr (MODE == 2) {
      o.qbase = uniform_ptr(p.Q + (int64_t)row0 * p.ldq);
      o.iv_base = lds_addr(s_scl + o.slot * SCL + BM + BN) + (wm * WTM + lhalf * 4) * 4;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = tn * BN + wn * WTN + j * 32 + lrow;
      const bool ok = col < N;
      if constexpr (MODE == 2)
        o.voff[j] = ok ? (int)(lhalf * 4 * p.ldq + col) : kBufInvalid;
      else
        o.voff[j] = ok ? (int)(lhalf * 4 * ldc4 + col * 4) : kBufInvalid;
    }
    o.col0 = tn * BN;
    o.sr_base = lds_addr(s_scl + o.slot * SCL) + (wm * WTM + lhalf * 4) * 4;
    o.rk_base = lds_addr(s_rk + o.slot * BM) + (wm * WTM + lhalf * 4) * 4;
    o.sc_base = lds_addr(s_scl + o.slot * SCL + BM) + (wn * WTN + lrow) * 4;
    for (int rr = tid; rr < BM; rr += NT) s_rk[o.slot * BM + rr] = hash_row_key((unsigned int)(row0 + rr));
  };
  // Scales and row keys of the epilogue blocks, read and waited for inside
  // one asm statement each time (the compiler would otherwise wait for every
  // outstanding direct-to-LDS load before reading LDS that such loads write).
  // A half holds parts 2h and 2h+1 of a block: the row scales and row keys of
  // this lane's rows 16h + 4*(lane/32) + {0..3, 8..11}.
  struct DHalf {
    v4i sr[2];
    v4i rk[2];
    v4i iv[2];   // MODE 2: the output scale reciprocals of the same rows
  };
  // MODE 2: the reciprocals of a half, at the same offset as its row scales
  auto read_iv = [&](const Out& o, auto OFF, DHalf& d) __attribute__((always_inline)) {
    constexpr int off = decltype(OFF)::value;
    asm volatile(
        "ds_read_b128 %[i0], %[iv] offset:%[o0]\n\t"
        "ds_read_b128 %[i1], %[iv] offset:%[o1]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [i0] "=&v"(d.iv[0]), [i1] "=&v"(d.iv[1])
        : [iv] "v"(o.iv_base), [o0] "i"(off), [o1] "i"(off + 32));
  };
  // Byte offsets (immediates of the LDS reads): the row scales / keys of half
  // h of block row i start 32i + 16h rows into the wave's rows; the column
  // scale of block column j is 32j columns into the wave's columns.
  auto read_late_early = [&](const Out& o1, auto B, DHalf& late, const Out& o2, auto C, DHalf& early,
                             int& sc) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value, c = decltype(C)::value;
    constexpr int ol = (b / FN) * 128 + 64, oe = (c / FN) * 128, oc = (c % FN) * 128;
    asm volatile(
        "ds_read_b128 %[l0], %[sr1] offset:%[ol0]\n\t"
        "ds_read_b128 %[l1], %[sr1] offset:%[ol1]\n\t"
        "ds_read_b128 %[l2], %[rk1] offset:%[ol0]\n\t"
        "ds_read_b128 %[l3], %[rk1] offset:%[ol1]\n\t"
        "ds_read_b128 %[e0], %[sr2] offset:%[oe0]\n\t"
        "ds_read_b128 %[e1], %[sr2] offset:%[oe1]\n\t"
        "ds_read_b128 %[e2], %[rk2] offset:%[oe0]\n\t"
        "ds_read_b128 %[e3], %[rk2] offset:%[oe1]\n\t"
        "ds_read_b32 %[sc], %[sc2] offset:%[oc]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [l0] "=&v"(late.sr[0]), [l1] "=&v"(late.sr[1]), [l2] "=&v"(late.rk[0]),
          [l3] "=&v"(late.rk[1]), [e0] "=&v"(early.sr[0]), [e1] "=&v"(early.sr[1]),
          [e2] "=&v"(early.rk[0]), [e3] "=&v"(early.rk[1]), [sc] "=&v"(sc)
        : [sr1] "v"(o1.sr_base), [rk1] "v"(o1.rk_base), [sr2] "v"(o2.sr_base),
          [rk2] "v"(o2.rk_base), [sc2] "v"(o2.sc_base), [ol0] "i"(ol), [ol1] "i"(ol + 32),
          [oe0] "i"(oe), [oe1] "i"(oe + 32), [oc] "i"(oc));
    if constexpr (MODE == 2) {
      read_iv(o1, std::integral_constant<int, ol>(), late);
      read_iv(o2, std::integral_constant<int, oe>(), early);
    }
  };
  // the second half of block b of o
  auto read_late = [&](const Out& o, auto B, DHalf& late) __attribute__((always_inline)) {
    constexpr int b = decltype(B)::value;
    constexpr int ol = (b / FN) * 128 + 64;
    asm volatile(
        "ds_read_b128 %[l0], %[sr] offset:%[o0]\n\t"
        "ds_read_b128 %[l1], %[sr] offset:%[o1]\n\t"
        "ds_read_b128 %[l2], %[rk] offset:%[o0]\n\t"
        "ds_read_b128 %[l3], %[rk] offset:%[o1]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [l0] "=&v"(late.sr[0]), [l1] "=&v"(late.sr[1]), [l2] "=&v"(late.rk[0]),
          [l3] "=&v"(late.rk[1])
        : [sr] "v"(o.sr_base), [rk] "v"(o.rk_base), [o0] "i"(ol), [o1] "i"(ol + 32));
    if constexpr (MODE == 2) read_iv(o, std::integral_constant<int, ol>(), late);
  };
  // the first half and column scale of block c of o
  auto read_early = [&](const Out& o, auto C, DHalf& early, int& sc) __attribute__((always_inline)) {
    constexpr int c = decltype(C)::value;
    constexpr int oe = (c / FN) * 128, oc = (c % FN) * 128;
    asm volatile(
        "ds_read_b128 %[e0], %[sr] offset:%[o0]\n\t"
        "ds_read_b128 %[e1], %[sr] offset:%[o1]\n\t"
        "ds_read_b128 %[e2], %[rk] offset:%[o0]\n\t"
        "ds_read_b128 %[e3], %[rk] offset:%[o1]\n\t"
        "ds_read_b32 %[sc], %[sca] offset:%[oc]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [e0] "=&v"(early.sr[0]), [e1] "=&v"(early.sr[1]), [e2] "=&v"(early.rk[0]),
          [e3] "=&v"(early.rk[1]), [sc] "=&v"(sc)
        : [sr] "v"(o.sr_base), [rk] "v"(o.rk_base), [sca] "v"(o.sc_base), [o0] "i"(oe),
          [o1] "i"(oe + 32), [oc] "i"(oc));
    if constexpr (MODE == 2) read_iv(o, std::integral_constant<int, oe>(), early);
  };
  // Element 4q+e of block b = (i, j) of accumulator set Y: lane l holds
  // column l % 32 and row 8q + 4*(l/32) + e of the block.
  // The four elements of part q of block b = (i, j), in steps spread over the
  // slots of a k-step so that the four dependency chains overlap each other
  // and the MFMAs: step 0 converts the accumulators, 1 applies the row
  // scales, 2 the column scale (and ReLU), 3 adds the hash terms of elements
  // 0-1 and stores them, 4 the same for elements 2-3.
  unsigned int rmx[FM][16];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) rmx[i][v] = 0u;
  float xq[4];
  auto drain_step = [&](v16i (&Y)[FM][FN], const Out& o, const DHalf& d, int scb, auto IJ, auto Q,
                        auto STEP) __attribute__((always_inline)) {
    constexpr int b = decltype(IJ)::value, q = decltype(Q)::value, st = decltype(STEP)::value;
    constexpr int i = b / FN, j = b % FN;
    if constexpr (st == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) xq[e] = (float)Y[i][j][q * 4 + e];
    } else if constexpr (st == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) xq[e] = mul_rn(xq[e], __int_as_float(d.sr[q % 2][e]));
    } else if constexpr (st == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xq[e] = mul_rn(xq[e], __int_as_float(scb));
        if (RELU) xq[e] = relu_pos0(xq[e]);
      }
    } else if constexpr (MODE == 1) {
      constexpr int e0 = (st - 3) * 2;
#pragma unroll
      for (int e = e0; e < e0 + 2; ++e) {
        const unsigned int a = __float_as_uint(xq[e]) & 0x7FFFFFFFu;
        rmx[i][q * 4 + e] = a > rmx[i][q * 4 + e] ? a : rmx[i][q * 4 + e];
      }
    } else if constexpr (MODE == 2) {
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(o.qbase + (int64_t)(wm_s * WTM + i * 32) * p.ldq), 0, (int)kBufRecords, 0x00020000);
      constexpr int e0 = (st - 3) * 2;
#pragma unroll
      for (int e = e0; e < e0 + 2; ++e) {
        tcol[j] += (uint64_t)(unsigned int)d.rk[q % 2][e] * (uint64_t)__float_as_uint(xq[e]);
        const int qv = quantize1(xq[e], __int_as_float(d.iv[q % 2][e]));
        __builtin_amdgcn_raw_buffer_store_b8((unsigned char)qv, rsrc, o.voff[j], (q * 8 + e) * (int)p.ldq, 0);
      }
      if constexpr (st == 4) asm volatile("" : "+v"(tcol[j]));
    } else {
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(o.cbase + (int64_t)(wm_s * WTM + i * 32) * p.ldc), 0, (int)kBufRecords,
          0x00020000);
      constexpr int e0 = (st - 3) * 2;
#pragma unroll
      for (int e = e0; e < e0 + 2; ++e) {
        tcol[j] += (uint64_t)(unsigned int)d.rk[q % 2][e] * (uint64_t)__float_as_uint(xq[e]);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(xq[e]), rsrc, o.voff[j], (q * 8 + e) * (int)ldc4,
                                              NTSTORE ? kStoreNT : 0);
      }
      if constexpr (st == 4) asm volatile("" : "+v"(tcol[j]));
    }
  };
  // MODE 1: the maxima of |y| of the tile being drained, over this lane's
  // column, per element row of each block row: rows 8q + 4*(lane/32) + e of
  // block row i in rmx[i][4q + e].  close_tile_max reduces them over the 32
  // lanes of each half-wave (four halving exchanges, then a last one between
  // lane pairs, after which lanes 2v and 2v+1 hold the maximum of element
  // row v) and stores one word per row: the wave's partial maximum of that
  // row over its WTN columns of the tile.
  auto close_tile_max = [&](const Out& o) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      unsigned int x8[8], x4[4], x2[2];
      const bool b4 = (lrow & 16) != 0, b3 = (lrow & 8) != 0, b2 = (lrow & 4) != 0, b1 = (lrow & 2) != 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const unsigned int keep = b4 ? rmx[i][8 + k] : rmx[i][k];
        const unsigned int give = b4 ? rmx[i][k] : rmx[i][8 + k];
        const unsigned int got = (unsigned int)__shfl_xor((int)give, 16, 64);
        x8[k] = got > keep ? got : keep;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const unsigned int keep = b3 ? x8[4 + k] : x8[k];
        const unsigned int give = b3 ? x8[k] : x8[4 + k];
        const unsigned int got = (unsigned int)__shfl_xor((int)give, 8, 64);
        x4[k] = got > keep ? got : keep;
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const unsigned int keep = b2 ? x4[2 + k] : x4[k];
        const unsigned int give = b2 ? x4[k] : x4[2 + k];
        const unsigned int got = (unsigned int)__shfl_xor((int)give, 4, 64);
        x2[k] = got > keep ? got : keep;
      }
      unsigned int m;
      {
        const unsigned int keep = b1 ? x2[1] : x2[0];
        const unsigned int give = b1 ? x2[0] : x2[1];
        const unsigned int got = (unsigned int)__shfl_xor((int)give, 2, 64);
        m = got > keep ? got : keep;
      }
      const unsigned int other = (unsigned int)__shfl_xor((int)m, 1, 64);
      m = other > m ? other : m;
      // element row v = 8*b4 + 4*b3 + 2*b2 + b1 of this half: block row
      // 8*(v/4) + 4*(lane/32) + v%4
      const int v = (lrow >> 1) & 15;
      const int row = i * 32 + 8 * (v >> 2) + 4 * lhalf + (v & 3);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(o.pbase, 0, (int)kBufRecords, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b32(m, rs, (lrow & 1) == 0 ? row * 4 : kBufInvalid, 0, 0);
#pragma unroll
      for (int k = 0; k < 16; ++k) rmx[i][k] = 0u;
    }
  };
  auto close_tile_hash = [&](const Out& o) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = o.col0 + wn * WTN + j * 32 + lrow;
      lane_hash += (col < N ? hash_col_key((uint64_t)col) : 0ull) * tcol[j];
      tcol[j] = 0;
    }
  };

  // One k-step, laid out slot by slot (a scheduling fence after each): slot m
  // issues MFMA m of X (fragments fa/fb); slots 0-2 read the next k-step's
  // fragments (stage buffer nbuf, k-step nt) into na/nb; with a stage to
  // fetch, slots 0-4 issue its loads; slot(m) adds the epilogue work of the
  // slot.  Fixing the order keeps the two fragment sets in distinct registers
  // and the reads one to five MFMAs ahead of their use.
  constexpr int NSLOT = FM * FN;
  static_assert(NSLOT >= 4, "the epilogue's five steps need at least four slots");
  constexpr int LPSL = (LPS + NSLOT - 2) / (NSLOT - 1);   // loads per slot, slots 0 .. NSLOT-2
  // With three or more slots a stage's loads are split: the first LH, one
  // per slot, in k-step 3 after the barrier that frees their slot, the rest
  // in k-step 0 of the next stage (they still have ~1.75 stages to land).
  // Spread over ten MFMAs instead of five, the loads stall the one wave of
  // each SIMD less: measured 3-6% faster on the 128x192 tile (down-projection
  // 30.8 -> 29.8 us, LM-head weight gradient 417 -> 400 us).  The stores
  // counted in the waits are unchanged: the next stage's share is issued in
  // its slots 0-3, before that stage's first epilogue stores.
  constexpr bool SPLIT = STAGES >= 3 && LPS > NSLOT;
  constexpr int LH = SPLIT ? NSLOT : LPS;
  // MODE 1 with two workgroups per CU drains each tile right after its last
  // k-step instead of under the next tile's MFMAs: no second accumulator set
  // is live across the main loop (the interleaved drain's row maxima and
  // both sets exceed the 256 registers of a wave at two waves per SIMD), and
  // the other workgroup's MFMAs keep the SIMD busy meanwhile.
  constexpr bool SYNC = MODE == 1 && WPC >= 2;
  auto kstep = [&](v16i (&X)[FM][FN], const v4i (&fa)[FM], const v4i (&fb)[FN], auto ZERO, int nbuf,
                   int nt, v4i (&na)[FM], v4i (&nb)[FN], auto DMA, const Dma& dm, bool dma_on, auto LB, auto LE,
                   auto&& slot)
      __attribute__((always_inline)) {
    constexpr bool zero = decltype(ZERO)::value, dma = decltype(DMA)::value;
    const int8_t* sb = smem + nbuf * STAGE + kc[nt];
    static_for<0, NSLOT>([&](auto MI) __attribute__((always_inline)) {
      constexpr int m = decltype(MI)::value, i = m / FN, j = m % FN;
      X[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], zero ? v16i{} : X[i][j], 0, 0, 0);
      constexpr int r0 = 2 * m, r1 = (2 * m + 2 < FM + FN) ? 2 * m + 2 : FM + FN;
      static_for<r0, r1>([&](auto RI) __attribute__((always_inline)) {
        constexpr int r = decltype(RI)::value;
        if constexpr (r < FM)
          na[r] = *reinterpret_cast<const v4i*>(sb + a_row0 + r * 32 * BK2);
        else
          nb[r - FM] = *reinterpret_cast<const v4i*>(sb + b_row0 + (r - FM) * 32 * BK2);
      });
      if constexpr (dma) {   // loads [LB, LE) of a stage, LPSL (one when split) per slot
        constexpr int lb = decltype(LB)::value, le = decltype(LE)::value;
        constexpr int per = SPLIT ? 1 : LPSL;
        constexpr int l0 = lb + m * per < le ? lb + m * per : le;
        constexpr int l1 = lb + (m + 1) * per < le ? lb + (m + 1) * per : le;
        if (dma_on) dma_range(dm, std::integral_constant<int, l0>(), std::integral_constant<int, l1>());
      }
      slot(MI);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // the stage whose loads [LH, LPS) are still to be issued (SPLIT)
  Dma dm_prev{};
  bool dm_pend = false;
  // ---- the fetch cursor: the tile and stage whose loads are issued next ----
  Src fsrc;
  int fr = 0, fkt = 0;
  auto advance_fetch = [&]() __attribute__((always_inline)) {
    ++fkt;
    if (fkt == nst) {
      if (fr + 1 < my_tiles) {
        ++fr;
        int a, b;
        tile_coords(fr, a, b);
        make_src(fr, a, b, fsrc);
        fkt = 0;
        issue_scales(fsrc);
      } else {
        fkt = nst - 1;   // past the end: repeat a stage into a slot that is never read
      }
    }
  };

  // One stage g of tile r (tile-local position s).  X accumulates tile r.
  // If DRAIN, block BLK of Y (tile r-1, Out oy) is drained: parts 0-1 with
  // the operand half `early` (read during the previous stage), parts 2-3 with
  // `late`, which mid() reads just before the barrier together with the next
  // stage's early half.  ST: stage g+1's loads are waited for with this many
  // later memory operations allowed outstanding, a lower bound of those
  // issued after them: the loads of the STAGES-2 stages issued since, the
  // previous stage's stores that follow them (PREV_ST) and the stores of
  // k-steps 0-2 of this one, stores counted only where those stages drain.
  auto stage = [&](v16i (&X)[FM][FN], v16i (&Y)[FM][FN], int g, const Out& oy, const DHalf& early,
                   int scb, DHalf& late, auto FIRST, auto DRAIN, auto BLK, auto STV, auto&& mid)
      __attribute__((always_inline)) {
    constexpr bool D = decltype(DRAIN)::value;
    constexpr int ST = decltype(STV)::value;
    const int buf = g % STAGES;
    // epilogue part q: steps 0-4 of its four elements in slots 0-4
    auto part = [&](auto Q) __attribute__((always_inline)) {
      return [&, Q](auto MI) __attribute__((always_inline)) {
        constexpr int m = decltype(MI)::value, q = decltype(Q)::value;
        auto step = [&](auto STEP) __attribute__((always_inline)) {
          if constexpr (q < 2)
            drain_step(Y, oy, early, scb, BLK, Q, STEP);
          else
            drain_step(Y, oy, late, scb, BLK, Q, STEP);
        };
        if constexpr (D && m <= 4) step(std::integral_constant<int, m>());
        // four slots (2x2 blocks per wave): the last one takes steps 3 and 4
        if constexpr (D && NSLOT == 4 && m == 3) step(std::integral_constant<int, 4>());
      };
    };
    const Dma none{};
    kstep(X, fa0, fb0, FIRST, buf, 1, fa1, fb1, std::integral_constant<bool, SPLIT>(), dm_prev, dm_pend,
          std::integral_constant<int, LH>(), std::integral_constant<int, LPS>(), part(std::integral_constant<int, 0>()));
    kstep(X, fa1, fb1, std::false_type(), buf, 2, fa0, fb0, std::false_type(), none, false,
          std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), part(std::integral_constant<int, 1>()));
    mid();   // epilogue operands (read and waited for)
    kstep(X, fa0, fb0, std::false_type(), buf, 3, fa1, fb1, std::false_type(), none, false,
          std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), part(std::integral_constant<int, 2>()));
    // This wave's reads of stage g are complete and stage g+1 has landed for
    // it; after the barrier, for every wave: stage g's slot is free and
    // stage g+1 can be read.
    wait_vmcnt_lgkm0<ST>();
    barrier_nofence();
    // k-step 3 reads k-step 0 of stage g+1 and loads stage g+3 into stage g's slot
    const Dma dm = dma_setup(buf, fsrc, fkt);
    kstep(X, fa1, fb1, std::false_type(), (g + 1) % STAGES, 0, fa0, fb0, std::true_type(), dm, true,
          std::integral_constant<int, 0>(), std::integral_constant<int, LH>(), part(std::integral_constant<int, 3>()));
    dm_prev = dm;
    dm_pend = true;
    advance_fetch();
  };

  // One tile r: X accumulates it; if DRAIN, Y (tile r-1, Out out_prev) is
  // drained during its first NB stages.  The early halves alternate between
  // (e0, s0) and (e1, s1); block 0 of a tile always uses (e0, s0).
  DHalf e0, e1, late;
  int s0 = 0, s1 = 0;
  Out out_cur, out_prev;
  // a workgroup without tiles stores nothing: every offset lies outside the range
  out_cur.cbase = p.C;
  out_cur.qbase = p.Q;
  out_cur.pbase = p.rowmax;
#pragma unroll
  for (int j = 0; j < FN; ++j) out_cur.voff[j] = kBufInvalid;
  out_cur.sr_base = out_cur.rk_base = out_cur.sc_base = out_cur.iv_base = 0;
  out_cur.col0 = 0;
  out_cur.slot = 0;
  // Stores of the previous stage issued after the loads a stage waits for:
  // all sixteen with three or more slots (those loads were issued a stage
  // earlier), with two slots only the four of its k-step 3 (the loads share
  // that k-step and precede its stores).  MODE 1 drains without stores.
  // MODE 1 drains without stores; MODE 2 stores its codes one byte per
  // element, as many stores as MODE 0.
  constexpr int PREV_ST = MODE == 1 ? 0 : (STAGES >= 3 ? 16 : 4);
  constexpr int CUR_ST = MODE == 1 ? 0 : 12;   // stores of k-steps 0-2 of a draining stage
  auto run_tile = [&](v16i (&X)[FM][FN], v16i (&Y)[FM][FN], int r, auto DRAIN)
      __attribute__((always_inline)) {
    constexpr bool D = decltype(DRAIN)::value;
    const int g0 = r * nst;
    const bool has_next = r + 1 < my_tiles;
    static_for<0, NB>([&](auto BI) __attribute__((always_inline)) {
      constexpr int b = decltype(BI)::value;
      constexpr int ST = (STAGES - 2) * LPS + (D && b >= 1 ? PREV_ST : 0) + (D ? CUR_ST : 0);
      DHalf& ec = (b % 2 == 0) ? e0 : e1;
      DHalf& en = (b % 2 == 0) ? e1 : e0;
      int& sc_c = (b % 2 == 0) ? s0 : s1;
      int& sc_n = (b % 2 == 0) ? s1 : s0;
      auto mid = [&]() __attribute__((always_inline)) {
        if constexpr (D && b + 1 < NB) {
          read_late_early(out_prev, BI, late, out_prev, std::integral_constant<int, b + 1>(), en, sc_n);
        } else if constexpr (D) {
          // last block; if nst == NB the next stage is the next tile's first,
          // which drains block 0 of this tile
          if (nst == NB && has_next)
            read_late_early(out_prev, BI, late, out_cur, std::integral_constant<int, 0>(), en, sc_n);
          else
            read_late(out_prev, BI, late);
        } else if constexpr (b + 1 == NB && !SYNC) {
          if (nst == NB && has_next) read_early(out_cur, std::integral_constant<int, 0>(), en, sc_n);
        }
      };
      stage(X, Y, g0 + b, out_prev, ec, sc_c, late, std::integral_constant<bool, b == 0>(), DRAIN, BI,
            std::integral_constant<int, ST>(), mid);
    });
    if (D) {
      if constexpr (MODE == 1)
        close_tile_max(out_prev);
      else
        close_tile_hash(out_prev);
    }
    static_assert(NB % 2 == 0, "stage NB (if any) finds its next early half in e0");
    for (int s = NB; s < nst; ++s) {
      auto mid = [&]() __attribute__((always_inline)) {
        if constexpr (!SYNC)
          if (s + 1 == nst && has_next) read_early(out_cur, std::integral_constant<int, 0>(), e0, s0);
      };
      if (s == NB)
        stage(X, Y, g0 + s, out_prev, e0, s0, late, std::false_type(), std::false_type(),
              std::integral_constant<int, 0>(), std::integral_constant<int, (STAGES - 2) * LPS + (D ? PREV_ST : 0)>(), mid);
      else
        stage(X, Y, g0 + s, out_prev, e0, s0, late, std::false_type(), std::false_type(),
              std::integral_constant<int, 0>(), std::integral_constant<int, (STAGES - 2) * LPS>(), mid);
    }
  };

  // SYNC: the row maxima of tile o (in acc0) right after its last k-step.
  // Loads of later stages may still be landing in LDS, so the scales are
  // read by asm statements that wait for the LDS reads only.
  auto sync_max = [&](const Out& o) __attribute__((always_inline)) {
    static_for<0, FM>([&](auto II) __attribute__((always_inline)) {
      constexpr int i = decltype(II)::value;
      v4i sr[4];
      asm volatile(
          "ds_read_b128 %[s0], %[sr] offset:%[o0]\n\t"
          "ds_read_b128 %[s1], %[sr] offset:%[o1]\n\t"
          "ds_read_b128 %[s2], %[sr] offset:%[o2]\n\t"
          "ds_read_b128 %[s3], %[sr] offset:%[o3]\n\t"
          "s_waitcnt lgkmcnt(0)"
          : [s0] "=&v"(sr[0]), [s1] "=&v"(sr[1]), [s2] "=&v"(sr[2]), [s3] "=&v"(sr[3])
          : [sr] "v"(o.sr_base), [o0] "i"(i * 128), [o1] "i"(i * 128 + 32), [o2] "i"(i * 128 + 64),
            [o3] "i"(i * 128 + 96));
      static_for<0, FN>([&](auto JJ) __attribute__((always_inline)) {
        constexpr int j = decltype(JJ)::value;
        int sc;
        asm volatile("ds_read_b32 %[sc], %[sca] offset:%[oc]\n\ts_waitcnt lgkmcnt(0)"
                     : [sc] "=&v"(sc)
                     : [sca] "v"(o.sc_base), [oc] "i"(j * 128));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float y = epilogue1(acc0[i][j][v], __int_as_float(sr[v >> 2][v & 3]), __int_as_float(sc));
          if (RELU) y = relu_pos0(y);
          const unsigned int a = __float_as_uint(y) & 0x7FFFFFFFu;
          rmx[i][v] = a > rmx[i][v] ? a : rmx[i][v];
        }
      });
    });
    close_tile_max(o);
  };

  if (my_tiles > 0) {
    int tm, tn;
    tile_coords(0, tm, tn);
    make_src(0, tm, tn, fsrc);
    make_out(0, tm, tn, out_cur);
    // prologue: scales and the first STAGES stages of tile 0
    issue_scales(fsrc);
    static_for<0, STAGES>([&](auto SI) __attribute__((always_inline)) {
      issue_ops(decltype(SI)::value, fsrc, decltype(SI)::value);
    });
    fkt = STAGES;   // nst >= STAGES
    wait_vmcnt_lgkm0<(STAGES - 1) * LPS>();   // stage 0 landed; the row keys of tile 0 written
    barrier_nofence();
    load_frags(0, 0, fa0, fb0);
#pragma unroll
    for (int j = 0; j < FN; ++j) tcol[j] = 0;

    run_tile(acc0, acc1, 0, std::false_type());
    if constexpr (SYNC) {
      for (int r = 1; r < my_tiles; ++r) {
        sync_max(out_cur);
        int a, b;
        tile_coords(r, a, b);
        make_out(r, a, b, out_cur);
        run_tile(acc0, acc1, r, std::false_type());
      }
    } else {
      for (int r = 1; r < my_tiles; ++r) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc1[i][j] = acc0[i][j];
        out_prev = out_cur;
        int a, b;
        tile_coords(r, a, b);
        make_out(r, a, b, out_cur);
        run_tile(acc0, acc1, r, std::true_type());
      }
    }
    // The last tile: no MFMAs left to hide its epilogue under.  Its hash
    // terms come first and its stores last, so that publishing this
    // workgroup's share of S (whose acknowledgement the ticket waits for,
    // and vmcnt retires in order) does not wait behind the tile's stores.
    // Every direct-to-LDS load has landed here, so plain LDS reads are used.
    wait_vmcnt<0>();
    if constexpr (SYNC) {
      sync_max(out_cur);
    } else if constexpr (MODE == 1) {
      static_for<0, NB>([&](auto BI) __attribute__((always_inline)) {
        constexpr int b = decltype(BI)::value, i = b / FN, j = b % FN;
        const int r0 = wm * WTM + i * 32 + lhalf * 4;
        const float* srp = s_scl + out_cur.slot * SCL + r0;
        const float sc = s_scl[out_cur.slot * SCL + BM + wn * WTN + j * 32 + lrow];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = (v >> 2) * 8 + (v & 3);
          float y = epilogue1(acc0[i][j][v], srp[rr], sc);
          if (RELU) y = relu_pos0(y);
          const unsigned int a = __float_as_uint(y) & 0x7FFFFFFFu;
          rmx[i][v] = a > rmx[i][v] ? a : rmx[i][v];
        }
      });
      close_tile_max(out_cur);
    } else if (p.do_hash) {
      static_for<0, NB>([&](auto BI) __attribute__((always_inline)) {
        constexpr int b = decltype(BI)::value, i = b / FN, j = b % FN;
        const int r0 = wm * WTM + i * 32 + lhalf * 4;
        const float* srp = s_scl + out_cur.slot * SCL + r0;
        const unsigned int* rkp = s_rk + out_cur.slot * BM + r0;
        const float sc = s_scl[out_cur.slot * SCL + BM + wn * WTN + j * 32 + lrow];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = (v >> 2) * 8 + (v & 3);
          float y = epilogue1(acc0[i][j][v], srp[rr], sc);
          if (RELU) y = relu_pos0(y);
          tcol[j] += (uint64_t)rkp[rr] * (uint64_t)__float_as_uint(y);
        }
      });
      close_tile_hash(out_cur);
    }
  }
  // The grid-wide sum of S (see hash_share_and_finalize), with its two
  // round trips to the coherence point overlapped with the last tile's
  // stores: thread 0 stores this workgroup's share; wave 0 then issues the
  // stores of the first half of its blocks (vmcnt retires in order, so
  // waiting until at most those stores are outstanding means the share is
  // acknowledged), takes its ticket, and issues the second half before it
  // needs the ticket's value.
  // pass 1 of the requantizing epilogue ends here: no output, no hash
  if constexpr (MODE == 1) return;
  constexpr int HALF = NB / 2;
  auto store_block = [&](auto BI) __attribute__((always_inline)) {
    constexpr int b = decltype(BI)::value, i = b / FN, j = b % FN;
    const int r0 = wm * WTM + i * 32 + lhalf * 4;
    const float* srp = s_scl + out_cur.slot * SCL + r0;
    const float sc = s_scl[out_cur.slot * SCL + BM + wn * WTN + j * 32 + lrow];
    if constexpr (MODE == 2) {
      const float* ivp = s_scl + out_cur.slot * SCL + BM + BN + r0;
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(out_cur.qbase + (int64_t)(wm_s * WTM + i * 32) * p.ldq), 0, (int)kBufRecords, 0x00020000);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = (v >> 2) * 8 + (v & 3);
        float y = epilogue1(acc0[i][j][v], srp[rr], sc);
        if (RELU) y = relu_pos0(y);
        const int qv = quantize1(y, ivp[rr]);
        __builtin_amdgcn_raw_buffer_store_b8((unsigned char)qv, rq, out_cur.voff[j], rr * (int)p.ldq, 0);
      }
      return;
    }
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(out_cur.cbase + (int64_t)(wm_s * WTM + i * 32) * p.ldc), 0, (int)kBufRecords,
        0x00020000);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rr = (v >> 2) * 8 + (v & 3);
      float y = epilogue1(acc0[i][j][v], srp[rr], sc);
      if (RELU) y = relu_pos0(y);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), rsrc, out_cur.voff[j], rr * (int)ldc4,
                                            NTSTORE ? kStoreNT : 0);
    }
  };
  // The share store and the ticket are issued by every lane of every wave,
  // with offsets outside their buffers (dropped stores, no-op atomics) for
  // all but thread 0: no branch, so the ticket's value is waited for only
  // where it is used.
  uint64_t part = 0;
  if (p.do_hash) part = block_sum_u64<NT>(lane_hash, s_red);   // ends with a barrier
  const bool t0h = p.do_hash && tid == 0;
  {
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(p.hash_parts), 0, (int)kBufRecords, 0x00020000);
    const v2u pv = {(unsigned int)part, (unsigned int)(part >> 32)};
    __builtin_amdgcn_raw_buffer_store_b64(pv, rs, t0h ? (int)blockIdx.x * 8 : kBufInvalid, 0, 16 /* sc1 */);
  }
  asm volatile("" ::: "memory");
  static_for<0, HALF>(store_block);
  asm volatile("" ::: "memory");
  wait_vmcnt<HALF * 16>();   // the share store has been acknowledged
  const __amdgpu_buffer_rsrc_t rt =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.ticket), 0, (int)kBufRecords, 0x00020000);
  const unsigned int ticket = (unsigned int)buffer_atomic_add_ret(rt, 1, t0h ? 0 : kBufInvalid);
  asm volatile("" ::: "memory");
  static_for<HALF, NB>(store_block);
  asm volatile("" ::: "memory");
  if (p.do_hash) {
    int* flag = reinterpret_cast<int*>(s_red + NWAVES);
    if (threadIdx.x == 0) *flag = (ticket == (unsigned int)(p.n_shares - 1));
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only: the flag is written
    barrier_nofence();
    if (*flag) {   // the last workgroup: every other share is complete
      uint64_t t = 0;
      for (int k = tid; k < p.n_shares; k += NT)
        t += __hip_atomic_load(p.hash_parts + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      t = block_sum_u64<NT>(t, s_red);
      if (threadIdx.x == 0) {
        *p.hash_out = hash_finalize(t, (uint64_t)M, (uint64_t)N);
        __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// split-K combine: acc = sum over splits (exact), then the same epilogue and
// hash shares as the GEMM kernel; each thread owns 4 consecutive columns of a
// band of p.comb_rows rows (chosen so that the grid has about a thousand
// workgroups: the sums are memory-bound and need the whole chip).
// ---------------------------------------------------------------------------
constexpr int COMB_ROWS_MAX = 32;

__global__ void __launch_bounds__(256)
splitk_combine_kernel(const GemmParams p) {
  __shared__ unsigned long long red[4];
  const int M = p.M, N = p.N;
  const int tid = threadIdx.x;
  const int c0 = (blockIdx.x * 256 + tid) * 4;
  const int r0 = blockIdx.y * p.comb_rows;
  const int r1 = r0 + p.comb_rows < M ? r0 + p.comb_rows : M;
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
      int sp = 0;
      if (vec) {
        // four splits' loads in flight together (integer sums: exact in any
        // order)
        for (; sp + 4 <= p.splits; sp += 4) {
          v4i v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + (sp + u) * plane));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            a[0] += v[u][0]; a[1] += v[u][1]; a[2] += v[u][2]; a[3] += v[u][3];
          }
        }
      }
      for (; sp < p.splits; ++sp) {
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
  if (p.do_hash) {
    uint64_t part = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c0 + e < N) part += hash_col_key((uint64_t)(c0 + e)) * t[e];
    // this workgroup's share; hash_parts_finalize_kernel, the next launch,
    // sums the shares (no cross-workgroup wait at the end of this kernel,
    // whose workgroups all finish together)
    part = block_sum_u64<256>(part, red);
    if (tid == 0) p.hash_parts[blockIdx.y * gridDim.x + blockIdx.x] = part;
  }
}

// H from the n shares of S written by the previous launch.
__global__ void __launch_bounds__(256)
hash_parts_finalize_kernel(const unsigned long long* __restrict__ parts, int n, uint64_t M, uint64_t N,
                           uint64_t* hash_out) {
  __shared__ unsigned long long red[4];
  uint64_t s = 0;
  for (int i0 = 0; i0 < n; i0 += 256 * 8) {   // eight loads in flight per thread
    uint64_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = i0 + k * 256 + (int)threadIdx.x;
      v[k] = i < n ? parts[i] : 0ull;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  s = block_sum_u64<256>(s, red);
  if (threadIdx.x == 0) *hash_out = hash_finalize(s, M, N);
}

hipError_t launch_hash_parts_finalize(const unsigned long long* parts, int n, int64_t M, int64_t N,
                                      uint64_t* hash_out, hipStream_t stream) {
  hipLaunchKernelGGL(hash_parts_finalize_kernel, dim3(1), dim3(256), 0, stream, parts, n, (uint64_t)M,
                     (uint64_t)N, hash_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host side: plan and launch
// ---------------------------------------------------------------------------
// Tile configurations: macro tile, LDS stages, workgroups resident per CU,
// and the int8 MAC rate one workgroup sustains in the steady-state loop
// (measured on MI355X with operands streaming through L2: LM-head weight
// gradient 768x50304x8192, down-projection 8192x768x3072).
// Tile configurations and the cost model that picks one.  Estimated time of
// a non-persistent plan: rounds of resident workgroups x (MAC time of a tile
// at `wg_macs` + its output tile at `wg_out_bw`); of a persistent plan:
// tiles per workgroup x (MAC time + `tile_overhead`).  The rates were fitted
// to timings on MI355X of the GPT-2-small shapes (8192x3072x768,
// 8192x768x3072, 8192x50304x768, 768x50304x8192): at K = 768 the epilogue
// and output write cost as much as the MACs.  A persistent configuration with two
// workgroups per CU runs twice as many at once (grid = 2 x CUs), each at about
// half the MAC rate.
struct TileCfg {
  int bm, bn, per_cu;
  double wg_macs;        // MAC/s of one resident workgroup in its main loop
  double wg_out_bw;      // bytes/s of output one workgroup writes in its epilogue
  double tile_overhead;  // persistent: seconds per tile beyond its MACs
  double tile_overhead_nt;  // the same with nontemporal output stores (outputs > 128 MB)
  bool persistent;       // one workgroup per CU walking tiles, epilogue drained under the next tile
  int kstage;            // bytes of K per LDS stage
};
static const TileCfg kCfgs[] = {
    {256, 256, 1, 4.5e12, 20e9, 0, 0, false, 64},    // eight waves (two per SIMD), 128x64 each
    {256, 128, 1, 3.3e12, 9.8e9, 0, 0, false, 64},   // four waves, 128x64 each
    {128, 128, 2, 1.43e12, 6.9e9, 0, 0, false, 64},  // four waves, 64x64 each
    {256, 256, 1, 4.0e12, 20e9, 0, 0, false, 64},    // four waves, 128x128 each (tests only)
    {256, 128, 1, 3.0e12, 0, 6.0e-6, 6.0e-6, true, 64},   // persistent, 128x64 per wave (tests only)
    {128, 192, 1, 3.0e12, 0, 5.2e-6, 5.2e-6, true, 64},   // persistent, four waves, 64x96 each
    {128, 192, 1, 3.7e12, 0, 5.5e-6, 2.1e-6, true, 128},  // persistent, 128-byte stages, 64x96 per wave
    {128, 128, 2, 1.75e12, 0, 4.5e-6, 1.3e-6, true, 128}, // the same, 64x64 per wave, two workgroups per CU
};
constexpr int kNumCfgs = kNumGemmCfgs;
static_assert(sizeof(kCfgs) / sizeof(kCfgs[0]) == kNumCfgs, "one entry per configuration");
constexpr int kPersistStages = 4;

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Plan overrides set by i8g_set_test_overrides (tests only; the output
// never depends on the plan).  Read once per plan, never from the
// environment.
static std::atomic<int> g_force_tile{-1}, g_force_splits{0}, g_qcols_path{0}, g_int4_direct{0};

void set_test_overrides(int force_tile, int force_splits, int qcols_path, int int4_direct) {
  g_force_tile.store(force_tile, std::memory_order_relaxed);
  g_force_splits.store(force_splits, std::memory_order_relaxed);
  g_qcols_path.store(qcols_path, std::memory_order_relaxed);
  g_int4_direct.store(int4_direct, std::memory_order_relaxed);
}

int qcols_path_requested() { return g_qcols_path.load(std::memory_order_relaxed); }

constexpr int kCfgInt4 = kNumCfgs;   // gemm_i4_kernel, planned as the 128x128 tile

GemmPlan plan_gemm_int4(int64_t M, int64_t N, int64_t K, int force_splits) {
  GemmPlan plan = plan_gemm_forced(M, N, K, false, 2,
                                   force_splits < 0 ? g_force_splits.load(std::memory_order_relaxed)
                                                    : force_splits);
  if (plan.bm != 0) plan.cfg = kCfgInt4;
  return plan;
}

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool allow_persistent) {
  return plan_gemm_forced(M, N, K, allow_persistent, g_force_tile.load(std::memory_order_relaxed),
                          g_force_splits.load(std::memory_order_relaxed));
}

GemmPlan plan_gemm_forced(int64_t M, int64_t N, int64_t K, bool allow_persistent, int force_tile,
                          int force_splits) {
  GemmPlan best{};
  if (M <= 0 || N <= 0) return best;
  const int cus = device_cus();
  // outputs above half the last-level cache are written with nontemporal
  // stores (the launch sets GemmParams::stream_out by the same rule)
  const bool stream_out = (double)M * (double)N * 4.0 > kStreamOutBytes;
  // Estimated seconds (see TileCfg), plus the split-K partial round trip;
  // no plan beats the whole output written at ~5 TB/s.
  const double mem_bw = 4.0e12;
  const double write_bw = 5.0e12;
  double best_cost = 1e300;
  const int64_t kstages = (K + BK - 1) / BK;
  for (int c = 0; c < kNumCfgs; ++c) {
    if (force_tile >= 0 && c != force_tile) continue;
    if (force_tile < 0 && (c == 3 || c == 4)) continue;   // tests only
    const TileCfg& t = kCfgs[c];
    const int64_t tm = (M + t.bm - 1) / t.bm, tn = (N + t.bn - 1) / t.bn;
    const int64_t tiles = tm * tn;
    if (t.persistent) {
      if (!allow_persistent || tiles > INT32_MAX / 2) continue;
      if (t.kstage == BK && (K % BK != 0 || kstages < kPersistStages - 1)) continue;
      // 128-byte stages: at least one stage per 32x32 block of a wave (2x2
      // waves; 64x96 wave tiles: 6, 64x64: 4), and no ragged tile-row
      const int wave_blocks = (t.bm / 64) * (t.bn / 64);
      if (t.kstage == BK2 && (K % BK2 != 0 || K / BK2 < wave_blocks || M % t.bm != 0)) continue;
      if (force_splits > 1) continue;
      const int64_t slots_p = (int64_t)cus * t.per_cu;
      const int64_t grid = tiles < slots_p ? tiles : slots_p;
      // two workgroups per CU measured faster only for short K and a few
      // rounds of tiles (MLP up-projection 8192x3072x768: 35 against 38 us);
      // slower on the LM head's 50 rounds at K = 768 (706 against ~680 us
      // for tile 0) and its K = 8192 weight gradient (375 against ~355 us)
      // (with nontemporal stores, for outputs above 128 MB, it also wins on
      // many rounds: LM-head forward ~425 us against ~680 for tile 0)
      if (t.per_cu > 1 && force_tile < 0 && (K > 1024 || (tiles > 8 * grid && !stream_out))) continue;
      const double rounds = std::ceil((double)tiles / (double)grid);
      double cost = rounds * ((double)t.bm * t.bn * K / t.wg_macs +
                              (stream_out ? t.tile_overhead_nt : t.tile_overhead));
      const double wr = (double)M * N * 4 / write_bw;
      if (wr > cost) cost = wr;
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        best.cfg = c;
        best.bm = t.bm;
        best.bn = t.bn;
        best.tiles_m = (int)tm;
        best.tiles_n = (int)tn;
        best.splits = 1;
        best.k_per_split = (int)K;
        best.grid = (int)grid;
        best.persistent = true;
      }
      continue;
    }
    const double slots = (double)cus * t.per_cu;
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
                            (double)t.bm * t.bn * 4 / t.wg_out_bw;
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
        best.grid = (int)(tiles * s_eff);
        best.persistent = false;
      }
    }
  }
  if (best.bm == 0) {   // only when a forced configuration cannot run this shape
    best.cfg = 2; best.bm = best.bn = 128;
    best.tiles_m = (int)((M + 127) / 128); best.tiles_n = (int)((N + 127) / 128);
    best.splits = 1; best.k_per_split = (int)((K + BK - 1) / BK * BK);
    best.grid = best.tiles_m * best.tiles_n;
    best.persistent = false;
  }
  if (best.splits > 1) {
    best.comb_x = (int)((N + 1023) / 1024);
    int64_t rows_per = (M * best.comb_x + 1023) / 1024;   // about 1024 workgroups
    rows_per = rows_per < 1 ? 1 : (rows_per > COMB_ROWS_MAX ? COMB_ROWS_MAX : rows_per);
    best.comb_rows = (int)rows_per;
    best.comb_y = (int)((M + rows_per - 1) / rows_per);
    best.hash_parts = best.comb_x * best.comb_y;
  } else {
    best.hash_parts = best.grid;    // one share per workgroup
  }
  size_t bytes = kWsHeader + ((size_t)best.hash_parts * 8 + 255) / 256 * 256;
  best.partials_offset = bytes;
  if (best.splits > 1) bytes += (size_t)best.splits * M * N * 4;
  best.workspace_bytes = bytes;
  return best;
}

// Persistent kernels: the ReLU and store-policy variants of one tile.
template <int BM, int BN>
static void launch_persist(const GemmParams& p, unsigned int grid, hipStream_t stream) {
  if (p.relu) {
    if (p.stream_out) hipLaunchKernelGGL((gemm_i8_persist_kernel<BM, BN, 2, 2, 4, true, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((gemm_i8_persist_kernel<BM, BN, 2, 2, 4, true, false>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (p.stream_out) hipLaunchKernelGGL((gemm_i8_persist_kernel<BM, BN, 2, 2, 4, false, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((gemm_i8_persist_kernel<BM, BN, 2, 2, 4, false, false>), dim3(grid), dim3(256), 0, stream, p);
  }
}

template <int BM, int BN, int STAGES, int WPC>
static void launch_persist128(const GemmParams& p, unsigned int grid, hipStream_t stream) {
  if (p.relu) {
    if (p.stream_out) hipLaunchKernelGGL((gemm_i8_persist128_kernel<BM, BN, 2, 2, true, STAGES, WPC, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((gemm_i8_persist128_kernel<BM, BN, 2, 2, true, STAGES, WPC, false>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (p.stream_out) hipLaunchKernelGGL((gemm_i8_persist128_kernel<BM, BN, 2, 2, false, STAGES, WPC, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((gemm_i8_persist128_kernel<BM, BN, 2, 2, false, STAGES, WPC, false>), dim3(grid), dim3(256), 0, stream, p);
  }
}

hipError_t launch_gemm(const GemmParams& p, const GemmPlan& plan, hipStream_t stream) {
  const unsigned int grid = (unsigned int)plan.grid;
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
    case 3:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<256, 256, 2, 2, 4>), dim3(grid), dim3(256), 0, stream, p);
      break;
    case 4:
      launch_persist<256, 128>(p, grid, stream);
      break;
    case 5:
      launch_persist<128, 192>(p, grid, stream);
      break;
    case kCfgInt4:
      if (p.a4 && p.b4)
        hipLaunchKernelGGL((gemm_i4_kernel<128, 128, 2, 2, true, true>), dim3(grid), dim3(256), 0, stream, p);
      else if (p.a4)
        hipLaunchKernelGGL((gemm_i4_kernel<128, 128, 2, 2, true, false>), dim3(grid), dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL((gemm_i4_kernel<128, 128, 2, 2, false, true>), dim3(grid), dim3(256), 0, stream, p);
      break;
    case 7:
      launch_persist128<128, 128, 2, 2>(p, grid, stream);
      break;
    default:
      launch_persist128<128, 192, 3, 1>(p, grid, stream);
      break;
  }
  if (plan.splits > 1) {
    hipLaunchKernelGGL(splitk_combine_kernel, dim3(plan.comb_x, plan.comb_y), dim3(256), 0, stream, p);
    if (p.do_hash) {
      const hipError_t e =
          launch_hash_parts_finalize(p.hash_parts, plan.comb_x * plan.comb_y, p.M, p.N, p.hash_out, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// requantizing epilogue: pass 1 (row maxima of |y|), the row scales, pass 2
// (codes, hash).  Both passes run the same tile walk and the same exact
// contraction, so pass 2 sees exactly the y that pass 1 reduced.
//  * Persistent (the 128x128 tile with two workgroups per CU for K <= 1024,
//    else the 128x192 tile; 128-byte stages): pass 1 stores each wave's partial maximum of every row of
//    its tile (no atomics: [tiles_n * 2][M] words), requant_scales_kernel
//    reduces them to the row scales and their reciprocals, and pass 2 loads
//    the reciprocals into the tile's scale slot beside the row and column
//    scales.
//  * Otherwise (the non-persistent tiles): the row maxima are zeroed, pass 1
//    raises them with integer atomicMax, pass 2 turns them into scales.
// ---------------------------------------------------------------------------
__global__ void fill_zero_u32_kernel(unsigned int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// s = max(RN(a/127), RN(1e-8)) of the largest partial maximum of row i, and
// its reciprocal RN(1/s) -- the scale and reciprocal quantize_rows would
// compute for row i of y.  A workgroup takes 64 rows; its four waves read
// every fourth partial (coalesced along the rows) and meet in LDS.
__global__ void __launch_bounds__(256) requant_scales_kernel(const unsigned int* part, int P, int M,
                                                             float* s_out, float* inv) {
  __shared__ unsigned int red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  unsigned int m = 0;
  if (i < M) {
#pragma unroll 4
    for (int k = wave; k < P; k += 4) {
      const unsigned int v = part[(int64_t)k * M + i];
      m = v > m ? v : m;
    }
  }
  red[wave][lane] = m;
  __syncthreads();
  if (wave == 0 && i < M) {
#pragma unroll
    for (int w = 1; w < 4; ++w) m = red[w][lane] > m ? red[w][lane] : m;
    const float sc = scale_of_absmax(__uint_as_float(m));
    s_out[i] = sc;
    inv[i] = recip_rn(sc);
  }
}

// The persistent tiles of the two passes, in order of preference: 128x128
// with two workgroups per CU (K <= 1024), then 128x192.
constexpr int kRequantPersistCfgs[2] = {7, 6};

GemmPlan plan_gemm_requant(int64_t M, int64_t N, int64_t K, int64_t ldq) {
  int force = g_force_tile.load(std::memory_order_relaxed);
  if (ldq <= (int64_t(1) << 24)) {
    for (const int c : kRequantPersistCfgs) {
      if (force >= 0 && force != c) continue;
      if (c == 7 && K > 1024) continue;
      const GemmPlan pp = plan_gemm_forced(M, N, K, true, c, 1);
      if (pp.cfg == c) return pp;
    }
  }
  if (force > 2) force = -1;
  return plan_gemm_forced(M, N, K, false, force, 1);
}

RequantLayout requant_layout(const GemmPlan& plan, int64_t M) {
  RequantLayout l;
  l.max_offset = (plan.workspace_bytes + 255) / 256 * 256;
  if (plan.persistent) {
    l.partials = plan.tiles_n * 2;
    l.inv_offset = l.max_offset + ((size_t)l.partials * M * 4 + 255) / 256 * 256;
    l.bytes = l.inv_offset + (size_t)M * 4;
  } else {
    l.partials = 0;
    l.inv_offset = 0;
    l.bytes = l.max_offset + (size_t)M * 4;
  }
  return l;
}

template <int MODE>
static void launch_dma_mode(const GemmParams& p, int cfg, unsigned int grid, hipStream_t stream) {
  switch (cfg) {
    case 0:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<256, 256, 2, 4, 4, MODE>), dim3(grid), dim3(512), 0, stream, p);
      break;
    case 1:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<256, 128, 2, 2, 4, MODE>), dim3(grid), dim3(256), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL((gemm_i8_dma_kernel<128, 128, 2, 2, 4, MODE>), dim3(grid), dim3(256), 0, stream, p);
      break;
  }
}

template <int MODE, int BM, int BN, int STAGES, int WPC>
static void launch_persist_mode(const GemmParams& p, unsigned int grid, hipStream_t stream) {
  if (p.relu)
    hipLaunchKernelGGL((gemm_i8_persist128_kernel<BM, BN, 2, 2, true, STAGES, WPC, false, MODE>), dim3(grid),
                       dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_i8_persist128_kernel<BM, BN, 2, 2, false, STAGES, WPC, false, MODE>), dim3(grid),
                       dim3(256), 0, stream, p);
}

hipError_t launch_gemm_requant(GemmParams p, const GemmPlan& plan, const RequantLayout& l, hipStream_t stream) {
  const int do_hash = p.do_hash;
  if (plan.persistent) {
    const bool t7 = plan.cfg == 7;
    p.do_hash = 0;
    if (t7)
      launch_persist_mode<1, 128, 128, 2, 2>(p, (unsigned int)plan.grid, stream);
    else
      launch_persist_mode<1, 128, 192, 3, 1>(p, (unsigned int)plan.grid, stream);
    hipLaunchKernelGGL(requant_scales_kernel, dim3((unsigned int)((p.M + 63) / 64)), dim3(256), 0, stream,
                       p.rowmax, l.partials, p.M, p.s_out, const_cast<float*>(p.inv_row));
    p.do_hash = do_hash;
    if (t7)
      launch_persist_mode<2, 128, 128, 2, 2>(p, (unsigned int)plan.grid, stream);
    else
      launch_persist_mode<2, 128, 192, 3, 1>(p, (unsigned int)plan.grid, stream);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(fill_zero_u32_kernel, dim3((unsigned int)((p.M + 255) / 256)), dim3(256), 0, stream,
                     p.rowmax, p.M);
  p.do_hash = 0;
  launch_dma_mode<1>(p, plan.cfg, (unsigned int)plan.grid, stream);
  p.do_hash = do_hash;
  launch_dma_mode<2>(p, plan.cfg, (unsigned int)plan.grid, stream);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// int4 operand widened to int8 codes (the value q itself) in rows of
// int4_widened_ld(K) bytes, so that the int8 kernels (and their planner) run
// the GEMM: one thread per 16-byte packed group.  A nibble n becomes the
// byte n | (bit 3 of n) * 0xF0, its sign extension.
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned int sext_nibble_bytes(unsigned int n) {
  return n | (((n >> 3) & 0x01010101u) * 0xF0u);
}

__global__ void __launch_bounds__(256)
widen_int4_kernel(const int8_t* __restrict__ P, int64_t ldp, int64_t rows, int64_t groups,
                  int8_t* __restrict__ Q, int64_t ldq) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * groups) return;
  const int64_t r = t / groups, gi = t % groups;
  const v4i w = *reinterpret_cast<const v4i*>(P + r * ldp + gi * 16);
  v4i lo, hi;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = (int)sext_nibble_bytes((unsigned int)w[e] & 0x0F0F0F0Fu);
    hi[e] = (int)sext_nibble_bytes(((unsigned int)w[e] >> 4) & 0x0F0F0F0Fu);
  }
  int8_t* q = Q + r * ldq + gi * 32;
  *reinterpret_cast<v4i*>(q) = lo;
  *reinterpret_cast<v4i*>(q + 16) = hi;
}

int64_t int4_widened_ld(int64_t K) { return (K + 31) / 32 * 32; }

hipError_t launch_widen_int4(const int8_t* P, int64_t ldp, int64_t rows, int64_t K, int8_t* Q,
                             hipStream_t stream) {
  const int64_t groups = (K + 31) / 32;
  const int64_t n = rows * groups;
  if (n > 0)
    hipLaunchKernelGGL(widen_int4_kernel, dim3((unsigned int)((n + 255) / 256)), dim3(256), 0, stream, P, ldp,
                       rows, groups, Q, int4_widened_ld(K));
  return hipGetLastError();
}

bool int4_direct_requested() { return g_int4_direct.load(std::memory_order_relaxed) != 0; }

}  // namespace i8g
