// verify.hip -- the library checking itself on the device it runs on, after
// the defence layers of the DaisyChain-Train page "Verification -- why you
// can trust the numbers":
//   * "Layer 1: exact init gates": i8g_gate runs the quantize passes, the
//     GEMM in every tile configuration and the output hash on a sweep of
//     ragged shapes and compares every output bit with an exact host mirror
//     of the method (below).  The inputs carry the cases that separate the
//     method from nearby wrong specifications (a tie x*inv = k + 0.5, a
//     product just below 0.5 where a fused multiply-add floors differently,
//     the order of the two scale multiplies, ReLU's +0), and the gate checks
//     on the host that they do separate them: a pass is something a wrong
//     device would fail ("gate the gate").  On a mismatch the gate refuses
//     with I8G_EGATE; the library never computes outputs on the CPU.
//   * "Layer 2: continuous audit": i8g_audit_gemm recomputes sampled cells
//     of a live GEMM output with a plain scalar dot product (not the MFMA
//     path) and compares bits; i8g_audit_quantize does the same for sampled
//     lines of a quantize pass.  Stride and padding bugs at live shapes show
//     up there.
//   * "Layer 3: the kernel probe": i8g_probe_hash runs a seeded GEMM through
//     the live kernels and returns its output hash; inputs come from the
//     SplitMix64 generator (Steele, Lea and Flood, OOPSLA 2014), so any
//     device (and the CPU) reproduces them.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/int8_gemm.h"
#include "i8g_device.h"
#include "i8g_launch.h"

namespace i8g {

// ---------------------------------------------------------------------------
// SplitMix64: output k (k = 0, 1, ...) of the generator seeded with `seed` is
// mix(seed + (k+1) * 0x9E3779B97F4A7C15).
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t k) {
  uint64_t z = seed + (k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The probe's input value of generator output z: the top 24 bits as a
// signed integer over 2^21, so in [-4, 4) and exact in binary32.
__host__ __device__ __forceinline__ float probe_value(uint64_t z) {
  return (float)((int32_t)(z >> 40) - (1 << 23)) * (1.0f / 2097152.0f);
}

namespace mirror {

// Exact host arithmetic of the method: binary32 round-to-nearest-even for
// every operation (x86-64 SSE scalar arithmetic; the library is built with
// -ffp-contract=off, so no multiply-add is fused).
static inline float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static inline uint32_t to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
static inline float scale_of(float a) {
  const float s = a / 127.0f;
  const float fl = from_bits(0x322BCC77u);
  return s > fl ? s : fl;
}
static inline int quant(float x, float inv) {
  const float t = x * inv;
  const float u = t + 0.5f;
  return (int)floorf(u);
}
// One line (row of X, or column of X with stride ldx): scale and codes.
static void quantize_line(const float* x, int64_t n, int64_t stride, int8_t* q, float* s) {
  float a = 0.0f;
  for (int64_t k = 0; k < n; ++k) {
    const float v = fabsf(x[k * stride]);
    a = v > a ? v : a;
  }
  *s = scale_of(a);
  const float inv = 1.0f / *s;
  for (int64_t k = 0; k < n; ++k) q[k] = (int8_t)quant(x[k * stride], inv);
}
// Storage formats (the presk page, section "Integer weights"): qmax 7 for
// int4, the scale rounded up to a power of two for pow2.
static inline float scale_of_fmt(float a, int fmt) {
  const float s0 = a / ((fmt & FMT_INT4) ? 7.0f : 127.0f);
  const float fl = from_bits(0x322BCC77u);
  float s = s0 > fl ? s0 : fl;
  if (fmt & FMT_POW2) {
    int e = 0;
    const float m = frexpf(s, &e);   // s = m * 2^e, m in [0.5, 1)
    s = ldexpf(1.0f, m == 0.5f ? e - 1 : e);
  }
  return s;
}
static void quantize_line_fmt(const float* x, int64_t n, int64_t stride, int8_t* q, float* s, int fmt) {
  float a = 0.0f;
  for (int64_t k = 0; k < n; ++k) {
    const float v = fabsf(x[k * stride]);
    a = v > a ? v : a;
  }
  *s = scale_of_fmt(a, fmt);
  const float inv = 1.0f / *s;
  for (int64_t k = 0; k < n; ++k) q[k] = (int8_t)quant(x[k * stride], inv);
}
// int4 line layout: value k in byte 16*(k/32) + k%16, low nibble when
// k%32 < 16, else high; 16*ceil(n/32) bytes, unused nibbles 0.
static void pack_int4(const int8_t* q, int64_t n, uint8_t* out) {
  const int64_t bytes = (n + 31) / 32 * 16;
  for (int64_t b = 0; b < bytes; ++b) out[b] = 0;
  for (int64_t k = 0; k < n; ++k) {
    const int64_t b = 16 * (k / 32) + k % 16;
    out[b] |= (uint8_t)(((unsigned)q[k] & 0xFu) << ((k % 32) < 16 ? 0 : 4));
  }
}
static float epilogue(int32_t acc, float sr, float sc, bool relu) {
  float y = (float)acc;
  y = y * sr;
  y = y * sc;
  if (relu) y = y > 0.0f ? y : 0.0f;
  return y;
}
// The output hash of include/int8_gemm.h (output_hash), written here from
// that definition on its own, without the device code's key functions, and
// summed row by row where the kernels sum column by column: the gate's
// hash check does not share code with the path it checks.
static uint64_t mirror_fmix64(uint64_t k) {
  const uint64_t m1 = 0xFF51AFD7ED558CCDull, m2 = 0xC4CEB9FE1A85EC53ull;
  k = (k ^ (k >> 33)) * m1;
  k = (k ^ (k >> 33)) * m2;
  return k ^ (k >> 33);
}
static uint64_t mirror_row_key(uint64_t i) {
  uint64_t x = i % 2147483648ull;   // i mod 2^31, then products mod 2^31
  x ^= x >> 16;
  x = (x * 0x3B9C5A1Dull) % 2147483648ull;
  x ^= x >> 13;
  x = (x * 0x2F6E8B35ull) % 2147483648ull;
  x ^= x >> 16;
  return 2 * x + 1;
}
static uint64_t hash_of(const float* C, int64_t M, int64_t N) {
  std::vector<uint64_t> ck((size_t)N);
  for (int64_t j = 0; j < N; ++j) ck[(size_t)j] = mirror_fmix64((uint64_t)j + 0x9E3779B97F4A7C15ull) | 1ull;
  uint64_t S = 0;
  for (int64_t i = 0; i < M; ++i) {
    uint64_t row = 0;
    for (int64_t j = 0; j < N; ++j) row += ck[(size_t)j] * (uint64_t)to_bits(C[i * N + j]);
    S += mirror_row_key((uint64_t)i) * row;
  }
  return mirror_fmix64(S ^ mirror_fmix64(((uint64_t)M << 32) + (uint64_t)N));
}

// Deterministic gate inputs: heavy-tailed values (a ratio of two uniforms)
// from the SplitMix64 stream.
static float gate_value(uint64_t seed, uint64_t k) {
  const uint64_t z = splitmix64_at(seed, k);
  const float u = (float)((z >> 40) & 0xFFFFFF) * (1.0f / 16777216.0f) - 0.5f;
  const float w = (float)((z >> 8) & 0xFFFF) * (1.0f / 65536.0f) + 0.0625f;
  return u / w;
}

// Plants, in a line whose scale is s (inv = RN(1/s)), the discriminating
// values at positions p0 and p1 (if they exist below the line's maximum):
// p0 gets x with RN(x*inv) == 0.5 exactly (floor(t + 0.5) = 1, round-half-
// even 0), p1 gets x with RN(x*inv) == 0.5 - 2^-25, where the two-rounding
// form gives 1 and a fused multiply-add gives 0.  Returns how many it found.
static int plant_discriminators(float* x0, float* x1, float s) {
  const float inv = 1.0f / s;
  const float half = 0.5f * s;
  int found = 0;
  float c = half;
  for (int d = 0; d < 16; ++d) c = nextafterf(c, -INFINITY);
  bool got0 = false, got1 = false;
  for (int d = 0; d < 33; ++d, c = nextafterf(c, INFINITY)) {
    const float t = c * inv;
    if (!got0 && t == 0.5f) {
      *x0 = c;
      got0 = true;
      ++found;
    }
    if (!got1 && t == from_bits(0x3EFFFFFFu) && floorf(fmaf(c, inv, 0.5f)) == 0.0f) {
      *x1 = c;
      got1 = true;
      ++found;
    }
  }
  return found;
}

}  // namespace mirror

// ---------------------------------------------------------------------------
// audit kernels
// ---------------------------------------------------------------------------
__global__ void audit_init_kernel(unsigned long long* r) {
  if (threadIdx.x == 0) {
    r[0] = 0ull;
    r[1] = ~0ull;
  }
}

// Value k of a stored line: int8, or int4 in the layout of
// quantize_rows_fmt (byte 16*(k/32) + k%16, low nibble for k%32 < 16, else
// high; 4-bit two's complement).
__device__ __forceinline__ int code_at(const int8_t* line, int64_t k, int int4) {
  if (!int4) return line[k];
  const int b = (unsigned char)line[16 * (k / 32) + k % 16];
  const int n = (k % 32) < 16 ? (b & 0xF) : (b >> 4);
  return n >= 8 ? n - 16 : n;
}

__global__ void __launch_bounds__(256)
audit_gemm_kernel(const int8_t* __restrict__ QA, int64_t lda, const float* __restrict__ s_row,
                  const int8_t* __restrict__ QB, int64_t ldb, const float* __restrict__ s_col,
                  int64_t M, int64_t N, int64_t K, const float* __restrict__ C, int64_t ldc, int relu,
                  int a4, int b4, uint64_t seed, int samples, unsigned long long* r) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= samples) return;
  const uint64_t h = splitmix64_at(seed, (uint64_t)s);
  const int64_t i = (int64_t)((h >> 32) % (uint64_t)M);
  const int64_t j = (int64_t)((h & 0xFFFFFFFFull) % (uint64_t)N);
  const int8_t* a = QA + i * lda;
  const int8_t* b = QB + j * ldb;
  int32_t acc = 0;
  int64_t k = 0;
  if (a4 || b4) {
    for (; k < K; ++k) acc += code_at(a, k, a4) * code_at(b, k, b4);
  }
  for (; k + 4 <= K; k += 4) {   // rows are 16-byte aligned (lda, ldb multiples of 16)
    const int av = *reinterpret_cast<const int*>(a + k);
    const int bv = *reinterpret_cast<const int*>(b + k);
    acc += (int32_t)(int8_t)(av) * (int8_t)(bv) + (int32_t)(int8_t)(av >> 8) * (int8_t)(bv >> 8) +
           (int32_t)(int8_t)(av >> 16) * (int8_t)(bv >> 16) + (int32_t)(int8_t)(av >> 24) * (int8_t)(bv >> 24);
  }
  for (; k < K; ++k) acc += (int32_t)a[k] * (int32_t)b[k];
  float y = epilogue1(acc, s_row[i], s_col[j]);
  if (relu) y = relu_pos0(y);
  if (__float_as_uint(y) != __float_as_uint(C[i * ldc + j])) {
    atomicAdd(&r[0], 1ull);
    atomicMin(&r[1], (unsigned long long)(i * N + j));
  }
}

// One workgroup per sampled line (a row of X for by_col == 0, a column for
// by_col == 1): recomputes the line's scale and every code.
__global__ void __launch_bounds__(256)
audit_quantize_kernel(const float* __restrict__ X, int64_t rows, int64_t cols, int64_t ldx,
                      const int8_t* __restrict__ Q, int64_t ldq, const float* __restrict__ scale,
                      int by_col, int fmt, uint64_t seed, unsigned long long* r) {
  __shared__ float red[4];
  __shared__ int bad_any;
  const int64_t nlines = by_col ? cols : rows, len = by_col ? rows : cols;
  const int64_t line = (int64_t)(splitmix64_at(seed, blockIdx.x) % (uint64_t)nlines);
  auto xat = [&](int64_t e) { return by_col ? X[e * ldx + line] : X[line * ldx + e]; };
  float a = 0.0f;
  for (int64_t e = threadIdx.x; e < len; e += 256) a = fmaxf(a, fabsf(xat(e)));
  a = wave_max_f32(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  if (threadIdx.x == 0) bad_any = 0;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = fmt == 0 ? scale_of_absmax_fmt<0>(a)
                  : fmt == FMT_POW2 ? scale_of_absmax_fmt<FMT_POW2>(a)
                  : fmt == FMT_INT4 ? scale_of_absmax_fmt<FMT_INT4>(a)
                                    : scale_of_absmax_fmt<FMT_INT4 | FMT_POW2>(a);
  const float inv = recip_rn(s);
  const int int4 = (fmt & FMT_INT4) != 0;
  int bad = (threadIdx.x == 0) && (__float_as_uint(s) != __float_as_uint(scale[line]));
  // int4 lines: the nibbles after the last value (to the end of its 16-byte
  // group) must be 0 as well
  const int64_t stored = int4 ? (len + 31) / 32 * 32 : len;
  for (int64_t e = threadIdx.x; e < stored; e += 256) {
    const int want = e < len ? quantize1(xat(e), inv) : 0;
    if (code_at(Q + line * ldq, e, int4) != want) bad = 1;
  }
  if (bad) atomicOr(&bad_any, 1);
  __syncthreads();
  if (threadIdx.x == 0 && bad_any) {
    atomicAdd(&r[0], 1ull);
    atomicMin(&r[1], (unsigned long long)line);
  }
}

__global__ void __launch_bounds__(256)
probe_fill_kernel(float* __restrict__ dst, int64_t n, uint64_t seed, uint64_t first) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    dst[e] = probe_value(splitmix64_at(seed, first + (uint64_t)e));
}

__global__ void zero_header_kernel(unsigned int* p) { p[threadIdx.x] = 0u; }

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int64_t round16(int64_t n) { return (n + 15) / 16 * 16; }
inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// the gate
// ---------------------------------------------------------------------------
struct QCase { int64_t rows, cols; bool by_col; int fmt; bool batch; };
struct GCase { int64_t M, N, K; int splits; };
// the cases marked batch run as quantize_batch calls (with a second job);
// the aligned rows of 2048 and 3072 values take the batch's long-row body
const QCase kQCases[] = {{37, 301, false, 0, false},  {5, 4500, false, 0, false},
                         {1, 1, false, 0, false},     {300, 37, true, 0, false},
                         {8200, 33, true, 0, false},  {700, 64, true, 0, false},
                         {37, 301, false, FMT_INT4, false},  {300, 37, true, FMT_INT4 | FMT_POW2, false},
                         {64, 100, false, FMT_POW2, false},  {100, 64, true, FMT_POW2, false},
                         {65, 1000, false, 0, true},  {1000, 65, true, 0, true},
                         {33, 700, false, FMT_POW2, true}, {700, 33, true, 0, true},
                         {24, 2048, false, 0, true}, {9, 3072, false, FMT_POW2, true}};
const GCase kGCases[] = {{17, 33, 15, 0}, {130, 190, 70, 0}, {300, 520, 192, 0},
                         {256, 200, 768, 0}, {64, 64, 4096, 4}};
constexpr int kGateCfgs = 8;   // tile configurations of the GEMM planner
constexpr size_t kGateWorkspace = 16u << 20;

struct GateRun {
  char* ws;
  hipStream_t st;
  i8g_gate_report* rep;
  size_t cursor;
  char* take(size_t n) {
    char* p = ws + cursor;
    cursor += align256(n);
    return p;
  }
};

int fail(i8g_gate_report* rep, int check, int cfg, int64_t m, int64_t n, int64_t k, int64_t idx,
         uint32_t got, uint32_t want) {
  if (rep) {
    rep->check = check;
    rep->config = cfg;
    rep->m = m;
    rep->n = n;
    rep->k = k;
    rep->index = idx;
    rep->got = got;
    rep->want = want;
  }
  return I8G_EGATE;
}

int hipok(hipError_t e) { return e == hipSuccess ? I8G_OK : I8G_EHIP; }

// Quantize cases: per line, the maximum planted first, then the two
// discriminators; the mirror's own outputs then show whether the plants
// separate the method from round-half-even and from the fused form.
int gate_quantize(GateRun& g, const QCase& c, int case_id, int64_t counts[2]) {
  const int64_t R = c.rows, Cc = c.cols, n = R * Cc;
  std::vector<float> X(n);
  for (int64_t e = 0; e < n; ++e) X[e] = mirror::gate_value(0x6A7E0000ull + case_id, e);
  const int64_t nlines = c.by_col ? Cc : R, len = c.by_col ? R : Cc;
  auto at = [&](int64_t line, int64_t e) -> float& {
    return c.by_col ? X[e * Cc + line] : X[line * Cc + e];
  };
  for (int64_t l = 0; l < nlines; ++l) {
    if (l % 7 == 3) {   // some all-zero lines (scale = the floor), with a -0
      for (int64_t e = 0; e < len; ++e) at(l, e) = 0.0f;
      at(l, 0) = -0.0f;
      continue;
    }
    if (len < 3) continue;
    float a = 0.0f;
    for (int64_t e = 0; e < len; ++e) a = fmaxf(a, fabsf(at(l, e)));
    at(l, 0) = (l & 1) ? -a : a;   // the maximum, with either sign
    const float s = mirror::scale_of(a);
    float x0 = 0.0f, x1 = 0.0f;
    if (mirror::plant_discriminators(&x0, &x1, s) == 2) {
      at(l, 1) = x0;
      at(l, 2) = x1;
    }
  }
  // the mirror, and how often wrong specifications would differ from it
  std::vector<int8_t> Qw(n);
  std::vector<float> Sw(nlines);
  for (int64_t l = 0; l < nlines; ++l) {
    const float* base = c.by_col ? &X[l] : &X[l * Cc];
    mirror::quantize_line_fmt(base, len, c.by_col ? Cc : 1, &Qw[l * len], &Sw[l], c.fmt);
    const float inv = 1.0f / Sw[l];
    for (int64_t e = 0; e < len; ++e) {
      const float x = base[e * (c.by_col ? Cc : 1)];
      const int q = Qw[l * len + e];
      if ((int)rintf(x * inv) != q) ++counts[0];                    // round-half-even
      if ((int)floorf(fmaf(x, inv, 0.5f)) != q) ++counts[1];        // fused multiply-add
    }
  }
  // the device (int4: lines of whole 16-byte groups; a batch adds the
  // other direction of the same X as a second job, which must not disturb it)
  const bool int4 = (c.fmt & FMT_INT4) != 0;
  g.cursor = 256;
  float* dX = reinterpret_cast<float*>(g.take(n * 4));
  const int64_t ldq = int4 ? (len + 31) / 32 * 16 : len;
  int8_t* dQ = reinterpret_cast<int8_t*>(g.take(nlines * ldq + 16));
  float* dS = reinterpret_cast<float*>(g.take(nlines * 4));
  const int64_t olines = c.by_col ? R : Cc, olen = c.by_col ? Cc : R;
  int8_t* dQ2 = reinterpret_cast<int8_t*>(g.take(olines * olen + 16));
  float* dS2 = reinterpret_cast<float*>(g.take(olines * 4));
  if (g.cursor > kGateWorkspace) return I8G_EWORKSPACE;
  int st = hipok(hipMemcpyAsync(dX, X.data(), n * 4, hipMemcpyHostToDevice, g.st));
  if (st) return st;
  if (c.batch) {
    i8g_quantize_job jobs[2] = {
        {dX, R, Cc, Cc, dQ, ldq, dS, c.by_col ? 1u : 0u, (uint32_t)c.fmt},
        {dX, R, Cc, Cc, dQ2, olen, dS2, c.by_col ? 0u : 1u, 0u}};
    st = quantize_batch(jobs, 2, g.st);
  } else {
    st = c.by_col ? quantize_cols_fmt(dX, R, Cc, Cc, dQ, ldq, dS, (uint32_t)c.fmt, g.st)
                  : quantize_rows_fmt(dX, R, Cc, Cc, dQ, ldq, dS, (uint32_t)c.fmt, g.st);
  }
  if (st) return st;
  std::vector<int8_t> Qg(nlines * ldq);
  std::vector<float> Sg(nlines);
  st = hipok(hipMemcpyAsync(Qg.data(), dQ, nlines * ldq, hipMemcpyDeviceToHost, g.st));
  if (!st) st = hipok(hipMemcpyAsync(Sg.data(), dS, nlines * 4, hipMemcpyDeviceToHost, g.st));
  if (!st) st = hipok(hipStreamSynchronize(g.st));
  if (st) return st;
  const int check = c.by_col ? 2 : 1;
  std::vector<uint8_t> packed(ldq);
  for (int64_t l = 0; l < nlines; ++l) {
    if (mirror::to_bits(Sg[l]) != mirror::to_bits(Sw[l]))
      return fail(g.rep, check, c.fmt, R, Cc, 0, l, mirror::to_bits(Sg[l]), mirror::to_bits(Sw[l]));
    if (int4) {
      mirror::pack_int4(&Qw[l * len], len, packed.data());
      for (int64_t b = 0; b < ldq; ++b)
        if ((uint8_t)Qg[l * ldq + b] != packed[b])
          return fail(g.rep, check, c.fmt, R, Cc, 0, l * ldq + b, (uint8_t)Qg[l * ldq + b], packed[b]);
      continue;
    }
    for (int64_t e = 0; e < len; ++e)
      if (Qg[l * ldq + e] != Qw[l * len + e])
        return fail(g.rep, check, c.fmt, R, Cc, 0, l * len + e, (uint8_t)Qg[l * ldq + e], (uint8_t)Qw[l * len + e]);
  }
  if (c.batch) {   // the second job: int8, the other direction
    std::vector<int8_t> Q2(olines * olen), Q2w(olen);
    std::vector<float> S2(olines);
    st = hipok(hipMemcpyAsync(Q2.data(), dQ2, olines * olen, hipMemcpyDeviceToHost, g.st));
    if (!st) st = hipok(hipMemcpyAsync(S2.data(), dS2, olines * 4, hipMemcpyDeviceToHost, g.st));
    if (!st) st = hipok(hipStreamSynchronize(g.st));
    if (st) return st;
    for (int64_t l = 0; l < olines; ++l) {
      float sw = 0.0f;
      const float* base = c.by_col ? &X[l * Cc] : &X[l];
      mirror::quantize_line_fmt(base, olen, c.by_col ? 1 : Cc, Q2w.data(), &sw, 0);
      if (mirror::to_bits(S2[l]) != mirror::to_bits(sw))
        return fail(g.rep, c.by_col ? 1 : 2, 0, R, Cc, 0, l, mirror::to_bits(S2[l]), mirror::to_bits(sw));
      for (int64_t e = 0; e < olen; ++e)
        if (Q2[l * olen + e] != Q2w[e])
          return fail(g.rep, c.by_col ? 1 : 2, 0, R, Cc, 0, l * olen + e, (uint8_t)Q2[l * olen + e], (uint8_t)Q2w[e]);
    }
  }
  return I8G_OK;
}

// GEMM cases: operands quantized by the mirror; every tile configuration;
// ReLU on for odd configurations; the fused hash and the standalone hash.
int gate_gemm(GateRun& g, const GCase& c, int case_id, int64_t counts[3], int* ncases) {
  const int64_t M = c.M, N = c.N, K = c.K, ld = round16(K);
  std::vector<float> A(M * K), B(N * K);   // B given as N x K (its columns as rows)
  for (int64_t e = 0; e < M * K; ++e) A[e] = mirror::gate_value(0x6E3A0000ull + case_id, e);
  for (int64_t e = 0; e < N * K; ++e) B[e] = mirror::gate_value(0x6E3B0000ull + case_id, e);
  std::vector<int8_t> QA(M * ld, 0), QB(N * ld, 0);
  std::vector<float> sr(M), sc(N);
  for (int64_t i = 0; i < M; ++i) mirror::quantize_line(&A[i * K], K, 1, &QA[i * ld], &sr[i]);
  for (int64_t j = 0; j < N; ++j) mirror::quantize_line(&B[j * K], K, 1, &QB[j * ld], &sc[j]);
  std::vector<int32_t> acc(M * N);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      int32_t t = 0;
      for (int64_t k = 0; k < K; ++k) t += (int32_t)QA[i * ld + k] * (int32_t)QB[j * ld + k];
      acc[i * N + j] = t;
    }
  std::vector<float> Cw[2];
  uint64_t Hw[2];
  for (int r = 0; r < 2; ++r) {
    Cw[r].resize(M * N);
    for (int64_t e = 0; e < M * N; ++e) Cw[r][e] = mirror::epilogue(acc[e], sr[e / N], sc[e % N], r == 1);
    Hw[r] = mirror::hash_of(Cw[r].data(), M, N);
  }
  for (int64_t e = 0; e < M * N; ++e) {
    const float a = (float)acc[e], s1 = sr[e / N], s2 = sc[e % N];
    if (mirror::to_bits((a * s2) * s1) != mirror::to_bits(Cw[0][e])) ++counts[0];   // column scale first
    if (mirror::to_bits(a * (s1 * s2)) != mirror::to_bits(Cw[0][e])) ++counts[1];   // scales multiplied first
    if (acc[e] < 0) ++counts[2];                                                       // ReLU gives +0
  }
  g.cursor = 256;
  int8_t* dA = reinterpret_cast<int8_t*>(g.take(M * ld));
  int8_t* dB = reinterpret_cast<int8_t*>(g.take(N * ld));
  float* dsr = reinterpret_cast<float*>(g.take(M * 4));
  float* dsc = reinterpret_cast<float*>(g.take(N * 4));
  float* dC = reinterpret_cast<float*>(g.take(M * N * 4));
  uint64_t* dH = reinterpret_cast<uint64_t*>(g.take(16));
  char* hws = g.take(output_hash_workspace_bytes());
  const size_t gws_off = g.cursor;
  int st = hipok(hipMemcpyAsync(dA, QA.data(), M * ld, hipMemcpyHostToDevice, g.st));
  if (!st) st = hipok(hipMemcpyAsync(dB, QB.data(), N * ld, hipMemcpyHostToDevice, g.st));
  if (!st) st = hipok(hipMemcpyAsync(dsr, sr.data(), M * 4, hipMemcpyHostToDevice, g.st));
  if (!st) st = hipok(hipMemcpyAsync(dsc, sc.data(), N * 4, hipMemcpyHostToDevice, g.st));
  if (st) return st;
  std::vector<float> Cg(M * N);
  for (int cfg = 0; cfg < kGateCfgs; ++cfg) {
    const int relu = cfg & 1;
    const GemmPlan plan = plan_gemm_forced(M, N, K, true, cfg, c.splits);
    const size_t gws = plan.workspace_bytes;
    if (gws_off + align256(gws) > kGateWorkspace) return I8G_EWORKSPACE;
    // the GEMM's workspace header shares the gate's zero header: it is left
    // zero by every call, and the gate's own header is zeroed at the start
    char* gw = g.ws + gws_off;
    hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(64), 0, g.st, reinterpret_cast<unsigned int*>(gw));
    st = enqueue_gemm(dA, ld, dsr, dB, ld, dsc, M, N, K, dC, N, (relu ? I8G_RELU : 0u) | I8G_HASH, dH,
                      gw, gws, g.st, cfg, c.splits);
    if (st) return st;
    uint64_t Hg = 0, Hs = 0;
    st = hipok(hipMemcpyAsync(Cg.data(), dC, M * N * 4, hipMemcpyDeviceToHost, g.st));
    if (!st) st = hipok(hipMemcpyAsync(&Hg, dH, 8, hipMemcpyDeviceToHost, g.st));
    if (!st) st = hipok(hipStreamSynchronize(g.st));
    if (st) return st;
    for (int64_t e = 0; e < M * N; ++e)
      if (mirror::to_bits(Cg[e]) != mirror::to_bits(Cw[relu][e]))
        return fail(g.rep, 3, plan.cfg, M, N, K, e, mirror::to_bits(Cg[e]), mirror::to_bits(Cw[relu][e]));
    if (Hg != Hw[relu]) return fail(g.rep, 4, plan.cfg, M, N, K, -1, (uint32_t)Hg, (uint32_t)Hw[relu]);
    // the standalone hash of the same output
    hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(64), 0, g.st, reinterpret_cast<unsigned int*>(hws));
    st = output_hash(dC, M, N, N, dH, hws, output_hash_workspace_bytes(), g.st);
    if (!st) st = hipok(hipMemcpyAsync(&Hs, dH, 8, hipMemcpyDeviceToHost, g.st));
    if (!st) st = hipok(hipStreamSynchronize(g.st));
    if (st) return st;
    if (Hs != Hw[relu]) return fail(g.rep, 4, -1, M, N, K, -1, (uint32_t)Hs, (uint32_t)Hw[relu]);
    ++*ncases;
  }
  return I8G_OK;
}

// int4 operands: the mirror quantizes A and/or B with qmax 7 (B with
// power-of-two scales) and packs the codes; the device runs the GEMM on the
// packed bytes.  The expected output is the mirror's exact contraction of
// the codes and its epilogue.
struct G4Case { int64_t M, N, K; bool a4, b4; };
const G4Case kG4Cases[] = {{130, 190, 70, false, true}, {256, 200, 768, true, false}, {65, 33, 1000, true, true}};

int upload_operand(GateRun& g, const std::vector<int8_t>& codes, int64_t rows, int64_t K, bool int4,
                   int64_t* ld_out, int8_t** dptr) {
  const int64_t ld = int4 ? (K + 31) / 32 * 16 : round16(K);
  std::vector<uint8_t> buf(rows * ld, 0);
  for (int64_t r = 0; r < rows; ++r) {
    if (int4) mirror::pack_int4(&codes[r * K], K, &buf[r * ld]);
    else memcpy(&buf[r * ld], &codes[r * K], K);
  }
  *dptr = reinterpret_cast<int8_t*>(g.take(rows * ld));
  *ld_out = ld;
  return hipok(hipMemcpyAsync(*dptr, buf.data(), rows * ld, hipMemcpyHostToDevice, g.st));
}

int gate_gemm_int4(GateRun& g, const G4Case& c, int case_id, int* ncases) {
  const int64_t M = c.M, N = c.N, K = c.K;
  const bool relu = (case_id & 1) != 0;
  const int fa = c.a4 ? FMT_INT4 : 0, fb = c.b4 ? (FMT_INT4 | FMT_POW2) : FMT_POW2;
  std::vector<float> A(M * K), B(N * K);
  for (int64_t e = 0; e < M * K; ++e) A[e] = mirror::gate_value(0x6E4A0000ull + case_id, e);
  for (int64_t e = 0; e < N * K; ++e) B[e] = mirror::gate_value(0x6E4B0000ull + case_id, e);
  std::vector<int8_t> QA(M * K), QB(N * K);
  std::vector<float> sr(M), sc(N);
  for (int64_t i = 0; i < M; ++i) mirror::quantize_line_fmt(&A[i * K], K, 1, &QA[i * K], &sr[i], fa);
  for (int64_t j = 0; j < N; ++j) mirror::quantize_line_fmt(&B[j * K], K, 1, &QB[j * K], &sc[j], fb);
  std::vector<float> Cw(M * N);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      int32_t t = 0;
      for (int64_t k = 0; k < K; ++k) t += (int32_t)QA[i * K + k] * (int32_t)QB[j * K + k];
      Cw[i * N + j] = mirror::epilogue(t, sr[i], sc[j], relu);
    }
  const uint64_t Hw = mirror::hash_of(Cw.data(), M, N);
  g.cursor = 256;
  int8_t *dA = nullptr, *dB = nullptr;
  int64_t lda = 0, ldb = 0;
  int st = upload_operand(g, QA, M, K, c.a4, &lda, &dA);
  if (!st) st = upload_operand(g, QB, N, K, c.b4, &ldb, &dB);
  float* dsr = reinterpret_cast<float*>(g.take(M * 4));
  float* dsc = reinterpret_cast<float*>(g.take(N * 4));
  float* dC = reinterpret_cast<float*>(g.take(M * N * 4));
  uint64_t* dH = reinterpret_cast<uint64_t*>(g.take(16));
  const uint32_t flags = (relu ? I8G_RELU : 0u) | I8G_HASH | (c.a4 ? I8G_A_INT4 : 0u) | (c.b4 ? I8G_B_INT4 : 0u);
  const size_t wsb = gemm_i8_workspace_bytes_flags(M, N, K, flags);
  char* gw = g.take(wsb);
  if (g.cursor > kGateWorkspace) return I8G_EWORKSPACE;
  if (!st) st = hipok(hipMemcpyAsync(dsr, sr.data(), M * 4, hipMemcpyHostToDevice, g.st));
  if (!st) st = hipok(hipMemcpyAsync(dsc, sc.data(), N * 4, hipMemcpyHostToDevice, g.st));
  if (st) return st;
  std::vector<float> Cg(M * N);
  // both paths: operands widened for the int8 kernels (-2), and the kernel
  // that reads the packed bytes itself (-3)
  for (int path = -2; path >= -3; --path) {
    hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(64), 0, g.st, reinterpret_cast<unsigned int*>(gw));
    st = enqueue_gemm(dA, lda, dsr, dB, ldb, dsc, M, N, K, dC, N, flags, dH, gw, wsb, g.st, path, 0);
    if (st) return st;
    uint64_t Hg = 0;
    st = hipok(hipMemcpyAsync(Cg.data(), dC, M * N * 4, hipMemcpyDeviceToHost, g.st));
    if (!st) st = hipok(hipMemcpyAsync(&Hg, dH, 8, hipMemcpyDeviceToHost, g.st));
    if (!st) st = hipok(hipStreamSynchronize(g.st));
    if (st) return st;
    for (int64_t e = 0; e < M * N; ++e)
      if (mirror::to_bits(Cg[e]) != mirror::to_bits(Cw[e]))
        return fail(g.rep, 6, path, M, N, K, e, mirror::to_bits(Cg[e]), mirror::to_bits(Cw[e]));
    if (Hg != Hw) return fail(g.rep, 4, path, M, N, K, -1, (uint32_t)Hg, (uint32_t)Hw);
    ++*ncases;
  }
  return I8G_OK;
}

// The requantizing epilogue: codes and scales must be the mirror's per-row
// quantization of the mirror's output, and the hash that output's hash.
int gate_requant(GateRun& g, int* ncases) {
  const int64_t M = 300, N = 520, K = 192;
  std::vector<float> A(M * K), B(N * K);
  for (int64_t e = 0; e < M * K; ++e) A[e] = mirror::gate_value(0x6E5A0000ull, e);
  for (int64_t e = 0; e < N * K; ++e) B[e] = mirror::gate_value(0x6E5B0000ull, e);
  std::vector<int8_t> QA(M * K), QB(N * K);
  std::vector<float> sr(M), sc(N);
  for (int64_t i = 0; i < M; ++i) mirror::quantize_line_fmt(&A[i * K], K, 1, &QA[i * K], &sr[i], 0);
  for (int64_t j = 0; j < N; ++j) mirror::quantize_line_fmt(&B[j * K], K, 1, &QB[j * K], &sc[j], 0);
  std::vector<float> Cw(M * N);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      int32_t t = 0;
      for (int64_t k = 0; k < K; ++k) t += (int32_t)QA[i * K + k] * (int32_t)QB[j * K + k];
      Cw[i * N + j] = mirror::epilogue(t, sr[i], sc[j], true);
    }
  std::vector<int8_t> Qw(M * N);
  std::vector<float> Sw(M);
  for (int64_t i = 0; i < M; ++i) mirror::quantize_line_fmt(&Cw[i * N], N, 1, &Qw[i * N], &Sw[i], 0);
  const uint64_t Hw = mirror::hash_of(Cw.data(), M, N);
  g.cursor = 256;
  int8_t *dA = nullptr, *dB = nullptr;
  int64_t lda = 0, ldb = 0;
  int st = upload_operand(g, QA, M, K, false, &lda, &dA);
  if (!st) st = upload_operand(g, QB, N, K, false, &ldb, &dB);
  float* dsr = reinterpret_cast<float*>(g.take(M * 4));
  float* dsc = reinterpret_cast<float*>(g.take(N * 4));
  int8_t* dQ = reinterpret_cast<int8_t*>(g.take(M * N));
  float* dS = reinterpret_cast<float*>(g.take(M * 4));
  uint64_t* dH = reinterpret_cast<uint64_t*>(g.take(16));
  const size_t wsb = gemm_i8_requant_workspace_bytes(M, N, K);
  char* gw = g.take(wsb);
  if (g.cursor > kGateWorkspace) return I8G_EWORKSPACE;
  if (!st) st = hipok(hipMemcpyAsync(dsr, sr.data(), M * 4, hipMemcpyHostToDevice, g.st));
  if (!st) st = hipok(hipMemcpyAsync(dsc, sc.data(), N * 4, hipMemcpyHostToDevice, g.st));
  if (st) return st;
  hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(64), 0, g.st, reinterpret_cast<unsigned int*>(gw));
  st = gemm_i8_requant(dA, lda, dsr, dB, ldb, dsc, M, N, K, dQ, N, dS, I8G_RELU | I8G_HASH, dH, gw, wsb, g.st);
  if (st) return st;
  std::vector<int8_t> Qg(M * N);
  std::vector<float> Sg(M);
  uint64_t Hg = 0;
  st = hipok(hipMemcpyAsync(Qg.data(), dQ, M * N, hipMemcpyDeviceToHost, g.st));
  if (!st) st = hipok(hipMemcpyAsync(Sg.data(), dS, M * 4, hipMemcpyDeviceToHost, g.st));
  if (!st) st = hipok(hipMemcpyAsync(&Hg, dH, 8, hipMemcpyDeviceToHost, g.st));
  if (!st) st = hipok(hipStreamSynchronize(g.st));
  if (st) return st;
  for (int64_t i = 0; i < M; ++i)
    if (mirror::to_bits(Sg[i]) != mirror::to_bits(Sw[i]))
      return fail(g.rep, 7, -1, M, N, K, i, mirror::to_bits(Sg[i]), mirror::to_bits(Sw[i]));
  for (int64_t e = 0; e < M * N; ++e)
    if (Qg[e] != Qw[e]) return fail(g.rep, 7, -1, M, N, K, e, (uint8_t)Qg[e], (uint8_t)Qw[e]);
  if (Hg != Hw) return fail(g.rep, 4, -1, M, N, K, -1, (uint32_t)Hg, (uint32_t)Hw);
  ++*ncases;
  return I8G_OK;
}

}  // namespace
}  // namespace i8g

using namespace i8g;

extern "C" {

size_t i8g_gate_workspace_bytes(void) { return kGateWorkspace; }

int i8g_gate(void* workspace, size_t workspace_bytes, void* stream, i8g_gate_report* report) {
  if (report) memset(report, 0, sizeof(*report));
  if (!workspace || ((uintptr_t)workspace % 256) != 0 || workspace_bytes < kGateWorkspace)
    return I8G_EWORKSPACE;
  GateRun g{reinterpret_cast<char*>(workspace), as_stream(stream), report, 0};
  int cases = 0;
  int64_t qcounts[2] = {0, 0}, gcounts[3] = {0, 0, 0};
  int id = 0;
  for (const QCase& c : kQCases) {
    const int st = gate_quantize(g, c, id++, qcounts);
    if (st) return st;
    ++cases;
  }
  id = 0;
  for (const GCase& c : kGCases) {
    const int st = gate_gemm(g, c, id++, gcounts, &cases);
    if (st) return st;
  }
  id = 0;
  for (const G4Case& c : kG4Cases) {
    const int st = gate_gemm_int4(g, c, id++, &cases);
    if (st) return st;
  }
  {
    const int st = gate_requant(g, &cases);
    if (st) return st;
  }
  if (report) report->cases = cases;
  // gate the gate: each wrong specification must differ somewhere
  const int64_t sep[5] = {qcounts[0], qcounts[1], gcounts[0], gcounts[1], gcounts[2]};
  for (int v = 0; v < 5; ++v)
    if (sep[v] == 0) return fail(report, 5, -1, 0, 0, 0, v, 0, 0);
  return I8G_OK;
}

int i8g_audit_gemm(const int8_t* QA, int64_t lda, const float* s_row, const int8_t* QBt, int64_t ldb,
                   const float* s_col, int64_t M, int64_t N, int64_t K, const float* C, int64_t ldc,
                   uint32_t flags, uint64_t seed, int32_t samples, uint64_t* result, void* stream) {
  if (M < 0 || N < 0 || K < 0 || samples < 0 || !result) return I8G_EINVAL;
  if (flags & ~(uint32_t)(I8G_RELU | I8G_HASH | I8G_A_INT4 | I8G_B_INT4)) return I8G_EINVAL;
  const int a4 = (flags & I8G_A_INT4) ? 1 : 0, b4 = (flags & I8G_B_INT4) ? 1 : 0;
  const int64_t k4 = (K + 31) / 32 * 16;
  const hipStream_t st = as_stream(stream);
  unsigned long long* r = reinterpret_cast<unsigned long long*>(result);
  hipLaunchKernelGGL(audit_init_kernel, dim3(1), dim3(64), 0, st, r);
  if (M == 0 || N == 0 || samples == 0) return hipGetLastError() == hipSuccess ? I8G_OK : I8G_EHIP;
  if (!s_row || !s_col || !C || ldc < N || (K > 0 && (!QA || !QBt))) return I8G_EINVAL;
  if (K > 0 && (((uintptr_t)QA % 16) || ((uintptr_t)QBt % 16) || (lda % 16) || (ldb % 16) ||
                lda < (a4 ? k4 : K) || ldb < (b4 ? k4 : K)))
    return I8G_EALIGN;
  hipLaunchKernelGGL(audit_gemm_kernel, dim3((samples + 255) / 256), dim3(256), 0, st, QA, lda, s_row, QBt,
                     ldb, s_col, M, N, K, C, ldc, (flags & I8G_RELU) ? 1 : 0, a4, b4, seed, samples, r);
  return hipGetLastError() == hipSuccess ? I8G_OK : I8G_EHIP;
}

int i8g_audit_quantize_fmt(const float* X, int64_t rows, int64_t cols, int64_t ldx, const int8_t* Q,
                           int64_t ldq, const float* scale, int32_t by_col, uint32_t format, uint64_t seed,
                           int32_t samples, uint64_t* result, void* stream) {
  if (rows < 0 || cols < 0 || samples < 0 || !result) return I8G_EINVAL;
  if (format & ~(uint32_t)(I8G_FMT_POW2 | I8G_FMT_INT4)) return I8G_EINVAL;
  const hipStream_t st = as_stream(stream);
  unsigned long long* r = reinterpret_cast<unsigned long long*>(result);
  hipLaunchKernelGGL(audit_init_kernel, dim3(1), dim3(64), 0, st, r);
  const int64_t nlines = by_col ? cols : rows, len = by_col ? rows : cols;
  if (nlines == 0 || samples == 0) return hipGetLastError() == hipSuccess ? I8G_OK : I8G_EHIP;
  const int64_t line_bytes = (format & I8G_FMT_INT4) ? (len + 31) / 32 * 16 : len;
  if (!scale || (len > 0 && (!X || !Q)) || ldx < cols || ldq < line_bytes) return I8G_EINVAL;
  hipLaunchKernelGGL(audit_quantize_kernel, dim3(samples), dim3(256), 0, st, X, rows, cols, ldx, Q, ldq,
                     scale, by_col ? 1 : 0, (int)format, seed, r);
  return hipGetLastError() == hipSuccess ? I8G_OK : I8G_EHIP;
}

int i8g_audit_quantize(const float* X, int64_t rows, int64_t cols, int64_t ldx, const int8_t* Q,
                       int64_t ldq, const float* scale, int32_t by_col, uint64_t seed, int32_t samples,
                       uint64_t* result, void* stream) {
  return i8g_audit_quantize_fmt(X, rows, cols, ldx, Q, ldq, scale, by_col, 0u, seed, samples, result, stream);
}

size_t i8g_probe_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 256;
  const int64_t ld = round16(K);
  return 256 + align256((size_t)M * K * 4) + align256((size_t)K * N * 4) + align256((size_t)M * ld) +
         align256((size_t)N * ld) + align256((size_t)M * 4) + align256((size_t)N * 4) +
         align256((size_t)M * N * 4) + align256(gemm_i8_workspace_bytes(M, N, K));
}

int i8g_probe_hash(uint64_t seed, int64_t M, int64_t N, int64_t K, uint64_t* hash, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (M <= 0 || N <= 0 || K <= 0 || !hash) return I8G_EINVAL;
  if (M > (1 << 20) || N > (1 << 20) || K > I8G_K_MAX) return I8G_EINVAL;
  if (!workspace || ((uintptr_t)workspace % 256) || workspace_bytes < i8g_probe_workspace_bytes(M, N, K))
    return I8G_EWORKSPACE;
  const hipStream_t st = as_stream(stream);
  const int64_t ld = round16(K);
  char* p = reinterpret_cast<char*>(workspace) + 256;
  auto take = [&](size_t n) { char* q = p; p += align256(n); return q; };
  float* A = reinterpret_cast<float*>(take((size_t)M * K * 4));
  float* B = reinterpret_cast<float*>(take((size_t)K * N * 4));
  int8_t* QA = reinterpret_cast<int8_t*>(take((size_t)M * ld));
  int8_t* QB = reinterpret_cast<int8_t*>(take((size_t)N * ld));
  float* sr = reinterpret_cast<float*>(take((size_t)M * 4));
  float* sc = reinterpret_cast<float*>(take((size_t)N * 4));
  float* C = reinterpret_cast<float*>(take((size_t)M * N * 4));
  char* gws = take(gemm_i8_workspace_bytes(M, N, K));
  // the GEMM's workspace header is the probe workspace's own zero header
  // moved along: zero it (a kernel, so the call can be captured in a graph)
  hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(64), 0, st, reinterpret_cast<unsigned int*>(gws));
  // A (M x K) takes generator outputs 0 .. MK-1 in row-major order, B (K x N)
  // the next KN outputs, also row-major
  hipLaunchKernelGGL(probe_fill_kernel, dim3(256), dim3(256), 0, st, A, M * K, seed, (uint64_t)0);
  hipLaunchKernelGGL(probe_fill_kernel, dim3(256), dim3(256), 0, st, B, K * N, seed, (uint64_t)(M * K));
  if (hipGetLastError() != hipSuccess) return I8G_EHIP;
  int rc = quantize_rows(A, M, K, K, QA, ld, sr, stream);
  if (!rc) rc = quantize_cols(B, K, N, N, QB, ld, sc, stream);
  if (!rc)
    rc = gemm_i8_blockscaled(QA, ld, sr, QB, ld, sc, M, N, K, C, N, I8G_HASH, hash, gws,
                             gemm_i8_workspace_bytes(M, N, K), stream);
  return rc;
}

}  // extern "C"
