// sampler_kernel.hip -- the decode-step sampler's row kernel for gfx950.
//
// Sources (page titles; sections named where used):
//   [A] "SGLang's +75% sampler speedup skips Qwen3 chat requests"
//   [B] the SGLang 101 operations manual
//   [C] "采样参数对解码开销的影响：temperature、top_p 与采样核路径"
//   Philox4x32-10: Salmon, Moraes, Dror, Shaw, SC'11.
//
// One launch samples a whole batch.  A row is split into G contiguous slices;
// G workgroups of 512 threads (a "row group") own one slice each and keep
// their slice's processed logits z = penalised(x) / T in LDS, so the logits
// are read from HBM once.  The G workgroups of a group cooperate through
// per-group barrier words and exchange slots in device memory; the grid
// never exceeds the workgroups the device holds at once, and every wait is
// bounded.  A group walks rows group, group + n_groups, ...
//
// Per row (row_kernel):
//   1. load, NaN -> -inf, z = x / T as the loads land; logits processors and
//      penalties from LDS hashes of the bias/stop entries and of the history
//      counts (or from a counted list, for histories longer than the hash
//      holds), applied once per distinct id
//   2. the slice's max and first argmax; a histogram of the values on an
//      absolute grid of 1/32-nat bins over a 16-nat window below the slice
//      max (counts, 2^-31 fixed-point masses; deeper masses summed), or the
//      exact sum where every value is kept
//   3. exchange 2: every workgroup of the row merges the records and
//      histograms alike: the row max, status and argmax, min-p's boundary,
//      and in parallel the bins holding each threshold
//   4. exchange 3: the values of those bins are gathered, and every
//      workgroup sorts the merged list alike and fixes top-k, top-p, the
//      kept-set sum and the top logprobs exactly (rows whose thresholds fall
//      outside the window take the general path: a radix select with one
//      exchange per 8-bit digit)
//   5. Gumbel-max over the kept set with an in-kernel Philox draw, a
//      linear-domain bound that skips elements which cannot win, and an
//      fp64 score for every element that still can (or the seeded inverse
//      CDF); probs / logprobs of the kept set are written meanwhile
//   6. final exchange: the last workgroup to arrive merges the G winners
//      across one wave and writes the token and status
// Rows that need no merged max (ids only, no truncation) skip steps 2-4;
// a row held by one workgroup exchanges through registers and LDS only.
//
// Other kernels: rows_kernel (per-row parameters from device arrays),
// hist_list_kernel (counts of long histories, ahead of the row kernel) and
// raw_lp_kernel (the raw logprob mode at T != 1, after it).
#include <float.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sampler_internal.h"

namespace dsts {
namespace {

#define DEV __device__ __forceinline__

constexpr int kWaves = kBlock / 64;
// An element more than this many nats below the row max cannot win the
// Gumbel-max: its best score z + 22.874 (E at its smallest, 2^-33) is below
// the worst score of the max, m - ln(22.874) (E at its largest, 33 ln 2).
// 22.874 + 3.130 = 26.004; the margin covers fp32 rounding of m - z.
constexpr float kPruneNats = 26.25f;
constexpr float kLnInvEmin = 22.8738570f;  // 33 ln 2 = -ln of the least E
// Relative slack of the linear-domain Gumbel bound (covers the fp32
// rounding of the probability and of the uniform, ~1e-6).
constexpr float kSlack = 1.0009765625f;
constexpr double kMassScale = 17592186044416.0;  // 2^44 (general-path radix masses)
constexpr double kWinScale = 2147483648.0;        // 2^31 (window masses)
// A top-p crossing found from window masses must lie farther than this
// from its target (relative to the mass it is a fraction of) on each side
// where moving it one tie group would change the kept set, else the row
// takes the exact path.  The window sums' error is ~1e-8 (independent
// per-value errors of ~1e-7), so a decision this far from its target is
// the exact one.
constexpr double kTopPMarginRel = 1e-7;
constexpr float kLog2e = 1.44269504088896341f;
constexpr uint32_t kEmpty = 0xFFFFFFFFu;
constexpr uint32_t kNone = 0xFFFFFFFFu;

// LDS region layout after the penalty phase (byte offsets):
//   A: merged inclusive prefix counts lc[kWinBins] (u32) and masses
//      lm[kWinBins + 1] (u64), filled by a merging workgroup;
//   B: the local histogram wh[kWinBins] (packed u64); later the
//      per-wave candidate staging; later the merger's sorted candidate keys
//      sk[kCandCap] (u64) and prefix masses sq[kCandCap] (f64).
constexpr size_t kRegionLm = 4 * kWinBins;
constexpr size_t kRegionB = (kRegionLm + 8 * (kWinBins + 1) + 15) & ~(size_t)15;
constexpr size_t kRegionBBytes = 16 * (size_t)kCandCap;
constexpr int kStagePerWave = (int)(kRegionBBytes / 8) / kWaves;
static_assert(kWinBins == kBlock, "the merge gives each thread one bin");
static_assert(2 * 256 * 12 <= kRegionBBytes, "radix histograms fit the region");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct alignas(16) SmemBase {
  double exp_tab[64];  // 2^(j/64)
  float red_f[kWaves];
  double red_d[kWaves];
  unsigned long long red_u[kWaves];
  int red_i[kWaves];
  uint32_t red_c[kWaves];
  uint32_t bu[40];
  double bd[16];
  uint32_t binmask[kWinBins / 32]; // the bins the gather collects
  double gd[kMaxG];              // per-workgroup values read by a merger
  double gf[kMaxG];
  double gs[kMaxG];
  unsigned long long gk[kMaxG];
  float ga[kMaxG];
  int gi[kMaxG];
  uint32_t gcnt[kMaxG];          // merger: candidates per workgroup
  uint32_t gpo[kMaxG + 1];       // merger: 16-byte pair offsets per workgroup
  uint32_t goff[kMaxG + 1];      // merger: candidate offsets per workgroup
  unsigned long long tl[kMaxTopLogprobs];
};

// ---------------------------------------------------------------- helpers
DEV uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DEV float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

template <typename T>
DEV T atomic_ld(const T *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
DEV void atomic_st(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The thread index behind an opaque copy: values derived from it are
// recomputed where used instead of being hoisted out of the row loop (where
// they would stay live across every phase).
DEV int tidx() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// One 16-byte read (16-byte aligned) at the point of coherence: the same
// access an agent-scope atomic load makes (sc1), issued as one instruction,
// so a thread fetches four exchange words in one round trip.  (The compiler
// waits after every atomic load, so a sequence of them costs one round trip
// each.)
DEV u32x4 coh_load16(const void *p) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(r) : "v"(p) : "memory");
  return r;
}
// Two such reads sharing one wait.
DEV void coh_load16x2(const void *p0, const void *p1, u32x4 &a, u32x4 &b) {
  asm volatile(
      "global_load_dwordx4 %0, %2, off sc1\n\t"
      "global_load_dwordx4 %1, %3, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(a), "=&v"(b)
      : "v"(p0), "v"(p1)
      : "memory");
}
// Three such reads sharing one wait.
DEV void coh_load16x3(const void *p0, const void *p1, const void *p2, u32x4 &a, u32x4 &b, u32x4 &c) {
  asm volatile(
      "global_load_dwordx4 %0, %3, off sc1\n\t"
      "global_load_dwordx4 %1, %4, off sc1\n\t"
      "global_load_dwordx4 %2, %5, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c)
      : "v"(p0), "v"(p1), "v"(p2)
      : "memory");
}
// Four and six such reads sharing one wait.
DEV void coh_load16x4(const void *p0, const void *p1, const void *p2, const void *p3, u32x4 &a, u32x4 &b, u32x4 &c,
                      u32x4 &d) {
  asm volatile(
      "global_load_dwordx4 %0, %4, off sc1\n\t"
      "global_load_dwordx4 %1, %5, off sc1\n\t"
      "global_load_dwordx4 %2, %6, off sc1\n\t"
      "global_load_dwordx4 %3, %7, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3)
      : "memory");
}
DEV void coh_load16x6(const void *p0, const void *p1, const void *p2, const void *p3, const void *p4, const void *p5,
                      u32x4 &a, u32x4 &b, u32x4 &c, u32x4 &d, u32x4 &e, u32x4 &f) {
  asm volatile(
      "global_load_dwordx4 %0, %6, off sc1\n\t"
      "global_load_dwordx4 %1, %7, off sc1\n\t"
      "global_load_dwordx4 %2, %8, off sc1\n\t"
      "global_load_dwordx4 %3, %9, off sc1\n\t"
      "global_load_dwordx4 %4, %10, off sc1\n\t"
      "global_load_dwordx4 %5, %11, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d), "=&v"(e), "=&v"(f)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "v"(p4), "v"(p5)
      : "memory");
}
DEV unsigned long long u64_of(uint32_t lo, uint32_t hi) { return ((unsigned long long)hi << 32) | lo; }
DEV double f64_of(uint32_t lo, uint32_t hi) { return __longlong_as_double((long long)u64_of(lo, hi)); }

// Wave-wide inclusive scans by DPP: row_shr:1,2,4,8 (Hillis-Steele within
// each 16-lane row, lanes shifted in from outside the row read 0), then
// row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and 3.  The
// combining order is fixed, so results are deterministic.
template <int CTRL, int ROWS>
DEV uint32_t dpp_mov(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, ROWS, 0xF, false);
}
#define DSTS_DPP_SCAN_STEPS(X) X(0x111, 0xF) X(0x112, 0xF) X(0x114, 0xF) X(0x118, 0xF) X(0x142, 0xA) X(0x143, 0xC)

DEV uint32_t wave_scan_u32(uint32_t v) {
#define X(C, R) v += dpp_mov<C, R>(v);
  DSTS_DPP_SCAN_STEPS(X)
#undef X
  return v;
}
DEV unsigned long long wave_scan_u64(unsigned long long v) {
#define X(C, R) v += u64_of(dpp_mov<C, R>((uint32_t)v), dpp_mov<C, R>((uint32_t)(v >> 32)));
  DSTS_DPP_SCAN_STEPS(X)
#undef X
  return v;
}
DEV double wave_scan_f64(double v) {
#define X(C, R)                                                                                              \
  {                                                                                                          \
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);                                \
    v += __longlong_as_double((long long)u64_of(dpp_mov<C, R>((uint32_t)b), dpp_mov<C, R>((uint32_t)(b >> 32)))); \
  }
  DSTS_DPP_SCAN_STEPS(X)
#undef X
  return v;
}
// running maximum (0 is the identity: unsigned keys)
DEV unsigned long long wave_scanmax_u64(unsigned long long v) {
#define X(C, R)                                                                        \
  {                                                                                    \
    const unsigned long long t = u64_of(dpp_mov<C, R>((uint32_t)v), dpp_mov<C, R>((uint32_t)(v >> 32))); \
    v = t > v ? t : v;                                                                 \
  }
  DSTS_DPP_SCAN_STEPS(X)
#undef X
  return v;
}
DEV uint32_t wave_scanmax_u32(uint32_t v) {
#define X(C, R)                              \
  {                                          \
    const uint32_t t = dpp_mov<C, R>(v);     \
    v = t > v ? t : v;                       \
  }
  DSTS_DPP_SCAN_STEPS(X)
#undef X
  return v;
}
DEV uint32_t lane63_u32(uint32_t v) { return __builtin_amdgcn_readlane(v, 63); }
DEV unsigned long long lane63_u64(unsigned long long v) {
  return u64_of(__builtin_amdgcn_readlane((uint32_t)v, 63), __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63));
}
DEV double wave_sum_d(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(wave_scan_f64(v));
  return __longlong_as_double((long long)lane63_u64(b));
}
DEV unsigned long long wave_max_u(unsigned long long v) { return lane63_u64(wave_scanmax_u64(v)); }
// maximum of non-negative floats (their bit patterns order as integers)
DEV float wave_max_nonneg_f(float v) { return __uint_as_float(lane63_u32(wave_scanmax_u32(__float_as_uint(v)))); }

// Workgroup reductions (every thread gets the result).
// Fixed order: lanes by the DPP scan, waves in index order (deterministic).
DEV double wg_sum_d(SmemBase &sm, double v) {
  v = wave_sum_d(v);
  if ((tidx() & 63) == 0) sm.red_d[tidx() >> 6] = v;
  __syncthreads();
  double r = sm.red_d[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += sm.red_d[w];
  __syncthreads();
  return r;
}
DEV unsigned long long wg_max_u(SmemBase &sm, unsigned long long v) {
  v = wave_max_u(v);
  if ((tidx() & 63) == 0) sm.red_u[tidx() >> 6] = v;
  __syncthreads();
  unsigned long long r = sm.red_u[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = sm.red_u[w] > r ? sm.red_u[w] : r;
  __syncthreads();
  return r;
}
// Sum of one u64 per thread over the workgroup (exact).
DEV unsigned long long wg_sum_u(SmemBase &sm, unsigned long long v) {
  v = lane63_u64(wave_scan_u64(v));
  if ((tidx() & 63) == 0) sm.red_u[tidx() >> 6] = v;
  __syncthreads();
  unsigned long long r = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r += sm.red_u[w];
  __syncthreads();
  return r;
}
// Best (score desc, index asc) pair over the workgroup.
DEV void wave_best(double &g, int &idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    double g2 = __shfl_xor(g, o, 64);
    int i2 = __shfl_xor(idx, o, 64);
    if (g2 > g || (g2 == g && i2 < idx)) {
      g = g2;
      idx = i2;
    }
  }
}
DEV void wg_best(SmemBase &sm, double &g, int &idx) {
  wave_best(g, idx);
  if ((tidx() & 63) == 0) {
    sm.red_d[tidx() >> 6] = g;
    sm.red_i[tidx() >> 6] = idx;
  }
  __syncthreads();
  g = sm.red_d[0];
  idx = sm.red_i[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    if (sm.red_d[w] > g || (sm.red_d[w] == g && sm.red_i[w] < idx)) {
      g = sm.red_d[w];
      idx = sm.red_i[w];
    }
  }
  __syncthreads();
}

// Inclusive scan of one value per thread over the workgroup (fixed order).
DEV uint32_t wave_scan(uint32_t v) { return wave_scan_u32(v); }
DEV unsigned long long wave_scan(unsigned long long v) { return wave_scan_u64(v); }
DEV double wave_scan(double v) { return wave_scan_f64(v); }
template <typename T>
DEV T block_scan_incl(T v, T *wave_tot) {
  const int lane = tidx() & 63, w = tidx() >> 6;
  v = wave_scan(v);
  if (lane == 63) wave_tot[w] = v;
  __syncthreads();
  T base = 0;
  for (int i = 0; i < w; ++i) base += wave_tot[i];
  __syncthreads();
  return v + base;
}

// Inclusive scans of a count and a mass per thread over the workgroup,
// sharing one barrier; the caller passes another barrier before it writes
// the wave totals again.
DEV void block_scan_incl2(uint32_t &c, unsigned long long &v, uint32_t *ctot, unsigned long long *vtot) {
  const int lane = tidx() & 63, w = tidx() >> 6;
  c = wave_scan(c);
  v = wave_scan(v);
  if (lane == 63) {
    ctot[w] = c;
    vtot[w] = v;
  }
  __syncthreads();
  uint32_t cb = 0;
  unsigned long long vb = 0;
  for (int i = 0; i < w; ++i) {
    cb += ctot[i];
    vb += vtot[i];
  }
  c += cb;
  v += vb;
}

// Philox4x32-10 block for counter (c0..c3) and key (k0, k1); each round
// takes both halves of the two 32x32-bit products.
DEV void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1,
                       uint32_t out[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t pa = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t pb = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t n0 = (uint32_t)(pb >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(pa >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = (uint32_t)pb;
    c2 = n2;
    c3 = (uint32_t)pa;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// Exp(1) from a 32-bit word, fp64: w = (x + 1/2) 2^-32, E = -ln(1 - w),
// clamped below at FLT_MIN ([A] "Nine lines, and exactly one call site").
DEV double exp1_f64(uint32_t x) {
  const double w = ((double)x + 0.5) * 0x1p-32;
  double e = -log1p(-w);
  return e < (double)FLT_MIN ? (double)FLT_MIN : e;
}

// exp(y) for y <= 0 in fp64: y = k ln2/64 + r with |r| <= ln2/128 (ln2/64 in
// two parts, the first exact in k * c), exp(r) by its degree-6 Taylor
// polynomial (truncation below 3e-20 relative), times 2^(k mod 64 / 64)
// from the table and 2^(k div 64).  y below -800 gives 0.
DEV double exp_nonpos(const double *tab, double y) {
  y = y < -800.0 ? -800.0 : y;
  const double kd = rint(y * 92.332482616893656);
  const double r = fma(-kd, -0x1.718432a1b0e26p-41, fma(-kd, 0x1.62e42ffp-7, y));
  double p = 1.0 / 720.0;
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int k = (int)kd;
  return ldexp(tab[k & 63] * p, k >> 6);
}

// A summand exp(z - m) (z <= m, m finite) of a normaliser that only scales
// outputs: t = (z - m) log2 e in fp64 (the difference of two fp32 values is
// exact, the product's error is below 1e-13 absolute), split into an
// integer k and a fraction f in [-1/2, 1/2]; 2^f by the hardware exp2 of f
// rounded to fp32 (1 ulp, and 2^-25 ln 2 from the rounding of f); 2^k
// exactly.  Relative error below 1.5e-7; -inf (and anything below 2^-1070)
// gives 0.
DEV double exp_term(float z, double m) {
  const double t = ((double)z - m) * 1.4426950408889634;
  if (!(t > -1070.0)) return 0.0;
  const double k = rint(t);
  const float e = __builtin_amdgcn_exp2f((float)(t - k));
  return ldexp((double)e, (int)k);
}

// Penalties on one logit ([C] "解码一步里采样做什么", _apply_penalties):
// repetition divides positive and multiplies non-positive logits, then
// frequency subtracts f * count, then presence subtracts p; each operation
// is rounded to fp32 on its own (the file builds with -ffp-contract=off).
DEV float apply_penalty(float x, uint32_t cnt, const RowParam &P) {
  const float t1 = (x > 0.0f) ? (x / P.rep) : (x * P.rep);
  const float fc = P.freq * (float)cnt;
  const float t2 = t1 - fc;
  return t2 - P.pres;
}

// A token's summed logit_bias added to its (sanitised) logit; NaN -> -inf.
DEV float add_bias(float x, float b) {
  const float y = x + b;
  return y == y ? y : -INFINITY;
}

// z = x / T, correctly rounded: q = x (1/T), then one FMA correction with
// the exact remainder (Markstein), valid while |q| lies in [2^-100, 2^100];
// elsewhere (and for infinities and zeros) the IEEE division.  -0 -> +0, so
// equal values share one key.  (The transform loop inlines the same
// computation with the out-of-range branch taken per group of four.)
DEV float div_temp(float x, float T, float rT) {
  const float q = x * rT;
  const float aq = fabsf(q);
  float z;
  if (__builtin_expect(aq >= 0x1p-100f && aq <= 0x1p100f, 1)) z = __builtin_fmaf(__builtin_fmaf(-q, T, x), rT, q);
  else z = x / T;
  return z + 0.0f;
}

template <typename TIn>
struct Loader;

// load4: four consecutive values at element offset `off` (16- or 8-byte
// aligned); load1: one value.  Streaming data: non-temporal loads.
template <>
struct Loader<float> {
  static DEV void load4(const void *base, int64_t off, float v[4]) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + off));
    v[0] = t.x;
    v[1] = t.y;
    v[2] = t.z;
    v[3] = t.w;
  }
  static DEV float load1(const void *base, int64_t off) {
    return __builtin_nontemporal_load(reinterpret_cast<const float *>(base) + off);
  }
};

template <>
struct Loader<uint16_t> {
  static DEV void load4(const void *base, int64_t off, float v[4]) {
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(base) + off));
    v[0] = __uint_as_float(t.x << 16);
    v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16);
    v[3] = __uint_as_float(t.y & 0xFFFF0000u);
  }
  static DEV float load1(const void *base, int64_t off) {
    const uint16_t b = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(base) + off);
    return __uint_as_float((uint32_t)b << 16);
  }
};

// ---------------------------------------------------------------- group sync
// Every word that workgroups exchange (slots, group records, barrier words)
// is read and written only with relaxed agent-scope atomics, which on gfx950
// go to the point of coherence instead of a per-XCD cache.  Ordering between
// them therefore needs no cache maintenance: a signalling workgroup waits
// for its own stores to complete (vmcnt 0 in every wave, then a workgroup
// barrier) before its signal, and a waiting workgroup issues its data loads
// only after the signal load has returned.  Agent-scope fences would also
// write back and invalidate the whole L2 (several microseconds per barrier)
// and are not used.
DEV void mem_quiesce() { __builtin_amdgcn_s_waitcnt(0); }
DEV void order_release() {
  mem_quiesce();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
}
DEV void order_acquire() {
  mem_quiesce();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Group words (the barrier word and the final-exchange counter) carry, in
// bits 32..63, the epoch of the launch that last used them; every launch has
// its own epoch (host launches count up from 1, launches whose epoch lives
// in device memory have bit 31 set).  A launch therefore never inherits an
// earlier launch's count, also after that launch aborted mid-count.  At its
// start a launch claims its groups' words with a fire-and-forget atomic max
// of epoch << 32 (epochs mostly increase, so the max resets a word to this
// launch's epoch with zero counts, and leaves a word it already claimed as
// it is).  An arrival adds one; an arrival that still finds an older epoch
// (the claim has not landed, or the epochs went back) claims the word by a
// compare-and-swap from what it holds, as if it were clear, or adds again
// once another arrival has claimed it.
//   barrier word: epoch << 32 | generation << 8 | arrivals
//   final word:   epoch << 32 | arrivals
// The last arrival at a barrier resets the count and advances the
// generation in one store; the others wait for the generation to change.
struct GroupCtx {
  GroupSync *s;
  uint32_t *abort_word;
  uint32_t epoch;
  uint32_t spin_limit;
  int G;
};

// The launch's claim of a group's two words (one thread per group).
DEV void claim_words(GroupSync *s, uint32_t epoch) {
  const unsigned long long mine = (unsigned long long)epoch << 32;
  __hip_atomic_fetch_max(&s->word, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_max(&s->fin, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One arrival at a group word; returns the word's value before it (the
// count of an older epoch reads as 0).
DEV unsigned long long arrive_word(unsigned long long *w, uint32_t epoch) {
  const unsigned long long mine = (unsigned long long)epoch << 32;
  const unsigned long long old = __hip_atomic_fetch_add(w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((uint32_t)(old >> 32) == epoch) return old;
  // an older epoch's word (the add above went to its count, which the claim
  // discards)
  unsigned long long cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while ((uint32_t)(cur >> 32) != epoch) {
    if (__hip_atomic_compare_exchange_strong(w, &cur, mine | 1ull, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return mine;
  }
  return __hip_atomic_fetch_add(w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The wait is bounded (~2 s by default): on expiry the launch is marked
// aborted (the abort word takes this launch's epoch), every later wait of
// the launch returns at once and the rows report status 3, so a logic error
// cannot hang the device.
constexpr uint32_t kSpinLimit = 1u << 26;
DEV void spin_gen(const GroupCtx &gc, uint32_t g0) {
  // one coherent load per iteration; the abort word (a peer's expired wait)
  // and the bound are checked every 256 iterations (every iteration under a
  // bound below 256)
  const uint32_t mask = gc.spin_limit < 256u ? 0u : 255u;
  uint32_t spins = 0;
  while (((uint32_t)__hip_atomic_load(&gc.s->word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 8) == g0) {
    if ((++spins & mask) == 0u) {
      if (__hip_atomic_load(gc.abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gc.epoch) break;
      if (spins > gc.spin_limit) {
        __hip_atomic_store(gc.abort_word, gc.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Barrier: every wave waits for its own stores, then one arrival; the last
// arrival resets the count and advances the generation in one store, the
// others wait for it.
DEV void group_barrier(SmemBase &sm, GroupCtx &gc) {
  order_release();
  __syncthreads();
  if (gc.G == 1) {  // a one-workgroup group: its own stores are all there is to wait for
    if (tidx() == 0) order_acquire();
    __syncthreads();
    return;
  }
  if (tidx() == 0) {
    const unsigned long long old = arrive_word(&gc.s->word, gc.epoch);
    const uint32_t g0 = ((uint32_t)old >> 8) & 0xFFFFFFu;
    if ((old & 0xFFull) == (unsigned long long)gc.G - 1ull)
      __hip_atomic_store(&gc.s->word, ((unsigned long long)gc.epoch << 32) | ((unsigned long long)((g0 + 1u) & 0xFFFFFFu) << 8),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else spin_gen(gc, g0);
    order_acquire();
  }
  __syncthreads();
}

// Arrival at the final exchange of a row: true in the last workgroup to
// arrive, which resets the count (one lane calls it).
DEV bool final_arrive(const GroupCtx &gc) {
  if (gc.G == 1) return true;
  const unsigned long long old = arrive_word(&gc.s->fin, gc.epoch);
  const bool last = (old & 0xFFull) == (unsigned long long)gc.G - 1ull;
  if (last) __hip_atomic_store(&gc.s->fin, (unsigned long long)gc.epoch << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// An exchange slot's address, computed where it is used from an opaque
// index (a slot pointer kept live across the row would be spilled).
DEV WgSlots *slot_at(const KernelParams &kp, int i) {
  i = __builtin_amdgcn_readfirstlane(i);
  asm volatile("" : "+s"(i));
  return kp.slots + i;
}

// Per-row context shared by the phases.
struct RowCtx {
  int row, gid, G, n, n4, s0;
  GroupCtx gc;
  WgSlots *my;
  WgSlots *peers;
  unsigned *xseq;
};

DEV void row_barrier(SmemBase &sm, RowCtx &rc) { group_barrier(sm, rc.gc); }

// Bins on an absolute grid: abin(z) = floor(z (32 wsc)) with wsc = min(1, T),
// so a bin is 1/32 nat of the logits x = z T below T = 1 and of z above it.
// A value's window bin is A - abin(z), counted down from the anchor A =
// abin(row max); bins from kWinBins on are deep.  Every bin of the kernel is
// computed by these two expressions (float operations: monotone in z, so
// the bins partition the value axis in order, and an anchor shift between
// two slices is a whole number of bins while |z wsc 32| < 2^24).
DEV float abin(float z, float wsc) { return floorf(z * (wsc * (float)kBinsPerNat)); }
DEV float win_pos(float A, float z, float wsc) { return A - abin(z, wsc); }
DEV int win_bin(float A, float z, float wsc) {
  const float lb = win_pos(A, z, wsc);
  return lb < (float)kWinBins ? (int)lb : kWinBins;
}

// The smallest value z whose window position A - abin(z) is at most h (a
// whole number): the values at or above it are exactly those in bins 0..h.
// Found on the order keys of the floats with the same expressions the bins
// use: a guess from the inverse of abin, settled within a few key steps,
// else a bisection.
DEV float win_floor_z(float A, float h, float wsc) {
  auto in = [&](uint32_t k) { return win_pos(A, key_to_float(k), wsc) <= h; };
  const uint32_t kninf = fkey(-INFINITY), kinf = fkey(INFINITY);  // in(kninf) false, in(kinf) true
  uint32_t k = fkey(((A - h) * (1.0f / kBinsPerNat)) / wsc);
  k = k < kninf ? kninf : (k > kinf ? kinf : k);
  for (int s = 0; s < 4; ++s) {
    if (in(k)) {
      if (!in(k - 1u)) return key_to_float(k);
      --k;
    } else {
      ++k;
    }
  }
  uint32_t lo = kninf, hi = kinf;
  while (hi - lo > 1u) {
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (in(mid)) hi = mid;
    else lo = mid;
  }
  return key_to_float(hi);
}

// Window histogram entry of one value at distance d = max - z: a count of
// one in bits 48.. and the mass exp(-d) in 2^-31 units below (rounded to an
// integer); a workgroup's bin holds at most 2^15 values, so neither field
// overflows.  The mass is the hardware exp2 of the small argument -d log2 e,
// then scaled by 2^31 exactly.  Its relative error is at most about
// 1.2e-7 (exp2) + 1.2e-7 d (the fp32 roundings of d and of d log2 e), and
// the rounding to units adds 2^-32 of the max's mass; these masses place
// thresholds in bins, and sum the bins above a threshold (a top-p decision
// closer to its target than kTopPMarginRel is taken by the exact path).
DEV float mass_scaled(float d) { return __builtin_amdgcn_exp2f(-d * kLog2e) * 2147483648.0f; }
DEV unsigned long long hist_entry(float a) {
  return (1ull << 48) | (unsigned long long)(uint32_t)__builtin_rintf(a);
}

// Candidate order key: value key << 32 | ~index (descending key order is
// (value desc, index asc); 0 never occurs for a real value).
DEV unsigned long long cand_key(float z, int idx) {
  return ((unsigned long long)fkey(z) << 32) | (uint32_t)(~(uint32_t)idx);
}

// ---------------------------------------------------------------- general path
// Radix select over the order-preserving keys of the slice values with
// key >= lower, one group exchange per 8-bit digit (used when a threshold
// lies outside the window or too many values share its bin).
//   COUNT: the key of the value of rank k in descending order (ties share a
//          key): #{key > t} < k <= #{key >= t}.
//   MASS:  the largest key t whose cumulative mass C(t) = sum_{key >= t}
//          exp(z - m) reaches p * C(lower), in 2^-44 fixed point.
// Padding values are -inf: lowest bin, zero mass, so they never move a
// threshold above -inf.  The digit is found in parallel over the 256 bins
// (thread t holds bin 255 - t, so an inclusive scan runs from the top).
template <bool MASS>
DEV uint32_t radix_select(SmemBase &sm, RowCtx &rc, const float *zs, unsigned char *region, uint32_t lower,
                          uint32_t k, double p, double m) {
  uint32_t *hcnt = reinterpret_cast<uint32_t *>(region);
  unsigned long long *hmass = reinterpret_cast<unsigned long long *>(region + 1024);
  unsigned long long *cum = reinterpret_cast<unsigned long long *>(region + 3072);
  const int tid = tidx();
  uint32_t prefix = 0, mask = 0;
  uint32_t rem = k;
  unsigned long long above = 0;
  double target = 0.0;
  for (int round = 0; round < 4; ++round) {
    const int shift = 24 - 8 * round;
    for (int b = tid; b < 256; b += kBlock) {
      hcnt[b] = 0;
      hmass[b] = 0;
    }
    __syncthreads();
    for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float zz = v[c];
        const uint32_t key = fkey(zz);
        if (key >= lower && (key & mask) == prefix) {
          const uint32_t bin = (key >> shift) & 0xFFu;
          if (MASS) atomicAdd(&hmass[bin], (unsigned long long)(exp_nonpos(sm.exp_tab, (double)zz - m) * kMassScale));
          else atomicAdd(&hcnt[bin], 1u);
        }
      }
    }
    __syncthreads();
    const unsigned par = (*rc.xseq)++ & 1u;
    for (int b = tid; b < 256; b += kBlock) {
      if (MASS) atomic_st(&rc.my->hmass[par][b], hmass[b]);
      else atomic_st(&rc.my->hcnt[par][b], hcnt[b]);
    }
    row_barrier(sm, rc);
    unsigned long long v = 0;
    if (tid < 256)
      for (int g = 0; g < rc.G; ++g)
        v += MASS ? atomic_ld(&rc.peers[g].hmass[par][255 - tid]) : (unsigned long long)atomic_ld(&rc.peers[g].hcnt[par][255 - tid]);
    const unsigned long long incl = block_scan_incl<unsigned long long>(v, sm.red_u);
    if (tid < 256) cum[tid] = incl;
    if (MASS && round == 0 && tid == 255) sm.bd[0] = p * (double)incl;
    if (tid == 0) sm.bu[0] = 255;
    __syncthreads();
    if (MASS && round == 0) target = sm.bd[0];
    if (tid < 256) {
      auto pred = [&](int t) {
        return t == 255 || (MASS ? ((double)(above + cum[t]) >= target) : (cum[t] >= (unsigned long long)rem));
      };
      if (pred(tid) && (tid == 0 || !pred(tid - 1))) sm.bu[0] = (uint32_t)tid;
    }
    __syncthreads();
    const int t = (int)sm.bu[0];
    const unsigned long long before = t > 0 ? cum[t - 1] : 0ull;
    if (MASS) above += before;
    else rem -= (uint32_t)before;
    prefix |= (uint32_t)(255 - t) << shift;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  return prefix;
}

// Packed hash entry: slice-local index << 13 | count.
DEV uint32_t hash_slot(uint32_t local, uint32_t slots) { return (local * 2654435761u) & (slots - 1u); }

// The summed bias of slice-local token `local`, if the row lists one.
DEV bool bias_lookup(const unsigned long long *bhash, uint32_t slots, uint32_t local, float &b) {
  uint32_t sl = hash_slot(local, slots);
  while (true) {
    const unsigned long long e = bhash[sl];
    if ((uint32_t)e == local) {
      b = __uint_as_float((uint32_t)(e >> 32));
      return true;
    }
    if ((uint32_t)e == 0xFFFFFFFFu) return false;
    sl = (sl + 1u) & (slots - 1u);
  }
}

// Whether slice-local token `local` has a history entry.
DEV bool hist_contains(const uint32_t *hash, uint32_t slots, uint32_t local) {
  uint32_t sl = hash_slot(local, slots);
  while (true) {
    const uint32_t e = hash[sl];
    if (e == 0xFFFFFFFFu) return false;
    if ((e >> 13) == local) return true;
    sl = (sl + 1u) & (slots - 1u);
  }
}

// min-p keeps exp(z - m) >= min_p (fp64).  That set is an upper set of keys
// (keys above the max's count as passing); its boundary is the smallest
// passing key.  Serial form: from the closed-form guess m + ln(min_p),
// bracket and bisect.
DEV uint32_t min_p_key_serial(double m, float min_p) {
  const double mp = (double)min_p;
  auto pass = [&](uint32_t k) { return exp((double)key_to_float(k) - m) >= mp; };
  const uint32_t top = fkey((float)m);  // passes: exp(0) = 1 >= min_p
  uint32_t g = fkey((float)(m + log(mp)));
  if (g > top) g = top;
  uint32_t lo, hi;  // pass(hi), !pass(lo)
  if (pass(g)) {
    hi = g;
    uint32_t step = 1;
    lo = g;
    while (true) {
      lo = (lo > step) ? lo - step : 0;
      if (lo == 0 || !pass(lo)) break;
      hi = lo;
      step *= 2;
    }
    if (lo == 0 && pass(0)) return 0;
  } else {
    lo = g;
    uint32_t step = 1;
    hi = g;
    while (true) {
      hi = (top - hi > step) ? hi + step : top;
      if (pass(hi)) break;
      lo = hi;
      step *= 2;
    }
  }
  while (hi - lo > 1u) {
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (pass(mid)) hi = mid;
    else lo = mid;
  }
  return hi;
}

// Parallel form: the boundary lies within a few keys of the guess, so two
// waves test the 128 keys around it, one key per lane, and the boundary is
// the lowest passing key of their ballots (pass is monotone in the key).
// Outside that span, the serial search.  lmp = ln(min_p), taken by the
// caller ahead of the exchange so its latency hides in the wait.  The
// ballots go to bu[32..35], read after one barrier; the caller passes
// other barriers before this function runs again.
DEV uint32_t min_p_key(SmemBase &sm, double m, double lmp, float min_p) {
  constexpr int kSpan = 128;
  const int tid = tidx();
  const double mp = (double)min_p;
  const uint32_t top = fkey((float)m);
  uint32_t g = fkey((float)(m + lmp));
  if (g > top) g = top;
  const int64_t k0 = (int64_t)g - kSpan / 2;
  if (tid < kSpan) {
    const int64_t k = k0 + tid;
    bool p;
    if (k > (int64_t)top) {
      p = true;
    } else if (k < 0) {
      p = false;
    } else {
      const double x = (double)key_to_float((uint32_t)k) - m;  // <= 0, or NaN below -inf's key
      p = x == x && exp_nonpos(sm.exp_tab, x) >= mp;
    }
    const unsigned long long bal = __ballot(p);
    if ((tid & 63) == 0) {
      sm.bu[32 + 2 * (tid >> 6)] = (uint32_t)bal;
      sm.bu[33 + 2 * (tid >> 6)] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();
  const unsigned long long b0 = u64_of(sm.bu[32], sm.bu[33]), b1 = u64_of(sm.bu[34], sm.bu[35]);
  const int first = b0 ? __ffsll((long long)b0) - 1 : b1 ? 64 + __ffsll((long long)b1) - 1 : -1;
  if (first <= 0) return min_p_key_serial(m, min_p);  // the boundary lies outside the span
  return (uint32_t)(k0 + first);
}

// Exchange 3 for at most 256 candidates: the waves have placed the sorted
// keys in sq; one wave then decides (position p = lane + 64 s in slot s of
// a lane) with no workgroup barrier: the same decisions as the workgroup
// form in the kernel (each gathered bin's first position and a check of
// the list against the merged counts, prefix masses, the end of the top-k
// tie group, the top-p crossing, the kept-set sum and the top logprobs),
// with wave scans and ballots in place of the searches.  lc becomes the
// bins' first positions.
constexpr int kE3Slots = 4;
struct E3In {
  int top_k;
  float top_p;
  double m, s_all;
  float Af, wsc;
  uint32_t t_m;
  int rklo, rkhi, r1lo, r1hi, K, row, gid;
  bool full_k, topk_on, topp, minp, truncated, want_S;
  bool lp_all;  // top logprobs list every token, valued with ln of the full sum
  double lnA;   // ln of the full sum (with lp_all)
};
struct E3Out {
  bool general;
  uint32_t tau;
  double lnS;
};
DEV E3Out e3_decide(SmemBase &sm, const int n, const double *sq, uint32_t *lc, const unsigned long long *lm, const E3In &in,
                    const KernelParams &kp) {
  const int lane = tidx() & 63;
  const unsigned long long *srt = reinterpret_cast<const unsigned long long *>(sq);
  bool has[kE3Slots];
  uint32_t kj[kE3Slots];  // the key at each of the lane's positions
#pragma unroll
  for (int s = 0; s < kE3Slots; ++s) {
    has[s] = lane + 64 * s < n;
    kj[s] = has[s] ? (uint32_t)(srt[lane + 64 * s] >> 32) : 0u;
  }
  // values above the top-k bin (merged inclusive counts, read before lc
  // becomes positions)
  const uint32_t c_rk = in.rklo > 0 ? lc[min(in.rklo - 1, kWinBins - 1)] : 0u;
  // the gathered bins' first positions: a masked scan of the merged counts,
  // eight bins per lane
  uint32_t tot;
  {
    uint32_t cbs[8], sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = 8 * lane + u;
      const bool gb = (sm.binmask[b >> 5] >> (b & 31)) & 1u;
      cbs[u] = gb ? lc[b] - (b > 0 ? lc[b - 1] : 0u) : 0u;
      sum += cbs[u];
    }
    const uint32_t incl = wave_scan_u32(sum);
    tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    uint32_t run = incl - sum;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      lc[8 * lane + u] = run;
      run += cbs[u];
    }
  }
  __builtin_amdgcn_wave_barrier();
  // the list against the merged counts: as many candidates as the gathered
  // bins hold, each at a position inside its bin's range (else the exact
  // path)
  bool bad = false;
#pragma unroll
  for (int s = 0; s < kE3Slots; ++s) {
    if (64 * s < n && has[s]) {
      const int p = lane + 64 * s;
      const int bj = win_bin(in.Af, key_to_float(kj[s]), in.wsc);
      bad |= bj < 0 || bj >= kWinBins || !((sm.binmask[bj >> 5] >> (bj & 31)) & 1u) || p < (int)lc[bj] ||
             p >= (bj + 1 < kWinBins ? (int)lc[bj + 1] : (int)tot);
    }
  }
  uint32_t flags = (__ballot(bad) || tot != (uint32_t)n) ? 1u : 0u;
  // inclusive prefix of the exact masses exp(z - m) along the list, slot by
  // slot
  // (slots past the list's end hold the running total; the test is
  // wave-uniform, so short lists skip their fp64 work)
  double pj[kE3Slots];
  {
    double carry = 0.0;
#pragma unroll
    for (int s = 0; s < kE3Slots; ++s) {
      if (64 * s < n) {
        pj[s] = carry + wave_scan_f64(has[s] ? exp_nonpos(sm.exp_tab, (double)key_to_float(kj[s]) - in.m) : 0.0);
        carry = __shfl(pj[s], 63);
      } else {
        pj[s] = carry;
      }
    }
  }
  // a position's key and prefix mass (j wave-uniform, 0 <= j < n)
  auto keyof = [&](int j) {
    const int s = j >> 6, l = j & 63;
    const uint32_t v = s == 0 ? kj[0] : s == 1 ? kj[1] : s == 2 ? kj[2] : kj[3];
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
  };
  auto pre_at = [&](int j) {
    const int s = j >> 6, l = j & 63;
    const double v = s == 0 ? pj[0] : s == 1 ? pj[1] : s == 2 ? pj[2] : pj[3];
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    return __longlong_as_double((long long)u64_of((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l),
                                                  (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l)));
  };
  auto fpos = [&](int b) { return b >= kWinBins ? n : (int)lc[b]; };
  auto qsum = [&](int a, int e) { return (e < a) ? 0.0 : pre_at(e) - (a > 0 ? pre_at(a - 1) : 0.0); };
  auto cmass = [&](int b) { return b < 0 ? 0.0 : (double)lm[b < kWinBins ? b : kWinBins] / kWinScale; };
  // the number of positions whose key is at least t (a prefix of the list)
  auto count_ge = [&](uint32_t t) {
    int c = 0;
#pragma unroll
    for (int s = 0; s < kE3Slots; ++s)
      if (64 * s < n) c += __popcll(__ballot(has[s] && kj[s] >= t));
    return c;
  };
  const int fp_k = fpos(in.rklo), fp_p0 = fpos(in.r1lo), fp_p1 = fpos(in.r1hi + 1);
  // top-k: the value of rank k, and the end of its tie group
  uint32_t tk = 0;
  int ek = n - 1;
  if (!flags && in.topk_on) {
    const int jk = in.full_k ? in.top_k - 1 : fp_k + (in.top_k - (int)c_rk) - 1;
    if (jk < 0 || jk >= n) {
      flags |= 1u;
    } else {
      tk = keyof(jk);
      ek = count_ge(tk) - 1;
    }
  }
  // top-p: the first tie-group end in the crossing range whose cumulative
  // mass reaches p times the top-k set's mass
  uint32_t t = tk;
  if (!flags && in.topp) {
    const double ctot = in.topk_on ? (in.full_k ? qsum(0, ek) : cmass(in.rklo - 1) + qsum(fp_k, ek)) : cmass(kWinBins);
    const double target = (double)in.top_p * ctot;
    const double base = in.full_k ? 0.0 : cmass(in.r1lo - 1) - (fp_p0 > 0 ? pre_at(fp_p0 - 1) : 0.0);
    int e = -1;
#pragma unroll
    for (int s = 0; s < kE3Slots; ++s) {
      if (64 * s >= n) break;  // wave-uniform: past the list's end
      // the key one position on: the next lane, or the next slot's lane 0
      const uint32_t nx = s + 1 < kE3Slots ? (uint32_t)__builtin_amdgcn_readlane((int)kj[s + 1 < kE3Slots ? s + 1 : s], 0) : 0u;
      const uint32_t dn = (uint32_t)__shfl_down((int)kj[s], 1);
      const uint32_t knext = lane == 63 ? nx : dn;
      const int p = lane + 64 * s;
      const bool end = p == n - 1 || knext != kj[s];
      const unsigned long long bal = __ballot(has[s] && p >= fp_p0 && p < fp_p1 && end && base + pj[s] >= target);
      if (e < 0 && bal) e = 64 * s + __ffsll((long long)bal) - 1;
    }
    if (e < 0) {
      flags |= 1u;
    } else {
      // the crossing's distance from the target on both sides (the
      // cumulative mass at the end of its tie group and before the group)
      const uint32_t ke = keyof(e);
      int gs = 0;  // the group's first position: the count of larger keys
#pragma unroll
      for (int s = 0; s < kE3Slots; ++s)
        if (64 * s < n) gs += __popcll(__ballot(has[s] && kj[s] > ke));
      const double c_new = base + pre_at(e), c_prev = base + (gs > 0 ? pre_at(gs - 1) : 0.0);
      // a side matters when moving the crossing there changes max(t_p,
      // t_k, t_m): one group later lowers t_p below ke, one group earlier
      // raises it to the previous group's key (a bin above when the group
      // opens the list)
      const uint32_t tkm = max(t, in.minp ? in.t_m : 0u);
      const uint32_t kprev = gs > 0 ? keyof(gs - 1) : 0xFFFFFFFFu;
      const bool close_lo = c_new - target < kTopPMarginRel * ctot && ke > tkm;
      const bool close_hi = target - c_prev < kTopPMarginRel * ctot && kprev > tkm;
      if (close_lo || close_hi) flags |= 1u;
      else t = max(t, ke);
    }
  }
  if (in.minp) t = max(t, in.t_m);
  // the kept set: positions [0, et); its sum and the top logprobs
  const int bt = t ? win_bin(in.Af, key_to_float(t), in.wsc) : kWinBins;
  const int et = t ? count_ge(t) : n;
  const int fp_bt = fpos(bt);
  double S_K = in.s_all;
  if (!flags && in.truncated && in.want_S) {
    if (in.full_k && bt <= in.rkhi) S_K = qsum(0, et - 1);
    else if (bt < kWinBins) S_K = cmass(bt - 1) + qsum(fp_bt, et - 1);
    else flags |= 1u;
  }
  const double lns = log(S_K);
  if (!flags && in.K > 0 && in.gid == 0) {
    const int kept_n = (in.truncated && !in.lp_all) ? et : n;
    const double lnl = in.lp_all ? in.lnA : lns;
    for (int q = lane; q < in.K; q += 64) {
      const int64_t o = (int64_t)in.row * in.K + q;
      if (q < kept_n) {
        const unsigned long long sq_ = srt[q];
        kp.top_lp_vals[o] = (float)(((double)key_to_float((uint32_t)(sq_ >> 32)) - in.m) - lnl);
        kp.top_lp_ids[o] = (int)(~(uint32_t)sq_);
      } else {
        kp.top_lp_vals[o] = -INFINITY;
        kp.top_lp_ids[o] = -1;
      }
    }
  }
  return E3Out{(flags & 1u) != 0u, t, lns};
}

// The last workgroup of a row writes it: the row max and first argmax (the
// largest of the slices' max keys; rows that skipped exchange 2 get their
// status here) and, with Gumbel-max, the best of the slices' best scores,
// ties to the lower index.  With `reduce`, one whole wave calls it: lane g
// < G holds slice g's record (max key mk, best score bg, its index bi), the
// other lanes the identities (0, -inf, 0x7FFFFFFF); the reductions run
// across the wave and lane 0 writes.  Without, lane 0 alone calls it with
// the row's only record.  aborted: lane 0's reading of the abort word.
DEV void finish_row(const KernelParams &kp, bool aborted, int row, bool gumbel, bool token_set, unsigned long long mk,
                    double bg, int bi, bool reduce) {
  if (reduce) {
    mk = wave_max_u(mk);
    wave_best(bg, bi);
    if ((tidx() & 63) != 0) return;
  }
  const float mx = key_to_float((uint32_t)(mk >> 32));
  const int status = (mx > -INFINITY && mx < INFINITY) ? 0 : (mx == INFINITY ? 2 : 1);
  int token = (int)(0xFFFFFFFFu - (uint32_t)(mk & 0xFFFFFFFFu));
  if (gumbel && bi != 0x7FFFFFFF) token = bi;
  // token_set: the inverse-CDF selection already wrote the token
  if (!token_set || aborted || status != 0) kp.token_ids[row] = (aborted || status != 0) ? -1 : token;
  if (kp.row_status) kp.row_status[row] = aborted ? 3 : status;
}

// The final-exchange records of a row's G workgroups and the abort word, read
// by one wave (lane g < G: slice g's record), then finish_row.
DEV void merge_final(const KernelParams &kp, const WgSlots *peers, unsigned fpar, uint32_t epoch, int row, int G,
                     bool gumbel, bool token_set) {
  const int lane = tidx() & 63;
  unsigned long long k = 0;
  double g = -INFINITY;
  int i = 0x7FFFFFFF;
  bool ab = false;
  if (lane < G) {
    u32x4 r0, r1, ra;
    coh_load16x3(&peers[lane].fin[fpar][0], &peers[lane].fin[fpar][2], kp.abort_word, r0, r1, ra);
    g = f64_of(r0.x, r0.y);
    i = (int)r0.z;
    k = u64_of(r1.x, r1.y);
    ab = ra.x == epoch;
  }
  finish_row(kp, ab, row, gumbel, token_set, k, g, i, true);
}

// A row's record from per-row arrays in device memory, normalised and
// checked with the rules the host applies to host arrays ([A] "One request
// with top_p takes the whole batch off the fast path": 0 <= T < 1e-6 is
// greedy, T := 1, top_k := 1; -1 means the whole vocabulary).  bad is set
// when a value breaks them.
DEV RowParam row_from_device(const KernelParams &kp, int r) {
  const DevRowArrays &d = kp.dev;
  const int V = kp.vocab;
  const float t = d.temperature ? d.temperature[r] : 1.0f;
  const float top_p = d.top_p ? d.top_p[r] : 1.0f;
  const float min_p = d.min_p ? d.min_p[r] : 0.0f;
  const float rep = d.rep ? d.rep[r] : 1.0f;
  const float pres = d.pres ? d.pres[r] : 0.0f;
  const float freq = d.freq ? d.freq[r] : 0.0f;
  int32_t k = d.top_k ? d.top_k[r] : -1;
  const int32_t hl = d.hist_len ? d.hist_len[r] : 0;
  const int64_t hs = d.hist_start ? d.hist_start[r] : 0;
  const int32_t bl = d.bias_len ? d.bias_len[r] : 0;
  const int64_t bs = d.bias_start ? d.bias_start[r] : 0;
  const bool stop_on = d.min_tokens && d.output_len && d.output_len[r] < d.min_tokens[r];
  const int32_t sl = (stop_on && d.stop_len) ? d.stop_len[r] : 0;
  const int64_t ss = d.stop_start ? d.stop_start[r] : 0;
  const bool bad = !(t >= 0.0f && __builtin_isfinite(t)) || !(top_p > 0.0f && top_p <= 1.0f) || !(k == -1 || k >= 1) ||
        !(min_p >= 0.0f && min_p <= 1.0f) || !(rep > 0.0f && __builtin_isfinite(rep)) ||
        !__builtin_isfinite(pres) || !__builtin_isfinite(freq) || hl < 0 || hl > kp.max_hist ||
        (hl > 0 && (hs < 0 || !kp.history_ids)) || bl < 0 || sl < 0 ||
        (bl > 0 && (bs < 0 || !kp.bias_ids || !kp.bias_vals)) || (sl > 0 && (ss < 0 || !kp.stop_ids)) ||
        (int64_t)bl + sl > kp.max_bias;
  const bool greedy = t >= 0.0f && (double)t < 1e-6;
  if (greedy) k = 1;
  RowParam p;
  p.temperature = greedy ? 1.0f : t;
  p.top_p = top_p;
  p.min_p = min_p;
  p.rep = rep;
  p.pres = pres;
  p.freq = freq;
  p.top_k = (k == -1 || k >= V) ? V : k;
  uint32_t f = 0;
  if (greedy) f |= RF_GREEDY | RF_TOP1;
  else {
    if (k == 1) f |= RF_TOP1 | RF_TOPK;
    else if (k != -1 && k < V) f |= RF_TOPK;
    if (top_p < 1.0f) f |= RF_TOPP;
    if (min_p > 0.0f) f |= RF_MINP;
  }
  p.hist_start = 0;
  p.hist_len = 0;
  if ((rep != 1.0f || pres != 0.0f || freq != 0.0f) && hl > 0) {
    f |= RF_PEN;
    p.hist_start = hs;
    p.hist_len = hl;
  }
  p.bias_start = bl > 0 ? bs : 0;
  p.bias_len = bl > 0 ? bl : 0;
  p.stop_start = sl > 0 ? ss : 0;
  p.stop_len = sl > 0 ? sl : 0;
  if (p.bias_len + p.stop_len > 0) f |= RF_SPEC;
  p.flags = bad ? RF_BAD : f;
  p.seed = d.seed ? d.seed[r] : (kp.det ? 42ull : kp.seed);
  p.stream = d.stream ? d.stream[r] : (kp.det ? 0u : (uint32_t)r);
  p.offset = d.offset ? d.offset[r] : kp.offset;
  p.row = r;
  p.pad = 0;
  return p;
}

// One thread per row: the records of a step whose per-row parameters live
// in device memory (the row kernel then reads them like copied records).
// Thread 0 also advances the device epoch word that the kernels launched after
// it read (bit 31 set: never a host epoch), by two: the row kernel takes the
// new value and the raw-logprob kernel the one after it, so that a captured
// graph's replays are distinct launches.
__global__ __launch_bounds__(256) void rows_kernel(KernelParams kp, RowParam *out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < kp.n_rows) out[r] = row_from_device(kp, r);
  if (r == 0 && kp.epoch_dev) {
    const uint32_t e = *kp.epoch_dev;
    __hip_atomic_store(kp.epoch_dev, ((e + 2u) & 0x7FFFFFFEu) | 0x80000000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Block b runs on XCD b % 8 (the dispatcher deals blocks round-robin over
// the eight XCDs), so the G workgroups of a group are taken from one
// residue class: their exchanges then stay on one XCD (a group barrier
// measures ~0.86 us there against ~1.16 us across XCDs).  Only speed
// depends on this; every exchange is coherent device-wide either way.
// Groups beyond a multiple of 8 take consecutive blocks.
DEV void block_group(const KernelParams &kp, int &group, int &gid) {
  const int b = blockIdx.x, G = kp.G;
  const int gpx = kp.n_groups / 8;  // groups per XCD in the XCD-aware part
  const int nbx = gpx * 8 * G;
  if (b < nbx) {
    const int q = b / 8;
    group = (b % 8) * gpx + q / G;
    gid = q % G;
  } else {
    group = gpx * 8 + (b - nbx) / G;
    gid = (b - nbx) % G;
  }
}

// ---------------------------------------------------------------- phase stamps
// Builds with DSTS_PHASE_STAMPS record the real-time clock (s_memrealtime,
// a constant-rate counter shared by the whole device) at the phase
// boundaries of the first row each workgroup walks: thread 0 stores it to
// g_phase_stamps[block][k].  Other builds compile the stamps out.
#ifdef DSTS_PHASE_STAMPS
__device__ unsigned long long g_phase_stamps[kStampBlocks * kStampSlots];
#define PHASE_STAMP(k)                                                                                        \
  do {                                                                                                        \
    if (tidx() == 0 && it == 0u && blockIdx.x < (unsigned)kStampBlocks)                                       \
      g_phase_stamps[blockIdx.x * kStampSlots + (k)] = wall_clock64();                                        \
  } while (0)
// a stamp taken by whichever single thread reaches it (the caller ensures one)
#define PHASE_STAMP_ONE(k)                                                                                    \
  do {                                                                                                        \
    if (it == 0u && blockIdx.x < (unsigned)kStampBlocks) g_phase_stamps[blockIdx.x * kStampSlots + (k)] = wall_clock64(); \
  } while (0)
// a value instead of the clock (the row's index)
#define PHASE_RECORD(k, v)                                                                                    \
  do {                                                                                                        \
    if (tidx() == 0 && it == 0u && blockIdx.x < (unsigned)kStampBlocks)                                       \
      g_phase_stamps[blockIdx.x * kStampSlots + (k)] = (unsigned long long)(v);                               \
  } while (0)
#else
#define PHASE_RECORD(k, v) \
  do {                     \
  } while (0)
#define PHASE_STAMP(k) \
  do {                 \
  } while (0)
#define PHASE_STAMP_ONE(k) \
  do {                     \
  } while (0)
#endif

// ---------------------------------------------------------------- the kernel
template <typename TIn, bool PEN>
__global__ __launch_bounds__(kBlock) void row_kernel(KernelArgs ka) {
  const KernelParams &kp = ka.kp;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  SmemBase &sm = *reinterpret_cast<SmemBase *>(lds_raw);
  static_assert(sizeof(SmemBase) % 16 == 0, "the LDS slice must be 16-byte aligned");
  float *zs = reinterpret_cast<float *>(lds_raw + sizeof(SmemBase));
  unsigned char *region = reinterpret_cast<unsigned char *>(zs + kp.slice);
  // region views (see the layout above)
  uint32_t *hash = reinterpret_cast<uint32_t *>(region);
  // logit_bias / stop entries: slice-local index (low word, kEmpty = free)
  // and the token's summed bias (high word, fp32 bits)
  unsigned long long *bhash = reinterpret_cast<unsigned long long *>(region + 4 * (size_t)kp.hash_slots);
  uint32_t *lc = reinterpret_cast<uint32_t *>(region);
  unsigned long long *lm = reinterpret_cast<unsigned long long *>(region + kRegionLm);
  unsigned char *regB = region + kRegionB;
  unsigned long long *wh = reinterpret_cast<unsigned long long *>(regB);
  unsigned long long *stage = reinterpret_cast<unsigned long long *>(regB);
  unsigned long long *sk = reinterpret_cast<unsigned long long *>(regB);
  double *sq = reinterpret_cast<double *>(regB + 8 * kCandCap);

  const int G = kp.G;
  int group, gid;
  block_group(kp, group, gid);
  const int V = kp.vocab;
  const uint32_t hslots = (uint32_t)kp.hash_slots;
  const uint32_t bslots = (uint32_t)kp.bias_slots;
  unsigned xseq = 0;
  RowCtx rc;
  rc.gid = gid;
  rc.G = G;
  // the launch's epoch: from the host, or from the device word that the
  // records kernel ahead of this launch advanced
  const uint32_t epoch = kp.epoch_dev ? atomic_ld(kp.epoch_dev) + kp.epoch_dev_add : kp.epoch;
  rc.gc.s = kp.sync + group;
  rc.gc.abort_word = kp.abort_word;
  rc.gc.epoch = epoch;
  rc.gc.spin_limit = kp.spin_limit ? kp.spin_limit : kSpinLimit;
  rc.gc.G = G;
  if (gid == 0 && G > 1 && tidx() == 0) claim_words(rc.gc.s, epoch);
  // after the streaming kernel: the rows it left, counted in its epoch
  int n_rows = kp.n_rows;
  if (kp.n_rows_word) {
    const unsigned long long w = atomic_ld(kp.n_rows_word);
    n_rows = (uint32_t)(w >> 32) == kp.n_rows_epoch ? (int)(uint32_t)w : 0;
  }
  rc.my = kp.slots + (size_t)group * G + gid;
  rc.peers = kp.slots + (size_t)group * G;
  rc.xseq = &xseq;
  const bool want_out = kp.probs != nullptr || kp.logprobs != nullptr;
  // output mode: none; both outputs with 16-byte stores; anything else,
  // element by element
  const int omode = !want_out ? 0 : (((kp.vec_ok & 2) && kp.probs && kp.logprobs) ? 1 : 2);
  const int K = kp.top_lp;
  const bool want_S = want_out || K > 0;
  // [B] "Logprobs are temperature-scaled": returned logprobs (and top
  // logprobs) of every token under the untruncated distribution at the
  // row's temperature, instead of the distribution sampled from
  const bool lp_all = kp.lp_mode != 0 && (kp.logprobs != nullptr || K > 0);
  const int s0 = gid * kp.slice;
  const int s1 = min(V, s0 + kp.slice);
  rc.s0 = s0;
  rc.n = s1 - s0;
  rc.n4 = (rc.n + 3) & ~3;
  unsigned it = 0;
  PHASE_STAMP(kStampStart);
  for (int j = tidx(); j < 64; j += kBlock) sm.exp_tab[j] = exp2((double)j * (1.0 / 64.0));
  __syncthreads();
  PHASE_STAMP(kStampTable);

  // Record ri describes batch row rows[ri].row: the host puts the rows it
  // expects to take longest on the groups whose workgroups are dispatched
  // first.
  for (int ri = group; ri < n_rows; ri += kp.n_groups, ++it) {
    // the slice bounds, opaque per row: keeps per-element offsets and
    // compares from being hoisted out of the row loop (they would stay
    // live across it)
    int ln = __builtin_amdgcn_readfirstlane(rc.n);
    asm volatile("" : "+s"(ln));
    const int ln4 = (ln + 3) & ~3;
    // the thread index, opaque per row for the same reason (addresses
    // derived from it are recomputed per row)
    const int tid = tidx();
    const int lane = tid & 63, wave = tid >> 6;
    if (tid == 0) sm.bu[37] = 0u;  // waves done with Gumbel-max (end of the row)

    const RowParam P = kp.rows ? kp.rows[ri] : ka.rows[ri];
    const int row = P.row;
    rc.row = row;
    PHASE_STAMP(kStampRow);
    PHASE_RECORD(kStampRowIndex, row + 1);
    if (P.flags & RF_BAD) {
      // device-side parameters that break the rules: status 4
      if (want_out)
        for (int l = tid; l < ln; l += kBlock) {
          if (kp.probs) kp.probs[(int64_t)row * V + s0 + l] = 0.0f;
          if (kp.logprobs) kp.logprobs[(int64_t)row * V + s0 + l] = -INFINITY;
        }
      if (gid == 0 && tid == 0) {
        kp.token_ids[row] = -1;
        if (kp.row_status) kp.row_status[row] = 4;
        for (int t = 0; t < K; ++t) {
          kp.top_lp_vals[(int64_t)row * K + t] = -INFINITY;
          kp.top_lp_ids[(int64_t)row * K + t] = -1;
        }
      }
      __syncthreads();
      continue;
    }
    const bool greedy = P.flags & RF_GREEDY;
    const bool top1 = P.flags & RF_TOP1;
    const bool pen = PEN && (P.flags & RF_PEN);
    const bool spec = PEN && (P.flags & RF_SPEC);
    const bool topk = !greedy && (P.flags & RF_TOPK);
    const bool topp = !greedy && (P.flags & RF_TOPP);
    const bool minp = !greedy && (P.flags & RF_MINP);
    const bool truncated = topk || topp || minp;

    // ---- 1. issue the history and logit loads; z = x / T into the LDS
    // slice as each batch lands.  Loads use clamped in-bounds addresses;
    // with vector loads the row stride is a multiple of 4, so a group
    // starting below s1 lies inside the row.
    constexpr int kHistPer = kMaxHistPerRow / kBlock;
    int32_t hv[kHistPer];
    float xr[kHistPer];  // raw logit of each in-slice history entry
    // a history longer than the hash holds arrives counted, as this slice's
    // list of (local << 17 | count) entries; hv then holds its first ones
    const bool longh = pen && P.hist_len > kMaxHistPerRow;
    const uint32_t *hl = nullptr;
    int hl_n = 0;
    if (pen) {
      if (longh) {
        const int64_t li = (int64_t)row * G + gid;
        hl = kp.hist_list + li * kp.hist_list_cap;
        hl_n = kp.hist_list_n[li];
#pragma unroll
        for (int q = 0; q < kHistPer; ++q) {
          const int h = tid + q * kBlock;
          hv[q] = h < hl_n ? (int32_t)hl[h] : -1;
        }
      } else {
        const int32_t *hist = kp.history_ids + P.hist_start;
#pragma unroll
        for (int q = 0; q < kHistPer; ++q) {
          const int h = tid + q * kBlock;
          hv[q] = h < P.hist_len ? hist[h] : -1;
        }
      }
    }
    // this thread's logit_bias or stop entry (one per thread): the bias
    // list first, then the stop ids with bias -inf
    int32_t bid = -1;
    float bval = 0.0f;
    if (spec) {
      if (tid < P.bias_len) {
        bid = kp.bias_ids[P.bias_start + tid];
        bval = kp.bias_vals[P.bias_start + tid];
      } else if (tid < P.bias_len + P.stop_len) {
        bid = kp.stop_ids[P.stop_start + (tid - P.bias_len)];
        bval = -INFINITY;
      }
    }
    constexpr int kBatch = kMaxSlice / (4 * kBlock);
    static_assert(kBatch <= 32, "one bit per batch");
    float v[kBatch][4];
    const int64_t rbase = (int64_t)row * kp.row_stride + s0;
    const bool vec = kp.vec_ok & 1;
    const float T = P.temperature;
    const float rT = 1.0f / T;
    // |x| in [xlo, xhi] keeps q = x (1/T) within [2^-100, 2^100], where one
    // FMA correction of q gives the correctly rounded quotient (Markstein).
    // The test runs on the bits of |x| (NaN compares above every finite
    // value); other groups of four (NaN, zeros, infinities, extreme values)
    // take the IEEE division.
    const uint32_t xlo_b = __float_as_uint(T * 0x1p-99f);
    const uint32_t xhi_b = min(__float_as_uint(T * 0x1p99f), 0x7F7FFFFFu);
    // Groups outside the Markstein range keep their raw values in the slice
    // and a bit in slow_b; one loop after the transform divides them (the
    // division's code then appears once, not once per unrolled batch).
    uint32_t slow_b = 0;
    auto transform = [&](int b0, int b1) {  // batches [b0, b1) (constants after inlining)
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int l = 4 * tid + 4 * kBlock * b;
        if (b >= b0 && b < b1 && l < ln4) {
          uint32_t a[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(v[b][c]) & 0x7FFFFFFFu;
          const uint32_t amax = max(max(a[0], a[1]), max(a[2], a[3]));
          const uint32_t amin = min(min(a[0], a[1]), min(a[2], a[3]));
          f32x4 o;
          const bool fast = (amax <= xhi_b) & (amin >= xlo_b);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float q = v[b][c] * rT;
            o[c] = fast ? __builtin_fmaf(__builtin_fmaf(-q, T, v[b][c]), rT, q) : v[b][c];
          }
          slow_b |= fast ? 0u : 1u << b;
          if (l + 4 > ln) {  // the slice's last group: slots past its end hold -inf
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (l + c >= ln) o[c] = -INFINITY;
          }
          *reinterpret_cast<f32x4 *>(zs + l) = o;
        }
      }
    };
    // the groups outside the Markstein range (NaN, zeros, infinities,
    // extreme values): IEEE division, NaN -> -inf, -0 -> +0 (equal values
    // share one key); slots past the slice's end stay -inf
    auto transform_slow = [&]() {
      while (slow_b) {
        const int b = __builtin_ctz(slow_b);
        slow_b &= slow_b - 1u;
        const int l = 4 * tid + 4 * kBlock * b;
        f32x4 o = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float x = o[c] == o[c] ? o[c] : -INFINITY;
          o[c] = l + c < ln ? x / T + 0.0f : -INFINITY;
        }
        *reinterpret_cast<f32x4 *>(zs + l) = o;
      }
    };
    // History counts live in an LDS hash (id -> count), built between the
    // two halves of the transform while the second half of the logits is
    // still arriving: cleared right after the loads are issued, filled
    // once the history ids have landed.  The raw logits of the slice's
    // history entries are then read again from the input (the transform
    // overwrites the slice).
    int32_t osl[kHistPer];  // hash slot of an entry this thread created, else -1
    int32_t bsl = -1;       // bias-hash slot this thread created, else -1
    float xbr = 0.0f;       // raw logit of that slot's token
    auto build_hash = [&]() {
      if (pen || spec) __syncthreads();
      if (spec) {
        // logit_bias and stop entries of this slice: a token's entries sum
        // into one slot (LDS float adds)
        if (bid >= s0 && bid < s1) {
          const uint32_t local = (uint32_t)(bid - s0);
          uint32_t sl = hash_slot(local, bslots);
          uint32_t *lo = reinterpret_cast<uint32_t *>(bhash);
          while (true) {
            const uint32_t prev = atomicCAS(&lo[2 * sl], kEmpty, local);
            if (prev == kEmpty || prev == local) {
              if (prev == kEmpty) bsl = (int32_t)sl;
              atomicAdd(reinterpret_cast<float *>(&lo[2 * sl + 1]), bval);
              break;
            }
            sl = (sl + 1u) & (bslots - 1u);
          }
        }
        if (bsl >= 0) xbr = Loader<TIn>::load1(kp.logits, rbase + (bid - s0));
      }
      if (longh) {
        // the entries' tokens are marked in a bitmap over the slice (for the
        // bias entries below) and their raw logits read
#pragma unroll
        for (int q = 0; q < kHistPer; ++q) {
          osl[q] = -1;
          xr[q] = 0.0f;
          if (hv[q] != -1) {
            const uint32_t local = (uint32_t)hv[q] >> 17;
            atomicOr(&hash[local >> 5], 1u << (local & 31u));
            xr[q] = Loader<TIn>::load1(kp.logits, rbase + local);
          }
        }
        for (int h = kHistPer * kBlock + tid; h < hl_n; h += kBlock) {
          const uint32_t local = hl[h] >> 17;
          atomicOr(&hash[local >> 5], 1u << (local & 31u));
        }
      } else if (pen) {
#pragma unroll
        for (int q = 0; q < kHistPer; ++q) {
          const int32_t id = hv[q];
          osl[q] = -1;
          if (id >= s0 && id < s1) {
            const uint32_t local = (uint32_t)(id - s0);
            uint32_t sl = hash_slot(local, hslots);
            while (true) {
              const uint32_t prev = atomicCAS(&hash[sl], kEmpty, (local << 13) | 1u);
              if (prev == kEmpty) {
                osl[q] = (int32_t)sl;
                break;
              }
              if ((prev >> 13) == local) {
                atomicAdd(&hash[sl], 1u);
                break;
              }
              sl = (sl + 1u) & (hslots - 1u);
            }
          }
        }
#pragma unroll
        for (int q = 0; q < kHistPer; ++q) {
          const int32_t id = hv[q];
          xr[q] = 0.0f;
          if (id >= s0 && id < s1) xr[q] = Loader<TIn>::load1(kp.logits, rbase + (id - s0));
        }
      }
    };
    // vector loads in issue order (batch b is later waited for with the
    // batches behind it still in flight), or scalar loads for unaligned
    // rows (each path is straight-line code from its loads to their uses)
    if (vec) {
      const int lastg = (ln - 1) & ~3;
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        Loader<TIn>::load4(kp.logits, rbase + min(4 * tid + 4 * kBlock * b, lastg), v[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (pen)
        for (int t = tid; t < (int)hslots; t += kBlock) hash[t] = longh ? 0u : kEmpty;
      if (spec)
        for (int t = tid; t < (int)bslots; t += kBlock) bhash[t] = 0xFFFFFFFFull;  // free, bias +0
      transform(0, kBatch / 2);
      PHASE_STAMP(kStampHalf);
      build_hash();
      PHASE_STAMP(kStampHashed);
      transform(kBatch / 2, kBatch);
      transform_slow();
      PHASE_STAMP(kStampTransformed);
    } else {
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[b][c] = Loader<TIn>::load1(kp.logits, rbase + min(4 * tid + 4 * kBlock * b + c, ln - 1));
      if (pen)
        for (int t = tid; t < (int)hslots; t += kBlock) hash[t] = longh ? 0u : kEmpty;
      if (spec)
        for (int t = tid; t < (int)bslots; t += kBlock) bhash[t] = 0xFFFFFFFFull;  // free, bias +0
      transform(0, kBatch / 2);
      build_hash();
      transform(kBatch / 2, kBatch);
      transform_slow();
    }
    if (pen || spec) {
      // The thread that created a history entry recomputes that token once
      // from its raw logit: its bias (if any), then the penalties with the
      // final count.  A bias entry whose token has no history entry is
      // recomputed by the thread that created it.
      __syncthreads();
      if (longh) {
#pragma unroll
        for (int q = 0; q < kHistPer; ++q) {
          if (hv[q] != -1) {
            const uint32_t local = (uint32_t)hv[q] >> 17;
            float x = xr[q] == xr[q] ? xr[q] : -INFINITY;
            if (spec) {
              float b;
              if (bias_lookup(bhash, bslots, local, b)) x = add_bias(x, b);
            }
            zs[local] = div_temp(apply_penalty(x, (uint32_t)hv[q] & 0x1FFFFu, P), T, rT);
          }
        }
        for (int h = kHistPer * kBlock + tid; h < hl_n; h += kBlock) {
          const uint32_t e = hl[h], local = e >> 17;
          float x = Loader<TIn>::load1(kp.logits, rbase + local);
          x = x == x ? x : -INFINITY;
          if (spec) {
            float b;
            if (bias_lookup(bhash, bslots, local, b)) x = add_bias(x, b);
          }
          zs[local] = div_temp(apply_penalty(x, e & 0x1FFFFu, P), T, rT);
        }
      } else if (pen) {
#pragma unroll
        for (int q = 0; q < kHistPer; ++q) {
          if (osl[q] >= 0) {
            const uint32_t e = hash[osl[q]];
            float x = xr[q] == xr[q] ? xr[q] : -INFINITY;
            if (spec) {
              float b;
              if (bias_lookup(bhash, bslots, e >> 13, b)) x = add_bias(x, b);
            }
            zs[e >> 13] = div_temp(apply_penalty(x, e & 0x1FFFu, P), T, rT);
          }
        }
      }
      if (spec && bsl >= 0) {
        const unsigned long long e = bhash[bsl];
        const uint32_t local = (uint32_t)e;
        const bool in_hist =
            pen && (longh ? ((hash[local >> 5] >> (local & 31u)) & 1u) != 0u : hist_contains(hash, hslots, local));
        if (!in_hist) {
          const float x = xbr == xbr ? xbr : -INFINITY;
          zs[local] = div_temp(add_bias(x, __uint_as_float((uint32_t)(e >> 32))), T, rT);
        }
      }
    }
    __syncthreads();
    if (kp.vocab_mask) {
      // grammar bitmask: a cleared bit makes the value -inf.  Groups of four
      // start at multiples of 4 of the row, so their bits share one word.
      const uint32_t *mrow = kp.vocab_mask + (int64_t)row * kp.mask_stride;
      uint32_t mw[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int l = 4 * tid + 4 * kBlock * b;
        mw[b] = l < ln4 ? mrow[(s0 + l) >> 5] : 0xFFFFFFFFu;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int l = 4 * tid + 4 * kBlock * b;
        const uint32_t bits = (mw[b] >> ((s0 + l) & 31)) & 0xFu;
        if (l < ln4 && bits != 0xFu) {
          f32x4 o = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (!((bits >> c) & 1u)) o[c] = -INFINITY;
          *reinterpret_cast<f32x4 *>(zs + l) = o;
        }
      }
      __syncthreads();
    }
    // this thread's max and first argmax: the best group of four by a
    // strict compare (groups in index order), then the first match in it
    float lmax = -INFINITY;
    int lgrp = -1;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int l = 4 * tid + 4 * kBlock * b;
      if (l < ln4) {
        const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
        const float gm = fmaxf(fmaxf(zv[0], zv[1]), fmaxf(zv[2], zv[3]));
        if (gm > lmax) {
          lmax = gm;
          lgrp = l;
        }
      }
    }
    int lidx = 0x7FFFFFFF;
    if (lgrp >= 0) {
      const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + lgrp);
      lidx = s0 + lgrp + (zv[0] == lmax ? 0 : zv[1] == lmax ? 1 : zv[2] == lmax ? 2 : 3);
    }

    PHASE_STAMP(kStampLoaded);
    // ---- 2. this slice's max and first argmax as one order key (value key
    // << 32 | ~index: the largest key is the first argmax)
    const unsigned long long lkey = wg_max_u(sm, ((unsigned long long)fkey(lmax) << 32) | (0xFFFFFFFFu - (uint32_t)lidx));
    const float mg = key_to_float((uint32_t)(lkey >> 32));  // -inf: no finite value in this slice
    PHASE_STAMP(kStampMax);
    const unsigned par = it & 1u;
    const float wsc = T < 1.0f ? T : 1.0f;  // bin scale (see abin)
    const bool need_sel = topk || topp || K > 0 || (truncated && want_S);  // window + candidates
    const bool need_mass = topp || (truncated && want_S);
    const bool need_deep = topp && !topk;  // top-p's total includes the deep values
    const bool need_exact = want_S && (!truncated || lp_all);
    // rows that need the merged max: thresholds, sums or min-p's boundary.
    // The rest (no truncation, no outputs) prune against their own slice's
    // max and settle argmax and status in the final exchange.
    const bool icdf = kp.icdf && !top1 && kp.path != PATH_GREEDY;  // inverse-CDF selection
    const bool need_x = need_sel || need_exact || minp || icdf;
    double m = (double)mg;
    int argmax_idx = (int)(0xFFFFFFFFu - (uint32_t)lkey);
    uint32_t t_m = 0;
    float Af = 0.0f;  // window anchor abin(row max)
    bool general = false;
    bool full_k = false;
    bool topk_on = topk;  // top-k decides (part of) the kept set
    uint32_t tau = 0;
    double lnS = 0.0;
    double s_all = 0.0;  // the exact sum of every value's mass, when needed
    double lnA = 0.0;    // its log (the logprob normaliser with lp_all)
    int r0hi = -1, r1lo = 1, r1hi = 0, rklo = 1, rkhi = 0, bm = -1;
    if (need_x) {
      // ---- 3. window histogram of this slice on the absolute bin grid,
      // anchored at its own max, masses relative to its own max; the fp64
      // sum when every token is kept.  Exchange 2: every workgroup of the
      // row finds the row max, shifts each histogram by whole bins,
      // rescales its masses and decides in parallel, alike.
      const bool finite_g = mg > -INFINITY && mg < INFINITY;
      const float Ag = finite_g ? abin(mg, wsc) : 0.0f;
      if (need_sel) {
        // this slice's histogram, and the row's merged bins (exchange 2)
        wh[tid] = 0;
        lc[tid] = 0;
        lm[tid] = 0;
        if (tid == 0) lm[kWinBins] = 0;
        __syncthreads();
      }
      double deep_a = 0.0;  // deeper masses, 2^-31 units
      double sx = 0.0;
      if (finite_g && (need_sel || need_exact)) {
        // Specialised on what the row needs (window bins, their deeper mass,
        // the exact sum).  Eight groups of four per step: all reads first
        // (from clamped addresses; only the work is guarded), then the bins
        // (LDS operations complete in order, so a read issued after the
        // previous step's atomics would wait for them).
        auto hist_pass = [&](auto SEL, auto DEEP, auto EXACT) __attribute__((always_inline)) {
          constexpr bool sel = decltype(SEL)::value, deep = decltype(DEEP)::value, exact = decltype(EXACT)::value;
          constexpr int kStep = 8;
          for (int b0 = 0; b0 < kBatch; b0 += kStep) {
            f32x4 zr[kStep];
#pragma unroll
            for (int u = 0; u < kStep; ++u)
              zr[u] = *reinterpret_cast<const f32x4 *>(zs + min(4 * tid + 4 * kBlock * (b0 + u), ln4 - 4));
#pragma unroll
            for (int u = 0; u < kStep; ++u) {
              if (4 * tid + 4 * kBlock * (b0 + u) < ln4) {
                float dsum = 0.0f;  // deep masses of the group (each below 2^8 units)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                  const float zz = zr[u][c];
                  if (sel) {
                    const float lb = win_pos(Ag, zz, wsc);  // padding: +inf
                    const bool near = lb < (float)kWinBins;
                    const float a = mass_scaled(mg - zz);
                    if (near) atomicAdd(&wh[(int)lb], hist_entry(a));
                    if (deep) dsum += near ? 0.0f : a;
                  }
                  if (exact) sx += exp_term(zz, (double)mg);
                }
                if (deep) deep_a += (double)dsum;
              }
            }
          }
        };
        using T1 = std::integral_constant<bool, true>;
        using F1 = std::integral_constant<bool, false>;
        if (need_sel) {
          if (need_deep) {
            if (need_exact) hist_pass(T1{}, T1{}, T1{});
            else hist_pass(T1{}, T1{}, F1{});
          } else if (need_exact) hist_pass(T1{}, F1{}, T1{});
          else hist_pass(T1{}, F1{}, F1{});
        } else {
          hist_pass(F1{}, F1{}, T1{});
        }
      }
      const double wdm = need_deep ? wg_sum_d(sm, deep_a) : 0.0;
      const double wsx = need_exact ? wg_sum_d(sm, sx) : 0.0;
      __syncthreads();
      // this workgroup's record and histogram -> its exchange slot (a row's
      // only workgroup keeps them: the merge reads registers and LDS)
      const unsigned xp = xseq++ & 1u;
      if (need_sel && G > 1) atomic_st(&rc.my->whist[xp][tid], wh[tid]);
      if (tid == 0 && G > 1) {
        atomic_st(&rc.my->x1[xp][0], lkey);
        atomic_st(&rc.my->x1[xp][1], (unsigned long long)__float_as_uint(Ag));
        atomic_st(&rc.my->x1[xp][2], (unsigned long long)__double_as_longlong(wdm));
        atomic_st(&rc.my->x1[xp][3], (unsigned long long)__double_as_longlong(wsx));
      }
      const double lmp = minp ? log((double)P.min_p) : 0.0;  // min-p's guess, taken before the wait
      PHASE_STAMP(kStampHist);
      group_barrier(sm, rc.gc);
      PHASE_STAMP(kStampX2);
      // ---- exchange 2, merged by every workgroup of the row alike: the
      // records and the first histogram pairs in one batch of 16-byte reads,
      // the row max, each slice's bin shift and mass scale, integer LDS adds
      // (order-free), prefix sums and decisions.  Every workgroup reads the
      // same words and runs the same code, so all take the same decisions.
      constexpr int kPairs = kWinBins / 2;
      const int npairs = need_sel ? G * kPairs : 0;
      u32x4 hr[4];
      if (G == 1) {
        // the local histogram is still in LDS (region B), the record in
        // registers
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pk = min(tid + k * kBlock, max(npairs - 1, 0));
          hr[k] = *reinterpret_cast<const u32x4 *>(&wh[2 * (pk % kPairs)]);
        }
        if (tid == 0) {
          sm.gk[0] = lkey;
          sm.ga[0] = Ag;
          sm.gf[0] = wdm;
          sm.gd[0] = wsx;
        }
      } else {
        const int g1 = tid < G ? tid : G - 1;
        u32x4 r0, r1;
        if (npairs > 0) {
          const void *ph[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int pk = min(tid + k * kBlock, npairs - 1);
            ph[k] = &rc.peers[pk / kPairs].whist[xp][2 * (pk % kPairs)];
          }
          coh_load16x6(&rc.peers[g1].x1[xp][0], &rc.peers[g1].x1[xp][2], ph[0], ph[1], ph[2], ph[3], r0, r1, hr[0], hr[1],
                       hr[2], hr[3]);
        } else {
          coh_load16x2(&rc.peers[g1].x1[xp][0], &rc.peers[g1].x1[xp][2], r0, r1);
        }
        if (tid < G) {
          sm.gk[tid] = u64_of(r0.x, r0.y);
          sm.ga[tid] = __uint_as_float(r0.z);
          sm.gf[tid] = f64_of(r1.x, r1.y);  // deep mass (scaled below)
          sm.gd[tid] = f64_of(r1.z, r1.w);  // exact sum (scaled below)
        }
      }
      __syncthreads();
      unsigned long long mk = 0;
      for (int g = 0; g < G; ++g) mk = sm.gk[g] > mk ? sm.gk[g] : mk;
      const float mfx = key_to_float((uint32_t)(mk >> 32));
      m = (double)mfx;
      argmax_idx = (int)(0xFFFFFFFFu - (uint32_t)(mk & 0xFFFFFFFFu));
      const uint32_t status = (mfx > -INFINITY && mfx < INFINITY) ? 0u : (mfx == INFINITY ? 2u : 1u);
      if (status != 0) {
        // ---- no finite logit (status 1) or a +inf value (status 2)
        if (want_out) {
          for (int l = tid; l < ln; l += kBlock) {
            if (kp.probs) kp.probs[(int64_t)row * V + s0 + l] = 0.0f;
            if (kp.logprobs) kp.logprobs[(int64_t)row * V + s0 + l] = -INFINITY;
          }
        }
        if (gid == 0 && tid == 0) {
          kp.token_ids[row] = -1;
          if (kp.row_status) kp.row_status[row] = (int)status;
          for (int t = 0; t < K; ++t) {
            kp.top_lp_vals[(int64_t)row * K + t] = -INFINITY;
            kp.top_lp_ids[(int64_t)row * K + t] = -1;
          }
        }
        __syncthreads();
        continue;
      }
      const float A = abin(mfx, wsc);
      Af = A;
      if (minp) t_m = min_p_key(sm, m, lmp, P.min_p);
      // per-workgroup mass scale exp(m_g - m) and bin shift A - A_g
      if (tid < G) {
        const float mgg = key_to_float((uint32_t)(sm.gk[tid] >> 32));
        const double f = mgg > -INFINITY ? exp_nonpos(sm.exp_tab, (double)mgg - m) : 0.0;
        const float sh = A - sm.ga[tid];  // whole bins, >= 0
        sm.gi[tid] = (mgg > -INFINITY && sh < (float)kWinBins) ? (int)sh : kWinBins;
        sm.gd[tid] *= f;
        sm.gf[tid] *= f;
        sm.gs[tid] = f;
      }
      __syncthreads();
      if (need_exact) {
        for (int g = 0; g < G; ++g) s_all += sm.gd[g];
        lnS = log(s_all);
        lnA = lnS;
      }
      if (need_sel) {
        const int b = tid;
        double deep_x = 0.0;  // window bins of a slice that fall past the row's window
        // two bins per 16-byte pair; integer LDS adds of each slice's
        // rescaled, rounded masses: order-free
        auto add_pair = [&](int p, const u32x4 &r) {
          const int g = p / kPairs;
          const unsigned long long e2[2] = {u64_of(r.x, r.y), u64_of(r.z, r.w)};
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const unsigned long long e = e2[i];
            if (e) {
              const int bin = 2 * (p % kPairs) + i + sm.gi[g];
              const double ms = (double)(e & 0xFFFFFFFFFFFFull) * sm.gs[g];
              if (bin < kWinBins) {
                atomicAdd(&lc[bin], (uint32_t)(e >> 48));
                if (need_mass) atomicAdd(&lm[bin], (unsigned long long)__double2ll_rn(ms));
              } else {
                deep_x += ms;
              }
            }
          }
        };
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (tid + k * kBlock < npairs) add_pair(tid + k * kBlock, hr[k]);
        // more than eight slices: the remaining pairs, two reads per pass
        for (int pi = tid + 4 * kBlock; pi < npairs; pi += 2 * kBlock) {
          const int pj = pi + kBlock < npairs ? pi + kBlock : pi;
          u32x4 ra, rb;
          coh_load16x2(&rc.peers[pi / kPairs].whist[xp][2 * (pi % kPairs)], &rc.peers[pj / kPairs].whist[xp][2 * (pj % kPairs)],
                       ra, rb);
          add_pair(pi, ra);
          if (pj != pi) add_pair(pj, rb);
        }
        const double deep_w = need_deep ? wg_sum_d(sm, deep_x) : 0.0;
        __syncthreads();
        const uint32_t cb = lc[b];
        const unsigned long long mb = lm[b];
        unsigned long long deep = 0;
        if (need_deep) {
          double dt = deep_w;
          for (int g = 0; g < G; ++g) dt += sm.gf[g];
          deep = (unsigned long long)__double2ll_rn(dt);
        }
        uint32_t runc = cb;
        unsigned long long runm = mb;
        block_scan_incl2(runc, runm, sm.red_c, sm.red_u);
        lc[b] = runc;
        lm[b] = runm;
        if (b == kWinBins - 1) lm[kWinBins] = runm + deep;
        if (tid == 0) {
          sm.bu[16] = kNone;
          sm.bu[17] = kNone;
          sm.bu[18] = kNone;
          sm.bu[19] = kNone;
        }
        __syncthreads();
        // bins of the k-th and the K-th value
        const uint32_t cprev = b > 0 ? lc[b - 1] : 0u;
        if (topk && cprev < (uint32_t)P.top_k && runc >= (uint32_t)P.top_k) sm.bu[16] = (uint32_t)b;
        if (K > 0 && cprev < (uint32_t)K && runc >= (uint32_t)K) sm.bu[17] = (uint32_t)b;
        __syncthreads();
        const uint32_t bk = sm.bu[16], r0 = sm.bu[17];
        bool gen = false;
        const int bmin = minp ? win_bin(A, key_to_float(t_m), wsc) : kWinBins;
        if (K > 0) {
          if (r0 != kNone) r0hi = (int)r0;
          else if (truncated && !lp_all) r0hi = kWinBins - 1;  // fewer than K values in the window: all of them
          else gen = true;
        }
        if (topk) {
          if (bk != kNone) {
            if (lc[bk] <= (uint32_t)kCandCap) {
              full_k = true;
              rklo = 0;
              rkhi = (int)bk;
            } else {
              rklo = rkhi = (int)bk;
            }
          } else if (topp || !(minp && bmin < kWinBins)) {
            gen = true;  // the k-th value is deeper than the window and decides the kept set
          } else {
            topk_on = false;
          }
        }
        // top-p: the bins where the cumulative mass crosses p times the
        // total mass of the top-k set (bounded below and above)
        double tlo = 0.0, thi = 0.0;
        if (topp && !gen) {
          if (topk) {
            tlo = (double)P.top_p * (bk > 0 ? (double)lm[bk - 1] : 0.0);
            thi = (double)P.top_p * (double)lm[bk];
          } else {
            tlo = thi = (double)P.top_p * (double)lm[kWinBins];
          }
          const double mprev = b > 0 ? (double)lm[b - 1] : 0.0, mcur = (double)lm[b];
          if (mprev < tlo && mcur >= tlo) sm.bu[18] = (uint32_t)b;
          if (mprev < thi && mcur >= thi) sm.bu[19] = (uint32_t)b;
        }
        __syncthreads();
        if (topp && !gen) {
          const uint32_t lo = tlo <= 0.0 ? 0u : sm.bu[18], hi = sm.bu[19];
          if (hi == kNone) {
            gen = true;  // the crossing lies deeper than the window
          } else {
            r1lo = (int)(lo == kNone ? hi : lo);
            r1hi = (int)hi;
            if (topk) {
              r1lo = min(r1lo, (int)bk);
              r1hi = min(r1hi, (int)bk);
            }
          }
        }
        if (minp && !gen) {
          if (bmin < kWinBins) bm = bmin;
          else if (!topk && !topp) gen = true;  // min-p alone keeps values deeper than the window
        }
        // the bin grid overflows for |m / T| beyond ~1e37: exact path
        if (!(A > -INFINITY && A < INFINITY)) gen = true;
        // gathered bins (mask for the gather) and their total count
        const bool in = !gen && (b <= r0hi || (b >= r1lo && b <= r1hi) || (b >= rklo && b <= rkhi) || b == bm);
        const unsigned long long bal = __ballot(in);
        if (lane == 0) {
          sm.binmask[2 * wave] = (uint32_t)bal;
          sm.binmask[2 * wave + 1] = (uint32_t)(bal >> 32);
        }
        const uint32_t ncand = (uint32_t)wg_sum_u(sm, in ? (unsigned long long)cb : 0ull);
        if (ncand > (uint32_t)kCandCap) gen = true;
        general = gen;
      } else if (minp) {
        tau = t_m;  // min-p alone without outputs: the closed-form boundary
      }
      __syncthreads();
    }
    // A row without exchanges meets its peers only in the final exchange; a
    // group that walks several rows then passes one barrier first, so that
    // no workgroup arrives at the next row's final exchange (or rewrites its
    // record of this row, two rows on) before this row's last arrival has
    // read the records.
    PHASE_STAMP(kStampDecided);
    if (!need_x && n_rows > kp.n_groups) row_barrier(sm, rc);
    const float mf = (float)m;

    // ---- 4. exact thresholds from the gathered candidates (exchange 3,
    // sorted and decided by every workgroup of the row alike)
    if (need_sel && !general) {
      // compact this slice's candidates into per-wave LDS staging (ballot
      // order: deterministic), then copy them to this workgroup's slot
      uint32_t cnt = 0;  // wave-uniform
      unsigned long long *wst = stage + wave * kStagePerWave;
      // the gathered bins as runs, from the (up to four) ranges the merge
      // chose: sorted by start and joined where they touch; the first two
      // runs are tested by value, any further bins through the mask
      int rl0 = 1, rh0 = 0, rl1 = 1, rh1 = 0;  // the first two runs (empty: hi < lo)
      bool more = false;
      {
        int lo[4] = {0, r1lo, rklo, bm}, hi[4] = {r0hi, r1hi, rkhi, bm};
        if (bm < 0) hi[3] = -1;
#pragma unroll
        for (int i = 1; i < 4; ++i)  // insertion sort by start (empty ranges have hi < lo)
#pragma unroll
          for (int j = i; j > 0; --j)
            if (lo[j] < lo[j - 1]) {
              const int tl = lo[j], th = hi[j];
              lo[j] = lo[j - 1];
              hi[j] = hi[j - 1];
              lo[j - 1] = tl;
              hi[j - 1] = th;
            }
        // join touching ranges; scalars only (a run index would put the
        // runs in scratch memory)
        int nrun = 0, clo = 0, chi = -1;
        auto close_run = [&]() {
          if (chi >= clo) {
            if (nrun == 0) {
              rl0 = clo;
              rh0 = chi;
            } else if (nrun == 1) {
              rl1 = clo;
              rh1 = chi;
            } else {
              more = true;
            }
            ++nrun;
          }
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (hi[i] < lo[i]) continue;
          if (chi >= clo && lo[i] <= chi + 1) {
            chi = max(chi, hi[i]);
          } else {
            close_run();
            clo = lo[i];
            chi = hi[i];
          }
        }
        close_run();
      }
      // each run [lo, hi] as a value range [zlo, zhi): bins lo..hi hold
      // exactly the values with zmin(hi) <= z < zmin(lo - 1)
      if (tid < 4) {
        const int rlo = (tid >> 1) ? rl1 : rl0, rhi = (tid >> 1) ? rh1 : rh0;
        const bool upper = tid & 1;
        float zb;
        if (rhi < rlo) zb = upper ? -INFINITY : INFINITY;  // empty run
        else if (!upper) zb = win_floor_z(Af, (float)rhi, wsc);
        else zb = rlo > 0 ? win_floor_z(Af, (float)(rlo - 1), wsc) : INFINITY;
        sm.bu[28 + tid] = __float_as_uint(zb);
      }
      __syncthreads();
      const float z0lo = __uint_as_float(sm.bu[28]), z0hi = __uint_as_float(sm.bu[29]);
      const float z1lo = __uint_as_float(sm.bu[30]), z1hi = __uint_as_float(sm.bu[31]);
      // membership by value (one or two runs), or (more than two runs,
      // rare) by the bin mask; groups of four in a fixed, unrolled order so
      // the LDS reads overlap; the staging branch runs only for the waves
      // that hold a candidate
      auto gather = [&](auto is_cand) __attribute__((always_inline)) {
        constexpr int kStep = 8;  // groups read before any is tested
        for (int q0 = 0; q0 < kBatch; q0 += kStep) {  // (a loop: the body's code is large)
          f32x4 zr[kStep];
#pragma unroll
          for (int u = 0; u < kStep; ++u) zr[u] = *reinterpret_cast<const f32x4 *>(zs + min(4 * tid + 4 * kBlock * (q0 + u), ln4 - 4));
#pragma unroll
          for (int u = 0; u < kStep; ++u) {
          const int l = 4 * tid + 4 * kBlock * (q0 + u);
          const f32x4 zv = zr[u];
          const bool in_slice = l < ln4;  // (a clamped read repeats the last group)
          bool isc[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) isc[c] = in_slice && is_cand(zv[c]);
          if (__ballot(isc[0] | isc[1] | isc[2] | isc[3])) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const unsigned long long bal = __ballot(isc[c]);
              if (bal) {
                const uint32_t off = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                if (isc[c] && cnt + off < (uint32_t)kStagePerWave) wst[cnt + off] = cand_key(zv[c], s0 + l + c);
                cnt += (uint32_t)__popcll(bal);
              }
            }
          }
          }
        }
      };
      if (more) {
        gather([&](float z) -> bool {
          const float lb = win_pos(Af, z, wsc);
          const int bb = min((int)lb, kWinBins - 1);
          return (lb < (float)kWinBins) & (bool)((sm.binmask[bb >> 5] >> (bb & 31)) & 1u);
        });
      } else if (rh1 < rl1) {
        gather([&](float z) -> bool { return (z >= z0lo) & (z < z0hi); });
      } else {
        gather([&](float z) -> bool { return ((z >= z0lo) & (z < z0hi)) | ((z >= z1lo) & (z < z1hi)); });
      }
      if (lane == 0) sm.red_c[wave] = cnt;
      __syncthreads();
      // every wave copies its own candidates to the slot, at its offset among
      // the waves' counts (each wave sums the counts itself)
      uint32_t acc = 0, woff = 0;
      bool ovf = false;
      for (int w = 0; w < kWaves; ++w) {
        const uint32_t c = sm.red_c[w];
        if (w == wave) woff = acc;
        ovf |= c > (uint32_t)kStagePerWave;
        acc += c;
      }
      ovf |= acc > (uint32_t)kCandCap;
      const uint32_t my_n = ovf ? (uint32_t)kCandCap + 1u : acc;
      const unsigned xq = xseq++ & 1u;
      {
        WgSlots *my = slot_at(kp, group * G + gid);
        if (my_n <= (uint32_t)kCandCap)
          for (int j = lane; j < (int)cnt; j += 64) atomic_st(&my->cand[xq][woff + j], wst[j]);
        if (tid == 0) atomic_st(&my->cand_n[xq][0], my_n);
      }
      // the addresses wave 0 reads in exchange 3 (below), taken before the wait
      constexpr int kPL = 5;
      const int pps = min(64 * kPL / G, kCandCap / 2);  // pairs read at first per slice
      WgSlots *peers = slot_at(kp, group * G);
      const void *pp[kPL];
      int pg[kPL], po[kPL];  // each pair's slice (G: none) and key offset in it
#pragma unroll
      for (int j = 0; j < kPL; ++j) {
        const int pj = lane + 64 * j;
        pg[j] = min(pj / pps, G);
        po[j] = 2 * (pj - pg[j] * pps);
        pp[j] = &peers[min(pg[j], G - 1)].cand[xq][pg[j] < G ? po[j] : 0];
      }
      PHASE_STAMP(kStampGathered);
      group_barrier(sm, rc.gc);
      PHASE_STAMP(kStampX3);
      // ---- exchange 3, in every workgroup alike: wave 0 reads the counts and
      // the first candidates of every slice in one batch (pairs of keys; a
      // slot's array has room past an odd count), places them in the list
      // by the slices' offsets (a scan of the counts within the wave), and
      // reads the rest only when a slice gathered more
      if (wave == 0) {
        const int g1 = lane < G ? lane : G - 1;
        u32x4 rn, rp[kPL];
        coh_load16x6(&peers[g1].cand_n[xq][0], pp[0], pp[1], pp[2], pp[3], pp[4], rn, rp[0], rp[1], rp[2], rp[3], rp[4]);
        // slice g's count and offset sit in lane g
        const bool bad = lane < G && rn.x > (uint32_t)kCandCap;
        const uint32_t cc = (lane < G && !bad) ? rn.x : 0u;
        const uint32_t incl = wave_scan(cc);
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, G - 1);
        const bool ovf = __ballot(bad) != 0ull || tot > (uint32_t)kCandCap;
        const uint32_t goff = incl - cc;
        if (lane == 0) {
          sm.goff[G] = tot;
          sm.bu[12] = ovf ? 1u : 0u;
        }
        bool fast = false;
        if (!ovf) {
#pragma unroll
          for (int j = 0; j < kPL; ++j) {
            const int g = min(pg[j], G - 1);
            const int c = pg[j] < G ? __shfl((int)cc, g) : 0, o = __shfl((int)goff, g);
            if (po[j] < c) sk[o + po[j]] = u64_of(rp[j].x, rp[j].y);
            if (po[j] + 1 < c) sk[o + po[j] + 1] = u64_of(rp[j].z, rp[j].w);
          }
          // slices with more than 2 pps candidates: the rest
          for (int g = 0; g < G; ++g) {
            const int c = __builtin_amdgcn_readlane((int)cc, g), o = __builtin_amdgcn_readlane((int)goff, g);
            for (int j = 2 * pps + 2 * lane; j < c; j += 128) {
              const u32x4 r = coh_load16(&peers[g].cand[xq][j]);
              sk[o + j] = u64_of(r.x, r.y);
              if (j + 1 < c) sk[o + j + 1] = u64_of(r.z, r.w);
            }
          }
          fast = tot <= (uint32_t)(64 * kE3Slots);
        }
        if (lane == 0) sm.bu[13] = fast ? 1u : 0u;
      }
      PHASE_STAMP(kStampX3Read);
      __syncthreads();
      // rank of each key: the number of larger keys (keys are distinct:
      // each holds its index), so the list is in (value desc, index asc)
      // order, a total order.  On a short list S adjacent lanes share a key
      // (S a power of two; at most the workgroup): each counts over its own
      // part of the list, eight keys read before any compare, and the parts
      // add up within the wave.
      auto rank_place = [&](int n, unsigned long long *srt) __attribute__((always_inline)) {
        int S = 1;
        while (S < 8 && 2 * S * ((n + 63) & ~63) <= kBlock) S *= 2;
        const int k = tid / S, p = tid & (S - 1);
        const int j0 = (p * n) / S, j1 = ((p + 1) * n) / S;
        uint32_t r = 0;
        unsigned long long c = ~0ull;
        if (k < n) {
          c = sk[k];
          int j = j0;
          for (; j + 8 <= j1; j += 8) {
            unsigned long long kk[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) kk[u] = sk[j + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) r += kk[u] > c ? 1u : 0u;
          }
          for (; j < j1; ++j) r += sk[j] > c ? 1u : 0u;
        }
        for (int o = 1; o < S; o <<= 1) r += (uint32_t)__shfl_xor((int)r, o);
        if (k < n && p == 0) srt[r] = c;
      };
      if (sm.bu[13] != 0u) {
        // a list of at most 256: sorted by every wave, decided by wave 0
        const int n = (int)sm.goff[G];
        rank_place(n, reinterpret_cast<unsigned long long *>(sq));
        __syncthreads();
        PHASE_STAMP(kStampX3Ranked);
        if (wave == 0) {
          E3In in;
          in.top_k = P.top_k;
          in.top_p = P.top_p;
          in.m = m;
          in.s_all = s_all;
          in.Af = Af;
          in.wsc = wsc;
          in.t_m = t_m;
          in.rklo = rklo;
          in.rkhi = rkhi;
          in.r1lo = r1lo;
          in.r1hi = r1hi;
          in.K = K;
          in.row = row;
          in.gid = gid;
          in.full_k = full_k;
          in.topk_on = topk_on;
          in.topp = topp;
          in.minp = minp;
          in.truncated = truncated;
          in.want_S = want_S;
          in.lp_all = lp_all;
          in.lnA = lnA;
          const E3Out o = e3_decide(sm, n, sq, lc, lm, in, kp);
          if (lane == 0) {
            sm.bu[26] = o.general ? 1u : 0u;
            sm.bu[27] = o.tau;
            sm.bd[5] = o.lnS;
          }
          PHASE_STAMP(kStampX3Decided);
        }
        __syncthreads();
        general = sm.bu[26] != 0u;
        tau = sm.bu[27];
        lnS = sm.bd[5];
      } else {
        bool ovf = sm.bu[12] != 0u;
        const int n = ovf ? 0 : (int)sm.goff[G];
        // sort by rank counting: a candidate's position is the number of
        // larger keys (keys are distinct: each holds its index), so the list
        // is in (value desc, index asc) order, a total order, and it and
        // every sum over it do not depend on the gather order.  Only the
        // waves holding candidates count, eight keys per step.
        // The gathered bins are complete, so a masked scan of the merged
        // histogram's counts gives each bin's first position in the list
        // (lc becomes those positions), checked against the sorted keys.
        const uint32_t c_rk = rklo > 0 ? lc[min(rklo - 1, kWinBins - 1)] : 0u;  // values above the top-k bin
        unsigned long long *srt = reinterpret_cast<unsigned long long *>(sq);  // the sorted keys
        double *pre = reinterpret_cast<double *>(sk);                          // then their prefix masses
        {
          const int b = tid;
          const bool gb = (sm.binmask[b >> 5] >> (b & 31)) & 1u;
          const uint32_t cb = gb ? lc[b] - (b > 0 ? lc[b - 1] : 0u) : 0u;
          const uint32_t incl = block_scan_incl<uint32_t>(cb, sm.red_c);
          lc[b] = incl - cb;
          auto rank_of = [&](unsigned long long c) {
            uint32_t r = 0;
            int j = 0;
            for (; j + 8 <= n; j += 8) {  // eight keys read before any compare
              unsigned long long kk[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) kk[u] = sk[j + u];
#pragma unroll
              for (int u = 0; u < 8; ++u) r += kk[u] > c ? 1u : 0u;
            }
            for (; j < n; ++j) r += sk[j] > c ? 1u : 0u;
            return r;
          };
          if (n <= kBlock) {
            rank_place(n, srt);
          } else {
            if (wave * 64 < n) {
              const unsigned long long c0 = tid < n ? sk[tid] : ~0ull;
              const uint32_t r0 = rank_of(c0);
              if (tid < n) srt[r0] = c0;
            }
            if (kBlock + wave * 64 < n) {
              const unsigned long long c1 = tid + kBlock < n ? sk[tid + kBlock] : ~0ull;
              const uint32_t r1 = rank_of(c1);
              if (tid + kBlock < n) srt[r1] = c1;
            }
          }
          __syncthreads();
          // each gathered bin's first and last positions hold keys of that
          // bin (else the exact path)
          bool bad = false;
          if (cb > 0) {
            const int f = (int)(incl - cb), e = (int)incl - 1;
            bad = e >= n || win_bin(Af, key_to_float((uint32_t)(srt[f] >> 32)), wsc) != b ||
                  win_bin(Af, key_to_float((uint32_t)(srt[e] >> 32)), wsc) != b;
          }
          if (__syncthreads_or(bad)) ovf = true;
        }
        auto keyof = [&](int j) { return (uint32_t)(srt[j] >> 32); };
        auto zof = [&](int j) { return key_to_float(keyof(j)); };
        auto idxof = [&](int j) { return (int)(~(uint32_t)srt[j]); };
        auto fpos = [&](int b) { return b >= kWinBins ? n : (int)lc[b]; };  // first position of bin b
        // inclusive prefix of exact masses exp(z - m) along the sorted list;
        // each thread owns kCandCap / kBlock consecutive positions
        {
          constexpr int kPerC = kCandCap / kBlock;
          static_assert(kCandCap % kBlock == 0, "candidate split");
          double qv[kPerC];
          double own = 0.0;
#pragma unroll
          for (int u = 0; u < kPerC; ++u) {
            const int j = tid * kPerC + u;
            qv[u] = j < n ? exp_nonpos(sm.exp_tab, (double)zof(j) - m) : 0.0;
            own += qv[u];
          }
          double run = block_scan_incl<double>(own, sm.red_d) - own;
#pragma unroll
          for (int u = 0; u < kPerC; ++u) {
            const int j = tid * kPerC + u;
            run += qv[u];
            if (j < n) pre[j] = run;
          }
        }
        auto qsum = [&](int a, int e) { return (e < a) ? 0.0 : pre[e] - (a > 0 ? pre[a - 1] : 0.0); };
        auto cmass = [&](int b) { return b < 0 ? 0.0 : (double)lm[b < kWinBins ? b : kWinBins] / kWinScale; };
        const int fp_k = fpos(rklo), fp_p0 = fpos(r1lo), fp_p1 = fpos(r1hi + 1);
        // top-k: the value of rank k, and the end of its tie group
        uint32_t flags = ovf ? 1u : 0u;
        uint32_t tk = 0;
        if (!flags && topk_on) {
          const int jk = full_k ? P.top_k - 1 : fp_k + (P.top_k - (int)c_rk) - 1;
          if (jk < 0 || jk >= n) flags |= 1u;
          else tk = keyof(jk);
        }
        if (tid == 0) sm.bu[23] = (uint32_t)n;
        __syncthreads();
        if (!flags && topk_on)
          for (int j = tid; j < n; j += kBlock)
            if (keyof(j) < tk && (j == 0 || keyof(j - 1) >= tk)) sm.bu[23] = (uint32_t)j;
        __syncthreads();
        const int ek = (int)sm.bu[23] - 1;
        // top-p: the first tie-group end whose cumulative mass reaches p
        // times the top-k set's mass (parallel over the crossing range)
        uint32_t t = tk;
        if (!flags && topp) {
          const double ctot = topk_on ? (full_k ? qsum(0, ek) : cmass(rklo - 1) + qsum(fp_k, ek)) : cmass(kWinBins);
          const double target = (double)P.top_p * ctot;
          const double base = full_k ? 0.0 : cmass(r1lo - 1) - (fp_p0 > 0 ? pre[fp_p0 - 1] : 0.0);
          if (tid == 0) sm.bu[24] = 0x7FFFFFFFu;
          __syncthreads();
          for (int e = fp_p0 + tid; e < fp_p1; e += kBlock) {
            const bool end = (e == n - 1) || (keyof(e + 1) != keyof(e));
            // positions rise with the lane: the wave's first passing lane
            // holds its smallest passing position
            const unsigned long long bal = __ballot(end && base + pre[e] >= target);
            if (bal && lane == __ffsll((long long)bal) - 1) atomicMin(&sm.bu[24], (uint32_t)e);
          }
          __syncthreads();
          const uint32_t e = sm.bu[24];
          if (e == 0x7FFFFFFFu) {
            flags |= 1u;
          } else {
            // the crossing's distance from the target on both sides (the
            // cumulative mass at the end of its tie group and before the
            // group, whose first position is found in parallel)
            const uint32_t ke = keyof((int)e);
            if (tid == 0) sm.bu[22] = 0u;
            __syncthreads();
            for (int j = tid; j <= (int)e; j += kBlock)
              if (keyof(j) == ke && (j == 0 || keyof(j - 1) != ke)) sm.bu[22] = (uint32_t)j;
            __syncthreads();
            const int gs = (int)sm.bu[22];
            const double c_new = base + pre[e], c_prev = base + (gs > 0 ? pre[gs - 1] : 0.0);
            // a side matters when moving the crossing there changes the
            // kept set's threshold (as in the wave form)
            const uint32_t tkm = max(t, minp ? t_m : 0u);
            const uint32_t kprev = gs > 0 ? keyof(gs - 1) : 0xFFFFFFFFu;
            const bool close_lo = c_new - target < kTopPMarginRel * ctot && ke > tkm;
            const bool close_hi = target - c_prev < kTopPMarginRel * ctot && kprev > tkm;
            if (close_lo || close_hi) flags |= 1u;
            else t = max(t, ke);
          }
        }
        if (minp) t = max(t, t_m);
        // the kept set: positions [0, et); its sum and the top logprobs
        const int bt = t ? win_bin(Af, key_to_float(t), wsc) : kWinBins;
        if (tid == 0) sm.bu[25] = (uint32_t)n;
        __syncthreads();
        if (t)
          for (int j = tid; j < n; j += kBlock)
            if (keyof(j) < t && (j == 0 || keyof(j - 1) >= t)) sm.bu[25] = (uint32_t)j;
        __syncthreads();
        const int et = (int)sm.bu[25], fp_bt = fpos(bt);
        double S_K = s_all;
        if (!flags && truncated && want_S) {
          if (full_k && bt <= rkhi) S_K = qsum(0, et - 1);
          else if (bt < kWinBins) S_K = cmass(bt - 1) + qsum(fp_bt, et - 1);
          else flags |= 1u;
        }
        const double lns = log(S_K);
        if (!flags && K > 0 && gid == 0) {
          const int kept_n = (truncated && !lp_all) ? et : n;
          const double lnl = lp_all ? lnA : lns;
          for (int q = tid; q < K; q += kBlock) {
            const int64_t o = (int64_t)row * K + q;
            if (q < kept_n) {
              kp.top_lp_vals[o] = (float)(((double)zof(q) - m) - lnl);
              kp.top_lp_ids[o] = idxof(q);
            } else {
              kp.top_lp_vals[o] = -INFINITY;
              kp.top_lp_ids[o] = -1;
            }
          }
        }
        general = flags & 1u;
        tau = t;
        lnS = lns;
      }
      __syncthreads();
    }

    PHASE_STAMP(kStampThresholds);
    // ---- general path: radix selects and an exact kept-set sum
    if (general) {
      tau = 0;
      if (topk) tau = radix_select<false>(sm, rc, zs, region, 0u, (uint32_t)P.top_k, 0.0, m);
      if (topp) {
        const uint32_t tp = radix_select<true>(sm, rc, zs, region, tau, 0u, (double)P.top_p, m);
        tau = tp > tau ? tp : tau;
      }
      if (minp) tau = t_m > tau ? t_m : tau;
      double ls = 0.0;
      for (int l = 4 * tid; l < ln4; l += 4 * kBlock) {
        const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (fkey(zv[c]) >= tau) ls += exp_nonpos(sm.exp_tab, (double)zv[c] - m);
      }
      const double ws = wg_sum_d(sm, ls);
      const unsigned p2 = xseq++ & 1u;
      if (tid == 0) atomic_st(&rc.my->ssum[p2], ws);
      row_barrier(sm, rc);
      if (tid == 0) {
        double t = 0.0;
        for (int g = 0; g < G; ++g) t += atomic_ld(&rc.peers[g].ssum[p2]);
        sm.bd[3] = t;
      }
      __syncthreads();
      lnS = log(sm.bd[3]);
      __syncthreads();
      // local top-logprob candidates: K rounds of a (value, index) max
      if (K > 0) {
        unsigned long long last = ~0ull;
        for (int t = 0; t < K; ++t) {
          unsigned long long cand = 0;
          for (int l = 4 * tid; l < ln4; l += 4 * kBlock) {
            const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if (zv[c] > -INFINITY && (lp_all || fkey(zv[c]) >= tau)) {
                const unsigned long long ck =
                    ((unsigned long long)fkey(zv[c]) << 32) | (0xFFFFFFFFu - (uint32_t)(s0 + l + c));
                if (ck < last && ck > cand) cand = ck;
              }
            }
          }
          cand = wg_max_u(sm, cand);
          if (tid == 0) sm.tl[t] = cand;
          last = cand;
          if (cand == 0) {
            if (tid == 0)
              for (int t2 = t + 1; t2 < K; ++t2) sm.tl[t2] = 0;
            break;
          }
        }
        __syncthreads();
      }
    }

    // ---- 5. Gumbel-max over the kept set, before any output store
    // Linear scores s_i = q_i / E_i with q_i = exp(z_i - m).  bound is a
    // lower bound of the best exact score (shared by the wave): an element
    // with w_i bound > q_i cannot reach it, because E_i >= w_i.  Groups of
    // four that hold a candidate (kept, and within kPruneNats of the max)
    // join a per-wave ring in LDS; Philox runs on full waves of such groups.
    const bool gumbel = !top1 && kp.path != PATH_GREEDY && !icdf;
    const float tauf = tau == 0 ? -INFINITY : key_to_float(tau);
    double best_g = -INFINITY;
    int best_i = 0x7FFFFFFF;
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const uint32_t off0 = (uint32_t)P.offset, off1 = (uint32_t)(P.offset >> 32);

    // ---- 4b. inverse-CDF selection (the seeded multinomial of [A] "One
    // request with top_p takes the whole batch off the fast path" and [B]
    // "What the flag switches"): the first kept token, in index order,
    // whose running kept mass q = exp(z - m) exceeds u times the kept total.
    // Each thread sums a contiguous segment of the slice in index order, a
    // fixed-order scan over threads and one exchange over the slices place
    // every segment on the row's cumulative axis, and the workgroup whose
    // range holds u S walks its segments.  (Summation order differs from a
    // single running sum only by rounding.)
    if (icdf) {
      double *cum = reinterpret_cast<double *>(regB);
      const int segl = (ln + kBlock - 1) / kBlock;
      const int a0 = min(tid * segl, ln), a1 = min(a0 + segl, ln);
      double ms = 0.0;
      int lastk = -1;
      for (int l = a0; l < a1; ++l) {
        const float zz = zs[l];
        if (zz >= tauf && zz > -INFINITY) {
          ms += exp_nonpos(sm.exp_tab, (double)zz - m);
          lastk = l;
        }
      }
      const double incl = block_scan_incl(ms, sm.red_d);
      cum[tid] = incl;
      if (tid == 0) {
        sm.bu[38] = 0xFFFFFFFFu;  // first slice position past u S
        sm.bu[39] = 0u;           // 1 + the slice's last kept position
      }
      __syncthreads();
      const double excl = tid > 0 ? cum[tid - 1] : 0.0;
      const double Mg = cum[kBlock - 1];
      if (lastk >= 0) atomicMax(&sm.bu[39], (uint32_t)lastk + 1u);
      const unsigned p2 = xseq++ & 1u;
      if (tid == 0) atomic_st(&rc.my->ssum[p2], Mg);
      row_barrier(sm, rc);
      if (tid == 0) {
        // the slices in index order: this slice's range [P_g, P_g+1) and
        // the total; the last slice with mass also takes u S >= the total
        double acc = 0.0, pg = 0.0, pg1 = 0.0;
        int lastg = -1;
        for (int g = 0; g < G; ++g) {
          const double mg_ = atomic_ld(&rc.peers[g].ssum[p2]);
          if (g == gid) pg = acc;
          acc += mg_;
          if (g == gid) pg1 = acc;
          if (mg_ > 0.0) lastg = g;
        }
        uint32_t w[4];
        philox4x32_10(0xFFFFFFFFu, P.stream, off0, off1, key0, key1, w);
        const double u = (double)((((unsigned long long)w[1] << 32) | w[0]) >> 11) * 0x1p-53;
        const double t = u * acc;
        sm.bd[6] = pg;
        sm.bd[7] = t;
        sm.bu[36] = (Mg > 0.0 && pg <= t && (t < pg1 || gid == lastg)) ? 1u : 0u;
      }
      __syncthreads();
      if (sm.bu[36]) {
        const double t = sm.bd[7];
        double c = sm.bd[6] + excl;
        if (c <= t) {
          for (int l = a0; l < a1; ++l) {
            const float zz = zs[l];
            if (zz >= tauf && zz > -INFINITY) {
              c += exp_nonpos(sm.exp_tab, (double)zz - m);
              if (c > t) {
                atomicMin(&sm.bu[38], (uint32_t)l);
                break;
              }
            }
          }
        }
        __syncthreads();
        if (tid == 0) {
          const uint32_t f = sm.bu[38];
          kp.token_ids[row] = s0 + (int)(f != 0xFFFFFFFFu ? f : sm.bu[39] - 1u);
        }
      }
    }
    float bound = 0.0f;
    float cut = kPruneNats;  // listing cut in nats below the max (set by the pass)
    // Groups of four that hold a Gumbel candidate (kept, and within
    // kPruneNats of the max) are listed per wave in LDS (16-bit group
    // numbers; every group the wave visits fits), then finished on full
    // waves: Philox and the filter.
    uint16_t *ring = reinterpret_cast<uint16_t *>(regB);  // this wave's list (set by the pass)
    uint32_t qh = 0, qt = 0;  // wave-uniform head and tail
#ifdef DSTS_PHASE_STAMPS
    uint32_t g_rounds = 0;  // fp64 scoring rounds of this wave (stamps builds)
#endif
    auto gumbel_batch = [&](uint32_t cnt) __attribute__((always_inline)) {  // one queued group per lane, cnt <= 64
      bool improved = false;
#ifdef DSTS_PHASE_STAMPS
      uint32_t surv_n = 0;
#endif
      if ((uint32_t)lane < cnt) {
        const int l = 4 * (int)ring[qh + lane];
        const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
        const int i0 = s0 + l;
        uint32_t w[4];
        philox4x32_10((uint32_t)i0 >> 2, P.stream, off0, off1, key0, key1, w);
        // the values of the group that may still beat the bound (bit c)
        uint32_t surv = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (zv[c] >= tauf && (mf - zv[c] <= cut)) {
            // lower bound of w: (float)x rounds to nearest
            const float wl = (float)w[c] * 0x1.fffffcp-33f;
            const float qv = __builtin_amdgcn_exp2f((zv[c] - mf) * kLog2e);
            if (wl * bound <= qv * kSlack) surv |= 1u << c;
          }
        }
        // their exact fp64 scores, one survivor per lane per round (in
        // index order): the wave runs as many rounds as its busiest lane
        // has survivors, not one per position that any lane needs
#ifdef DSTS_PHASE_STAMPS
        surv_n = (uint32_t)__popc(surv);
#endif
        while (surv) {
          const int c = __builtin_ctz(surv);
          surv &= surv - 1u;
          const float zc = c == 0 ? zv[0] : c == 1 ? zv[1] : c == 2 ? zv[2] : zv[3];
          const uint32_t wc = c == 0 ? w[0] : c == 1 ? w[1] : c == 2 ? w[2] : w[3];
          const double ge = (double)zc - log(exp1_f64(wc));
          if (ge > best_g || (ge == best_g && i0 + c < best_i)) {
            best_g = ge;
            best_i = i0 + c;
            improved = true;
          }
        }
      }
      qh += cnt;
#ifdef DSTS_PHASE_STAMPS
      g_rounds += lane63_u32(wave_scanmax_u32(surv_n));  // the wave's scoring rounds in this batch
#endif
      if (__ballot(improved)) {
        float mb = improved ? (float)exp(best_g - m) * 0.99999f : 0.0f;
        mb = wave_max_nonneg_f(mb);
        bound = fmaxf(bound, mb);
      }
    };
    // Gumbel candidates of the slice, NT threads from thread 0 (a list per
    // wave), then Philox on full waves of listed groups.
    auto gumbel_pass = [&](auto NTC) __attribute__((always_inline)) {
      constexpr int NT = decltype(NTC)::value;
      constexpr uint32_t kRingW = kMaxSlice / 4 / (NT / 64);  // groups one wave visits at most
      static_assert((NT / 64) * kRingW * sizeof(uint16_t) <= kRegionBBytes, "candidate lists fit the region");
      ring = reinterpret_cast<uint16_t *>(regB) + wave * kRingW;
      // the bound starts at the argmax's own score 1 / E (the argmax is
      // always kept).  A value's score is at most q 2^33 (E >= 2^-33), so
      // one with m - z above 33 ln 2 - ln(bound) cannot beat the argmax:
      // the listing cut, never looser than kPruneNats (1 / E >= 1 / (33
      // ln 2)), with the same margin for the fp32 rounding of m - z.
      uint32_t w4[4];
      philox4x32_10((uint32_t)argmax_idx >> 2, P.stream, off0, off1, key0, key1, w4);
      bound = (float)(1.0 / exp1_f64(w4[argmax_idx & 3])) * 0.99999f;
      cut = fminf(kPruneNats, kLnInvEmin + (kPruneNats - 26.004f) - logf(bound));
      PHASE_STAMP(kStampGumbelBound);
      const int its = (ln4 + 4 * NT - 1) / (4 * NT);
      constexpr int kStep = 8;  // groups read before any is tested
      for (int q0 = 0; q0 < its; q0 += kStep) {
        f32x4 zr[kStep];  // (clamped addresses)
#pragma unroll
        for (int u = 0; u < kStep; ++u) zr[u] = *reinterpret_cast<const f32x4 *>(zs + min(4 * tid + 4 * NT * (q0 + u), ln4 - 4));
#pragma unroll
        for (int u = 0; u < kStep; ++u) {
          const int l = 4 * tid + 4 * NT * (q0 + u);
          const bool act = l < ln4;
          // both tests are monotone in z (float subtraction rounds
          // monotonically), so a group holds a candidate exactly when its
          // largest value passes them; padding (-inf) never does
          const float zmax = fmaxf(fmaxf(zr[u][0], zr[u][1]), fmaxf(zr[u][2], zr[u][3]));
          const bool any_cand = zmax >= tauf && (mf - zmax <= cut);
          const unsigned long long bal = __ballot(act && any_cand);
          if (bal) {
            const uint32_t off = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (act && any_cand) ring[qt + off] = (uint16_t)(l >> 2);
            qt += (uint32_t)__popcll(bal);
          }
        }
      }
      PHASE_STAMP(kStampGumbelListed);
      PHASE_RECORD(kStampGumbelListedCount, qt);
      for (; qh < qt;) gumbel_batch(min(qt - qh, 64u));
      PHASE_STAMP(kStampGumbelBatched);
      PHASE_RECORD(kStampGumbelRounds, g_rounds);
    };

    // ---- 6. final exchange: the last workgroup to arrive writes the row.
    // One wave arrives before it issues any output store, so its wait for
    // its own stores covers only the exchange data, and the exchange runs
    // while the outputs are written.  Rows that merge top-logprob lists
    // (general path) need every thread and exchange after the emit.
    const unsigned fpar = it & 1u;
    const bool late_fin = general && K > 0;
    auto final_exchange = [&]() __attribute__((always_inline)) {  // one wave
      if (G == 1) {  // the row's only workgroup: the exchange stays in registers
        // (a one-workgroup launch never waits, so it cannot have aborted)
        if (lane == 0) {
          finish_row(kp, false, row, gumbel, icdf, lkey, best_g, best_i, false);
          PHASE_STAMP_ONE(kStampToken);
        }
        return;
      }
      if (lane == 0) {
        atomic_st(&rc.my->fin[fpar][0], (unsigned long long)__double_as_longlong(best_g));
        atomic_st(&rc.my->fin[fpar][1], (unsigned long long)(uint32_t)best_i);
        atomic_st(&rc.my->fin[fpar][2], lkey);
      }
      order_release();
      if (lane == 0) PHASE_STAMP_ONE(kStampReleased);
      uint32_t last = 0;
      if (lane == 0) {
        last = final_arrive(rc.gc) ? 1u : 0u;
        if (last) order_acquire();
        PHASE_STAMP_ONE(kStampArrived);
      }
      if (__builtin_amdgcn_readfirstlane(last)) {
        merge_final(kp, rc.peers, fpar, rc.gc.epoch, row, G, gumbel, icdf);
        if (lane == 0) PHASE_STAMP_ONE(kStampToken);
      }
    };

    // Outputs: the loop is specialised on the output mode (both outputs
    // with 16-byte stores; anything else, element by element) and on the
    // number of storing threads, with the per-row constants it uses held in
    // vector registers.
    auto emit_loop = [&](auto MODE, auto NTC, auto LPA) __attribute__((always_inline)) {
      constexpr int mode = decltype(MODE)::value;
      constexpr int NT = decltype(NTC)::value;  // the last NT threads store
      constexpr bool lpa = decltype(LPA)::value;  // logprobs of every token (ln S_all)
      const int et = tid - (kBlock - NT);
      const int its = (ln4 + 4 * NT - 1) / (4 * NT);
      double mv = m, lnsv = lnS, lnav = lnA;
      float tv = tauf;
      int64_t ob = (int64_t)row * V + s0;  // output offset of the slice
      // the slice's output rows, as global pointers held in vector registers
      typedef __attribute__((address_space(1))) f32x4 gf32x4;
      gf32x4 *pq = nullptr, *lq = nullptr;
      if (mode == 1) {
        pq = (gf32x4 *)(kp.probs + ob);
        lq = (gf32x4 *)(kp.logprobs + ob);
      }
      asm volatile("" : "+v"(mv), "+v"(lnsv), "+v"(tv), "+v"(ob), "+v"(pq), "+v"(lq));
      if (lpa) asm volatile("" : "+v"(lnav));
      for (int q0 = 0; q0 < its; q0 += 4) {
        f32x4 zr[4];  // the chunk's four groups, read first (clamped addresses)
#pragma unroll
        for (int u = 0; u < 4; ++u) zr[u] = *reinterpret_cast<const f32x4 *>(zs + min(4 * et + 4 * NT * (q0 + u), ln4 - 4));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int l = 4 * et + 4 * NT * (q0 + u);
          const bool act = l < ln4;
          const f32x4 zv = zr[u];
          // padding (-inf) only passes when tau is 0
          const bool anyk = fmaxf(fmaxf(zv[0], zv[1]), fmaxf(zv[2], zv[3])) >= tv;
          // a wave whose groups keep nothing stores 0 / -inf without the math
          if (!lpa && act && !__ballot(act && anyk)) {
            if (mode == 1 && l + 3 < ln) {
              __builtin_nontemporal_store(f32x4{0.0f, 0.0f, 0.0f, 0.0f}, pq + (l >> 2));
              __builtin_nontemporal_store(f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY}, lq + (l >> 2));
            } else {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                if (l + c < ln) {
                  if (kp.probs) kp.probs[ob + l + c] = 0.0f;
                  if (kp.logprobs) kp.logprobs[ob + l + c] = -INFINITY;
                }
              }
            }
          } else if (act) {
            float lv[4], pv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              // logprob: one rounding of the fp64 value; prob = 2^(lp log2 e)
              // by the hardware exp2 (absolute error below 2e-7)
              const bool kk = zv[c] >= tv;
              const float lp = kk ? (float)(((double)zv[c] - mv) - lnsv) : -INFINITY;
              lv[c] = lpa ? (float)(((double)zv[c] - mv) - lnav) : lp;
              pv[c] = kk ? __builtin_amdgcn_exp2f(lp * kLog2e) : 0.0f;
            }
            const int64_t o = ob + l;
            if (mode == 1 && l + 3 < ln) {
              __builtin_nontemporal_store(f32x4{pv[0], pv[1], pv[2], pv[3]}, pq + (l >> 2));
              __builtin_nontemporal_store(f32x4{lv[0], lv[1], lv[2], lv[3]}, lq + (l >> 2));
            } else {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                if (l + c < ln) {
                  if (kp.probs) kp.probs[o + c] = pv[c];
                  if (kp.logprobs) kp.logprobs[o + c] = lv[c];
                }
              }
            }
          }
        }
      }
    };
    using NT256 = std::integral_constant<int, 256>;
    using NT512 = std::integral_constant<int, kBlock>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using B0 = std::integral_constant<bool, false>;
    using B1 = std::integral_constant<bool, true>;
    PHASE_STAMP(kStampSelect);
    if (omode != 0 && !late_fin && tau != 0) {
      // A truncated row: waves 4..7 write the outputs from the start; waves
      // 0..3 run Gumbel-max over the whole slice meanwhile (the kept set is
      // small), and the last of them to finish (an LDS counter, cleared at
      // the row start) merges the four bests and runs the final exchange.
      // Rows that keep every value need all waves for Philox (below).
      static_assert(kBlock == 512, "four Gumbel waves and four storing waves");
      if (wave < 4) {
        if (gumbel) {
          gumbel_pass(NT256{});
          wave_best(best_g, best_i);
        }
        PHASE_STAMP(kStampGumbel);
        if (lane == 0) {
          sm.red_d[wave] = best_g;
          sm.red_i[wave] = best_i;
        }
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(&sm.bu[37], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(old) == 3u) {
          best_g = sm.red_d[0];
          best_i = sm.red_i[0];
#pragma unroll
          for (int w = 1; w < 4; ++w) {
            if (sm.red_d[w] > best_g || (sm.red_d[w] == best_g && sm.red_i[w] < best_i)) {
              best_g = sm.red_d[w];
              best_i = sm.red_i[w];
            }
          }
          final_exchange();
        }
      } else if (lp_all) {
        if (omode == 1) emit_loop(I1{}, NT256{}, B1{});
        else emit_loop(I2{}, NT256{}, B1{});
      } else if (omode == 1) {
        emit_loop(I1{}, NT256{}, B0{});
      } else {
        emit_loop(I2{}, NT256{}, B0{});
      }
    } else {
      if (gumbel) {
        gumbel_pass(NT512{});
        wg_best(sm, best_g, best_i);
      }
      PHASE_STAMP(kStampGumbel);
      if (!late_fin && wave == 0) final_exchange();
      if (lp_all) {
        if (omode == 1) emit_loop(I1{}, NT512{}, B1{});
        else if (omode == 2) emit_loop(I2{}, NT512{}, B1{});
      } else if (omode == 1) {
        emit_loop(I1{}, NT512{}, B0{});
      } else if (omode == 2) {
        emit_loop(I2{}, NT512{}, B0{});
      }
    }

    if (late_fin) {
      if (tid == 0) {
        atomic_st(&rc.my->fin[fpar][0], (unsigned long long)__double_as_longlong(best_g));
        atomic_st(&rc.my->fin[fpar][1], (unsigned long long)(uint32_t)best_i);
        atomic_st(&rc.my->fin[fpar][2], lkey);
      }
      for (int t = tid; t < K; t += kBlock) atomic_st(&rc.my->toplist[fpar][t], sm.tl[t]);
      order_release();
      __syncthreads();
      if (tid == 0) {
        const bool last = final_arrive(rc.gc);
        if (last) order_acquire();
        sm.bu[15] = last ? 1u : 0u;
      }
      __syncthreads();
      if (sm.bu[15]) {
        if (wave == 0) merge_final(kp, rc.peers, fpar, rc.gc.epoch, row, G, gumbel, icdf);
        // merge the G local top-logprob lists (keys are distinct: each holds
        // its index): an entry's rank among all entries is its output slot
        unsigned long long *ent = reinterpret_cast<unsigned long long *>(region);
        const int ne = G * K;
        for (int e = tid; e < ne; e += kBlock) ent[e] = atomic_ld(&rc.peers[e / K].toplist[fpar][e % K]);
        __syncthreads();
        uint32_t nz = 0;
        for (int e = tid; e < ne; e += kBlock) {
          const unsigned long long key = ent[e];
          if (key == 0) continue;
          ++nz;
          int r = 0;
          for (int j = 0; j < ne; ++j) r += ent[j] > key ? 1 : 0;
          if (r < K) {
            const int64_t o = (int64_t)row * K + r;
            const float zz = key_to_float((uint32_t)(key >> 32));
            kp.top_lp_vals[o] = (float)(((double)zz - m) - (lp_all ? lnA : lnS));
            kp.top_lp_ids[o] = (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
          }
        }
        const uint32_t nzt = (uint32_t)wg_sum_u(sm, nz);
        for (int r = (int)nzt + tid; r < K; r += kBlock) {
          kp.top_lp_vals[(int64_t)row * K + r] = -INFINITY;
          kp.top_lp_ids[(int64_t)row * K + r] = -1;
        }
      }
    }
    __syncthreads();
    PHASE_STAMP(kStampEnd);
  }
}

// ---------------------------------------------------------------- long histories
// [C] "解码一步里采样做什么" (_apply_penalties): the penalties take each
// token's count in the sequence so far.  A history longer than the row
// kernel's LDS hash holds is counted here, ahead of the row kernel:
// workgroup (record, slice) counts the ids that fall in its slice in a
// dense LDS array, then writes the nonzero counts in index order as
// local << 17 | count, and their number.  Each thread compacts a contiguous
// run of the slice, so the list's order is fixed.  Rows that do not need it
// leave at once.
__global__ __launch_bounds__(kBlock) void hist_list_kernel(KernelArgs ka) {
  const KernelParams &kp = ka.kp;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  uint32_t *cnt = reinterpret_cast<uint32_t *>(lds_raw);
  __shared__ uint32_t wave_tot[kWaves];
  const int G = kp.G;
  const int ri = (int)blockIdx.x / G, gid = (int)blockIdx.x % G;
  const RowParam *pp = kp.rows ? kp.rows + ri : ka.rows + ri;
  const uint32_t flags = pp->flags;
  const int32_t hist_len = pp->hist_len;
  if ((flags & RF_BAD) || !(flags & RF_PEN) || hist_len <= kMaxHistPerRow) return;
  const int64_t hist_start = pp->hist_start;
  const int row = pp->row;
  const int tid = (int)threadIdx.x;
  const int s0 = gid * kp.slice, s1 = min(kp.vocab, s0 + kp.slice), ln = s1 - s0;
  for (int l = tid; l < ln; l += kBlock) cnt[l] = 0u;
  __syncthreads();
  const int32_t *hist = kp.history_ids + hist_start;
#pragma unroll 8
  for (int h = tid; h < hist_len; h += kBlock) {
    const int32_t id = hist[h];
    if (id >= s0 && id < s1) atomicAdd(&cnt[id - s0], 1u);
  }
  __syncthreads();
  const int per = (ln + kBlock - 1) / kBlock;
  const int l0 = min(ln, tid * per), l1 = min(ln, l0 + per);
  uint32_t c = 0;
  for (int l = l0; l < l1; ++l) c += cnt[l] != 0u ? 1u : 0u;
  const uint32_t incl = block_scan_incl(c, wave_tot);
  const int64_t li = (int64_t)row * G + gid;
  uint32_t *out = kp.hist_list + li * kp.hist_list_cap;
  uint32_t k = incl - c;
  for (int l = l0; l < l1; ++l)
    if (cnt[l] != 0u) out[k++] = ((uint32_t)l << 17) | cnt[l];
  if (tid == kBlock - 1) kp.hist_list_n[li] = (int32_t)incl;
}

// ---------------------------------------------------------------- raw logprobs
// [B] "Logprobs are temperature-scaled": with the original-logprob switch
// the returned logprobs are log_softmax of the processed logits x' (logits
// processors and penalties applied, no temperature).  The row kernel holds
// z = x' / T, from which x' cannot be recovered exactly, so for the rows
// whose effective temperature is not 1 this kernel runs after it: each
// workgroup of a row group rebuilds x' for its slice (the raw logits again,
// NaN -> -inf, the grammar mask, then the owners of history and bias
// entries recompute their tokens as the row kernel does), takes the slice's
// max and exact fp64 sum, exchanges them with its peers, and overwrites the
// row's logprobs and the values of its top logprobs (whose ids and order
// the row kernel chose, by z over all tokens).  Rows at temperature 1 are
// already right (z = x').
template <typename TIn>
__global__ __launch_bounds__(kBlock) void raw_lp_kernel(KernelArgs ka) {
  const KernelParams &kp = ka.kp;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  SmemBase &sm = *reinterpret_cast<SmemBase *>(lds_raw);
  float *xs = reinterpret_cast<float *>(lds_raw + sizeof(SmemBase));
  unsigned char *region = reinterpret_cast<unsigned char *>(xs + kp.slice);
  uint32_t *hash = reinterpret_cast<uint32_t *>(region);
  unsigned long long *bhash = reinterpret_cast<unsigned long long *>(region + 4 * (size_t)kp.hash_slots);
  const int G = kp.G, V = kp.vocab;
  int group, gid;
  block_group(kp, group, gid);
  const uint32_t hslots = (uint32_t)kp.hash_slots, bslots = (uint32_t)kp.bias_slots;
  GroupCtx gc;
  gc.s = kp.sync + group;
  gc.abort_word = kp.abort_word;
  gc.epoch = kp.epoch_dev ? atomic_ld(kp.epoch_dev) + kp.epoch_dev_add : kp.epoch;
  gc.spin_limit = kp.spin_limit ? kp.spin_limit : kSpinLimit;
  gc.G = G;
  if (gid == 0 && G > 1 && tidx() == 0) claim_words(gc.s, gc.epoch);
  const int s0 = gid * kp.slice, s1 = min(V, s0 + kp.slice), ln = s1 - s0;
  for (int j = tidx(); j < 64; j += kBlock) sm.exp_tab[j] = exp2((double)j * (1.0 / 64.0));
  unsigned it = 0;
  for (int ri = group; ri < kp.n_rows; ri += kp.n_groups) {
    const RowParam P = kp.rows ? kp.rows[ri] : ka.rows[ri];
    if ((P.flags & RF_BAD) || P.temperature == 1.0f) continue;  // the same on every workgroup of the row
    const int tid = tidx(), row = P.row;
    const bool pen = (P.flags & RF_PEN) != 0, spec = (P.flags & RF_SPEC) != 0;
    const int64_t rbase = (int64_t)row * kp.row_stride + s0;
    // x' = the sanitised raw logit, -inf where the grammar mask clears it
    const uint32_t *mrow = kp.vocab_mask ? kp.vocab_mask + (int64_t)row * kp.mask_stride : nullptr;
    for (int l = tid; l < ln; l += kBlock) {
      float x = Loader<TIn>::load1(kp.logits, rbase + l);
      if (x != x) x = -INFINITY;
      if (mrow && !((mrow[(s0 + l) >> 5] >> ((s0 + l) & 31)) & 1u)) x = -INFINITY;
      xs[l] = x;
    }
    // the history and bias hashes of the slice, as in the row kernel (a
    // history longer than the hash holds: its counted list and a bitmap)
    const bool longh = pen && P.hist_len > kMaxHistPerRow;
    const int64_t li = (int64_t)row * G + gid;
    const uint32_t *hl = longh ? kp.hist_list + li * kp.hist_list_cap : nullptr;
    const int hl_n = longh ? kp.hist_list_n[li] : 0;
    if (pen)
      for (int t = tid; t < (int)hslots; t += kBlock) hash[t] = longh ? 0u : kEmpty;
    if (spec)
      for (int t = tid; t < (int)bslots; t += kBlock) bhash[t] = 0xFFFFFFFFull;
    __syncthreads();
    int32_t bid = -1;
    float bval = 0.0f;
    if (spec) {
      if (tid < P.bias_len) {
        bid = kp.bias_ids[P.bias_start + tid];
        bval = kp.bias_vals[P.bias_start + tid];
      } else if (tid < P.bias_len + P.stop_len) {
        bid = kp.stop_ids[P.stop_start + (tid - P.bias_len)];
        bval = -INFINITY;
      }
    }
    if (spec && bid >= s0 && bid < s1) {
      const uint32_t local = (uint32_t)(bid - s0);
      uint32_t sl = hash_slot(local, bslots);
      uint32_t *lo = reinterpret_cast<uint32_t *>(bhash);
      while (true) {
        const uint32_t prev = atomicCAS(&lo[2 * sl], kEmpty, local);
        if (prev == kEmpty || prev == local) {
          atomicAdd(reinterpret_cast<float *>(&lo[2 * sl + 1]), bval);
          break;
        }
        sl = (sl + 1u) & (bslots - 1u);
      }
    }
    for (int h = tid; h < hl_n; h += kBlock) {
      const uint32_t local = hl[h] >> 17;
      atomicOr(&hash[local >> 5], 1u << (local & 31u));
    }
    if (pen && !longh) {
      const int32_t *hist = kp.history_ids + P.hist_start;
      for (int h = tid; h < P.hist_len; h += kBlock) {
        const int32_t id = hist[h];
        if (id >= s0 && id < s1) {
          const uint32_t local = (uint32_t)(id - s0);
          uint32_t sl = hash_slot(local, hslots);
          while (true) {
            const uint32_t prev = atomicCAS(&hash[sl], kEmpty, (local << 13) | 1u);
            if (prev == kEmpty) break;
            if ((prev >> 13) == local) {
              atomicAdd(&hash[sl], 1u);
              break;
            }
            sl = (sl + 1u) & (hslots - 1u);
          }
        }
      }
    }
    __syncthreads();
    // every occupied slot's token is recomputed from its raw logit: bias,
    // then the penalties with the final count (masked tokens stay -inf)
    if (pen && !longh)
      for (int t = tid; t < (int)hslots; t += kBlock) {
        const uint32_t e = hash[t];
        if (e == kEmpty) continue;
        const uint32_t local = e >> 13;
        float x = Loader<TIn>::load1(kp.logits, rbase + local), b;
        x = x == x ? x : -INFINITY;
        if (spec && bias_lookup(bhash, bslots, local, b)) x = add_bias(x, b);
        const bool masked = mrow && !((mrow[(s0 + local) >> 5] >> ((s0 + local) & 31)) & 1u);
        xs[local] = masked ? -INFINITY : apply_penalty(x, e & 0x1FFFu, P);
      }
    for (int h = tid; h < hl_n; h += kBlock) {
      const uint32_t e = hl[h], local = e >> 17;
      float x = Loader<TIn>::load1(kp.logits, rbase + local), b;
      x = x == x ? x : -INFINITY;
      if (spec && bias_lookup(bhash, bslots, local, b)) x = add_bias(x, b);
      const bool masked = mrow && !((mrow[(s0 + local) >> 5] >> ((s0 + local) & 31)) & 1u);
      xs[local] = masked ? -INFINITY : apply_penalty(x, e & 0x1FFFFu, P);
    }
    if (spec)
      for (int t = tid; t < (int)bslots; t += kBlock) {
        const unsigned long long e = bhash[t];
        const uint32_t local = (uint32_t)e;
        if (local == kEmpty) continue;
        if (pen && (longh ? ((hash[local >> 5] >> (local & 31u)) & 1u) != 0u : hist_contains(hash, hslots, local)))
          continue;
        float x = Loader<TIn>::load1(kp.logits, rbase + local);
        x = x == x ? x : -INFINITY;
        const bool masked = mrow && !((mrow[(s0 + local) >> 5] >> ((s0 + local) & 31)) & 1u);
        xs[local] = masked ? -INFINITY : add_bias(x, __uint_as_float((uint32_t)(e >> 32)));
      }
    __syncthreads();
    // the slice's max, then its exact sum relative to it
    float lm = -INFINITY;
    for (int l = tid; l < ln; l += kBlock) lm = fmaxf(lm, xs[l]);
    const unsigned long long mkey = wg_max_u(sm, (unsigned long long)fkey(lm));
    const float mg = key_to_float((uint32_t)mkey);
    double ls = 0.0;
    if (mg > -INFINITY && mg < INFINITY)
      for (int l = tid; l < ln; l += kBlock) ls += exp_nonpos(sm.exp_tab, (double)xs[l] - (double)mg);
    const double sg = wg_sum_d(sm, ls);
    const unsigned par = it++ & 1u;
    WgSlots *my = kp.slots + (size_t)group * G + gid;
    if (tid == 0) {
      atomic_st(&my->x1[par][0], (unsigned long long)__float_as_uint(mg));
      atomic_st(&my->x1[par][1], (unsigned long long)__double_as_longlong(sg));
    }
    group_barrier(sm, gc);
    if (tid == 0) {
      // every workgroup combines the slices in the same order
      float m = -INFINITY;
      for (int g = 0; g < G; ++g)
        m = fmaxf(m, __uint_as_float((uint32_t)atomic_ld(&kp.slots[(size_t)group * G + g].x1[par][0])));
      double S = 0.0;
      for (int g = 0; g < G; ++g) {
        const WgSlots &pg = kp.slots[(size_t)group * G + g];
        const float mgg = __uint_as_float((uint32_t)atomic_ld(&pg.x1[par][0]));
        const double sgg = __longlong_as_double((long long)atomic_ld(&pg.x1[par][1]));
        if (mgg > -INFINITY && m < INFINITY) S += sgg * exp_nonpos(sm.exp_tab, (double)mgg - (double)m);
      }
      sm.bd[0] = (double)m;
      sm.bd[1] = log(S);
      sm.bu[0] = (m > -INFINITY && m < INFINITY && atomic_ld(kp.abort_word) != gc.epoch) ? 1u : 0u;
      if (gid == 0 && atomic_ld(kp.abort_word) == gc.epoch && kp.row_status) kp.row_status[row] = 3;
    }
    __syncthreads();
    // rows without a finite value keep the row kernel's outputs (status 1 or 2)
    if (sm.bu[0]) {
      const double m = sm.bd[0], lns = sm.bd[1];
      if (kp.logprobs)
        for (int l = tid; l < ln; l += kBlock) kp.logprobs[(int64_t)row * V + s0 + l] = (float)(((double)xs[l] - m) - lns);
      for (int j = tid; j < kp.top_lp; j += kBlock) {
        const int id = kp.top_lp_ids[(int64_t)row * kp.top_lp + j];
        if (id >= s0 && id < s1) kp.top_lp_vals[(int64_t)row * kp.top_lp + j] = (float)(((double)xs[id - s0] - m) - lns);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- streaming rows
// Batches of many rows that want only tokens and top logprobs (no probs or
// logprobs), [C] "best_of 与 n 的放大": forks multiply the rows of a step.
// The row kernel holds a row's slices in LDS, so such a batch walks each
// row group through many rows one after the other.  Here one workgroup
// owns a whole row (two workgroups per CU) and reads it from memory in up
// to three passes, recomputing z = penalised(x) / T each time, so every row
// of the batch is in flight at once:
//   A. the row max and its first index;
//   B. (rows with thresholds or a top-logprob list) the window histogram of
//      the row kernel -- absolute bins of 1/32 nat, counts and approximate
//      masses -- which places each threshold in a range of values;
//   C. values in those ranges are gathered into LDS; values above them
//      (certainly kept) are counted, their masses summed exactly and their
//      Gumbel scores taken on the way (Philox, the linear-domain bound,
//      fp64 scores).
// The gathered list is then sorted and every decision taken exactly on it:
// the k-th value and its tie group, the top-p crossing on exact fp64
// cumulative masses, min-p's boundary key, tau, the kept-set sum, the top
// logprobs and the Gumbel scores of the kept values in the list.  A row
// whose thresholds lie outside the window, whose ranges hold more than
// kSCap values, or whose exact decision falls outside the ranges the
// histogram chose is not written: its record goes to a list that the row
// kernel, launched after this one, samples in full.
constexpr int kSCap = 2048;       // values gathered per row (one workgroup per CU has room)
constexpr int kSLoads = 4;        // 16-byte chunks each thread loads per step (one more step in flight)
static_assert(kSCap % kBlock == 0, "gathered values per thread");

// Window histogram entry of the streaming kernel: a count in bits 44.. (a
// row of up to 2^19 values fits) and the mass exp(z - max) in 2^-24 units
// below (a bin of 2^19 values at most 2^43).  These masses only place the
// top-p crossing in a range of bins; the decision itself is exact.
DEV unsigned long long hist_entry_s(float a) {
  return (1ull << 44) | (unsigned long long)(uint32_t)__builtin_rintf(a * 16777216.0f);
}

// A token's history count from the row's hash (token << 13 | count), or 0.
DEV uint32_t hist_count(const uint32_t *hash, uint32_t slots, uint32_t tok) {
  uint32_t sl = hash_slot(tok, slots);
  while (true) {
    const uint32_t e = hash[sl];
    if (e == kEmpty) return 0u;
    if ((e >> 13) == tok) return e & 0x1FFFu;
    sl = (sl + 1u) & (slots - 1u);
  }
}

// A 16-byte chunk of a row (16-byte aligned): kGroups groups of four
// values (one of fp32, two of bf16).  Ordinary loads: the passes read a row
// again soon after, so it should stay in the caches.
template <typename TIn>
struct Chunk16;
template <>
struct Chunk16<float> {
  static constexpr int kGroups = 1;
  static DEV u32x4 load(const void *base, int64_t off) {
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const float *>(base) + off);
  }
  static DEV u32x4 load_scalar(const void *base, int64_t rbase, int i0, int V) {
    const float *p = reinterpret_cast<const float *>(base) + rbase;
    u32x4 r;
    r.x = __float_as_uint(p[min(i0, V - 1)]);
    r.y = __float_as_uint(p[min(i0 + 1, V - 1)]);
    r.z = __float_as_uint(p[min(i0 + 2, V - 1)]);
    r.w = __float_as_uint(p[min(i0 + 3, V - 1)]);
    return r;
  }
  static DEV void unpack(const u32x4 &t, int j, float v[4]) {
    (void)j;
    v[0] = __uint_as_float(t.x);
    v[1] = __uint_as_float(t.y);
    v[2] = __uint_as_float(t.z);
    v[3] = __uint_as_float(t.w);
  }
};
template <>
struct Chunk16<uint16_t> {
  static constexpr int kGroups = 2;
  static DEV u32x4 load(const void *base, int64_t off) {
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(base) + off);
  }
  static DEV u32x4 load_scalar(const void *base, int64_t rbase, int i0, int V) {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + rbase;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)p[min(i0 + 2 * k, V - 1)] | ((uint32_t)p[min(i0 + 2 * k + 1, V - 1)] << 16);
    return u32x4{w[0], w[1], w[2], w[3]};
  }
  static DEV void unpack(const u32x4 &t, int j, float v[4]) {
    const uint32_t a = j == 0 ? t.x : t.z, b = j == 0 ? t.y : t.w;
    v[0] = __uint_as_float(a << 16);
    v[1] = __uint_as_float(a & 0xFFFF0000u);
    v[2] = __uint_as_float(b << 16);
    v[3] = __uint_as_float(b & 0xFFFF0000u);
  }
};
// One value (rows not aligned for vector loads).
DEV float load1_cached(const float *base, int64_t off) { return base[off]; }
DEV float load1_cached(const uint16_t *base, int64_t off) { return __uint_as_float((uint32_t)base[off] << 16); }

template <typename TIn, bool PEN>
__global__ __launch_bounds__(kBlock, 2) void stream_kernel(KernelArgs ka) {
  const KernelParams &kp = ka.kp;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  SmemBase &sm = *reinterpret_cast<SmemBase *>(lds_raw);
  const uint32_t hslots = PEN ? (uint32_t)kp.hash_slots : 0u;
  const int bwords = PEN ? stream_bitmap_words(kp.vocab) : 0;
  // LDS: with penalties, a bitmap of the tokens that have history, the hash
  // of their counts (token << 13 | count) and each entry's penalised value;
  // then the gathered keys sk (later their prefix masses) and the sorted
  // keys srt; the window histogram and its prefix sums use the same bytes
  // before the gather
  uint32_t *bmap = reinterpret_cast<uint32_t *>(lds_raw + sizeof(SmemBase));
  uint32_t *hash = bmap + bwords;
  float *hz = reinterpret_cast<float *>(hash + hslots);
  unsigned long long *sk = reinterpret_cast<unsigned long long *>(hz + hslots);
  unsigned long long *srt = sk + kSCap;
  double *pre = reinterpret_cast<double *>(sk);
  unsigned long long *wh = sk;                                     // [kWinBins]
  unsigned long long *lm = sk + kWinBins;                          // [kWinBins] inclusive masses
  uint32_t *lc = reinterpret_cast<uint32_t *>(sk + 2 * kWinBins);  // [kWinBins] inclusive counts
  static_assert(8 * 2 * kWinBins + 4 * kWinBins <= 16 * kSCap, "the histogram fits the list region");

  const int V = kp.vocab;
  const int n4 = (V + 3) >> 2;
  const int K = kp.top_lp;
  unsigned it = 0;  // (the phase stamps describe a workgroup's first row)
  PHASE_STAMP(kStampStreamStart);
  for (int j = tidx(); j < 64; j += kBlock) sm.exp_tab[j] = exp2((double)j * (1.0 / 64.0));
  __syncthreads();

  for (int ri = blockIdx.x; ri < kp.n_rows; ri += gridDim.x, ++it) {
    const int tid = tidx();
    const int lane = tid & 63;
    const RowParam P = kp.rows ? kp.rows[ri] : ka.rows[ri];
    const int row = P.row;
    PHASE_STAMP(kStampRow);
    PHASE_RECORD(kStampRowIndex, row + 1);
    // outputs of a row without a token (status 1, 2 or 4)
    auto write_status = [&](int status) {
      if (tid == 0) {
        kp.token_ids[row] = -1;
        if (kp.row_status) kp.row_status[row] = status;
      }
      for (int t = tid; t < K; t += kBlock) {
        kp.top_lp_vals[(int64_t)row * K + t] = -INFINITY;
        kp.top_lp_ids[(int64_t)row * K + t] = -1;
      }
    };
    // the row goes to the row kernel launched after this one (its record
    // is read again: keeping P live across the row would cost registers)
    auto defer_row = [&]() {
      if (tid == 0) {
        const uint32_t slot = (uint32_t)arrive_word(kp.defer_word, kp.epoch);
        kp.defer_rows[slot] = kp.rows ? kp.rows[ri] : ka.rows[ri];
      }
    };
    auto row_body = [&]() __attribute__((always_inline)) {
      if (P.flags & RF_BAD) {
        write_status(4);
        return;
      }
      const bool greedy = P.flags & RF_GREEDY;
      const bool top1 = P.flags & RF_TOP1;
      const bool pen = PEN && (P.flags & RF_PEN);
      const bool topk = !greedy && (P.flags & RF_TOPK);
      const bool topp = !greedy && (P.flags & RF_TOPP);
      const bool minp = !greedy && (P.flags & RF_MINP);
      const bool truncated = topk || topp || minp;
      const bool gumbel = !top1 && kp.path != PATH_GREEDY;
      const float T = P.temperature;
      const float rT = 1.0f / T;
      const uint32_t xlo_b = __float_as_uint(T * 0x1p-99f);
      const uint32_t xhi_b = min(__float_as_uint(T * 0x1p99f), 0x7F7FFFFFu);
      const int64_t rbase = (int64_t)row * kp.row_stride;
      const bool vec = kp.vec_ok & 4;  // rows aligned for 16-byte loads

      // ---- history counts: the hash, the bitmap, and each token's
      // penalised value (computed once, by the thread that created the entry,
      // from the token's raw logit).  The passes take the history tokens out
      // of the stream (their bits make them -inf there) and then visit them
      // from the hash: the "patch" step of each pass.
      if (pen) {
        for (int t = tid; t < bwords; t += kBlock) bmap[t] = 0u;
        for (int t = tid; t < (int)hslots; t += kBlock) hash[t] = kEmpty;
        __syncthreads();
        const int32_t *hist = kp.history_ids + P.hist_start;
        for (int h = tid; h < P.hist_len; h += kBlock) {
          const int32_t id = hist[h];
          if (id >= 0 && id < V) {
            const uint32_t tok = (uint32_t)id;
            uint32_t sl = hash_slot(tok, hslots);
            while (true) {
              const uint32_t prev = atomicCAS(&hash[sl], kEmpty, (tok << 13) | 1u);
              if (prev == kEmpty) {
                atomicOr(&bmap[tok >> 5], 1u << (tok & 31u));
                break;
              }
              if ((prev >> 13) == tok) {
                atomicAdd(&hash[sl], 1u);
                break;
              }
              sl = (sl + 1u) & (hslots - 1u);
            }
          }
        }
        __syncthreads();
        for (int t = tid; t < (int)hslots; t += kBlock) {
          const uint32_t e = hash[t];
          if (e != kEmpty) {
            float x = load1_cached(reinterpret_cast<const TIn *>(kp.logits), rbase + (e >> 13));
            x = x == x ? x : -INFINITY;
            hz[t] = div_temp(apply_penalty(x, e & 0x1FFFu, P), T, rT);
          }
        }
        __syncthreads();
      }
      PHASE_STAMP(kStampHashed);
      // the patch step: f(token, z) for every history token of the row
      auto patches = [&](auto &&f) __attribute__((always_inline)) {
        if (pen)
          for (int t = tid; t < (int)hslots; t += kBlock) {
            const uint32_t e = hash[t];
            if (e != kEmpty) f((int)(e >> 13), hz[t]);
          }
      };

      // The passes see every token without history: pass A and B its z =
      // x / T correctly rounded (Markstein while |x| lies in [T 2^-99,
      // T 2^99], else the IEEE division), NaN -> -inf, -0 -> +0; pass C its
      // raw logit, compared with thresholds mapped to the logits.  History
      // tokens and slots past the row are masked (they read -inf).
      // A chunk is a 16-byte load: kGPL groups of four values.
      constexpr int kGPL = Chunk16<TIn>::kGroups;
      constexpr int kCV = 4 * kGPL;  // values per chunk
      const int nch = (V + kCV - 1) / kCV;
      // the chunk's history bits (bit j: value j of the chunk)
      auto chunk_bits = [&](int c) -> uint32_t {
        if (!pen) return 0u;
        const uint32_t i0 = (uint32_t)(kCV * c);
        return (bmap[i0 >> 5] >> (i0 & 31u)) & ((1u << kCV) - 1u);
      };
      // z of an unmasked value: the Markstein form when the step is known
      // to lie in its range, else the general division
      auto zval = [&](float x, bool fast) __attribute__((always_inline)) {
        if (fast) {
          const float qq = x * rT;
          return __builtin_fmaf(__builtin_fmaf(-qq, T, x), rT, qq);
        }
        return div_temp(x == x ? x : -INFINITY, T, rT);
      };
      // One pass over the row: fstep(gi, v, mk, fast) for each step of kNG
      // groups per thread (their indices, raw values and masks of masked
      // values; fast: every value of the step is finite and in the Markstein
      // range, tested only when the pass asks for it).  Threads take chunks;
      // each workgroup starts at its own point of its row (rows lie at
      // multiples of one stride) and wraps around.  Loads run one step ahead
      // (the next step's chunks are in flight while this step's are
      // processed).  Lanes past the row's end see masked values, so
      // cross-lane operations in fstep run in uniform control flow.
      const int shift = (int)(((int64_t)blockIdx.x * nch) / (int64_t)gridDim.x);
      auto cmap = [&](int x) {  // x in [0, nch): the chunk it stands for
        const int y = x + shift;
        return y >= nch ? y - nch : y;
      };
      constexpr int kSL = kSLoads;  // loads per step
      constexpr int kNG = kSL * kGPL;  // groups per thread and step
      auto stream_pass = [&](auto NEEDZ, auto &&fstep) __attribute__((always_inline)) {
        constexpr bool needz = decltype(NEEDZ)::value;
        const int lastc = nch - 1;
        constexpr int kStep = kBlock * kSL;
        // a step: group indices, masks and the fast flag; values are
        // unpacked from the raw chunks where the pass uses them
        auto step = [&](int s0, const u32x4 (&ch)[kSL], const uint32_t (&bb)[kSL]) __attribute__((always_inline)) {
          int gi[kNG];
          uint32_t mk[kNG];
          uint32_t amax = 0u, amin = 0xFFFFFFFFu;
#pragma unroll
          for (int u = 0; u < kSL; ++u) {
            const int x = s0 + tid + u * kBlock;
            const int c = cmap(min(x, lastc));
#pragma unroll
            for (int j = 0; j < kGPL; ++j) {
              const int t = u * kGPL + j;
              gi[t] = kGPL * c + j;
              const int i0 = kCV * c + 4 * j;
              uint32_t m4 = (bb[u] >> (4 * j)) & 0xFu;
              if (x >= nch) m4 = 0xFu;
              if (i0 + 4 > V) m4 |= (0xFu << (V - i0 > 0 ? V - i0 : 0)) & 0xFu;
              mk[t] = m4;
              if (needz) {
                float v[4];
                Chunk16<TIn>::unpack(ch[u], j, v);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const uint32_t ab = ((m4 >> q) & 1u) ? __float_as_uint(1.0f) : __float_as_uint(v[q]) & 0x7FFFFFFFu;
                  amax = max(amax, ab);
                  amin = min(amin, ab);
                }
              }
            }
          }
          // (1.0 stands in for masked values: in range whenever T is)
          const bool fast = needz && (__float_as_uint(1.0f) <= xhi_b) && (__float_as_uint(1.0f) >= xlo_b) &&
                            __ballot(!((amax <= xhi_b) & (amin >= xlo_b))) == 0ull;  // (wave-uniform)
          fstep(gi, ch, mk, fast);
        };
        if (vec) {
          u32x4 cur[kSL];
#pragma unroll
          for (int u = 0; u < kSL; ++u)
            cur[u] = Chunk16<TIn>::load(kp.logits, rbase + kCV * (int64_t)cmap(min(tid + u * kBlock, lastc)));
          for (int s0 = 0; s0 < nch; s0 += kStep) {  // (workgroup-uniform trip count)
            u32x4 nxt[kSL];  // (clamped: the last step loads in bounds, unused)
#pragma unroll
            for (int u = 0; u < kSL; ++u)
              nxt[u] = Chunk16<TIn>::load(kp.logits, rbase + kCV * (int64_t)cmap(min(s0 + kStep + tid + u * kBlock, lastc)));
            uint32_t bb[kSL];
#pragma unroll
            for (int u = 0; u < kSL; ++u) bb[u] = chunk_bits(cmap(min(s0 + tid + u * kBlock, lastc)));
            step(s0, cur, bb);
#pragma unroll
            for (int u = 0; u < kSL; ++u) cur[u] = nxt[u];
          }
        } else {  // clamped scalar loads, packed into chunks
          for (int s0 = 0; s0 < nch; s0 += kStep) {
            u32x4 ch[kSL];
            uint32_t bb[kSL];
#pragma unroll
            for (int u = 0; u < kSL; ++u) {
              const int c = cmap(min(s0 + tid + u * kBlock, lastc));
              bb[u] = chunk_bits(c);
              ch[u] = Chunk16<TIn>::load_scalar(kp.logits, rbase, kCV * c, V);
            }
            step(s0, ch, bb);
          }
        }
      };
      // value q of group t of a step's raw chunks
      auto rawv = [&](const u32x4 (&ch)[kSL], int t, int q) __attribute__((always_inline)) {
        float v[4];
        Chunk16<TIn>::unpack(ch[t / kGPL], t % kGPL, v);
        return v[q];
      };
      // a pass whose work is per group of processed values: f(g, z)
      auto group_pass = [&](auto &&f) __attribute__((always_inline)) {
        stream_pass(std::true_type{}, [&](const int (&gi)[kNG], const u32x4 (&ch)[kSL], const uint32_t (&mk)[kNG], bool fast)
                                          __attribute__((always_inline)) {
          if (fast) {
#pragma unroll
            for (int t = 0; t < kNG; ++t) {
              float z[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) z[q] = ((mk[t] >> q) & 1u) ? -INFINITY : zval(rawv(ch, t, q), true);
              f(gi[t], z);
            }
          } else {
#pragma unroll
            for (int t = 0; t < kNG; ++t) {
              float z[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) z[q] = ((mk[t] >> q) & 1u) ? -INFINITY : zval(rawv(ch, t, q), false);
              f(gi[t], z);
            }
          }
        });
      };
      // the smallest logit whose z has a key of at least kz (z is monotone in
      // the logit), or NaN when none has: "key(z) >= kz" is then "x >= it"
      // for every unmasked value (NaN compares false, as -inf would)
      auto x_at_least = [&](uint32_t kz) -> float {
        if (kz > fkey(INFINITY)) return __uint_as_float(0x7FC00000u);
        uint32_t lo = fkey(-INFINITY), hi = fkey(INFINITY);  // key(z(lo)) < kz <= key(z(hi)) once lo is excluded
        if (fkey(div_temp(-INFINITY, T, rT)) >= kz) return -INFINITY;
        while (hi - lo > 1u) {
          const uint32_t mid = lo + (hi - lo) / 2u;
          if (fkey(div_temp(key_to_float(mid), T, rT)) >= kz) hi = mid;
          else lo = mid;
        }
        return key_to_float(hi);
      };

      // ---- A. the row max and its first index (the best group of four, the
      // earlier group on a tie, then the first match in it)
      float lmax = -INFINITY;
      int lgrp = -1;
      float lz[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (gumbel && !top1) {
        // Gumbel-max rows need the max z and any index holding it (its draw
        // seeds the bound), not the first: z is monotone in the logit, so
        // the pass takes the max of the raw logits (NaN never wins) and
        // divides only each thread's largest
        stream_pass(std::false_type{}, [&](const int (&gi)[kNG], const u32x4 (&ch)[kSL], const uint32_t (&mk)[kNG], bool)
                                           __attribute__((always_inline)) {
#pragma unroll
          for (int t = 0; t < kNG; ++t) {
            float x[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = ((mk[t] >> c) & 1u) ? -INFINITY : rawv(ch, t, c);
            const float gm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            const bool take = gm > lmax || (gm == lmax && gm > -INFINITY && gi[t] < lgrp);
            lmax = take ? gm : lmax;
            lgrp = take ? gi[t] : lgrp;
#pragma unroll
            for (int c = 0; c < 4; ++c) lz[c] = take ? x[c] : lz[c];
          }
        });
      } else {
        group_pass([&](int g, const float z[4]) __attribute__((always_inline)) {
          const float gm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
          const bool take = gm > lmax || (gm == lmax && gm > -INFINITY && g < lgrp);
          lmax = take ? gm : lmax;
          lgrp = take ? g : lgrp;
#pragma unroll
          for (int c = 0; c < 4; ++c) lz[c] = take ? z[c] : lz[c];
        });
      }
      int lidx = 0x7FFFFFFF;
      if (lgrp >= 0) lidx = 4 * lgrp + (lz[0] == lmax ? 0 : lz[1] == lmax ? 1 : lz[2] == lmax ? 2 : 3);
      if (gumbel && !top1) lmax = zval(lmax, false);  // (the raw maximum's z; -inf stays -inf)
      unsigned long long lkey = ((unsigned long long)fkey(lmax) << 32) | (0xFFFFFFFFu - (uint32_t)lidx);
      patches([&](int i, float zz) {
        const unsigned long long k2 = ((unsigned long long)fkey(zz) << 32) | (0xFFFFFFFFu - (uint32_t)i);
        lkey = k2 > lkey ? k2 : lkey;
      });
      const unsigned long long mk = wg_max_u(sm, lkey);
      const float mf = key_to_float((uint32_t)(mk >> 32));
      const int argmax = (int)(0xFFFFFFFFu - (uint32_t)mk);
      PHASE_STAMP(kStampMax);
      if (!(mf > -INFINITY && mf < INFINITY)) {
        write_status(mf == INFINITY ? 2 : 1);  // a +inf value, or no finite value
        return;
      }
      if ((!gumbel || top1) && K == 0) {  // the first argmax is all the row needs
        if (tid == 0) {
          kp.token_ids[row] = argmax;
          if (kp.row_status) kp.row_status[row] = 0;
        }
        return;
      }
      const double m = (double)mf;
      const float wsc = T < 1.0f ? T : 1.0f;
      uint32_t t_m = 0;
      if (minp) t_m = min_p_key(sm, m, log((double)P.min_p), P.min_p);

      // Value ranges, as order keys.  Values with key >= T_hi are certainly
      // kept ("above"), values with key in [T_lo, T_hi) may hold tau and are
      // gathered, values below T_lo are dropped; values with key >= K_lo
      // (the top-logprob range) are gathered too.  Without truncation every
      // finite value is above; min-p alone gives tau exactly.
      const uint32_t kFinite = fkey(-INFINITY) + 1u;
      uint32_t T_lo = kFinite, T_hi = kFinite, K_lo = 0xFFFFFFFFu;
      bool topk_on = topk;
      uint32_t lo_max = 0, hi_max = 0;  // the threshold ranges' bounds (pass B)
      uint32_t klo_bin = 0xFFFFFFFFu;   // the top-logprob range's lower bound (pass B)
      uint32_t klo_k = 0;               // the lower bound of the top-k value's bin (pass B)
      double C_all = 0.0;  // top-p without top-k: the row's whole mass (window masses, fp64 sum)

      // ---- B. window histogram (the row kernel's bins), when a threshold
      // or the top-logprob list needs placing
      if (topk || topp || K > 0) {
        const float A = abin(mf, wsc);
        if (!(A > -INFINITY && A < INFINITY)) {  // the bin grid overflows for |m / T| beyond ~1e37
          defer_row();
          return;
        }
        wh[tid] = 0;
        __syncthreads();
        const bool need_c = topp && !topk;
        double csum = 0.0;
        if (topp) {  // counts and masses (only the top-p crossing reads the masses)
          group_pass([&](int g, const float z[4]) __attribute__((always_inline)) {
            float dsum = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float lb = win_pos(A, z[c], wsc);  // -inf: +inf
              const float a = __builtin_amdgcn_exp2f((z[c] - mf) * kLog2e);
              if (lb < (float)kWinBins) atomicAdd(&wh[(int)lb], hist_entry_s(a));
              dsum += a;
            }
            if (need_c) csum += (double)dsum;
          });
        } else {  // counts only: a 32-bit add to the bin's high word (count bits 44 and up)
          uint32_t *whc = reinterpret_cast<uint32_t *>(wh);
          group_pass([&](int g, const float z[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float lb = win_pos(A, z[c], wsc);  // -inf: +inf
              if (lb < (float)kWinBins) atomicAdd(&whc[2 * (int)lb + 1], 1u << 12);
            }
          });
        }
        // (the same atomic width as the pass above: the passes of other
        // waves may still run)
        patches([&](int i, float zz) {
          const float lb = win_pos(A, zz, wsc);
          const float a = __builtin_amdgcn_exp2f((zz - mf) * kLog2e);
          if (lb < (float)kWinBins) {
            if (topp) atomicAdd(&wh[(int)lb], hist_entry_s(a));
            else atomicAdd(reinterpret_cast<uint32_t *>(wh) + 2 * (int)lb + 1, 1u << 12);
          }
          if (need_c) csum += (double)a;
        });
        C_all = need_c ? wg_sum_d(sm, csum) : 0.0;
        __syncthreads();
        PHASE_STAMP(kStampHist);
        const int b = tid;
        const unsigned long long e = wh[b];
        uint32_t runc = (uint32_t)(e >> 44);
        unsigned long long runm = e & ((1ull << 44) - 1ull);
        block_scan_incl2(runc, runm, sm.red_c, sm.red_u);
        lc[b] = runc;
        lm[b] = runm;
        if (tid == 0) {
          sm.bu[16] = kNone;
          sm.bu[17] = kNone;
          sm.bu[18] = kNone;
          sm.bu[19] = kNone;
        }
        __syncthreads();
        // bins of the k-th and the K-th value
        const uint32_t cprev = b > 0 ? lc[b - 1] : 0u;
        if (topk && cprev < (uint32_t)P.top_k && runc >= (uint32_t)P.top_k) sm.bu[16] = (uint32_t)b;
        if (K > 0 && cprev < (uint32_t)K && runc >= (uint32_t)K) sm.bu[17] = (uint32_t)b;
        __syncthreads();
        const uint32_t bk = sm.bu[16], r0 = sm.bu[17];
        bool gen = false;
        if (topk && bk == kNone) {
          // the k-th value is deeper than the window: it decides unless
          // min-p's boundary lies inside the window (and so above it)
          const bool minp_in = minp && win_bin(A, key_to_float(t_m), wsc) < kWinBins;
          if (topp || !minp_in) gen = true;
          else topk_on = false;
        }
        // top-p: the bins where the cumulative mass crosses p times the
        // total mass of the top-k set (bounded below and above), or of the
        // row
        double tlo = 0.0, thi = 0.0;
        if (topp && !gen) {
          if (topk) {
            tlo = (double)P.top_p * (bk > 0 ? (double)lm[bk - 1] : 0.0);
            thi = (double)P.top_p * (double)lm[bk];
          } else {
            tlo = thi = (double)P.top_p * C_all * 16777216.0;
          }
          const double mprev = b > 0 ? (double)lm[b - 1] : 0.0, mcur = (double)lm[b];
          if (mprev < tlo && mcur >= tlo) sm.bu[18] = (uint32_t)b;
          if (mprev < thi && mcur >= thi) sm.bu[19] = (uint32_t)b;
        }
        __syncthreads();
        int plo = 0, phi = -1;
        if (topp && !gen) {
          const uint32_t lo = tlo <= 0.0 ? 0u : sm.bu[18], hi = sm.bu[19];
          if (hi == kNone) {
            gen = true;  // the crossing lies deeper than the window
          } else {
            // one bin of slack on each side (the masses are approximate;
            // the decision on the gathered values is exact)
            plo = max((int)(lo == kNone ? hi : lo) - 1, 0);
            phi = min((int)hi + 1, kWinBins - 1);
            if (topk) {
              plo = min(plo, (int)bk);
              phi = min(phi, (int)bk);
            }
          }
        }
        int r0hi = -1;
        if (K > 0 && !gen) {
          if (r0 != kNone) r0hi = (int)r0;
          else if (truncated) r0hi = kWinBins - 1;  // fewer than K values in the window: all of them
          else gen = true;                          // the list reaches below the window
        }
        if (gen) {
          __syncthreads();
          defer_row();
          return;
        }
        // the key bounds of those bins: bins 0..h hold the values with key
        // >= lo(h); bin h the values in [lo(h), lo(h - 1))
        if (tid < 5) {
          const int h = tid == 0 ? (int)bk : tid == 1 ? (int)bk - 1 : tid == 2 ? phi : tid == 3 ? plo - 1 : r0hi;
          const bool act = tid <= 1 ? topk_on : tid <= 3 ? topp : K > 0;
          uint32_t k = 0xFFFFFFFFu;  // (no bin above bin 0)
          if (act && h >= 0) k = fkey(win_floor_z(A, (float)h, wsc));
          sm.bu[20 + tid] = k;
        }
        __syncthreads();
        if (topk_on) {
          lo_max = max(lo_max, sm.bu[20]);
          hi_max = max(hi_max, sm.bu[21]);
          klo_k = sm.bu[20];
        }
        if (topp) {
          lo_max = max(lo_max, sm.bu[22]);
          hi_max = max(hi_max, sm.bu[23]);
        }
        if (minp) {
          lo_max = max(lo_max, t_m);
          hi_max = max(hi_max, t_m + 1u);
        }
        klo_bin = sm.bu[24];
        __syncthreads();  // the histogram's bytes are reused by the gather
        PHASE_STAMP(kStampDecided);
      }
      if (truncated) {
        if (topk_on || topp) {
          T_lo = lo_max;
          T_hi = hi_max;
          // top-p takes its share of the top-k set's mass, so the values
          // down to the k-th one are gathered too (those below tau drop out)
          if (topk_on && topp) T_lo = klo_k;
        } else {
          T_lo = T_hi = t_m;  // min-p alone: tau exactly
        }
      }
      if (K > 0) K_lo = truncated ? max(klo_bin, T_lo) : klo_bin;

      // ---- C. gather the ranges; above them: count, exact masses, Gumbel
      const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
      const uint32_t off0 = (uint32_t)P.offset, off1 = (uint32_t)(P.offset >> 32);
      double best_g = -INFINITY;
      int best_i = 0x7FFFFFFF;
      float bound = 0.0f, cut = kPruneNats;
      if (gumbel) {
        // the argmax (always kept) scores 1 / E; a value more than 33 ln 2 -
        // ln(bound) nats below the max cannot beat it (as in the row kernel)
        uint32_t w4[4];
        philox4x32_10((uint32_t)argmax >> 2, P.stream, off0, off1, key0, key1, w4);
        bound = (float)(1.0 / exp1_f64(w4[argmax & 3])) * 0.99999f;
        cut = fminf(kPruneNats, kLnInvEmin + (kPruneNats - 26.004f) - logf(bound));
      }
      const bool need_s = topp || K > 0;  // the kept mass (crossing, normaliser)
      double s_above = 0.0;
      uint32_t n_above = 0;
      if (tid == 0) sm.bu[25] = 0u;
      __syncthreads();
      // whether a value is gathered, or above the gathered ranges (kept)
      auto is_gat = [&](uint32_t k) { return (k >= K_lo) | ((k >= T_lo) & (k < T_hi)); };
      auto is_abv = [&](uint32_t k, float z) { return !is_gat(k) & (k >= T_hi) & (z > -INFINITY); };
      // the ranges as logit thresholds (threads 0..2, by bisection)
      if (tid < 3) {
        const float xt = x_at_least(tid == 0 ? K_lo : tid == 1 ? T_lo : T_hi);
        sm.bu[32 + tid] = __float_as_uint(xt);
      }
      __syncthreads();
      const float xK = __uint_as_float(sm.bu[32]), xTlo = __uint_as_float(sm.bu[33]), xThi = __uint_as_float(sm.bu[34]);
      stream_pass(std::false_type{}, [&](const int (&gi)[kNG], const u32x4 (&ch)[kSL], const uint32_t (&mk)[kNG], bool)
                                         __attribute__((always_inline)) {
        // cheap per-group part on the raw logits: gathered values (their z
        // taken exactly) appended per wave in ballot order; groups holding a
        // value above the ranges marked in hv
        uint32_t hv = 0;
#pragma unroll
        for (int t = 0; t < kNG; ++t) {
          bool anya = false;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float x = ((mk[t] >> c) & 1u) ? -INFINITY : rawv(ch, t, c);  // (NaN compares false)
            const bool below_hi = !(x >= xThi);
            const bool gt = (x >= xK) | ((x >= xTlo) & below_hi);
            anya |= !gt & !below_hi & (x > -INFINITY);
            const unsigned long long bal = __ballot(gt);
            if (bal) {
              uint32_t base = 0;
              if (lane == 0) base = atomicAdd(&sm.bu[25], (uint32_t)__popcll(bal));
              base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
              const uint32_t off = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
              if (gt && base + off < (uint32_t)kSCap) sk[base + off] = cand_key(zval(x, false), 4 * gi[t] + c);
            }
          }
          hv |= anya ? 1u << t : 0u;
        }
        // the groups above the ranges, one per lane per round (one copy of
        // the heavy code): count, exact masses, Philox, the linear-domain
        // bound and the fp64 scores of the values that can still win
        bool improved = false;
        if (!truncated) {
          // a row that keeps every value: nearly every group is above the
          // ranges, so the step's groups run unrolled (their Philox chains
          // interleave); the values that pass the linear-domain bound are
          // marked (bit 4 t + c) and scored in fp64 after the step, one
          // copy of that code
          uint32_t sv = 0;
#pragma unroll
          for (int t = 0; t < kNG; ++t) {
            if (!((hv >> t) & 1u)) continue;
            uint32_t am = 0;
            bool cand = false;
            float z[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float x = ((mk[t] >> c) & 1u) ? -INFINITY : rawv(ch, t, c);
              const bool ab = (x >= xThi) & !(x >= xK) & (x > -INFINITY);
              z[c] = ab ? zval(x, false) : -INFINITY;
              am |= ab ? 1u << c : 0u;
              cand |= ab && (mf - z[c] <= cut);
            }
            n_above += (uint32_t)__popc(am);
            // each value's mass exp(z - m) in fp32 (0 for -inf), for the sum
            // and the bound alike
            float qv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) qv[c] = __builtin_amdgcn_exp2f((z[c] - mf) * kLog2e);
            if (need_s) {
#pragma unroll
              for (int c = 0; c < 4; ++c) s_above += (double)qv[c];
            }
            if (gumbel && cand) {
              uint32_t w[4];
              philox4x32_10((uint32_t)gi[t], P.stream, off0, off1, key0, key1, w);
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const float wl = (float)w[c] * 0x1.fffffcp-33f;
                sv |= (((am >> c) & 1u) && (mf - z[c] <= cut) && wl * bound <= qv[c] * kSlack) ? 1u << (4 * t + c) : 0u;
              }
            }
          }
          while (sv) {
            const int bit = __builtin_ctz(sv);
            sv &= sv - 1u;
            const int t0 = bit >> 2, c0 = bit & 3;
            int g = 0;
            float xv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < kNG; ++t)
              if (t == t0) {
                g = gi[t];
#pragma unroll
                for (int c = 0; c < 4; ++c) xv[c] = rawv(ch, t, c);
              }
            const float zc = zval(c0 == 0 ? xv[0] : c0 == 1 ? xv[1] : c0 == 2 ? xv[2] : xv[3], false);
            uint32_t w[4];
            philox4x32_10((uint32_t)g, P.stream, off0, off1, key0, key1, w);
            const uint32_t wc = c0 == 0 ? w[0] : c0 == 1 ? w[1] : c0 == 2 ? w[2] : w[3];
            const double ge = (double)zc - log(exp1_f64(wc));
            if (ge > best_g || (ge == best_g && 4 * g + c0 < best_i)) {
              best_g = ge;
              best_i = 4 * g + c0;
              improved = true;
            }
          }
        } else {
          while (hv) {
            const int t0 = __builtin_ctz(hv);
            hv &= hv - 1u;
            int g = 0;
            float xr[4];
            uint32_t m4 = 0;
#pragma unroll
            for (int t = 0; t < kNG; ++t)
              if (t == t0) {
                g = gi[t];
                m4 = mk[t];
#pragma unroll
                for (int c = 0; c < 4; ++c) xr[c] = rawv(ch, t, c);
              }
            bool cand = false;
            uint32_t am = 0;
            float z[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float x = ((m4 >> c) & 1u) ? -INFINITY : xr[c];
              const bool ab = (x >= xThi) & !(x >= xK) & (x > -INFINITY);
              z[c] = ab ? zval(x, false) : -INFINITY;
              am |= ab ? 1u << c : 0u;
              cand |= ab && (mf - z[c] <= cut);
            }
            n_above += (uint32_t)__popc(am);
            if (need_s) {
              for (uint32_t mm = am; mm; mm &= mm - 1u) {
                const int c = __builtin_ctz(mm);
                const float zc = c == 0 ? z[0] : c == 1 ? z[1] : c == 2 ? z[2] : z[3];
                s_above += truncated ? exp_nonpos(sm.exp_tab, (double)zc - m) : exp_term(zc, m);
              }
            }
            if (gumbel && cand) {
              uint32_t w[4];
              philox4x32_10((uint32_t)g, P.stream, off0, off1, key0, key1, w);
              // lower bound of E (E >= w) against the best score so far
              uint32_t surv = 0;
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const float wl = (float)w[c] * 0x1.fffffcp-33f;
                const float qv = __builtin_amdgcn_exp2f((z[c] - mf) * kLog2e);
                surv |= (((am >> c) & 1u) && (mf - z[c] <= cut) && wl * bound <= qv * kSlack) ? 1u << c : 0u;
              }
              while (surv) {
                const int c = __builtin_ctz(surv);
                surv &= surv - 1u;
                const float zc = c == 0 ? z[0] : c == 1 ? z[1] : c == 2 ? z[2] : z[3];
                const uint32_t wc = c == 0 ? w[0] : c == 1 ? w[1] : c == 2 ? w[2] : w[3];
                const double ge = (double)zc - log(exp1_f64(wc));
                if (ge > best_g || (ge == best_g && 4 * g + c < best_i)) {
                  best_g = ge;
                  best_i = 4 * g + c;
                  improved = true;
                }
              }
            }
          }
        }
        if (gumbel && __ballot(improved)) {
          float mb = improved ? (float)exp(best_g - m) * 0.99999f : 0.0f;
          mb = wave_max_nonneg_f(mb);
          bound = fmaxf(bound, mb);
        }
      });
      patches([&](int i, float zz) {
        const uint32_t k = fkey(zz);
        if (is_gat(k)) {
          const uint32_t slot = atomicAdd(&sm.bu[25], 1u);
          if (slot < (uint32_t)kSCap) sk[slot] = cand_key(zz, i);
        } else if (is_abv(k, zz)) {
          ++n_above;
          if (need_s) s_above += truncated ? exp_nonpos(sm.exp_tab, (double)zz - m) : exp_term(zz, m);
          if (gumbel) {
            uint32_t w[4];
            philox4x32_10((uint32_t)i >> 2, P.stream, off0, off1, key0, key1, w);
            const uint32_t wc = (i & 3) == 0 ? w[0] : (i & 3) == 1 ? w[1] : (i & 3) == 2 ? w[2] : w[3];
            const double ge = (double)zz - log(exp1_f64(wc));
            if (ge > best_g || (ge == best_g && i < best_i)) {
              best_g = ge;
              best_i = i;
            }
          }
        }
      });
      const uint32_t cnt_above = (uint32_t)wg_sum_u(sm, n_above);  // (its barriers also order the appends)
      const double S_above = need_s ? wg_sum_d(sm, s_above) : 0.0;
      const uint32_t n_g = sm.bu[25];
      PHASE_STAMP(kStampGathered);
      if (n_g > (uint32_t)kSCap) {
        defer_row();
        return;
      }
      const int n = (int)n_g;

      // ---- the gathered list, sorted by (value desc, index asc): a key's
      // position is the number of larger keys (keys are distinct)
      for (int j = tid; j < n; j += kBlock) {
        const unsigned long long c = sk[j];
        uint32_t r = 0;
        int i = 0;
        for (; i + 8 <= n; i += 8) {
          unsigned long long kk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) kk[u] = sk[i + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) r += kk[u] > c ? 1u : 0u;
        }
        for (; i < n; ++i) r += sk[i] > c ? 1u : 0u;
        srt[r] = c;
      }
      __syncthreads();
      PHASE_STAMP(kStampX3Ranked);
      auto keyof = [&](int j) { return (uint32_t)(srt[j] >> 32); };
      auto zof = [&](int j) { return key_to_float(keyof(j)); };
      auto idxof = [&](int j) { return (int)(~(uint32_t)srt[j]); };
      // inclusive prefix of exact masses exp(z - m) along the list (each
      // thread owns kSCap / kBlock consecutive positions)
      {
        constexpr int kPer = kSCap / kBlock;
        double qv[kPer];
        double own = 0.0;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int j = tid * kPer + u;
          qv[u] = j < n ? exp_nonpos(sm.exp_tab, (double)zof(j) - m) : 0.0;
          own += qv[u];
        }
        double run = block_scan_incl<double>(own, sm.red_d) - own;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int j = tid * kPer + u;
          run += qv[u];
          if (j < n) pre[j] = run;
        }
      }
      // the list's head (keys >= K_lo) lies above the above-range, the rest
      // below it; nK = the head's length (the whole list when nothing is above)
      const bool has_above = cnt_above > 0u;
      if (tid == 0) {
        sm.bu[26] = (uint32_t)n;  // nK
        sm.bu[27] = (uint32_t)n;  // end of the top-k tie group
        sm.bu[28] = 0x7FFFFFFFu;  // top-p crossing
        sm.bu[29] = 0u;           // first position of the crossing's tie group
        sm.bu[30] = (uint32_t)n;  // end of the kept list
      }
      __syncthreads();
      if (has_above)
        for (int j = tid; j < n; j += kBlock)
          if (keyof(j) < K_lo && (j == 0 || keyof(j - 1) >= K_lo)) sm.bu[26] = (uint32_t)j;
      __syncthreads();
      const int nK = (int)sm.bu[26];
      const double ab = has_above ? S_above : 0.0;
      auto cum = [&](int j) { return pre[j] + (j >= nK ? ab : 0.0); };               // mass up to and with j
      auto cumb = [&](int j) { return (j > 0 ? pre[j - 1] : 0.0) + (j >= nK ? ab : 0.0); };  // mass before j
      bool bad = false;
      // top-k: the value of rank k (values above the list's tail count too);
      // past the list's end it lies below T_lo, under another threshold's
      // range, and does not bind (kout)
      uint32_t tk = 0;
      bool kout = false;
      if (topk_on) {
        const int r = P.top_k - 1;
        const int j = (!has_above || r < nK) ? r : (r < nK + (int)cnt_above ? -1 : r - (int)cnt_above);
        if (j < 0) bad = true;
        else if (j >= n) kout = true;
        else tk = keyof(j);
        if (!bad && !kout)
          for (int q = tid; q < n; q += kBlock)
            if (keyof(q) < tk && (q == 0 || keyof(q - 1) >= tk)) sm.bu[27] = (uint32_t)q;
      }
      __syncthreads();
      const int ek = (int)sm.bu[27];
      // top-p: the first tie-group end whose cumulative mass reaches p times
      // the top-k set's mass (exact) or the row's (window masses)
      uint32_t tp = 0;
      double ctot = 0.0, target = 0.0;
      if (topp && topk_on && kout) bad = true;  // (the list reaches down to the k-th value's bin)
      if (topp && !bad) {
        ctot = topk_on ? (ek > 0 ? cum(ek - 1) : 0.0) : C_all;
        target = (double)P.top_p * ctot;
        for (int e = tid; e < n; e += kBlock) {
          const bool end = (e == n - 1) || (keyof(e + 1) != keyof(e));
          const unsigned long long bal = __ballot(end && cum(e) >= target);
          if (bal && lane == __ffsll((long long)bal) - 1) atomicMin(&sm.bu[28], (uint32_t)e);
        }
      }
      __syncthreads();
      if (topp && !bad) {
        const uint32_t e = sm.bu[28];
        if (e == 0x7FFFFFFFu) {
          // no tie-group end reaches the target: the crossing lies below
          // T_lo, where another threshold's range keeps tau above it -- if
          // the mass of everything from T_lo up is short of the target by
          // more than the total's error
          const double tot = n > 0 ? cum(n - 1) : ab;
          if (tot >= target || target - tot < kTopPMarginRel * ctot) bad = true;
        } else {
          const uint32_t ke = keyof((int)e);
          for (int j = tid; j <= (int)e; j += kBlock)
            if (keyof(j) == ke && (j == 0 || keyof(j - 1) != ke)) sm.bu[29] = (uint32_t)j;
          __syncthreads();
          const int gs = (int)sm.bu[29];
          const double c_new = cum((int)e), c_prev = cumb(gs);
          if (c_prev >= target) bad = true;  // the crossing lies among the values above the list
          if (!topk_on) {
            // the row's mass is approximate: a crossing this close to its
            // target, on a side where moving it would change tau, goes to
            // the row kernel
            const uint32_t tkm = minp ? t_m : 0u;
            const uint32_t kprev = (gs > 0 && !(has_above && gs == nK)) ? keyof(gs - 1) : 0xFFFFFFFFu;
            const bool close_lo = c_new - target < kTopPMarginRel * ctot && ke > tkm;
            const bool close_hi = target - c_prev < kTopPMarginRel * ctot && kprev > tkm;
            if (close_lo || close_hi) bad = true;
          }
          tp = ke;
        }
      }
      // tau, the kept list [0, et), and the checks that the ranges held it
      uint32_t tau = truncated ? 0u : kFinite;
      if (topk_on) tau = max(tau, tk);
      if (topp) tau = max(tau, tp);
      if (minp) tau = max(tau, t_m);
      if (truncated && (tau < T_lo || (has_above && tau > T_hi))) bad = true;
      if (!bad)
        for (int j = tid; j < n; j += kBlock)
          if (keyof(j) < tau && (j == 0 || keyof(j - 1) >= tau)) sm.bu[30] = (uint32_t)j;
      __syncthreads();
      const int et = (int)sm.bu[30];
      // the top-logprob list must come from the head when values lie above
      if (K > 0 && has_above && et > nK && nK < K) bad = true;
      if (__syncthreads_or(bad)) {
        defer_row();
        return;
      }
      PHASE_STAMP(kStampThresholds);
      const double lnS = need_s ? log(cumb(et)) : 0.0;
      for (int q = tid; q < K; q += kBlock) {
        const int64_t o = (int64_t)row * K + q;
        if (q < et) {
          kp.top_lp_vals[o] = (float)(((double)zof(q) - m) - lnS);
          kp.top_lp_ids[o] = idxof(q);
        } else {
          kp.top_lp_vals[o] = -INFINITY;
          kp.top_lp_ids[o] = -1;
        }
      }
      // Gumbel-max: the kept values of the list, then the best over the
      // workgroup (ties to the smaller index)
      if (gumbel) {
        for (int j = tid; j < et; j += kBlock) {
          const int i = idxof(j);
          uint32_t w[4];
          philox4x32_10((uint32_t)i >> 2, P.stream, off0, off1, key0, key1, w);
          const uint32_t wc = (i & 3) == 0 ? w[0] : (i & 3) == 1 ? w[1] : (i & 3) == 2 ? w[2] : w[3];
          const double ge = (double)zof(j) - log(exp1_f64(wc));
          if (ge > best_g || (ge == best_g && i < best_i)) {
            best_g = ge;
            best_i = i;
          }
        }
        wg_best(sm, best_g, best_i);
      }
      if (tid == 0) {
        kp.token_ids[row] = gumbel ? best_i : argmax;
        if (kp.row_status) kp.row_status[row] = 0;
      }
    };
    row_body();
    __syncthreads();
    PHASE_STAMP(kStampEnd);
  }
}

// ln E in fp32 for the word x, E = -ln(1 - w), w = (x + 1/2) 2^-32 (the
// draw of exp1_f64), for ranking only: below w = 1/16 by the series of
// -ln(1 - w) to w^6 (relative truncation below 1e-8), above it from 1 - w
// taken from the complement of x (relative error 6e-8, so E's relative error
// stays below 3e-6 where -ln(1 - w) >= 1/16).  The result is within 1e-5 of
// ln E; kChunkMargin leaves a hundredfold slack for two scores' errors.
DEV float ln_exp1_f32(uint32_t x) {
  const float w = ((float)x + 0.5f) * 0x1p-32f;
  const float q = ((float)(0xFFFFFFFFu - x) + 0.5f) * 0x1p-32f;
  const float es = w * (1.0f + w * (0.5f + w * (1.0f / 3.0f + w * (0.25f + w * (0.2f + w * (1.0f / 6.0f))))));
  const float el = -__logf(q);
  return __logf(w < 0.0625f ? es : el);  // (both sides computed: no branch)
}
constexpr float kChunkMargin = 0x1p-10f;
constexpr uint32_t kChunkExact = 4u;  // chunk record: the score word holds an exact fp64 score
// Order keys of fp64 values (larger value, larger key; -0 < +0), and back.
DEV unsigned long long dkey(double d) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
DEV double key_to_double(unsigned long long k) {
  return __longlong_as_double((long long)((k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k));
}

// A workgroup's Gumbel-max pick among its values whose fp32 score is at
// least thr (a set that holds the exact winner, thr lying within
// kChunkMargin of the best fp32 score).  Most often the set has one value:
// then it is the winner, found without any fp64 work (single; its index,
// z and word in pk).  Otherwise the set's exact fp64 scores z - ln E decide
// (ties: the smaller index) through two LDS atomics (pk.best_key,
// pk.best_idx).  NG groups of four per thread, ng of them used, value c of
// group u at index base + 4 (tid + NT u) + c.  The caller clears pk.n,
// pk.best_key and pk.best_idx before the barrier that follows thr's inputs.
struct PickLds {
  unsigned long long best_key;
  int best_idx;
  uint32_t n;  // values in the set
  int idx;     // the set's value, when it has one
  uint32_t w;
  float z;
};
template <int NG, int NT>
DEV bool pick_candidate(const float (&z)[NG][4], const float (&g32)[NG][4], const uint32_t (&wv)[NG][4], int ng,
                        int base, float thr, PickLds &pk) {
  const int tid = tidx();
  uint32_t myc = 0;
  int myi = 0x7FFFFFFF;
  uint32_t myw = 0;
  float myz = 0.0f;
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    if (u >= ng) break;
    const int i0 = base + 4 * (tid + NT * u);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (g32[u][c] >= thr) {
        ++myc;
        myi = i0 + c;
        myw = wv[u][c];
        myz = z[u][c];
      }
  }
  if (myc != 0u) atomicAdd(&pk.n, myc);
  if (myc == 1u) {  // (read only when no other thread has a value in the set)
    pk.idx = myi;
    pk.w = myw;
    pk.z = myz;
  }
  __syncthreads();
  if (pk.n == 1u) return true;  // (workgroup-uniform)
  double tg = -INFINITY;
  int ti = 0x7FFFFFFF;
#pragma unroll
  for (int u = 0; u < NG; ++u) {
    if (u >= ng) break;
    const int i0 = base + 4 * (tid + NT * u);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (g32[u][c] >= thr) {
        const double ge = ((double)z[u][c] - log(exp1_f64(wv[u][c]))) + 0.0;  // (+0 for -0)
        if (ge > tg || (ge == tg && i0 + c < ti)) {
          tg = ge;
          ti = i0 + c;
        }
      }
  }
  const unsigned long long tk = dkey(tg);
  if (ti != 0x7FFFFFFF) atomicMax(&pk.best_key, tk);
  __syncthreads();
  const unsigned long long bk = pk.best_key;
  if (ti != 0x7FFFFFFF && tk == bk) atomicMin(&pk.best_idx, ti);
  __syncthreads();
  return false;
}

// ---------------------------------------------------------------- small rows
// Rows of at most kSmallV values that keep every value -- Gumbel-max over
// the whole row, or greedy ([A] "Nine lines, and exactly one call site": the
// path with no truncation) -- with no penalties, logits processors or
// top-logprob list.  The row kernel's general machinery (tables, exchanges,
// candidate lists) is all latency for them: here one workgroup of
// kSmallBlock threads takes a row with every value in registers, and the
// row's steps meet at a handful of workgroup barriers.  The arithmetic is
// the row kernel's: z = x / T correctly rounded, the first argmax, the fp64
// sum of exp(z - m) (in another order, so it may round differently), the
// fp64 Gumbel scores z - ln E (here only for the values whose fp32 score is
// near the best, which provably holds the winner), lp = fl32(z - m - ln S)
// and p = 2^(lp log2 e).
constexpr int kSmallBlock = 256;
constexpr int kSmallG = kSmallV / 4 / kSmallBlock;  // groups of four per thread
static_assert(kSmallV % (4 * kSmallBlock) == 0, "whole groups per thread");

// z = x / T, correctly rounded, of the group of four raw values at index l
// (in place); NaN gives -inf, indices from V on give -inf.  Values whose
// magnitude lies in [T 2^-99, T 2^99] (xlo_b, xhi_b: those bounds' bits)
// take one reciprocal product and one fma correction, others the division.
DEV void temper4(float (&v)[4], int l, int V, float T, float rT, uint32_t xlo_b, uint32_t xhi_b) {
  uint32_t a[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(v[c]) & 0x7FFFFFFFu;
  const bool fast = (max(max(a[0], a[1]), max(a[2], a[3])) <= xhi_b) & (min(min(a[0], a[1]), min(a[2], a[3])) >= xlo_b);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float x = v[c];
    const float q = x * rT;
    float zz = __builtin_fmaf(__builtin_fmaf(-q, T, x), rT, q);
    if (!fast) zz = (x == x ? x : -INFINITY) / T + 0.0f;
    v[c] = l + c < V ? zz : -INFINITY;
  }
}

template <typename TIn>
__global__ __launch_bounds__(kSmallBlock) void small_kernel(KernelArgs ka) {
  const KernelParams &kp = ka.kp;
  constexpr int kW = kSmallBlock / 64;
  __shared__ unsigned long long red_u[kW];
  __shared__ double red_d[kW];
  __shared__ int red_i[kW];
  __shared__ PickLds pk;
  const int tid = tidx();
  const int lane = tid & 63, wave = tid >> 6;
  const unsigned it = 0;  // (stamps)
  PHASE_STAMP(kStampStart);
  const RowParam P = kp.rows ? kp.rows[blockIdx.x] : ka.rows[blockIdx.x];
  const int row = P.row;
  const int V = kp.vocab;
  PHASE_STAMP(kStampRow);
  PHASE_RECORD(kStampRowIndex, row + 1);
  // groups of four per thread that the row fills (the same for every thread)
  const int ng = min(kSmallG, (V + 4 * kSmallBlock - 1) / (4 * kSmallBlock));
  const float T = P.temperature;
  const float rT = 1.0f / T;
  const uint32_t xlo_b = __float_as_uint(T * 0x1p-99f);
  const uint32_t xhi_b = min(__float_as_uint(T * 0x1p99f), 0x7F7FFFFFu);
  const int64_t rbase = (int64_t)row * kp.row_stride;
  const bool vec = kp.vec_ok & 1;
  const bool gumbel = !(P.flags & RF_TOP1) && kp.path != PATH_GREEDY;
  const int lastg = (V - 1) & ~3;
  // the values: group u of this thread starts at 4 (tid + kSmallBlock u)
  float z[kSmallG][4];
#pragma unroll
  for (int u = 0; u < kSmallG; ++u) {
    if (u >= ng) break;
    const int l = 4 * (tid + kSmallBlock * u);
    if (vec) {
      Loader<TIn>::load4(kp.logits, rbase + min(l, lastg), z[u]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) z[u][c] = Loader<TIn>::load1(kp.logits, rbase + min(l + c, V - 1));
    }
  }
#pragma unroll
  for (int u = 0; u < kSmallG && u < ng; ++u) temper4(z[u], 4 * (tid + kSmallBlock * u), V, T, rT, xlo_b, xhi_b);
  PHASE_STAMP(kStampLoaded);
  // the row max and its first index (the best group by a strict compare,
  // groups in index order, then the first match in it)
  float lmax = -INFINITY;
  int lidx = 0x7FFFFFFF;
#pragma unroll
  for (int u = 0; u < kSmallG; ++u) {
    if (u >= ng) break;
    const float gm = fmaxf(fmaxf(z[u][0], z[u][1]), fmaxf(z[u][2], z[u][3]));
    if (gm > lmax) {
      lmax = gm;
      lidx = 4 * (tid + kSmallBlock * u) + (z[u][0] == gm ? 0 : z[u][1] == gm ? 1 : z[u][2] == gm ? 2 : 3);
    }
  }
  unsigned long long mk = wave_max_u(((unsigned long long)fkey(lmax) << 32) | (0xFFFFFFFFu - (uint32_t)lidx));
  if (lane == 0) red_u[wave] = mk;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kW; ++w) mk = red_u[w] > mk ? red_u[w] : mk;
  const float mf = key_to_float((uint32_t)(mk >> 32));
  const int argmax = (int)(0xFFFFFFFFu - (uint32_t)mk);
  PHASE_STAMP(kStampMax);
  const bool want_out = kp.probs != nullptr || kp.logprobs != nullptr;
  if (!(mf > -INFINITY && mf < INFINITY)) {  // no finite value (status 1) or a +inf value (status 2)
    if (want_out)
      for (int l = tid; l < V; l += kSmallBlock) {
        if (kp.probs) kp.probs[(int64_t)row * V + l] = 0.0f;
        if (kp.logprobs) kp.logprobs[(int64_t)row * V + l] = -INFINITY;
      }
    if (tid == 0) {
      kp.token_ids[row] = -1;
      if (kp.row_status) kp.row_status[row] = mf == INFINITY ? 2 : 1;
    }
    return;
  }
  const double m = (double)mf;
  // the normaliser: the fp64 sum of exp(z - m) (per thread in index order,
  // then across the wave and the waves in a fixed order)
  double lnS = 0.0;
  if (want_out) {
    double sx = 0.0;
#pragma unroll
    for (int u = 0; u < kSmallG && u < ng; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) sx += exp_term(z[u][c], m);
    sx = wave_sum_d(sx);
    if (lane == 0) red_d[wave] = sx;
    __syncthreads();
    double t = red_d[0];
#pragma unroll
    for (int w = 1; w < kW; ++w) t += red_d[w];
    lnS = log(t);
  }
  PHASE_STAMP(kStampThresholds);
  // Gumbel-max: every finite value gets an fp32 score z - ln E; the values
  // within kChunkMargin of the best one hold the winner (pick_candidate)
  int best_i = 0x7FFFFFFF;
  if (gumbel) {
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const uint32_t off0 = (uint32_t)P.offset, off1 = (uint32_t)(P.offset >> 32);
    float g32[kSmallG][4];
    uint32_t wv[kSmallG][4];
    float gmx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSmallG; ++u) {
      if (u >= ng) break;
      const int i0 = 4 * (tid + kSmallBlock * u);
      const float gm = fmaxf(fmaxf(z[u][0], z[u][1]), fmaxf(z[u][2], z[u][3]));
      if (i0 < V && gm > -INFINITY) {
        philox4x32_10((uint32_t)i0 >> 2, P.stream, off0, off1, key0, key1, wv[u]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          g32[u][c] = z[u][c] - ln_exp1_f32(wv[u][c]);  // (-inf stays -inf)
          gmx = fmaxf(gmx, g32[u][c]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) g32[u][c] = -INFINITY;
      }
    }
    uint32_t gk = lane63_u32(wave_scanmax_u32(fkey(gmx)));
    if (lane == 0) red_i[wave] = (int)gk;
    if (tid == 0) {
      pk.best_key = 0ull;
      pk.best_idx = 0x7FFFFFFF;
      pk.n = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kW; ++w) gk = max(gk, (uint32_t)red_i[w]);
    const float G32 = key_to_float(gk);
    const float thr = G32 - (kChunkMargin + fabsf(G32) * 0x1p-20f);
    best_i = pick_candidate<kSmallG, kSmallBlock>(z, g32, wv, ng, 0, thr, pk) ? pk.idx : pk.best_idx;
  }
  PHASE_STAMP(kStampGumbel);
  if (tid == 0) {
    kp.token_ids[row] = gumbel ? best_i : argmax;
    if (kp.row_status) kp.row_status[row] = 0;
  }
  // outputs: every value is kept
  if (want_out) {
#pragma unroll
    for (int u = 0; u < kSmallG; ++u) {
    if (u >= ng) break;
      const int l = 4 * (tid + kSmallBlock * u);
      float lv[4], pv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lv[c] = z[u][c] > -INFINITY ? (float)(((double)z[u][c] - m) - lnS) : -INFINITY;
        pv[c] = z[u][c] > -INFINITY ? __builtin_amdgcn_exp2f(lv[c] * kLog2e) : 0.0f;
      }
      const int64_t o = (int64_t)row * V + l;
      if ((kp.vec_ok & 2) && l + 3 < V) {
        if (kp.probs) *reinterpret_cast<f32x4 *>(kp.probs + o) = f32x4{pv[0], pv[1], pv[2], pv[3]};
        if (kp.logprobs) *reinterpret_cast<f32x4 *>(kp.logprobs + o) = f32x4{lv[0], lv[1], lv[2], lv[3]};
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (l + c < V) {
            if (kp.probs) kp.probs[o + c] = pv[c];
            if (kp.logprobs) kp.logprobs[o + c] = lv[c];
          }
      }
    }
  }
  PHASE_STAMP(kStampEnd);
}

// ---------------------------------------------------------------- chunked rows
// Rows longer than kSmallV of the same kind (every value kept, Gumbel-max or
// greedy, no penalties, processors or top-logprob list) in a step that wants
// only token ids.  Neither the normaliser nor the row max is needed for
// that: the Gumbel-max winner is the first index of the largest fp64 score
// z - ln E ([A] "Nine lines, and exactly one call site"), greedy's the first
// index of the largest z.  So each workgroup scores one chunk of the row on
// its own and the last chunk of the row to arrive merges the chunks' bests.
// No workgroup waits for another.
template <typename TIn>
__global__ __launch_bounds__(kChunkBlock) void chunk_kernel(KernelArgs ka) {
  const KernelParams &kp = ka.kp;
  constexpr int kW = kChunkBlock / 64;
  __shared__ unsigned long long red_u[kW];
  __shared__ int red_i[kW];
  __shared__ uint32_t last_s;
  __shared__ PickLds pk;
  const int tid = tidx();
  const int lane = tid & 63, wave = tid >> 6;
  const int ri = blockIdx.y;   // the record
  const int ch = blockIdx.x;   // the chunk
  const int U = kp.chunk_u;
  const unsigned it = blockIdx.y;  // (stamps: the first row's chunks)
  PHASE_STAMP(kStampStart);
  const RowParam P = kp.rows ? kp.rows[ri] : ka.rows[ri];
  const int row = P.row;
  PHASE_STAMP(kStampRow);
  PHASE_RECORD(kStampRowIndex, row + 1);
  const int V = kp.vocab;
  const float T = P.temperature;
  const float rT = 1.0f / T;
  const uint32_t xlo_b = __float_as_uint(T * 0x1p-99f);
  const uint32_t xhi_b = min(__float_as_uint(T * 0x1p99f), 0x7F7FFFFFu);
  const int64_t rbase = (int64_t)row * kp.row_stride;
  const bool vec = kp.vec_ok & 1;
  const bool gumbel = !(P.flags & RF_TOP1) && kp.path != PATH_GREEDY;
  const int lastg = (V - 1) & ~3;
  const int c0 = ch * 4 * kChunkBlock * U;  // the chunk's first index
  // group u of this thread starts at c0 + 4 (tid + kChunkBlock u)
  float z[kChunkMaxU][4];
#pragma unroll
  for (int u = 0; u < kChunkMaxU; ++u) {
    if (u >= U) break;
    const int l = c0 + 4 * (tid + kChunkBlock * u);
    if (vec) {
      Loader<TIn>::load4(kp.logits, rbase + min(l, lastg), z[u]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) z[u][c] = Loader<TIn>::load1(kp.logits, rbase + min(l + c, V - 1));
    }
  }
#pragma unroll
  for (int u = 0; u < kChunkMaxU; ++u) {
    if (u >= U) break;
    temper4(z[u], c0 + 4 * (tid + kChunkBlock * u), V, T, rT, xlo_b, xhi_b);
  }
  PHASE_STAMP(kStampLoaded);
  // the chunk's max and its first index
  float lmax = -INFINITY;
  int lidx = 0x7FFFFFFF;
#pragma unroll
  for (int u = 0; u < kChunkMaxU; ++u) {
    if (u >= U) break;
    const float gm = fmaxf(fmaxf(z[u][0], z[u][1]), fmaxf(z[u][2], z[u][3]));
    if (gm > lmax) {
      lmax = gm;
      lidx = c0 + 4 * (tid + kChunkBlock * u) + (z[u][0] == gm ? 0 : z[u][1] == gm ? 1 : z[u][2] == gm ? 2 : 3);
    }
  }
  unsigned long long mk = wave_max_u(((unsigned long long)fkey(lmax) << 32) | (0xFFFFFFFFu - (uint32_t)lidx));
  if (lane == 0) red_u[wave] = mk;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kW; ++w) mk = red_u[w] > mk ? red_u[w] : mk;
  const float mf = key_to_float((uint32_t)(mk >> 32));
  const int amax = (int)(0xFFFFFFFFu - (uint32_t)mk);
  PHASE_STAMP(kStampMax);
  // Gumbel-max within the chunk: every finite value gets an fp32 score; the
  // values within kChunkMargin of the chunk's best one hold its winner
  // (pick_candidate: usually one value, else settled by fp64 scores)
  double best_g = -INFINITY;
  int best_i = 0x7FFFFFFF;
  bool single = false;  // the chunk's winner is its one value near the best fp32 score (pk)
  float win32 = -INFINITY;  // then its fp32 score
  const uint32_t cst = mf == INFINITY ? 2u : mf > -INFINITY ? 0u : 1u;  // +inf / no finite value
  if (gumbel && cst == 0u) {
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const uint32_t off0 = (uint32_t)P.offset, off1 = (uint32_t)(P.offset >> 32);
    float g32[kChunkMaxU][4];
    uint32_t wv[kChunkMaxU][4];
    float gmx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kChunkMaxU; ++u) {
      if (u >= U) break;
      const int i0 = c0 + 4 * (tid + kChunkBlock * u);
      const float gm = fmaxf(fmaxf(z[u][0], z[u][1]), fmaxf(z[u][2], z[u][3]));
      if (i0 < V && gm > -INFINITY) {
        philox4x32_10((uint32_t)i0 >> 2, P.stream, off0, off1, key0, key1, wv[u]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          g32[u][c] = z[u][c] - ln_exp1_f32(wv[u][c]);  // (-inf stays -inf)
          gmx = fmaxf(gmx, g32[u][c]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) g32[u][c] = -INFINITY;
      }
    }
    PHASE_STAMP(kStampGumbelListed);
    // the chunk's best fp32 score (finite: the chunk max is finite)
    uint32_t gk = lane63_u32(wave_scanmax_u32(fkey(gmx)));
    if (lane == 0) red_i[wave] = (int)gk;
    if (tid == 0) {
      pk.best_key = 0ull;
      pk.best_idx = 0x7FFFFFFF;
      pk.n = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kW; ++w) gk = max(gk, (uint32_t)red_i[w]);
    const float G32 = key_to_float(gk);
    const float thr = G32 - (kChunkMargin + fabsf(G32) * 0x1p-20f);
    single = pick_candidate<kChunkMaxU, kChunkBlock>(z, g32, wv, U, c0, thr, pk);
    win32 = G32;
    PHASE_STAMP(kStampGumbelBatched);
    if (!single) {
      best_g = key_to_double(pk.best_key);
      best_i = pk.best_idx;
    }
  }
  PHASE_STAMP(kStampGumbel);
  // the chunk's result (Gumbel-max rows: its winner's z and word, or its
  // exact fp64 score when several values were near its best, with the
  // winner's index and the chunk's status; greedy rows: the max's order
  // key), then its arrival: one atomic add on the row's word, whose count the
  // last chunk to arrive resets to zero for the next launch (every launch
  // runs to its end: no chunk waits for another)
  ChunkRec *recs = kp.chunk_recs + (int64_t)ri * kp.chunk_stride;
  if (tid == 0) {
    if (gumbel) {
      // b: the winner's fp32 score << 32 | flags << 28 | its index (< 2^20)
      if (single) {
        atomic_st(&recs[ch].a, ((unsigned long long)__float_as_uint(pk.z) << 32) | pk.w);
        atomic_st(&recs[ch].b, ((unsigned long long)__float_as_uint(cst == 0u ? win32 : -INFINITY) << 32) |
                                   (cst << 28) | (uint32_t)pk.idx);
      } else {
        atomic_st(&recs[ch].a, (unsigned long long)__double_as_longlong(best_g));
        atomic_st(&recs[ch].b, ((unsigned long long)__float_as_uint(cst == 0u ? (float)best_g : -INFINITY) << 32) |
                                   ((cst | kChunkExact) << 28) | ((uint32_t)best_i & 0x0FFFFFFFu));
      }
    } else {
      atomic_st(&recs[ch].a, mk);
    }
    order_release();
    PHASE_STAMP(kStampReleased);
    unsigned long long *word = kp.chunk_words + (int64_t)kChunkWordStride * ri;
    const unsigned long long old = __hip_atomic_fetch_add(word, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == (unsigned long long)(kp.chunk_n - 1);
    if (last) {
      atomic_st(word, 0ull);
      order_acquire();
    }
    last_s = last ? 1u : 0u;
    PHASE_STAMP(kStampArrived);
  }
  __syncthreads();
  if (!last_s || wave != 0) return;
  // the merge (one wave): lane l holds chunks l, l + 64, l + 128, l + 192,
  // read in one round trip
  const int C = kp.chunk_n;
  u32x4 r[4];
  coh_load16x4(&recs[min(lane, C - 1)], &recs[min(lane + 64, C - 1)], &recs[min(lane + 128, C - 1)],
               &recs[min(lane + 192, C - 1)], r[0], r[1], r[2], r[3]);
  unsigned long long k = 0;  // greedy: the max's order key; Gumbel-max: the row's status as a key
  double g = -INFINITY;
  int gi = 0x7FFFFFFF;
  if (gumbel) {
    // each chunk's best score in fp32 (its fp32 score, or its exact score
    // rounded): the chunks within kChunkMargin of the best hold the row's
    // winner; one such chunk is the winner, several are settled by their
    // exact fp64 scores
    float a32[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a32[t] = -INFINITY;
      if (lane + 64 * t >= C) continue;
      const uint32_t st = (r[t].z >> 28) & 3u;
      const unsigned long long sk = (unsigned long long)fkey(st == 2u ? INFINITY : st == 1u ? -INFINITY : 0.0f) << 32;
      k = sk > k ? sk : k;
      if (st == 0u) a32[t] = __uint_as_float(r[t].w);
    }
    const float G = key_to_float(lane63_u32(wave_scanmax_u32(fkey(fmaxf(fmaxf(a32[0], a32[1]), fmaxf(a32[2], a32[3]))))));
    if (G > -INFINITY) {
      const float thr = G - (kChunkMargin + fabsf(G) * 0x1p-20f);
      uint32_t nc = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) nc += (uint32_t)__popcll(__ballot(a32[t] >= thr));
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (a32[t] >= thr) {
          const int ij = (int)(r[t].z & 0x0FFFFFFFu);
          double gj = 0.0;  // one candidate: any finite score
          if (nc > 1u)
            gj = ((r[t].z >> 28) & kChunkExact) ? f64_of(r[t].x, r[t].y)
                                                : ((double)__uint_as_float(r[t].y) - log(exp1_f64(r[t].x))) + 0.0;
          if (gj > g || (gj == g && ij < gi)) {
            g = gj;
            gi = ij;
          }
        }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (lane + 64 * t >= C) break;
      const unsigned long long kj = u64_of(r[t].x, r[t].y);
      k = kj > k ? kj : k;
    }
  }
  finish_row(kp, false, row, gumbel, false, k, g, gi, true);
  if (lane == 0) PHASE_STAMP_ONE(kStampToken);
}

template <typename TIn, bool PEN>
hipError_t launch_t(const KernelArgs &ka, bool cooperative, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const KernelParams &kp = ka.kp;
  const size_t lds = kernel_lds_bytes(kp.slice, kp.hash_slots, kp.bias_slots, PEN);
  const dim3 grid(kp.n_groups * kp.G), block(kBlock);
  void *args[] = {const_cast<KernelArgs *>(&ka)};
  if (cooperative) {
    hipError_t e;
    if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&row_kernel<TIn, PEN>), grid, block, args,
                                   (unsigned)lds, stream);
    if (e == hipSuccess && ev1) e = hipEventRecord(ev1, stream);
    return e;
  }
  // the event pair (when given) brackets the kernel's own execution
  return hipExtLaunchKernel(reinterpret_cast<const void *>(&row_kernel<TIn, PEN>), grid, block, args, lds, stream,
                            ev0, ev1, 0);
}

template <typename TIn, bool PEN>
hipError_t set_lds_attr(size_t lds) {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&row_kernel<TIn, PEN>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

}  // namespace

hipError_t phase_stamps_take(unsigned long long *host, size_t n) {
#ifdef DSTS_PHASE_STAMPS
  const size_t total = (size_t)kStampBlocks * kStampSlots;
  if (n > total) n = total;
  hipError_t e = hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_stamps), n * sizeof(unsigned long long), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  void *p = nullptr;
  if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_phase_stamps))) != hipSuccess) return e;
  return hipMemset(p, 0, total * sizeof(unsigned long long));
#else
  (void)host;
  (void)n;
  return hipErrorNotSupported;
#endif
}

size_t hist_list_lds_bytes(int slice) { return sizeof(uint32_t) * (size_t)slice; }

hipError_t launch_hist_list(const KernelArgs &ka, hipStream_t stream) {
  const KernelParams &kp = ka.kp;
  const size_t lds = hist_list_lds_bytes(kp.slice);  // the attribute allows any slice (resident_blocks)
  void *args[] = {const_cast<KernelArgs *>(&ka)};
  return hipExtLaunchKernel(reinterpret_cast<const void *>(&hist_list_kernel), dim3(kp.n_rows * kp.G), dim3(kBlock),
                            args, lds, stream, nullptr, nullptr, 0);
}


size_t kernel_lds_fixed() { return sizeof(SmemBase); }

size_t kernel_lds_region(int slice, int hash_slots, int bias_slots, bool penalties) {
  size_t r = kRegionB + kRegionBBytes;
  const size_t radix = 3072 + 8 * 256;
  r = r > radix ? r : radix;
  const size_t merge = 8 * (size_t)kMaxG * kMaxTopLogprobs;
  r = r > merge ? r : merge;
  if (penalties) {
    const size_t pen = sizeof(uint32_t) * (size_t)hash_slots + 8 * (size_t)bias_slots;
    r = r > pen ? r : pen;
  }
  return (r + 15) & ~(size_t)15;
}

size_t kernel_lds_bytes(int slice, int hash_slots, int bias_slots, bool penalties) {
  return kernel_lds_fixed() + sizeof(float) * (size_t)slice +
         kernel_lds_region(slice, hash_slots, bias_slots, penalties);
}

hipError_t launch_raw_lp(const KernelArgs &ka, int dtype, hipStream_t stream) {
  const KernelParams &kp = ka.kp;
  const size_t lds = kernel_lds_bytes(kp.slice, kp.hash_slots, kp.bias_slots, true);
  const dim3 grid(kp.n_groups * kp.G), block(kBlock);
  void *args[] = {const_cast<KernelArgs *>(&ka)};
  const void *fn = dtype == 0 ? reinterpret_cast<const void *>(&raw_lp_kernel<float>)
                              : reinterpret_cast<const void *>(&raw_lp_kernel<uint16_t>);
  return hipExtLaunchKernel(fn, grid, block, args, lds, stream, nullptr, nullptr, 0);
}

size_t stream_lds_bytes(int hash_slots, bool penalties, int vocab) {
  return sizeof(SmemBase) +
         (penalties ? sizeof(uint32_t) * (size_t)stream_bitmap_words(vocab) + 8 * (size_t)hash_slots : 0) +
         2 * sizeof(unsigned long long) * (size_t)kSCap;
}

namespace {
template <typename TIn, bool PEN>
const void *stream_fn() {
  return reinterpret_cast<const void *>(&stream_kernel<TIn, PEN>);
}
}  // namespace

hipError_t launch_stream(const KernelArgs &ka, int dtype, bool penalties, int grid, hipStream_t stream, hipEvent_t ev0,
                         hipEvent_t ev1) {
  const KernelParams &kp = ka.kp;
  const size_t lds = stream_lds_bytes(kp.hash_slots, penalties, kp.vocab);
  const void *fn = dtype == 0 ? (penalties ? stream_fn<float, true>() : stream_fn<float, false>())
                              : (penalties ? stream_fn<uint16_t, true>() : stream_fn<uint16_t, false>());
  void *args[] = {const_cast<KernelArgs *>(&ka)};
  return hipExtLaunchKernel(fn, dim3(grid), dim3(kBlock), args, lds, stream, ev0, ev1, 0);
}

hipError_t stream_resident(int device, size_t lds_bytes, int *out) {
  const void *fns[] = {stream_fn<float, true>(), stream_fn<float, false>(), stream_fn<uint16_t, true>(),
                       stream_fn<uint16_t, false>()};
  hipError_t e;
  hipDeviceProp_t prop;
  if ((e = hipGetDeviceProperties(&prop, device)) != hipSuccess) return e;
  if (lds_bytes > prop.sharedMemPerBlock) {  // (the largest vocabularies with the longest histories)
    *out = 0;
    return hipSuccess;
  }
  int pc = 1 << 30;
  for (const void *f : fns) {
    if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes)) != hipSuccess) return e;
    int per_cu = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kBlock, lds_bytes)) != hipSuccess) return e;
    pc = per_cu < pc ? per_cu : pc;
  }
  *out = pc * prop.multiProcessorCount;
  return hipSuccess;
}

hipError_t launch_small(const KernelArgs &ka, int dtype, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const void *fn = dtype == 0 ? reinterpret_cast<const void *>(&small_kernel<float>)
                              : reinterpret_cast<const void *>(&small_kernel<uint16_t>);
  void *args[] = {const_cast<KernelArgs *>(&ka)};
  return hipExtLaunchKernel(fn, dim3(ka.kp.n_rows), dim3(kSmallBlock), args, 0, stream, ev0, ev1, 0);
}

hipError_t launch_chunk(const KernelArgs &ka, int dtype, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const void *fn = dtype == 0 ? reinterpret_cast<const void *>(&chunk_kernel<float>)
                              : reinterpret_cast<const void *>(&chunk_kernel<uint16_t>);
  void *args[] = {const_cast<KernelArgs *>(&ka)};
  return hipExtLaunchKernel(fn, dim3(ka.kp.chunk_n, ka.kp.n_rows), dim3(kChunkBlock), args, 0, stream, ev0, ev1, 0);
}

hipError_t launch_rows(const KernelParams &kp, RowParam *out, hipStream_t stream) {
  hipLaunchKernelGGL(rows_kernel, dim3((kp.n_rows + 255) / 256), dim3(256), 0, stream, kp, out);
  return hipGetLastError();
}

hipError_t launch_step(const KernelArgs &ka, int dtype, bool penalties, bool cooperative, hipStream_t stream,
                       hipEvent_t ev0, hipEvent_t ev1) {
  if (dtype == 0)
    return penalties ? launch_t<float, true>(ka, cooperative, stream, ev0, ev1)
                     : launch_t<float, false>(ka, cooperative, stream, ev0, ev1);
  return penalties ? launch_t<uint16_t, true>(ka, cooperative, stream, ev0, ev1)
                   : launch_t<uint16_t, false>(ka, cooperative, stream, ev0, ev1);
}

hipError_t kernel_lds_static(size_t *out) {
  const void *fns[] = {reinterpret_cast<const void *>(&row_kernel<float, true>),
                       reinterpret_cast<const void *>(&row_kernel<float, false>),
                       reinterpret_cast<const void *>(&row_kernel<uint16_t, true>),
                       reinterpret_cast<const void *>(&row_kernel<uint16_t, false>)};
  size_t m = 0;
  for (const void *f : fns) {
    hipFuncAttributes attr;
    const hipError_t e = hipFuncGetAttributes(&attr, f);
    if (e != hipSuccess) return e;
    m = attr.sharedSizeBytes > m ? attr.sharedSizeBytes : m;
  }
  *out = m;
  return hipSuccess;
}

hipError_t resident_blocks(int device, size_t lds_bytes, int *out) {
  hipError_t e;
  if ((e = set_lds_attr<float, true>(lds_bytes)) != hipSuccess) return e;
  if ((e = set_lds_attr<float, false>(lds_bytes)) != hipSuccess) return e;
  if ((e = set_lds_attr<uint16_t, true>(lds_bytes)) != hipSuccess) return e;
  if ((e = set_lds_attr<uint16_t, false>(lds_bytes)) != hipSuccess) return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(&raw_lp_kernel<float>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(&raw_lp_kernel<uint16_t>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(&hist_list_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)hist_list_lds_bytes(kMaxSlice))) !=
      hipSuccess)
    return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&row_kernel<float, true>),
                                                   kBlock, lds_bytes);
  if (e != hipSuccess) return e;
  int per_cu2 = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu2, reinterpret_cast<const void *>(&row_kernel<uint16_t, true>),
                                                   kBlock, lds_bytes);
  if (e != hipSuccess) return e;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return e;
  const int pc = per_cu < per_cu2 ? per_cu : per_cu2;
  *out = pc * prop.multiProcessorCount;
  return hipSuccess;
}

}  // namespace dsts
