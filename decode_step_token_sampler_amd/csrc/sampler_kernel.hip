// sampler_kernel.hip -- the decode-step sampler's row kernel for gfx950.
//
// Sources (page titles; sections named where used):
//   [A] "SGLang's +75% sampler speedup skips Qwen3 chat requests"
//   [B] the SGLang 101 operations manual
//   [C] "采样参数对解码开销的影响：temperature、top_p 与采样核路径"
//   Philox4x32-10: Salmon, Moraes, Dror, Shaw, SC'11.
//
// One launch samples a whole batch.  A row is split into G contiguous slices;
// G workgroups of 1024 threads (a "row group") own one slice each and keep
// their slice's processed logits z = penalised(x) / T in LDS, so the logits
// are read from HBM once.  The G workgroups of a group cooperate
// through per-group barrier words and exchange slots in device memory (the
// launch is cooperative, so all workgroups are resident).  A group walks
// rows group, group + n_groups, ...
//
// Per row:
//   1. load, NaN -> -inf, penalties (LDS hash of history counts, each
//      distinct id applied once), z = x / T
//   2. exchange 1: row max and first argmax
//   3. exchange 2: a histogram of d = max - z in 1/16-nat bins (counts over
//      32 nats, 2^-44 fixed-point masses over 16 nats, deeper values summed
//      in registers), merged by the last workgroup to arrive, which picks the
//      bins holding each threshold; min-p's fp64 test bounds an upper set of
//      keys, found by bisection
//   4. exchange 3: the values of those bins are gathered, ranked exactly by
//      the last workgroup to arrive, which fixes top-k, top-p, the kept-set
//      sum and the top logprobs (rows whose thresholds fall outside the
//      window take the general path: a radix select with one exchange per
//      8-bit digit)
//   5. emit probs / logprobs of the kept set; Gumbel-max with an in-kernel
//      Philox draw, an fp32 log-domain filter and an fp64 check of every
//      element that can still win
//   6. the last workgroup to arrive merges the Gumbel candidates and writes
//      the token and status
#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

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
// fp32 log-domain Gumbel scores are within ~1e-5 of the exact ones; any
// element whose fp32 score is within this margin of the running best is
// rescored in fp64.
constexpr float kVerifyMargin = 1e-3f;
constexpr double kMassScale = 17592186044416.0;  // 2^44
constexpr uint32_t kEmpty = 0xFFFFFFFFu;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct alignas(16) SmemBase {
  float red_f[kWaves];
  double red_d[kWaves];
  unsigned long long red_u[kWaves];
  int red_i[kWaves];
  uint32_t red_c[kWaves];
  uint32_t bu[16];
  double bd[16];
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

DEV float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEV unsigned long long wave_max_u(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// Workgroup reductions (every thread gets the result).
DEV float wg_max_f(SmemBase &sm, float v) {
  v = wave_max_f(v);
  if ((threadIdx.x & 63) == 0) sm.red_f[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sm.red_f[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, sm.red_f[w]);
  __syncthreads();
  return r;
}
// Fixed order: lanes by xor tree, waves in index order (deterministic).
DEV double wg_sum_d(SmemBase &sm, double v) {
  v = wave_sum_d(v);
  if ((threadIdx.x & 63) == 0) sm.red_d[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = sm.red_d[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r += sm.red_d[w];
  __syncthreads();
  return r;
}
DEV unsigned long long wg_max_u(SmemBase &sm, unsigned long long v) {
  v = wave_max_u(v);
  if ((threadIdx.x & 63) == 0) sm.red_u[threadIdx.x >> 6] = v;
  __syncthreads();
  unsigned long long r = sm.red_u[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = sm.red_u[w] > r ? sm.red_u[w] : r;
  __syncthreads();
  return r;
}
// Best (score desc, index asc) pair over the workgroup.
DEV void wg_best(SmemBase &sm, double &g, int &idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    double g2 = __shfl_xor(g, o, 64);
    int i2 = __shfl_xor(idx, o, 64);
    if (g2 > g || (g2 == g && i2 < idx)) {
      g = g2;
      idx = i2;
    }
  }
  if ((threadIdx.x & 63) == 0) {
    sm.red_d[threadIdx.x >> 6] = g;
    sm.red_i[threadIdx.x >> 6] = idx;
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

// Philox4x32-10 block for counter (c0..c3) and key (k0, k1).
DEV void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1,
                       uint32_t out[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo_a = c0 * 0xD2511F53u, hi_a = __umulhi(c0, 0xD2511F53u);
    const uint32_t lo_b = c2 * 0xCD9E8D57u, hi_b = __umulhi(c2, 0xCD9E8D57u);
    const uint32_t n0 = hi_b ^ c1 ^ k0;
    const uint32_t n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
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
// ln E in fp32 (filter only).  For x >= 2^31 use 1 - w = (~x + 1/2) 2^-32,
// which is exact in the integer complement.
DEV float ln_exp1_f32(uint32_t x) {
  float e;
  if (x < 0x80000000u) {
    const float w = ((float)x + 0.5f) * 0x1p-32f;
    e = -log1pf(-w);
  } else {
    const float u = ((float)(~x) + 0.5f) * 0x1p-32f;
    e = -logf(u);
  }
  return logf(e);
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
// Exchange data is written with agent-scope stores; every wave drains its
// memory counters before the workgroup barrier, then one thread fences
// (agent-scope release, once per workgroup) and arrives.  Waiters poll the
// generation word with relaxed loads and take one acquire fence when it
// moves.  The last arrival resets the count, so the words are reusable
// without clearing.
DEV void mem_quiesce() { __builtin_amdgcn_s_waitcnt(0); }

// Returns true in exactly one workgroup, the last to arrive, which merges
// the exchange and then calls group_release; the others call group_wait.
DEV bool group_arrive(SmemBase &sm, GroupSync *s, int G) {
  mem_quiesce();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t g0 = __hip_atomic_load(&s->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = __hip_atomic_fetch_add(&s->count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == (uint32_t)G - 1u;
    if (last) {
      __hip_atomic_store(&s->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    sm.bu[14] = g0;
    sm.bu[15] = last ? 1u : 0u;
  }
  __syncthreads();
  const bool last = sm.bu[15] != 0u;
  __syncthreads();
  return last;
}

DEV void group_release(GroupSync *s) {
  mem_quiesce();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(&s->gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The wait is bounded (~2 s): on expiry the launch is marked aborted (the
// abort word takes this launch's epoch), every later wait of the launch
// returns at once and the rows report status 3, so a logic error cannot hang
// the device.
constexpr uint32_t kSpinLimit = 1u << 26;
DEV void group_wait(SmemBase &sm, GroupSync *s, uint32_t *abort_word, uint32_t epoch) {
  if (threadIdx.x == 0) {
    const uint32_t g0 = sm.bu[14];
    uint32_t spins = 0;
    while (__hip_atomic_load(&s->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
      if (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) break;
      if (++spins > kSpinLimit) {
        __hip_atomic_store(abort_word, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Plain barrier: arrive, and the last arrival releases at once.
DEV void group_barrier(SmemBase &sm, GroupSync *s, int G, uint32_t *abort_word, uint32_t epoch) {
  if (group_arrive(sm, s, G)) group_release(s);
  else group_wait(sm, s, abort_word, epoch);
}

// ---------------------------------------------------------------- block scans
// Inclusive scan of one value per thread over the workgroup (fixed order).
template <typename T>
DEV T block_scan_incl(T v, T *wave_tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wave_tot[w] = v;
  __syncthreads();
  T base = 0;
  for (int i = 0; i < w; ++i) base += wave_tot[i];
  __syncthreads();
  return v + base;
}

// Sum of one u64 per thread over the workgroup (exact).
DEV unsigned long long wg_sum_u(SmemBase &sm, unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sm.red_u[threadIdx.x >> 6] = v;
  __syncthreads();
  unsigned long long r = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r += sm.red_u[w];
  __syncthreads();
  return r;
}

// Per-row context shared by the phases.
struct RowCtx {
  int row, gid, G, n, n4, s0;
  GroupSync *gsync;
  GroupRec *rec;
  uint32_t *abort_word;
  uint32_t epoch;
  WgSlots *my;
  WgSlots *peers;
  unsigned *xseq;
};

DEV void row_barrier(SmemBase &sm, RowCtx &rc) { group_barrier(sm, rc.gsync, rc.G, rc.abort_word, rc.epoch); }

// Window bin of a value: d = max - z in 1/16-nat steps, kWinBins past 32
// nats.  Monotone in z, so the bins partition the value axis in order.
DEV int win_bin(float mf, float z) {
  const float d = mf - z;
  return d < 32.0f ? (int)(d * kBinsPerNat) : kWinBins;
}

// exp(-d) for d >= 0 as 2^-44 fixed point (fp32 exp; exact scaling by 2^12
// and 2^32, truncating conversions).
DEV unsigned long long mass_fixed(float d) {
  const float q = expf(-d);
  const float a = q * 4096.0f;
  const uint32_t hi = (uint32_t)a;
  const uint32_t lo = (uint32_t)((a - (float)hi) * 4294967296.0f);
  return ((unsigned long long)hi << 32) | lo;
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
// threshold above -inf.
template <bool MASS>
DEV uint32_t radix_select(SmemBase &sm, RowCtx &rc, const float *zs, unsigned char *region, uint32_t lower,
                          uint32_t k, double p, double m) {
  uint32_t *hcnt = reinterpret_cast<uint32_t *>(region);
  uint32_t *mcnt = hcnt + 256;
  unsigned long long *hmass = reinterpret_cast<unsigned long long *>(mcnt + 256);
  unsigned long long *mmass = hmass + 256;
  uint32_t prefix = 0, mask = 0;
  uint32_t rem_cnt = k;
  unsigned long long above = 0;
  double target = 0.0;
  for (int round = 0; round < 4; ++round) {
    const int shift = 24 - 8 * round;
    for (int b = threadIdx.x; b < 256; b += kBlock) {
      hcnt[b] = 0;
      hmass[b] = 0;
    }
    __syncthreads();
    for (int l = 4 * threadIdx.x; l < rc.n4; l += 4 * kBlock) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float zz = v[c];
        const uint32_t key = fkey(zz);
        if (key >= lower && (key & mask) == prefix) {
          const uint32_t bin = (key >> shift) & 0xFFu;
          if (MASS) atomicAdd(&hmass[bin], (unsigned long long)(exp((double)zz - m) * kMassScale));
          else atomicAdd(&hcnt[bin], 1u);
        }
      }
    }
    __syncthreads();
    const unsigned par = (*rc.xseq)++ & 1u;
    for (int b = threadIdx.x; b < 256; b += kBlock) {
      if (MASS) atomic_st(&rc.my->hmass[par][b], hmass[b]);
      else atomic_st(&rc.my->hcnt[par][b], hcnt[b]);
    }
    row_barrier(sm, rc);
    for (int b = threadIdx.x; b < 256; b += kBlock) {
      if (MASS) {
        unsigned long long t = 0;
        for (int g = 0; g < rc.G; ++g) t += atomic_ld(&rc.peers[g].hmass[par][b]);
        mmass[b] = t;
      } else {
        uint32_t t = 0;
        for (int g = 0; g < rc.G; ++g) t += atomic_ld(&rc.peers[g].hcnt[par][b]);
        mcnt[b] = t;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t digit = 0;
      if (MASS) {
        if (round == 0) {
          unsigned long long tot = 0;
          for (int b = 0; b < 256; ++b) tot += mmass[b];
          target = p * (double)tot;
        }
        unsigned long long acc = above;
        for (int b = 255; b >= 0; --b) {
          const unsigned long long nxt = acc + mmass[b];
          if ((double)nxt >= target || b == 0) {
            digit = (uint32_t)b;
            break;
          }
          acc = nxt;
        }
        sm.bd[0] = target;
        sm.bu[1] = (uint32_t)(acc & 0xFFFFFFFFu);
        sm.bu[2] = (uint32_t)(acc >> 32);
      } else {
        uint32_t acc = 0;
        for (int b = 255; b >= 0; --b) {
          if (acc + mcnt[b] >= rem_cnt || b == 0) {
            digit = (uint32_t)b;
            break;
          }
          acc += mcnt[b];
        }
        sm.bu[1] = rem_cnt - acc;
      }
      sm.bu[0] = digit;
    }
    __syncthreads();
    const uint32_t digit = sm.bu[0];
    if (MASS) {
      target = sm.bd[0];
      above = ((unsigned long long)sm.bu[2] << 32) | sm.bu[1];
    } else {
      rem_cnt = sm.bu[1];
    }
    prefix |= digit << shift;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  return prefix;
}

// Packed hash entry: slice-local index << 13 | count.
DEV uint32_t hash_slot(uint32_t local, uint32_t slots) { return (local * 2654435761u) & (slots - 1u); }

// min-p keeps exp(z - m) >= min_p (fp64).  That set is an upper set of keys;
// its boundary key is the smallest key passing the same test, found from the
// closed-form guess m + ln(min_p) by bracketing and bisection.
DEV uint32_t min_p_key(double m, float min_p) {
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

// Decision words of GroupRec::dec
enum : int {
  D_FLAGS = 0,  // bit 0: general path; bit 1: [0, RKHI] gathered whole (top-k prefix)
  D_R0HI = 1,   // gathered bins: [0, R0HI] (top logprobs), [R1LO, R1HI] (top-p crossing),
  D_R1LO = 2,   //   [RKLO, RKHI] (top-k crossing bin, or the whole top-k prefix), BM (min-p boundary)
  D_R1HI = 3,
  D_RKLO = 4,
  D_RKHI = 5,
  D_BM = 6,
  D_TAU = 7,
};

// Ranges of window bins whose values are gathered (hi < lo: empty).
struct CandRanges {
  int r0hi, r1lo, r1hi, rklo, rkhi, bm;
  DEV bool has(int b) const {
    return b <= r0hi || (b >= r1lo && b <= r1hi) || (b >= rklo && b <= rkhi) || b == bm;
  }
};

// Exchange-2 decisions, by one thread of the merging workgroup, from the
// merged inclusive prefix counts lc[0..kWinBins] and masses lm[0..kMassBins]
// (LDS; the last entry of each includes the values deeper than the window).
DEV void decide_window(GroupRec *rec, const uint32_t *lc, const unsigned long long *lm, const RowParam &P,
                       bool topk, bool topp, bool minp, bool need_thr, int K, float mf, uint32_t t_m, double S_all) {
  uint32_t flags = 0;
  auto cc = [&](int b) { return b < 0 ? 0u : lc[b < kWinBins ? b : kWinBins]; };
  auto cm = [&](int b) { return b < 0 ? 0.0 : (double)lm[b < kMassBins ? b : kMassBins]; };
  auto bin_for_count = [&](uint32_t want) {  // first bin reaching `want`; kWinBins + 1 if none
    if (lc[kWinBins] < want) return kWinBins + 1;
    int lo = 0, hi = kWinBins;
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (lc[mid] >= want) hi = mid;
      else lo = mid + 1;
    }
    return lo;
  };
  auto bin_for_mass = [&](double want) {  // first mass bin reaching `want`; kMassBins: the deep values
    int lo = 0, hi = kMassBins;
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if ((double)lm[mid] >= want) hi = mid;
      else lo = mid + 1;
    }
    return lo;
  };
  int r0hi = -1, r1lo = 1, r1hi = 0, rklo = 1, rkhi = 0, bm = -1;
  if (K > 0) r0hi = min(bin_for_count((uint32_t)K), kWinBins);
  int bk = -1;
  if (topk) {
    bk = bin_for_count((uint32_t)P.top_k);
    if (cc(bk) <= (uint32_t)kCandCap) {  // the whole top-k prefix fits: gather it
      flags |= 2u;
      rklo = 0;
      rkhi = bk;
    } else if (bk < kMassBins) {
      rklo = rkhi = bk;
    } else {
      flags |= 1u;
    }
  }
  if (topp && !(flags & 1u)) {
    double clo, chi;
    if (topk) {
      clo = cm(min(bk, kMassBins) - 1);
      chi = bk < kMassBins ? cm(bk) : cm(kMassBins);
    } else {
      clo = chi = cm(kMassBins);
    }
    r1lo = bin_for_mass((double)P.top_p * clo);
    r1hi = bin_for_mass((double)P.top_p * chi);
    if (r1hi >= kMassBins) flags |= 1u;
    if (topk) {
      r1lo = min(r1lo, bk);
      r1hi = min(r1hi, bk);
    }
  }
  if (minp && !(flags & 1u)) {
    bm = win_bin(mf, key_to_float(t_m));
    if (bm >= kMassBins && !((flags & 2u) && bm <= rkhi)) flags |= 1u;
  }
  if (!(flags & 1u) && need_thr) {
    // values to gather: the union of the ranges, counted bin by bin
    uint32_t n = 0;
    for (int b = 0; b <= kWinBins; ++b) {
      const bool in = b <= r0hi || (b >= r1lo && b <= r1hi) || (b >= rklo && b <= rkhi) || b == bm;
      if (in) n += cc(b) - cc(b - 1);
    }
    if (n > (uint32_t)kCandCap) flags |= 1u;
  }
  atomic_st(&rec->dec[D_FLAGS], flags);
  atomic_st(&rec->dec[D_R0HI], (uint32_t)r0hi);
  atomic_st(&rec->dec[D_R1LO], (uint32_t)r1lo);
  atomic_st(&rec->dec[D_R1HI], (uint32_t)r1hi);
  atomic_st(&rec->dec[D_RKLO], (uint32_t)rklo);
  atomic_st(&rec->dec[D_RKHI], (uint32_t)rkhi);
  atomic_st(&rec->dec[D_BM], (uint32_t)bm);
  atomic_st(&rec->dd[0], S_all);
  atomic_st(&rec->cand_n, 0u);
}

// ---------------------------------------------------------------- the kernel
template <typename TIn, bool PEN>
__global__ __launch_bounds__(kBlock) void row_kernel(KernelParams kp) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  SmemBase &sm = *reinterpret_cast<SmemBase *>(lds_raw);
  static_assert(sizeof(SmemBase) % 16 == 0, "the LDS slice must be 16-byte aligned");
  float *zs = reinterpret_cast<float *>(lds_raw + sizeof(SmemBase));
  unsigned char *region = reinterpret_cast<unsigned char *>(zs + kp.slice);
  // region views (used one at a time)
  uint32_t *hash = reinterpret_cast<uint32_t *>(region);
  uint32_t *bitmap = hash + kp.hash_slots;
  unsigned long long *wm = reinterpret_cast<unsigned long long *>(region);              // [kMassBins + 1]
  uint32_t *wc = reinterpret_cast<uint32_t *>(wm + (kMassBins + 1));                     // [kWinBins + 1]
  float *cz = reinterpret_cast<float *>(wc + (kWinBins + 4));                            // leader: candidates
  int32_t *ci = reinterpret_cast<int32_t *>(cz + kCandCap);
  float *sz = reinterpret_cast<float *>(ci + kCandCap);
  int32_t *si = reinterpret_cast<int32_t *>(sz + kCandCap);
  double *sq = reinterpret_cast<double *>(si + kCandCap);

  const int tid = threadIdx.x;
  const int G = kp.G;
  const int gid = blockIdx.x % G;
  const int group = blockIdx.x / G;
  const int V = kp.vocab;
  const uint32_t hslots = (uint32_t)kp.hash_slots;
  unsigned xseq = 0;
  RowCtx rc;
  rc.gid = gid;
  rc.G = G;
  rc.gsync = kp.sync + group;
  rc.rec = kp.recs + group;
  rc.abort_word = kp.abort_word;
  rc.epoch = kp.epoch;
  rc.my = kp.slots + blockIdx.x;
  rc.peers = kp.slots + (size_t)group * G;
  rc.xseq = &xseq;
  GroupRec *rec = rc.rec;
  const bool want_out = kp.probs != nullptr || kp.logprobs != nullptr;
  const int K = kp.top_lp;
  const bool want_S = want_out || K > 0;
  const int s0 = gid * kp.slice;
  const int s1 = min(V, s0 + kp.slice);
  rc.s0 = s0;
  rc.n = s1 - s0;
  rc.n4 = (rc.n + 3) & ~3;

  unsigned it = 0;
  for (int row = group; row < kp.n_rows; row += kp.n_groups, ++it) {
    const RowParam P = kp.rows[row];
    rc.row = row;
    const bool greedy = P.flags & RF_GREEDY;
    const bool top1 = P.flags & RF_TOP1;
    const bool pen = PEN && (P.flags & RF_PEN);
    const bool topk = !greedy && (P.flags & RF_TOPK);
    const bool topp = !greedy && (P.flags & RF_TOPP);
    const bool minp = !greedy && (P.flags & RF_MINP);
    const bool truncated = topk || topp || minp;

    // ---- 1. issue the history and logit loads, build the penalty counts
    // while they are in flight, then sanitise, penalise and divide by the
    // temperature into the LDS slice.  Loads use clamped in-bounds
    // addresses; with vector loads the row stride is a multiple of 4, so a
    // group starting below s1 lies inside the row.
    int32_t hv[kMaxHistPerRow / kBlock];
    if (pen) {
      const int32_t *hist = kp.history_ids + P.hist_start;
#pragma unroll
      for (int q = 0; q < kMaxHistPerRow / kBlock; ++q) {
        const int h = tid + q * kBlock;
        hv[q] = h < P.hist_len ? hist[h] : -1;
      }
    }
    constexpr int kBatch = kMaxSlice / (4 * kBlock);
    float v[kBatch][4];
    {
      // opaque per row: keeps the per-load offsets from being hoisted out of
      // the row loop (they would stay live across it and spill)
      int ln = __builtin_amdgcn_readfirstlane(rc.n);
      asm volatile("" : "+s"(ln));
      const int64_t rbase = (int64_t)row * kp.row_stride + s0;
      const int lastg = (ln - 1) & ~3;
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int l = 4 * tid + 4 * kBlock * b;
        if (kp.vec_ok & 1) {
          Loader<TIn>::load4(kp.logits, rbase + min(l, lastg), v[b]);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) v[b][c] = Loader<TIn>::load1(kp.logits, rbase + min(l + c, ln - 1));
        }
      }
    }
    if (pen) {
      for (int t = tid; t < (int)hslots; t += kBlock) hash[t] = kEmpty;
      for (int t = tid; t < (rc.n4 + 31) / 32; t += kBlock) bitmap[t] = 0;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kMaxHistPerRow / kBlock; ++q) {
        const int32_t id = hv[q];
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
          atomicOr(&bitmap[local >> 5], 1u << (local & 31));
        }
      }
    }
    // raw values -> LDS (slots past the slice end: -inf)
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int l = 4 * tid + 4 * kBlock * b;
      if (l < rc.n4) {
        f32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = (l + c < rc.n) ? v[b][c] : -INFINITY;
        *reinterpret_cast<f32x4 *>(zs + l) = o;
      }
    }
    __syncthreads();
    // z = x / T, correctly rounded: q = x (1/T), then one FMA correction
    // with the exact remainder (Markstein), valid while q stays in the
    // normal range; elsewhere (and for infinities) the IEEE division.
    const float T = P.temperature;
    const float rT = 1.0f / T;
    float lmax = -INFINITY;
    int lidx = 0x7FFFFFFF;  // first index of the local max (slots are visited in index order)
    for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
      f32x4 o = *reinterpret_cast<const f32x4 *>(zs + l);
      const uint32_t pb = pen ? (bitmap[l >> 5] >> (l & 31)) & 0xFu : 0u;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x = o[c];
        x = (x == x) ? x : -INFINITY;
        if ((pb >> c) & 1u) {
          const uint32_t local = (uint32_t)(l + c);
          uint32_t sl = hash_slot(local, hslots);
          while ((hash[sl] >> 13) != local) sl = (sl + 1u) & (hslots - 1u);
          x = apply_penalty(x, hash[sl] & 0x1FFFu, P);
        }
        const float q = x * rT;
        const float aq = fabsf(q);
        float zz;
        if (aq >= 0x1p-100f && aq <= 0x1p100f) zz = __builtin_fmaf(__builtin_fmaf(-q, T, x), rT, q);
        else zz = x / T;
        zz = zz + 0.0f;  // -0 -> +0: equal values share one key
        o[c] = zz;
        if (zz > lmax) {
          lmax = zz;
          lidx = s0 + l + c;
        }
      }
      *reinterpret_cast<f32x4 *>(zs + l) = o;
    }

    // ---- 2. exchange 1: row max and first argmax
    const float wmax = wg_max_f(sm, lmax);
    const unsigned long long wam =
        wg_max_u(sm, lmax == wmax && lmax > -INFINITY ? ((unsigned long long)fkey(lmax) << 32) | (0xFFFFFFFFu - (uint32_t)lidx) : 0ull);
    const unsigned par = it & 1u;
    if (tid == 0) {
      atomic_st(&rc.my->small[par][0], (double)wmax);
      atomic_st(&rc.my->small[par][1], __longlong_as_double((long long)wam));
    }
    row_barrier(sm, rc);
    if (tid == 0) {
      double gm = -INFINITY;
      unsigned long long am = 0;
      for (int g = 0; g < G; ++g) {
        gm = fmax(gm, atomic_ld(&rc.peers[g].small[par][0]));
        const unsigned long long a = (unsigned long long)__double_as_longlong(atomic_ld(&rc.peers[g].small[par][1]));
        am = a > am ? a : am;
      }
      sm.bd[0] = gm;
      sm.bu[0] = 0xFFFFFFFFu - (uint32_t)(am & 0xFFFFFFFFu);
      if (minp && gm > -INFINITY && gm < INFINITY) sm.bu[3] = min_p_key(gm, P.min_p);
    }
    __syncthreads();
    const double m = sm.bd[0];
    const int argmax_idx = (int)sm.bu[0];
    const uint32_t t_m = minp ? sm.bu[3] : 0u;
    __syncthreads();

    // ---- rows with no finite logit (status 1) or a +inf value (status 2)
    if (!(m > -INFINITY) || m == INFINITY) {
      if (want_out) {
        for (int l = tid; l < rc.n; l += kBlock) {
          if (kp.probs) kp.probs[(int64_t)row * V + s0 + l] = 0.0f;
          if (kp.logprobs) kp.logprobs[(int64_t)row * V + s0 + l] = -INFINITY;
        }
      }
      if (gid == 0 && tid == 0) {
        kp.token_ids[row] = -1;
        if (kp.row_status) kp.row_status[row] = (m == INFINITY) ? 2 : 1;
        for (int t = 0; t < K; ++t) {
          kp.top_lp_vals[(int64_t)row * K + t] = -INFINITY;
          kp.top_lp_ids[(int64_t)row * K + t] = -1;
        }
      }
      __syncthreads();
      continue;
    }
    const float mf = (float)m;

    // ---- 3. window histogram (exchange 2, merged by the last workgroup to
    // arrive): counts for top-k and the top logprobs, masses for top-p and
    // the kept-set sum, and the exact fp64 sum when every token is kept.
    const bool need_cnt = topk || K > 0;
    const bool need_mass = truncated && (topp || want_S);
    const bool need_exact = !truncated && want_S;
    const bool need_thr = truncated || K > 0;  // thresholds / candidates needed
    bool general = false;
    bool full_k = false;
    uint32_t tau = 0;
    double lnS = 0.0;
    CandRanges cr = {-1, 1, 0, 1, 0, -1};
    if (need_cnt || need_mass || need_exact) {
      if (need_cnt || need_mass) {
        for (int b = tid; b < kWinBins + 1; b += kBlock) wc[b] = 0;
        for (int b = tid; b < kMassBins + 1; b += kBlock) wm[b] = 0;
        __syncthreads();
      }
      uint32_t deep_n = 0;
      unsigned long long deep_m = 0;
      double sx = 0.0;
      for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
        const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float zz = zv[c];
          const float d = mf - zz;
          if (need_cnt && l + c < rc.n) {
            if (d < 32.0f) atomicAdd(&wc[(int)(d * kBinsPerNat)], 1u);
            else ++deep_n;
          }
          if (need_mass) {
            if (d < 16.0f) atomicAdd(&wm[(int)(d * kBinsPerNat)], mass_fixed(d));
            else deep_m += mass_fixed(d);
          }
          if (need_exact) sx += d < 40.0f ? exp((double)zz - m) : (double)expf(-d);
        }
      }
      const uint32_t wdn = need_cnt ? (uint32_t)wg_sum_u(sm, deep_n) : 0u;
      const unsigned long long wdm = need_mass ? wg_sum_u(sm, deep_m) : 0ull;
      const double wsx = need_exact ? wg_sum_d(sm, sx) : 0.0;
      __syncthreads();
      // this workgroup's histogram -> its exchange slot
      if (need_cnt)
        for (int b = tid; b < kWinBins; b += kBlock) atomic_st(&rc.my->wcnt[b], wc[b]);
      if (need_mass)
        for (int b = tid; b < kMassBins; b += kBlock) atomic_st(&rc.my->wmass[b], wm[b]);
      if (tid == 0) {
        atomic_st(&rc.my->wcnt[kWinBins], wdn);
        atomic_st(&rc.my->wmass[kMassBins], wdm);
        atomic_st(&rc.my->spart, wsx);
      }
      if (group_arrive(sm, rc.gsync, G)) {
        // ---- merge (last arrival): inclusive prefix sums over the bins,
        // kept in LDS for the decisions and published for exchange 3
        static_assert(kWinBins == kBlock && kMassBins <= kBlock, "one bin per thread");
        {
          uint32_t c = 0;
          if (need_cnt)
            for (int g = 0; g < G; ++g) c += atomic_ld(&rc.peers[g].wcnt[tid]);
          const uint32_t run = block_scan_incl<uint32_t>(c, sm.red_c);
          wc[tid] = run;
          if (tid == kBlock - 1) {
            uint32_t o = 0;
            if (need_cnt)
              for (int g = 0; g < G; ++g) o += atomic_ld(&rc.peers[g].wcnt[kWinBins]);
            wc[kWinBins] = run + o;
          }
        }
        {
          unsigned long long mm = 0;
          if (need_mass && tid < kMassBins)
            for (int g = 0; g < G; ++g) mm += atomic_ld(&rc.peers[g].wmass[tid]);
          const unsigned long long run = block_scan_incl<unsigned long long>(mm, sm.red_u);
          if (tid < kMassBins) wm[tid] = run;
          if (tid == kMassBins - 1) {
            unsigned long long o = 0;
            if (need_mass)
              for (int g = 0; g < G; ++g) o += atomic_ld(&rc.peers[g].wmass[kMassBins]);
            wm[kMassBins] = run + o;
          }
        }
        __syncthreads();
        for (int b = tid; b <= kWinBins; b += kBlock) atomic_st(&rec->cum_cnt[b], wc[b]);
        for (int b = tid; b <= kMassBins; b += kBlock) atomic_st(&rec->cum_mass[b], wm[b]);
        if (tid == 0) {
          double S_all = 0.0;
          if (need_exact)
            for (int g = 0; g < G; ++g) S_all += atomic_ld(&rc.peers[g].spart);
          decide_window(rec, wc, wm, P, topk, topp, minp, need_thr, K, mf, t_m, S_all);
        }
        group_release(rc.gsync);
      } else {
        group_wait(sm, rc.gsync, rc.abort_word, rc.epoch);
      }
      if (tid == 0) {
        sm.bu[4] = atomic_ld(&rec->dec[D_FLAGS]);
        sm.bu[5] = atomic_ld(&rec->dec[D_R0HI]);
        sm.bu[6] = atomic_ld(&rec->dec[D_R1LO]);
        sm.bu[7] = atomic_ld(&rec->dec[D_R1HI]);
        sm.bu[8] = atomic_ld(&rec->dec[D_RKLO]);
        sm.bu[9] = atomic_ld(&rec->dec[D_RKHI]);
        sm.bu[10] = atomic_ld(&rec->dec[D_BM]);
        sm.bd[1] = atomic_ld(&rec->dd[0]);
      }
      __syncthreads();
      general = sm.bu[4] & 1u;
      full_k = sm.bu[4] & 2u;
      cr.r0hi = (int)sm.bu[5];
      cr.r1lo = (int)sm.bu[6];
      cr.r1hi = (int)sm.bu[7];
      cr.rklo = (int)sm.bu[8];
      cr.rkhi = (int)sm.bu[9];
      cr.bm = (int)sm.bu[10];
      if (need_exact) lnS = log(sm.bd[1]);
      __syncthreads();
    }

    // ---- 4. exact thresholds from the gathered candidates (exchange 3,
    // ranked and decided by the last workgroup to arrive)
    if (need_thr && !general) {
      // count, reserve, then write this slice's candidates
      uint32_t mine = 0;
      for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
        const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (l + c < rc.n && cr.has(win_bin(mf, zv[c]))) ++mine;
      }
      const uint32_t incl = block_scan_incl<uint32_t>(mine, sm.red_c);
      if (tid == kBlock - 1) sm.bu[11] = atomicAdd(&rec->cand_n, incl);
      __syncthreads();
      uint32_t pos = sm.bu[11] + incl - mine;
      if (mine > 0) {
        for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
          const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (l + c < rc.n && cr.has(win_bin(mf, zv[c]))) {
              if (pos < (uint32_t)kCandCap) {
                atomic_st(&rec->cz[pos], zv[c]);
                atomic_st(&rec->ci[pos], s0 + l + c);
              }
              ++pos;
            }
          }
        }
      }
      if (group_arrive(sm, rc.gsync, G)) {
        if (tid == 0) sm.bu[12] = atomic_ld(&rec->cand_n);
        __syncthreads();
        const uint32_t n_all = sm.bu[12];
        const int n = (int)min(n_all, (uint32_t)kCandCap);
        // merged prefix arrays and candidates -> LDS
        for (int b = tid; b <= kWinBins; b += kBlock) wc[b] = atomic_ld(&rec->cum_cnt[b]);
        for (int b = tid; b <= kMassBins; b += kBlock) wm[b] = atomic_ld(&rec->cum_mass[b]);
        for (int t = tid; t < n; t += kBlock) {
          cz[t] = atomic_ld(&rec->cz[t]);
          ci[t] = atomic_ld(&rec->ci[t]);
        }
        __syncthreads();
        // rank by (value desc, index asc): a total order, so the sorted list
        // (and every sum over it) does not depend on the gather order
        for (int t = tid; t < n; t += kBlock) {
          const float zt = cz[t];
          const int it_ = ci[t];
          int r = 0;
          for (int j = 0; j < n; ++j) r += (cz[j] > zt || (cz[j] == zt && ci[j] < it_)) ? 1 : 0;
          sz[r] = zt;
          si[r] = it_;
        }
        __syncthreads();
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
            qv[u] = j < n ? exp((double)sz[j] - m) : 0.0;
            own += qv[u];
          }
          double run = block_scan_incl<double>(own, sm.red_d) - own;
#pragma unroll
          for (int u = 0; u < kPerC; ++u) {
            const int j = tid * kPerC + u;
            run += qv[u];
            if (j < n) sq[j] = run;
          }
        }
        __syncthreads();
        // exact decisions; the sorted list holds every value of the gathered
        // bins, so the values of one bin are a contiguous run
        auto binof = [&](int j) { return win_bin(mf, sz[j]); };
        auto first_pos_bin = [&](int b) {  // first position whose bin is >= b
          int lo = 0, hi = n;
          while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (binof(mid) >= b) hi = mid;
            else lo = mid + 1;
          }
          return lo;
        };
        auto last_pos_ge = [&](uint32_t key) {  // last position with key >= `key` (-1: none)
          int lo = 0, hi = n;
          while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (fkey(sz[mid]) >= key) lo = mid + 1;
            else hi = mid;
          }
          return lo - 1;
        };
        auto qsum = [&](int a, int e) { return (e < a) ? 0.0 : sq[e] - (a > 0 ? sq[a - 1] : 0.0); };
        auto cmass = [&](int b) { return b < 0 ? 0.0 : (double)wm[b < kMassBins ? b : kMassBins] / kMassScale; };
        auto ccnt = [&](int b) { return b < 0 ? 0u : wc[b < kWinBins ? b : kWinBins]; };
        if (tid == 0) {
          uint32_t flags = n_all > (uint32_t)kCandCap ? 1u : 0u;
          uint32_t t = 0;
          double ctot = cmass(kMassBins);
          if (!flags && topk) {
            int j;
            if (full_k) {
              j = P.top_k - 1;
            } else {
              j = first_pos_bin(cr.rklo) + (P.top_k - (int)ccnt(cr.rklo - 1)) - 1;
            }
            if (j < 0 || j >= n) {
              flags |= 1u;
            } else {
              t = fkey(sz[j]);
              const int e = last_pos_ge(t);
              ctot = full_k ? qsum(0, e) : cmass(cr.rklo - 1) + qsum(first_pos_bin(cr.rklo), e);
            }
          }
          sm.bd[4] = ctot;
          sm.bu[0] = flags;
          sm.bu[1] = t;
          // top-p search range: positions of bins [r1lo, r1hi]
          const int p0 = first_pos_bin(cr.r1lo);
          sm.bu[2] = (uint32_t)p0;
          sm.bu[3] = (uint32_t)(first_pos_bin(cr.r1hi + 1) - 1);
          sm.bd[5] = (full_k ? 0.0 : cmass(cr.r1lo - 1)) - (p0 > 0 ? (full_k ? 0.0 : sq[p0 - 1]) : 0.0);
          sm.bd[6] = (double)P.top_p * ctot;
          sm.bu[5] = 0x7FFFFFFF;
        }
        __syncthreads();
        // top-p crossing: the first tie-group end e in range whose
        // cumulative mass reaches p * C_tot (parallel over positions)
        if (topp && !(sm.bu[0] & 1u)) {
          const int p0 = (int)sm.bu[2], p1 = (int)sm.bu[3];
          const double base = sm.bd[5], target = sm.bd[6];
          for (int e = p0 + tid; e <= p1; e += kBlock) {
            const bool end = (e == n - 1) || (sz[e + 1] != sz[e]);
            if (end && base + sq[e] >= target) atomicMin(&sm.bu[5], (uint32_t)e);
          }
        }
        __syncthreads();
        if (tid == 0) {
          uint32_t flags = sm.bu[0];
          uint32_t t = sm.bu[1];
          if (topp && !flags) {
            const uint32_t e = sm.bu[5];
            if (e == 0x7FFFFFFFu) flags |= 1u;
            else t = max(t, fkey(sz[e]));
          }
          if (minp) t = max(t, t_m);
          double S_K = atomic_ld(&rec->dd[0]);
          if (!flags && truncated && want_S) {
            const int e = last_pos_ge(t);
            const int bt = win_bin(mf, key_to_float(t));
            if (full_k && bt <= cr.rkhi) {
              S_K = qsum(0, e);
            } else if (bt < kMassBins) {
              S_K = cmass(bt - 1) + qsum(first_pos_bin(bt), e);
            } else {
              flags |= 1u;
            }
          }
          const double lns = log(S_K);
          if (!flags && K > 0) {
            const int kept_n = truncated ? last_pos_ge(t) + 1 : n;
            int w = 0;
            for (int j = 0; j < kept_n && w < K; ++j) {
              if (sz[j] > -INFINITY) {
                kp.top_lp_vals[(int64_t)row * K + w] = (float)(((double)sz[j] - m) - lns);
                kp.top_lp_ids[(int64_t)row * K + w] = si[j];
                ++w;
              }
            }
            for (; w < K; ++w) {
              kp.top_lp_vals[(int64_t)row * K + w] = -INFINITY;
              kp.top_lp_ids[(int64_t)row * K + w] = -1;
            }
          }
          atomic_st(&rec->dec[D_FLAGS], flags);
          atomic_st(&rec->dec[D_TAU], t);
          atomic_st(&rec->dd[1], lns);
        }
        group_release(rc.gsync);
      } else {
        group_wait(sm, rc.gsync, rc.abort_word, rc.epoch);
      }
      if (tid == 0) {
        sm.bu[4] = atomic_ld(&rec->dec[D_FLAGS]);
        sm.bu[13] = atomic_ld(&rec->dec[D_TAU]);
        sm.bd[2] = atomic_ld(&rec->dd[1]);
      }
      __syncthreads();
      general = sm.bu[4] & 1u;
      tau = sm.bu[13];
      lnS = sm.bd[2];
      __syncthreads();
    }

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
      for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
        const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (fkey(zv[c]) >= tau) ls += exp((double)zv[c] - m);
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
          for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
            const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if (zv[c] > -INFINITY && fkey(zv[c]) >= tau) {
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

    // ---- 5. emit probs / logprobs, Gumbel-max candidates
    const bool gumbel = !top1 && kp.path != PATH_GREEDY;
    double best_g = -INFINITY;
    float best_a = -INFINITY;
    int best_i = 0x7FFFFFFF;
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const uint32_t off0 = (uint32_t)P.offset, off1 = (uint32_t)(P.offset >> 32);
    for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
      const f32x4 zv = *reinterpret_cast<const f32x4 *>(zs + l);
      const int i0 = s0 + l;
      bool kk[4];
      bool any_cand = false;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kk[c] = fkey(zv[c]) >= tau;
        any_cand |= kk[c] && (mf - zv[c] <= kPruneNats);
      }
      if (want_out) {
        float pv[4], lv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float lp = kk[c] ? (float)(((double)zv[c] - m) - lnS) : -INFINITY;
          lv[c] = lp;
          pv[c] = kk[c] ? expf(lp) : 0.0f;
        }
        const int64_t o = (int64_t)row * V + i0;
        if ((kp.vec_ok & 2) && l + 3 < rc.n) {
          if (kp.probs) {
            const f32x4 t = {pv[0], pv[1], pv[2], pv[3]};
            __builtin_nontemporal_store(t, reinterpret_cast<f32x4 *>(kp.probs + o));
          }
          if (kp.logprobs) {
            const f32x4 t = {lv[0], lv[1], lv[2], lv[3]};
            __builtin_nontemporal_store(t, reinterpret_cast<f32x4 *>(kp.logprobs + o));
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (l + c < rc.n) {
              if (kp.probs) kp.probs[o + c] = pv[c];
              if (kp.logprobs) kp.logprobs[o + c] = lv[c];
            }
          }
        }
      }
      if (gumbel && any_cand) {
        uint32_t w[4];
        philox4x32_10((uint32_t)i0 >> 2, P.stream, off0, off1, key0, key1, w);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (kk[c] && (mf - zv[c] <= kPruneNats)) {
            const float ga = (zv[c] - mf) - ln_exp1_f32(w[c]);
            if (ga > best_a - kVerifyMargin) {
              const double ge = (double)zv[c] - log(exp1_f64(w[c]));
              if (ge > best_g) {
                best_g = ge;
                best_i = i0 + c;
                best_a = ga;
              }
            }
          }
        }
      }
    }
    if (gumbel) wg_best(sm, best_g, best_i);

    // ---- 6. final exchange: the last workgroup to arrive writes the row
    const unsigned fpar = it & 1u;
    if (tid == 0) {
      atomic_st(&rc.my->fin[fpar][0], best_g);
      atomic_st(&rc.my->fin[fpar][1], (double)best_i);
    }
    if (general)
      for (int t = tid; t < K; t += kBlock) atomic_st(&rc.my->toplist[fpar][t], sm.tl[t]);
    mem_quiesce();
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t old = __hip_atomic_fetch_add(&rc.gsync->fin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == (uint32_t)G - 1u;
      if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(&rc.gsync->fin, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int token = argmax_idx;
        if (gumbel) {
          double bg = -INFINITY;
          int bi = 0x7FFFFFFF;
          for (int g = 0; g < G; ++g) {
            const double gg = atomic_ld(&rc.peers[g].fin[fpar][0]);
            const int gi = (int)atomic_ld(&rc.peers[g].fin[fpar][1]);
            if (gg > bg || (gg == bg && gi < bi)) {
              bg = gg;
              bi = gi;
            }
          }
          if (bi != 0x7FFFFFFF) token = bi;
        }
        const bool aborted = atomic_ld(kp.abort_word) == kp.epoch;
        kp.token_ids[row] = aborted ? -1 : token;
        if (kp.row_status) kp.row_status[row] = aborted ? 3 : 0;
        if (general && K > 0) {
          // merge the G local lists: K rounds of a max below the previous pick
          unsigned long long lastk = ~0ull;
          for (int t = 0; t < K; ++t) {
            unsigned long long best = 0;
            for (int g = 0; g < G; ++g)
              for (int u = 0; u < K; ++u) {
                const unsigned long long c = atomic_ld(&rc.peers[g].toplist[fpar][u]);
                if (c < lastk && c > best) best = c;
              }
            lastk = best;
            const int64_t o = (int64_t)row * K + t;
            if (best == 0) {
              kp.top_lp_vals[o] = -INFINITY;
              kp.top_lp_ids[o] = -1;
            } else {
              const float zz = key_to_float((uint32_t)(best >> 32));
              kp.top_lp_vals[o] = (float)(((double)zz - m) - lnS);
              kp.top_lp_ids[o] = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

template <typename TIn, bool PEN>
hipError_t launch_t(const KernelParams &kp, hipStream_t stream) {
  void *args[] = {const_cast<KernelParams *>(&kp)};
  const size_t lds = kernel_lds_bytes(kp.slice, kp.hash_slots, PEN);
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&row_kernel<TIn, PEN>),
                                    dim3(kp.n_groups * kp.G), dim3(kBlock), args, (unsigned)lds, stream);
}

template <typename TIn, bool PEN>
hipError_t set_lds_attr(size_t lds) {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&row_kernel<TIn, PEN>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

}  // namespace

size_t kernel_lds_fixed() { return sizeof(SmemBase); }

size_t kernel_lds_region(int slice, int hash_slots, bool penalties) {
  // window histogram (masses first, 8-byte aligned), then the leader's
  // candidate arrays after it
  const size_t hist = sizeof(unsigned long long) * (kMassBins + 1) + sizeof(uint32_t) * (kWinBins + 4);
  size_t r = hist + (sizeof(float) + sizeof(int32_t)) * 2 * (size_t)kCandCap + sizeof(double) * kCandCap;
  const size_t radix = 2 * 256 * sizeof(uint32_t) + 2 * 256 * sizeof(unsigned long long);
  r = r > radix ? r : radix;
  if (penalties) {
    const size_t pen = sizeof(uint32_t) * ((size_t)hash_slots + ((size_t)slice + 31) / 32 + 1);
    r = r > pen ? r : pen;
  }
  return (r + 15) & ~(size_t)15;
}

size_t kernel_lds_bytes(int slice, int hash_slots, bool penalties) {
  return kernel_lds_fixed() + sizeof(float) * (size_t)slice + kernel_lds_region(slice, hash_slots, penalties);
}

hipError_t launch_step(const KernelParams &kp, int dtype, bool penalties, hipStream_t stream) {
  if (dtype == 0) return penalties ? launch_t<float, true>(kp, stream) : launch_t<float, false>(kp, stream);
  return penalties ? launch_t<uint16_t, true>(kp, stream) : launch_t<uint16_t, false>(kp, stream);
}

hipError_t resident_blocks(int device, size_t lds_bytes, int *out) {
  hipError_t e;
  if ((e = set_lds_attr<float, true>(lds_bytes)) != hipSuccess) return e;
  if ((e = set_lds_attr<float, false>(lds_bytes)) != hipSuccess) return e;
  if ((e = set_lds_attr<uint16_t, true>(lds_bytes)) != hipSuccess) return e;
  if ((e = set_lds_attr<uint16_t, false>(lds_bytes)) != hipSuccess) return e;
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
