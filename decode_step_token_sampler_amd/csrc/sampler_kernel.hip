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
//   2. exchange 1: row max, first argmax, sum of exp(z - max) (fp64)
//   3. filtered rows: thresholds by radix select on order-preserving keys,
//      one exchange per 8-bit digit: top-k by count, top-p by mass (2^-44
//      fixed point, so the sums do not depend on the summation order);
//      min-p's fp64 test bounds an upper set of keys, found by bisection;
//      then the kept-set sum (exchange)
//   4. emit probs / logprobs of the kept set; Gumbel-max with an in-kernel
//      Philox draw, an fp32 log-domain filter and an fp64 check of every
//      element that can still win; local top-logprob candidates
//   5. the last workgroup to arrive merges the candidates and writes the
//      token, status and top logprobs
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
  uint32_t hcnt[256];
  unsigned long long hmass[256];
  uint32_t mcnt[256];
  unsigned long long mmass[256];
  unsigned long long tl[kMaxTopLogprobs];
  uint32_t bu[8];
  double bd[8];
  uint32_t bitmap[kMaxSlice / 32];  // history ids of the slice (penalty rows)
};

// ---------------------------------------------------------------- helpers
// Opaque copy: per-element work derived from it stays inside the phase that
// needs it instead of being hoisted (and kept live) across phases.
DEV float opq(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
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

// Group barrier.  Wave 0 has written this workgroup's exchange data with
// agent-scope stores; its release fence orders them before the arrival.
// The last of the G arrivals resets the count and bumps the generation.
// The wait is bounded (~2 s): on expiry the launch is marked aborted (the
// abort word takes this launch's epoch), every waiter of the launch stops
// waiting, and the rows report status 3, so a logic error cannot hang the
// device.  Returns false once the launch is aborted.
constexpr uint32_t kSpinLimit = 1u << 26;
DEV bool group_barrier(GroupSync *s, int G, uint32_t *abort_word, uint32_t epoch) {
  if (threadIdx.x < 64) {
    __atomic_thread_fence(__ATOMIC_RELEASE);
    if (threadIdx.x == 0) {
      uint32_t g0 = __hip_atomic_load(&s->gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t old = __hip_atomic_fetch_add(&s->count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (old == (uint32_t)G - 1u) {
        __hip_atomic_store(&s->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(&s->gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        uint32_t spins = 0;
        while (__hip_atomic_load(&s->gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == g0) {
          if (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) break;
          if (++spins > kSpinLimit) {
            __hip_atomic_store(abort_word, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
  }
  __syncthreads();
  return __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch;
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

DEV double exp_d(double x) { return exp(x); }
DEV double log_d(double x) { return log(x); }

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

// Per-row context shared by the phases.
struct RowCtx {
  int row, gid, G, n;      // n: slice length (valid values); the LDS slice is padded to n4 with -inf
  int n4;
  GroupSync *gsync;
  uint32_t *abort_word;
  uint32_t epoch;
  WgSlots *my;
  WgSlots *peers;
  unsigned *xseq;
};

// Radix select over the order-preserving keys of the slice values with
// key >= lower, one group exchange per 8-bit digit.
//   COUNT: the key of the value of rank k in descending order (ties share a
//          key): #{key > t} < k <= #{key >= t}.
//   MASS:  the largest key t whose cumulative mass C(t) = sum_{key >= t}
//          exp(z - m) reaches p * C(lower); masses are summed in 2^-44 fixed
//          point so the totals do not depend on the summation order.
// Padding values are -inf: lowest bin, zero mass, so they never move a
// threshold above -inf.
template <bool MASS>
DEV uint32_t radix_select(SmemBase &sm, RowCtx &rc, const float *zs, uint32_t lower, uint32_t k, double p,
                          double m) {
  uint32_t prefix = 0, mask = 0;
  uint32_t rem_cnt = k;
  unsigned long long above = 0;  // mass strictly above the current prefix range
  double target = 0.0;
  for (int round = 0; round < 4; ++round) {
    const int shift = 24 - 8 * round;
    for (int b = threadIdx.x; b < 256; b += kBlock) {
      sm.hcnt[b] = 0;
      sm.hmass[b] = 0;
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
          if (MASS) {
            const double q = exp((double)zz - m);
            atomicAdd(&sm.hmass[bin], (unsigned long long)(q * kMassScale));
          } else {
            atomicAdd(&sm.hcnt[bin], 1u);
          }
        }
      }
    }
    __syncthreads();
    const unsigned par = (*rc.xseq)++ & 1u;
    if (threadIdx.x < 64) {
      for (int b = threadIdx.x; b < 256; b += 64) {
        if (MASS) atomic_st(&rc.my->hmass[par][b], sm.hmass[b]);
        else atomic_st(&rc.my->hcnt[par][b], sm.hcnt[b]);
      }
    }
    group_barrier(rc.gsync, rc.G, rc.abort_word, rc.epoch);
    if (threadIdx.x < 256) {
      const int b = threadIdx.x;
      if (MASS) {
        unsigned long long t = 0;
        for (int g = 0; g < rc.G; ++g) t += atomic_ld(&rc.peers[g].hmass[par][b]);
        sm.mmass[b] = t;
      } else {
        uint32_t t = 0;
        for (int g = 0; g < rc.G; ++g) t += atomic_ld(&rc.peers[g].hcnt[par][b]);
        sm.mcnt[b] = t;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t digit = 0;
      if (MASS) {
        if (round == 0) {
          unsigned long long tot = 0;
          for (int b = 0; b < 256; ++b) tot += sm.mmass[b];
          target = p * (double)tot;
        }
        unsigned long long acc = above;
        for (int b = 255; b >= 0; --b) {
          const unsigned long long nxt = acc + sm.mmass[b];
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
          if (acc + sm.mcnt[b] >= rem_cnt || b == 0) {
            digit = (uint32_t)b;
            break;
          }
          acc += sm.mcnt[b];
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

template <typename TIn, bool PEN>
__global__ __launch_bounds__(kBlock) void row_kernel(KernelParams kp) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  SmemBase &sm = *reinterpret_cast<SmemBase *>(lds_raw);
  static_assert(sizeof(SmemBase) % 16 == 0, "the LDS slice must be 16-byte aligned");
  float *zs = reinterpret_cast<float *>(lds_raw + sizeof(SmemBase));
  uint32_t *hash = reinterpret_cast<uint32_t *>(zs + kp.slice);

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
  rc.abort_word = kp.abort_word;
  rc.epoch = kp.epoch;
  rc.my = kp.slots + blockIdx.x;
  rc.peers = kp.slots + (size_t)group * G;
  rc.xseq = &xseq;
  const bool want_out = kp.probs != nullptr || kp.logprobs != nullptr;
  const int s0 = gid * kp.slice;
  const int s1 = min(V, s0 + kp.slice);
  rc.n = s1 - s0;
  rc.n4 = (rc.n + 3) & ~3;

  unsigned it = 0;
  for (int row = group; row < kp.n_rows; row += kp.n_groups, ++it) {
    const RowParam P = kp.rows[row];
    rc.row = row;
    const bool greedy = P.flags & RF_GREEDY;
    const bool top1 = P.flags & RF_TOP1;
    const bool pen = PEN && (P.flags & RF_PEN);

    // ---- penalties: counts of the history ids that fall in this slice,
    // plus a bitmap of those ids for the load pass
    if (pen) {
      for (int t = tid; t < (int)hslots; t += kBlock) hash[t] = kEmpty;
      for (int t = tid; t < kMaxSlice / 32; t += kBlock) sm.bitmap[t] = 0;
      __syncthreads();
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
          atomicOr(&sm.bitmap[local >> 5], 1u << (local & 31));
        }
      }
      __syncthreads();
    }

    // ---- 1. load, sanitise, divide by the temperature; history tokens are
    // stored raw and finished by the penalty pass below.  Loads of a thread
    // are issued together at clamped in-bounds addresses; with vector loads
    // the row stride is a multiple of 4, so a group starting below s1 lies
    // inside the row.
    {
      const int64_t rbase = (int64_t)row * kp.row_stride + s0;
      const int lastg = (rc.n - 1) & ~3;
      constexpr int kBatch = 8;
      for (int l0 = 4 * tid; l0 < rc.n4; l0 += 4 * kBlock * kBatch) {
        float v[kBatch][4];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int l = l0 + 4 * kBlock * b;
          if (kp.vec_ok & 1) {
            Loader<TIn>::load4(kp.logits, rbase + min(l, lastg), v[b]);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[b][c] = Loader<TIn>::load1(kp.logits, rbase + min(l + c, rc.n - 1));
          }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int l = l0 + 4 * kBlock * b;
          if (l < rc.n4) {
            const uint32_t pb = pen ? (sm.bitmap[l >> 5] >> (l & 31)) & 0xFu : 0u;
            f32x4 o;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              float x = v[b][c];
              x = (l + c < rc.n && x == x) ? x : -INFINITY;
              if (!((pb >> c) & 1u)) x = x / P.temperature + 0.0f;  // -0 -> +0: equal values share one key
              o[c] = x;
            }
            *reinterpret_cast<f32x4 *>(zs + l) = o;
          }
        }
      }
    }
    if (pen) {
      __syncthreads();
      // each distinct history id of the slice owns one hash slot
      for (int t = tid; t < (int)hslots; t += kBlock) {
        const uint32_t e = hash[t];
        if (e != kEmpty) {
          const uint32_t local = e >> 13, cnt = e & 0x1FFFu;
          zs[local] = apply_penalty(zs[local], cnt, P) / P.temperature + 0.0f;
        }
      }
    }
    __syncthreads();

    // ---- 2. exchange 1: max, first argmax, sum of exp(z - local max)
    float lmax = -INFINITY;
    unsigned long long lam = 0;  // (key << 32) | ~index : max = largest value, lowest index
    for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lmax = fmaxf(lmax, v[c]);
        const unsigned long long k = ((unsigned long long)fkey(v[c]) << 32) | (0xFFFFFFFFu - (uint32_t)(s0 + l + c));
        lam = k > lam ? k : lam;
      }
    }
    const float wmax = wg_max_f(sm, lmax);
    const unsigned long long wam = wg_max_u(sm, lam);
    double lsum = 0.0;
    if (wmax > -INFINITY && wmax < INFINITY) {
      for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
        for (int c = 0; c < 4; ++c) lsum += exp((double)v[c] - (double)wmax);
      }
    }
    const double wsum = wg_sum_d(sm, lsum);
    {
      const unsigned par = xseq++ & 1u;
      if (tid == 0) {
        atomic_st(&rc.my->small[par][0], (double)wmax);
        atomic_st(&rc.my->small[par][1], wsum);
        atomic_st(&rc.my->small[par][2], __longlong_as_double((long long)wam));
      }
      group_barrier(rc.gsync, G, rc.abort_word, rc.epoch);
      if (tid == 0) {
        double gm = -INFINITY;
        unsigned long long am = 0;
        for (int g = 0; g < G; ++g) {
          gm = fmax(gm, atomic_ld(&rc.peers[g].small[par][0]));
          const unsigned long long a =
              (unsigned long long)__double_as_longlong(atomic_ld(&rc.peers[g].small[par][2]));
          am = a > am ? a : am;
        }
        double S = 0.0;
        if (gm > -INFINITY && gm < INFINITY) {
          for (int g = 0; g < G; ++g) {
            const double mg = atomic_ld(&rc.peers[g].small[par][0]);
            if (mg > -INFINITY) S += atomic_ld(&rc.peers[g].small[par][1]) * exp(mg - gm);
          }
        }
        sm.bd[0] = gm;
        sm.bd[1] = S;
        sm.bu[0] = 0xFFFFFFFFu - (uint32_t)(am & 0xFFFFFFFFu);
      }
      __syncthreads();
    }
    const double m = sm.bd[0];
    double S_K = sm.bd[1];
    const int argmax_idx = (int)sm.bu[0];
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
        for (int t = 0; t < kp.top_lp; ++t) {
          kp.top_lp_vals[(int64_t)row * kp.top_lp + t] = -INFINITY;
          kp.top_lp_ids[(int64_t)row * kp.top_lp + t] = -1;
        }
      }
      __syncthreads();
      continue;
    }

    // ---- 3. truncation thresholds (filtered rows): kept <=> key >= tau
    uint32_t tau = 0;
    const bool truncated = !greedy && (P.flags & (RF_TOP1 | RF_TOPK | RF_TOPP | RF_MINP));
    if (!greedy) {
      if (top1) {
        tau = fkey((float)m);
      } else {
        if (P.flags & RF_TOPK) tau = radix_select<false>(sm, rc, zs, 0u, (uint32_t)P.top_k, 0.0, m);
        if (P.flags & RF_TOPP) {
          const uint32_t tp = radix_select<true>(sm, rc, zs, tau, 0u, (double)P.top_p, m);
          tau = tp > tau ? tp : tau;
        }
      }
      // min-p keeps exp(z - m) >= min_p (fp64).  That set is an upper set of
      // keys, so its boundary key is found once per row by bisection with
      // the same test.
      if (P.flags & RF_MINP) {
        if (tid == 0) {
          const double min_p = (double)P.min_p;
          uint32_t lo = 0, hi = fkey((float)m);  // the test holds at hi, fails at 0
          while (hi - lo > 1u) {
            const uint32_t mid = lo + (hi - lo) / 2u;
            if (exp((double)key_to_float(mid) - m) >= min_p) hi = mid;
            else lo = mid;
          }
          sm.bu[3] = hi;
        }
        __syncthreads();
        tau = sm.bu[3] > tau ? sm.bu[3] : tau;
        __syncthreads();
      }
    }
    if (truncated && (want_out || kp.top_lp > 0)) {
      double ls = 0.0;
      for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (fkey(v[c]) >= tau) ls += exp((double)v[c] - m);
      }
      const double ws = wg_sum_d(sm, ls);
      const unsigned par = xseq++ & 1u;
      if (tid == 0) atomic_st(&rc.my->small[par][3], ws);
      group_barrier(rc.gsync, G, rc.abort_word, rc.epoch);
      if (tid == 0) {
        double t = 0.0;
        for (int g = 0; g < G; ++g) t += atomic_ld(&rc.peers[g].small[par][3]);
        sm.bd[2] = t;
      }
      __syncthreads();
      S_K = sm.bd[2];
      __syncthreads();
    }
    const double lnS = log(S_K);

    // ---- 4. emit probs / logprobs, Gumbel-max candidates
    const bool gumbel = !top1 && kp.path != PATH_GREEDY;
    double best_g = -INFINITY;
    float best_a = -INFINITY;
    int best_i = 0x7FFFFFFF;
    const uint32_t key0 = (uint32_t)P.seed, key1 = (uint32_t)(P.seed >> 32);
    const uint32_t off0 = (uint32_t)P.offset, off1 = (uint32_t)(P.offset >> 32);
    const float mf = (float)m;
    for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(zs + l);
      const int i0 = s0 + l;
      bool kk[4];
      bool any_cand = false;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kk[c] = fkey(v[c]) >= tau;
        any_cand |= kk[c] && (mf - v[c] <= kPruneNats);
      }
      if (want_out) {
        float pv[4], lv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float lp = kk[c] ? (float)(((double)v[c] - m) - lnS) : -INFINITY;
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
          if (kk[c] && (mf - v[c] <= kPruneNats)) {
            const float ga = (v[c] - mf) - ln_exp1_f32(w[c]);
            if (ga > best_a - kVerifyMargin) {
              const double ge = (double)v[c] - log(exp1_f64(w[c]));
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

    // ---- local top-logprob candidates: K rounds of a (value, index) max
    const int K = kp.top_lp;
    if (K > 0) {
      unsigned long long last = ~0ull;
      for (int t = 0; t < K; ++t) {
        unsigned long long cand = 0;
        for (int l = 4 * tid; l < rc.n4; l += 4 * kBlock) {
          const f32x4 v = *reinterpret_cast<const f32x4 *>(zs + l);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (v[c] > -INFINITY && fkey(v[c]) >= tau) {
              const unsigned long long ck =
                  ((unsigned long long)fkey(v[c]) << 32) | (0xFFFFFFFFu - (uint32_t)(s0 + l + c));
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

    // ---- 5. final exchange: the last workgroup to arrive writes the row
    const unsigned fpar = it & 1u;
    if (tid < 64) {
      if (tid == 0) {
        atomic_st(&rc.my->fin[fpar][0], best_g);
        atomic_st(&rc.my->fin[fpar][1], (double)best_i);
      }
      for (int t = tid; t < K; t += 64) atomic_st(&rc.my->toplist[fpar][t], sm.tl[t]);
      __atomic_thread_fence(__ATOMIC_RELEASE);
      if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&rc.gsync->fin, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        sm.bu[4] = (old == (uint32_t)G - 1u) ? 1u : 0u;
      }
    }
    __syncthreads();
    if (sm.bu[4] && tid == 0) {
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
      // merge the G local lists: K rounds of a max below the previous pick
      unsigned long long last = ~0ull;
      for (int t = 0; t < K; ++t) {
        unsigned long long best = 0;
        for (int g = 0; g < G; ++g)
          for (int u = 0; u < K; ++u) {
            const unsigned long long c = atomic_ld(&rc.peers[g].toplist[fpar][u]);
            if (c < last && c > best) best = c;
          }
        last = best;
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

size_t kernel_lds_fixed() { return (sizeof(SmemBase) + 15) & ~(size_t)15; }

size_t kernel_lds_bytes(int slice, int hash_slots, bool penalties) {
  return kernel_lds_fixed() + sizeof(float) * (size_t)slice + (penalties ? sizeof(uint32_t) * (size_t)hash_slots : 0);
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
