/*
 * sampler_oracle.c -- plain, slow CPU oracle for the per-decode-step token
 * sampler.  TEST INFRASTRUCTURE ONLY: it exists to check the HIP library
 * against a transparent implementation.  Only tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product never does.
 *
 * It shares no code, header, table or constant generator with the HIP
 * library.  Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (scalar code; fp32 steps are rounded one operation at a time, everything
 * after the temperature division is fp64).
 *
 * Sources (the pages this follows; each function cites the passage):
 *   [A] "SGLang's +75% sampler speedup skips Qwen3 chat requests" (dev.to)
 *   [B] the SGLang 101 operations manual (aiengineeringfromscratch.com),
 *       sections "Logprobs are temperature-scaled" and "What the flag switches"
 *   [C] "采样参数对解码开销的影响：temperature、top_p 与采样核路径"
 *       (xbrilliance.ai note on sampling-parameter decode cost)
 *   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
 *       as easy as 1, 2, 3", SC'11.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - penalties: repetition (divide positive / multiply non-positive logits),
 *     then frequency (minus f*count), then presence (minus p), only where the
 *     token occurs in the row's history; each op rounded to fp32.
 *   - truncation order top-k -> top-p (on the top-k renormalised mass) ->
 *     min-p (relative to the row maximum); thresholds keep ties.
 *   - probs/logprobs are those of the distribution sampled from (after
 *     truncation); greedy rows are untruncated at temperature 1.
 *   - Gumbel-max over the kept set with Philox4x32-10 draws, counter
 *     (i>>2, stream, off_lo, off_hi), key (seed_lo, seed_hi), word i&3.
 *   - top-k logprobs list the K largest kept values by (z desc, index asc);
 *     entries with z = -inf are never listed; padding is (-inf, -1).
 *   - logits processors run first, in this order: grammar bitmask (cleared
 *     bit -> -inf), logit_bias (a token's entries summed, then added once;
 *     NaN -> -inf), min_tokens (stop ids -> -inf while fewer than min_tokens
 *     tokens were produced); then penalties and temperature.
 *   - logprob modes: processed (after truncation, the default), temperature
 *     (untruncated log_softmax(z)), raw (untruncated, before temperature).
 *   - inverse-CDF selection (the seeded multinomial): u from the Philox
 *     block at counter (0xFFFFFFFF, stream, off_lo, off_hi), 53 bits; the
 *     first kept token in index order whose running kept mass exceeds u
 *     times the kept total.
 *
 * Parity pins: see tests/test_oracle_*.py.  The penalty formula is not
 * fixed by the pages: its repetition term is pinned against the transformers
 * library's repetition-penalty processor, and the frequency and presence
 * terms by invariants (presence lowers a seen token by a constant whatever
 * its count, frequency lowers it linearly in the count, the two add).  The
 * order of the three is a reading the pages leave open: "parity unpinned".
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_TOP_K_ALL (1 << 30)   /* [A] "One request with top_p ..." : -1 becomes 1<<30 */
#define ORC_GREEDY_EPS 1e-6       /* [A] same section: temperature below 1e-6 is greedy */
#define ORC_NEAR_TIE 1e-6         /* relative gap under which a Gumbel row is flagged */
#define ORC_TOPP_MARGIN 1e-6      /* relative top-p margin under which a row is flagged */
#define ORC_MINP_MARGIN 1e-9      /* relative min-p boundary margin (flag) */

/* path codes */
#define ORC_PATH_GREEDY 0
#define ORC_PATH_GUMBEL 1
#define ORC_PATH_FILTERED 2
#define ORC_PATH_DETERMINISTIC 3

/* per-row diagnostic flags */
#define ORC_FLAG_GUMBEL_NEAR_TIE 1
#define ORC_FLAG_TOPP_MARGIN 2
#define ORC_FLAG_MINP_MARGIN 4
#define ORC_FLAG_SPELLING_MISMATCH 8
#define ORC_FLAG_ICDF_MARGIN 16
#define ORC_ICDF_MARGIN 1e-10       /* relative distance of u*S from a CDF step (flag) */

typedef struct {
  const void *logits;       /* [n_rows, row_stride] fp32 or bf16 bits (host) */
  int32_t dtype;            /* 0 = fp32, 1 = bf16 */
  int32_t n_rows;
  int32_t vocab;
  int64_t row_stride;       /* elements */
  const float *temperature; /* each array: n_rows entries, NULL = default */
  const float *top_p;
  const float *min_p;
  const float *repetition_penalty;
  const float *presence_penalty;
  const float *frequency_penalty;
  const int32_t *top_k;
  const int32_t *history_ids;   /* host copy of the id buffer */
  const int64_t *history_start; /* per row */
  const int32_t *history_len;   /* per row */
  uint64_t seed;
  uint64_t offset;
  const uint64_t *row_seed;
  const uint64_t *row_offset;
  const uint32_t *row_stream;
  int32_t deterministic;
  int32_t n_threads;
  /* outputs (host) */
  int32_t *token_ids;
  float *probs;             /* [n_rows, vocab] or NULL */
  float *logprobs;          /* [n_rows, vocab] or NULL */
  int32_t top_logprobs;
  float *top_logprob_vals;  /* [n_rows, top_logprobs] */
  int32_t *top_logprob_ids;
  int32_t *row_status;
  /* diagnostics, each [n_rows] or NULL */
  int32_t *diag_flags;
  double *diag_gumbel_gap;  /* (s1 - s2) / s1 of the Gumbel scores */
  double *diag_topp_margin; /* relative distance of the top-p crossing */
  int32_t *diag_kept;       /* |K| */
  /* logits processors, applied before the penalties (NULL = none) */
  const uint32_t *vocab_mask; /* [n_rows, mask_stride] words; bit i&31 of word i>>5: 1 = allowed */
  int64_t mask_stride;        /* words */
  const int32_t *bias_ids;    /* host copy of the bias id buffer */
  const float *bias_vals;     /* same length */
  const int64_t *bias_start;  /* per row */
  const int32_t *bias_len;    /* per row */
  const int32_t *stop_ids;    /* host copy of the stop id buffer */
  const int64_t *stop_start;  /* per row */
  const int32_t *stop_len;    /* per row */
  const int32_t *min_tokens;  /* per row */
  const int32_t *output_len;  /* per row: tokens generated so far */
  int32_t logprob_mode;       /* 0 processed, 1 temperature-scaled, 2 raw */
  int32_t inverse_cdf;        /* select by the seeded inverse CDF instead of Gumbel-max */
  int32_t *diag_token_alt;    /* [n_rows] or NULL: for a near-tie or inverse-CDF margin row, the token on
                                 the other side of the tie or step, else -1 */
} orc_args;

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11): ten rounds of the multiply /  */
/* xor round function; the key is bumped by the Weyl constants between */
/* rounds.                                                             */
/* ------------------------------------------------------------------ */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  const uint32_t MUL_A = 0xD2511F53u, MUL_B = 0xCD9E8D57u;
  const uint32_t WEYL_A = 0x9E3779B9u, WEYL_B = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += WEYL_A;
      k1 += WEYL_B;
    }
    uint64_t prod_a = (uint64_t)MUL_A * (uint64_t)c0;
    uint64_t prod_b = (uint64_t)MUL_B * (uint64_t)c2;
    uint32_t n0 = (uint32_t)(prod_b >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)prod_b;
    uint32_t n2 = (uint32_t)(prod_a >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)prod_a;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 32-bit word that vocabulary entry `i` of a row draws. */
uint32_t orc_draw_word(uint64_t seed, uint32_t stream, uint64_t offset, int64_t i) {
  uint32_t ctr[4] = {(uint32_t)((uint64_t)i >> 2), stream, (uint32_t)offset, (uint32_t)(offset >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[i & 3];
}

/* Exp(1) variate from one 32-bit word, as [A] "Nine lines..." draws it with
 * exponential_(1.0) followed by a clamp at the smallest normal float:
 * w = (x + 1/2) 2^-32 is uniform on (0,1); E = -ln(1 - w). */
double orc_exp1_from_word(uint32_t x) {
  double w = ((double)x + 0.5) * 0x1p-32;
  double e = -log1p(-w);
  if (e < (double)FLT_MIN) e = (double)FLT_MIN;
  return e;
}

/* The row's uniform for inverse-CDF selection: the Philox block at counter
 * (0xFFFFFFFF, stream, off_lo, off_hi) -- a counter no vocabulary entry
 * uses (entries use i >> 2 < 2^30) -- words 0 and 1 as a 64-bit integer,
 * its top 53 bits scaled to [0, 1). */
double orc_icdf_uniform(uint64_t seed, uint32_t stream, uint64_t offset) {
  uint32_t ctr[4] = {0xFFFFFFFFu, stream, (uint32_t)offset, (uint32_t)(offset >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  uint64_t x = ((uint64_t)out[1] << 32) | out[0];
  return (double)(x >> 11) * 0x1p-53;
}

/* Exp(1) variates of vocabulary entries 0..n-1 of one row (test helper). */
void orc_fill_exp1(uint64_t seed, uint32_t stream, uint64_t offset, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_exp1_from_word(orc_draw_word(seed, stream, offset, i));
}

/* bf16 -> fp32: the bf16 bits are the high half of the fp32 bits. */
static float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------ */
/* Normalisation and the batch predicate: [A] "One request with top_p  */
/* takes the whole batch off the fast path" (normalize and              */
/* path_for_batch, and the four-row path table).                        */
/* ------------------------------------------------------------------ */
int orc_row_is_greedy(float temperature) {
  return temperature >= 0.0f && (double)temperature < ORC_GREEDY_EPS;
}

int32_t orc_normalized_top_k(float temperature, int32_t top_k) {
  if (orc_row_is_greedy(temperature)) return 1;
  if (top_k == -1) return ORC_TOP_K_ALL;
  return top_k;
}

/* The path table of [A] "One request with top_p takes the whole batch off
 * the fast path", read as a function of the set of row classes present:
 * a batch with no sampling row (every row has top_k <= 1 after
 * normalisation) is greedy; one whose rows ask for no truncation at all
 * takes Gumbel-max (deterministic on a deterministic handle); a single row
 * with top-k (a greedy row counts: its top_k is 1), top-p or min-p makes
 * the whole batch filtered. */
enum { ORC_C_SAMPLING = 1, ORC_C_TOPK = 2, ORC_C_TOPP = 4, ORC_C_MINP = 8 };

static unsigned orc_row_classes(float temperature, int32_t top_k, float top_p, float min_p) {
  const int32_t k = orc_normalized_top_k(temperature, top_k);
  return (k > 1 ? ORC_C_SAMPLING : 0u) | (k != ORC_TOP_K_ALL ? ORC_C_TOPK : 0u) |
         (top_p != 1.0f ? ORC_C_TOPP : 0u) | (min_p > 0.0f ? ORC_C_MINP : 0u);
}

/* Returns 0 and writes the path, or -1 for an empty batch. */
int orc_select_path(int32_t n, const float *temperature, const int32_t *top_k, const float *top_p,
                    const float *min_p, int32_t deterministic, int32_t *path_out) {
  if (n <= 0) return -1;
  unsigned present = 0;
  for (int32_t r = 0; r < n; ++r)
    present |= orc_row_classes(temperature ? temperature[r] : 1.0f, top_k ? top_k[r] : -1,
                               top_p ? top_p[r] : 1.0f, min_p ? min_p[r] : 0.0f);
  const int32_t U = deterministic ? ORC_PATH_DETERMINISTIC : ORC_PATH_GUMBEL; /* untruncated sampling */
  const int32_t F = ORC_PATH_FILTERED, G = ORC_PATH_GREEDY;
  /* indexed by the classes present: bit 0 sampling, 1 top-k, 2 top-p, 3 min-p */
  const int32_t table[16] = {G, U, G, F, G, F, G, F, G, F, G, F, G, F, G, F};
  *path_out = table[present];
  return 0;
}

/* [C] "哪些参数会额外打开一趟全词表计算": do_penalties is raised by any row
 * whose presence, frequency or repetition penalty differs from its default
 * (compared exactly here). */
int orc_do_penalties(int32_t n, const float *rep, const float *pres, const float *freq) {
  for (int32_t r = 0; r < n; ++r) {
    if ((rep && rep[r] != 1.0f) || (pres && pres[r] != 0.0f) || (freq && freq[r] != 0.0f)) return 1;
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* One row.                                                            */
/* ------------------------------------------------------------------ */
typedef struct {
  float z;
  int32_t idx;
} orc_zi;

static int orc_cmp_desc(const void *pa, const void *pb) {
  const orc_zi *a = (const orc_zi *)pa, *b = (const orc_zi *)pb;
  if (a->z > b->z) return -1;
  if (a->z < b->z) return 1;
  return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

/* Neumaier-compensated sum (accuracy of the normaliser; order is index). */
typedef struct {
  double s, c;
} orc_ksum;
static void orc_kadd(orc_ksum *k, double v) {
  double t = k->s + v;
  if (fabs(k->s) >= fabs(v)) k->c += (k->s - t) + v;
  else k->c += (v - t) + k->s;
  k->s = t;
}
static double orc_kval(const orc_ksum *k) { return k->s + k->c; }

/* Working arrays of one row (one set per worker thread). */
typedef struct {
  float *z;              /* processed logits after temperature */
  float *xp;             /* processed logits before temperature (raw logprob mode) */
  orc_zi *ord;           /* the row in (z desc, index asc) order */
  double *q;             /* exp(z - m) */
  int32_t *cnt;          /* history counts */
  unsigned char *kept;   /* the kept set K */
} orc_work;

/* What steps 1-5 found for a row. */
#define ORC_MAX_NEAR 4
typedef struct {
  int status;            /* 0; 1: no finite value; 2: a +inf value */
  int greedy;
  int32_t k_eff;
  float m;
  int32_t n_p;           /* entries of the order that top-k and top-p keep */
  int32_t n_p_alt[2];    /* that prefix with the top-p crossing one tie group earlier / later; -1: not reachable */
  int32_t n_near;        /* values kept by top-k/top-p within the min-p margin of the boundary */
  float near_z[ORC_MAX_NEAR];
  double topp_margin;
  int32_t flags;
} orc_rowinfo;

/* Steps 1-4 of a row: load, logits processors, penalties, temperature,
 * row maximum and status. */
static void orc_row_values(const orc_args *a, int32_t r, orc_work *w, orc_rowinfo *info) {
  const int32_t V = a->vocab;
  float *z = w->z;
  const float T = a->temperature ? a->temperature[r] : 1.0f;
  const float rep = a->repetition_penalty ? a->repetition_penalty[r] : 1.0f;
  const float pres = a->presence_penalty ? a->presence_penalty[r] : 0.0f;
  const float freq = a->frequency_penalty ? a->frequency_penalty[r] : 0.0f;
  memset(info, 0, sizeof(*info));
  info->greedy = orc_row_is_greedy(T);
  info->k_eff = orc_normalized_top_k(T, a->top_k ? a->top_k[r] : -1);
  info->n_p_alt[0] = info->n_p_alt[1] = -1;
  info->topp_margin = INFINITY;
  const float T_eff = info->greedy ? 1.0f : T;

  /* 1. load; NaN becomes -inf ([B] "On Apple silicon" lists NaN
   *    sanitisation among the sampler options; here it is always on). */
  for (int32_t i = 0; i < V; ++i) {
    float x;
    if (a->dtype == 1) x = orc_bf16_to_f32(((const uint16_t *)a->logits)[(int64_t)r * a->row_stride + i]);
    else x = ((const float *)a->logits)[(int64_t)r * a->row_stride + i];
    if (isnan(x)) x = -INFINITY;
    z[i] = x;
  }

  /* 1b. logits processors, before the sampler's own steps.
   *    Grammar mask ([B] "Constrained decoding", step 4 "Mask": the grammar
   *    fills a vocabulary bitmask that is applied to the logits before
   *    sampling): a cleared bit makes the logit -inf.
   *    logit_bias (listed among the sampler options in [B] "On Apple
   *    silicon"): every entry of the row's list adds its value to its
   *    token's logit; entries of one token are summed first (in list
   *    order), then added once.  A NaN result becomes -inf.
   *    min_tokens ([C] "解码一步里采样做什么", step _apply_min_tokens_penalty):
   *    while the row has produced fewer than min_tokens tokens, each of
   *    its stop ids is made -inf.  Ids outside [0, V) are ignored. */
  if (a->vocab_mask) {
    const uint32_t *mw = a->vocab_mask + (int64_t)r * a->mask_stride;
    for (int32_t i = 0; i < V; ++i)
      if (((mw[i >> 5] >> (i & 31)) & 1u) == 0u) z[i] = -INFINITY;
  }
  if (a->bias_len && a->bias_len[r] > 0 && a->bias_ids && a->bias_vals && a->bias_start) {
    const int32_t *bi = a->bias_ids + a->bias_start[r];
    const float *bv = a->bias_vals + a->bias_start[r];
    const int32_t nb = a->bias_len[r];
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t id = bi[j];
      if (id < 0 || id >= V) continue;
      int first = 1;
      for (int32_t j2 = 0; j2 < j; ++j2)
        if (bi[j2] == id) first = 0;
      if (!first) continue; /* this token's total was added at its first entry */
      float total = bv[j];
      for (int32_t j2 = j + 1; j2 < nb; ++j2)
        if (bi[j2] == id) total = total + bv[j2];
      float x = z[id] + total;
      z[id] = isnan(x) ? -INFINITY : x;
    }
  }
  if (a->min_tokens && a->output_len && a->output_len[r] < a->min_tokens[r] && a->stop_ids && a->stop_start &&
      a->stop_len) {
    const int32_t *st = a->stop_ids + a->stop_start[r];
    for (int32_t j = 0; j < a->stop_len[r]; ++j)
      if (st[j] >= 0 && st[j] < V) z[st[j]] = -INFINITY;
  }

  /* 2. penalties ([C] "解码一步里采样做什么", step _apply_penalties):
   *    counts of each token in the row's history, then the three penalties
   *    on the tokens that occur.  Ids outside [0, V) are ignored. */
  if (a->history_len && a->history_len[r] > 0 && a->history_ids && a->history_start) {
    int32_t *cnt = w->cnt;
    memset(cnt, 0, sizeof(int32_t) * (size_t)V);
    const int32_t *h = a->history_ids + a->history_start[r];
    for (int32_t j = 0; j < a->history_len[r]; ++j) {
      int32_t id = h[j];
      if (id >= 0 && id < V) cnt[id] += 1;
    }
    for (int32_t i = 0; i < V; ++i) {
      if (cnt[i] > 0) {
        float x = z[i];
        float t1 = (x > 0.0f) ? (x / rep) : (x * rep);
        float fc = freq * (float)cnt[i];
        float t2 = t1 - fc;
        float t3 = t2 - pres;
        z[i] = t3;
      }
    }
  }

  /* the processed logits before temperature, for the raw logprob mode */
  if (a->logprob_mode == 2) memcpy(w->xp, z, sizeof(float) * (size_t)V);

  /* 3. temperature ([C] same section: logits.div_(temperatures)) */
  for (int32_t i = 0; i < V; ++i) z[i] = z[i] / T_eff;

  /* 4. row maximum */
  float m = -INFINITY;
  for (int32_t i = 0; i < V; ++i)
    if (z[i] > m) m = z[i];
  info->m = m;
  info->status = (m == INFINITY) ? 2 : (m > -INFINITY ? 0 : 1);
}

/* Step 5, truncation ([C] "解码一步里采样做什么": _apply_top_k_top_p, then
 * _apply_min_p), for a row with status 0: q_i = exp(z_i - m), the order,
 * the kept set K in w->kept, and the row's boundary diagnostics.  Greedy rows
 * keep every token (their distribution is the one at temperature 1).
 *
 * The diagnostics mark a rule's boundary only where that rule decides K:
 *   - top-p: the crossing's distance from the target mass, relative to the
 *     top-k mass.  Within ORC_TOPP_MARGIN, rounding of the masses could
 *     move the crossing one tie group earlier (hi side) or later (lo side);
 *     the row is flagged when such a move changes K, i.e. when min-p keeps
 *     the tie group that the move would add or drop.
 *   - min-p: values kept by top-k and top-p whose q lies within
 *     ORC_MINP_MARGIN (relative) of min_p. */
static void orc_row_truncate(const orc_args *a, int32_t r, orc_work *w, orc_rowinfo *info) {
  const int32_t V = a->vocab;
  const float *z = w->z;
  double *q = w->q;
  orc_zi *ord = w->ord;
  unsigned char *kept = w->kept;
  const float top_p = a->top_p ? a->top_p[r] : 1.0f;
  const float min_p = a->min_p ? a->min_p[r] : 0.0f;
  const double dm = (double)info->m;
  for (int32_t i = 0; i < V; ++i) q[i] = exp((double)z[i] - dm);
  for (int32_t i = 0; i < V; ++i) kept[i] = 1;
  info->n_p = V;
  if (info->greedy) return;
  for (int32_t i = 0; i < V; ++i) {
    ord[i].z = z[i];
    ord[i].idx = i;
  }
  qsort(ord, (size_t)V, sizeof(orc_zi), orc_cmp_desc);
  /* min-p keeps exp(z - m) >= min_p, i.e. a probability of at least min_p
   * times the largest one */
  const int minp_on = min_p > 0.0f;
#define ORC_MINP_KEEPS(zv) (!minp_on || exp((double)(zv) - dm) >= (double)min_p)

  /* top-k: keep every token whose value is >= the k-th largest value */
  int32_t n_k = V;
  if (info->k_eff < V) {
    const float t_k = ord[info->k_eff - 1].z;
    n_k = info->k_eff;
    while (n_k < V && ord[n_k].z == t_k) ++n_k;
  }
  /* top-p over the top-k set: the smallest tie-closed prefix (by value)
   * whose mass reaches top_p times the top-k mass */
  int32_t n_p = n_k;
  if (top_p < 1.0f) {
    double c_tot = 0.0;
    for (int32_t j = 0; j < n_k; ++j) c_tot += q[ord[j].idx];
    const double target = (double)top_p * c_tot;
    double c = 0.0;
    int32_t j = 0;
    while (j < n_k) {
      int32_t j2 = j;
      const float v = ord[j].z;
      double c_new = c;
      while (j2 < n_k && ord[j2].z == v) c_new += q[ord[j2++].idx];
      if (c_new >= target) {
        n_p = j2;
        const double lo = (c_new - target) / c_tot;                /* distance to the lo side */
        const double hi = j > 0 ? (target - c) / c_tot : INFINITY; /* distance to the hi side */
        info->topp_margin = lo < hi ? lo : hi;
        /* hi side: the crossing one group earlier drops this group */
        if (hi < ORC_TOPP_MARGIN) {
          info->n_p_alt[0] = j;
          if (ORC_MINP_KEEPS(v)) info->flags |= ORC_FLAG_TOPP_MARGIN;
        }
        /* lo side: one group later adds the next group of the top-k set */
        if (lo < ORC_TOPP_MARGIN && j2 < n_k) {
          int32_t j3 = j2;
          while (j3 < n_k && ord[j3].z == ord[j2].z) ++j3;
          info->n_p_alt[1] = j3;
          if (ORC_MINP_KEEPS(ord[j2].z)) info->flags |= ORC_FLAG_TOPP_MARGIN;
        }
        break;
      }
      c = c_new;
      j = j2;
    }
  }
  info->n_p = n_p;
  /* kept by top-k/top-p: the first n_p entries of the order; then min-p */
  for (int32_t i = 0; i < V; ++i) kept[i] = 0;
  for (int32_t j = 0; j < n_p; ++j) kept[ord[j].idx] = 1;
  if (minp_on) {
    /* the widest prefix any top-p alternative keeps, for the margin test */
    int32_t n_any = n_p;
    if (info->n_p_alt[1] > n_any) n_any = info->n_p_alt[1];
    for (int32_t j = 0; j < n_any; ++j) {
      const int32_t i = ord[j].idx;
      if (j < n_p && !ORC_MINP_KEEPS(z[i])) kept[i] = 0;
      if (fabs(q[i] / (double)min_p - 1.0) < ORC_MINP_MARGIN) {
        if (j < n_p) info->flags |= ORC_FLAG_MINP_MARGIN;
        int seen = 0;
        for (int32_t t = 0; t < info->n_near; ++t)
          if (info->near_z[t] == z[i]) seen = 1;
        if (!seen && info->n_near < ORC_MAX_NEAR) info->near_z[info->n_near++] = z[i];
      }
    }
  }
#undef ORC_MINP_KEEPS
}

/* Steps 6-8 of a row with status 0 and the kept set in w->kept: probs,
 * logprobs, the token and the top logprobs, written to row r of the
 * outputs; the diagnostics of the selection are added to info->flags. */
static void orc_row_emit(const orc_args *a, int32_t r, orc_work *w, orc_rowinfo *info) {
  const int32_t V = a->vocab;
  const float *z = w->z, *xp = w->xp;
  const double *q = w->q;
  const unsigned char *kept = w->kept;
  const double dm = (double)info->m;
  const int want_topk_out = a->top_logprobs > 0 && a->top_logprob_vals && a->top_logprob_ids;
  int32_t flags = info->flags;
  double gumbel_gap = INFINITY;
  int32_t token_alt = -1;

  /* 6. normaliser over the kept set, probs and logprobs
   *    ([C] softmax/log_softmax in fp32 of the processed logits). */
  orc_ksum ks = {0.0, 0.0};
  int32_t n_kept = 0;
  for (int32_t i = 0; i < V; ++i)
    if (kept[i]) {
      orc_kadd(&ks, q[i]);
      ++n_kept;
    }
  const double S = orc_kval(&ks);
  const double lnS = log(S);
  /* Returned logprobs ([B] "Logprobs are temperature-scaled"): mode 0 (the
   * default) reports the distribution sampled from, after truncation; mode
   * 1 the untruncated log_softmax(logits / temperature); mode 2 the
   * untruncated log_softmax of the processed logits without temperature
   * (the page's original-logprob switch).  Greedy rows are untruncated at
   * temperature 1, so the three modes agree on them. */
  double lp_m = dm, lp_lnS = lnS;
  if (a->logprob_mode == 1) {
    orc_ksum ka = {0.0, 0.0};
    for (int32_t i = 0; i < V; ++i) orc_kadd(&ka, q[i]);
    lp_lnS = log(orc_kval(&ka));
  } else if (a->logprob_mode == 2) {
    float mr = -INFINITY;
    for (int32_t i = 0; i < V; ++i)
      if (xp[i] > mr) mr = xp[i];
    lp_m = (double)mr;
    orc_ksum ka = {0.0, 0.0};
    for (int32_t i = 0; i < V; ++i) orc_kadd(&ka, exp((double)xp[i] - lp_m));
    lp_lnS = log(orc_kval(&ka));
  }
  const float *lp_x = a->logprob_mode == 2 ? xp : z;
  const int lp_all = a->logprob_mode != 0;
  for (int32_t i = 0; i < V; ++i) {
    if (a->probs) a->probs[(int64_t)r * V + i] = kept[i] ? (float)(q[i] / S) : 0.0f;
    if (a->logprobs)
      a->logprobs[(int64_t)r * V + i] =
          (kept[i] || lp_all) ? (float)(((double)lp_x[i] - lp_m) - lp_lnS) : -INFINITY;
  }

  /* 7. token selection.  Rows with top_k = 1 (greedy rows included) take
   *    the first index of the maximum ([C] "采样类型与选路": argmax); the
   *    others draw by Gumbel-max over the kept set ([A] "Nine lines, and
   *    exactly one call site": probs divided by Exp(1) draws, then argmax). */
  int32_t token = -1;
  const uint64_t seed = a->row_seed ? a->row_seed[r] : (a->deterministic ? 42u : a->seed);
  const uint32_t stream = a->row_stream ? a->row_stream[r] : (a->deterministic ? 0u : (uint32_t)r);
  const uint64_t off = a->row_offset ? a->row_offset[r] : a->offset;
  if (info->k_eff == 1) {
    for (int32_t i = 0; i < V; ++i)
      if (z[i] == info->m) {
        token = i;
        break;
      }
  } else if (a->inverse_cdf) {
    /* The seeded multinomial ([A] "One request with top_p ...", the
     * deterministic path's seeded multinomial; [B] "What the flag
     * switches"): one uniform u per row, then the first token (in index
     * order) whose cumulative kept mass exceeds u times the kept total.
     * Masses are summed one at a time in index order.  Where u S lies
     * within ORC_ICDF_MARGIN of a step, the token on the step's other side
     * is the row's alternative. */
    const double u = orc_icdf_uniform(seed, stream, off);
    double tot = 0.0;
    for (int32_t i = 0; i < V; ++i)
      if (kept[i]) tot += q[i];
    const double t = u * tot;
    double c = 0.0, c_prev = 0.0;
    int32_t prev = -1;
    for (int32_t i = 0; i < V; ++i) {
      if (!kept[i]) continue;
      c_prev = c;
      c += q[i];
      prev = token;
      token = i;
      if (c > t) break;
    }
    const double up = fabs(c - t) / tot, down = fabs(t - c_prev) / tot;
    if (up < ORC_ICDF_MARGIN || down < ORC_ICDF_MARGIN) {
      flags |= ORC_FLAG_ICDF_MARGIN;
      if (down <= up) {
        token_alt = prev;
      } else {
        for (int32_t i = token + 1; i < V; ++i)
          if (kept[i]) {
            token_alt = i;
            break;
          }
      }
    }
  } else {
    double s1 = -1.0, s2 = -1.0;
    int32_t tok2 = -1;
    double g_best = -INFINITY;
    int32_t tok_g = -1;
    for (int32_t i = 0; i < V; ++i) {
      if (!kept[i]) continue;
      double E = orc_exp1_from_word(orc_draw_word(seed, stream, off, i));
      double s = (q[i] / S) / E;
      if (s > s1) {
        s2 = s1;
        tok2 = token;
        s1 = s;
        token = i;
      } else if (s > s2) {
        s2 = s;
        tok2 = i;
      }
      /* second spelling (log domain), for the self-check */
      double g = (((double)z[i] - dm) - lnS) - log(E);
      if (g > g_best) {
        g_best = g;
        tok_g = i;
      }
    }
    gumbel_gap = (s2 >= 0.0 && s1 > 0.0) ? (s1 - s2) / s1 : INFINITY;
    if (gumbel_gap < ORC_NEAR_TIE) {
      flags |= ORC_FLAG_GUMBEL_NEAR_TIE;
      token_alt = tok2;
    } else if (tok_g != token) {
      flags |= ORC_FLAG_SPELLING_MISMATCH;
    }
  }
  a->token_ids[r] = token;

  /* 8. top logprobs: the largest listed values by (z desc, index asc),
   *    with the logprob mode's values; mode 0 lists kept tokens only,
   *    modes 1 and 2 every token with a finite value. */
  if (want_topk_out) {
    const int32_t K = a->top_logprobs;
    int32_t nfill = 0;
    /* simple selection by repeated scans (K is small) */
    float last_z = INFINITY;
    int32_t last_i = -1;
    for (; nfill < K; ++nfill) {
      int32_t best = -1;
      for (int32_t i = 0; i < V; ++i) {
        if ((!kept[i] && !lp_all) || z[i] == -INFINITY) continue;
        /* strictly after (last_z, last_i) in the (z desc, idx asc) order */
        if (z[i] > last_z || (z[i] == last_z && i <= last_i)) continue;
        if (best < 0 || z[i] > z[best]) best = i; /* index ascending keeps the first */
      }
      if (best < 0) break;
      a->top_logprob_vals[(int64_t)r * K + nfill] = (float)(((double)lp_x[best] - lp_m) - lp_lnS);
      a->top_logprob_ids[(int64_t)r * K + nfill] = best;
      last_z = z[best];
      last_i = best;
    }
    for (; nfill < K; ++nfill) {
      a->top_logprob_vals[(int64_t)r * K + nfill] = -INFINITY;
      a->top_logprob_ids[(int64_t)r * K + nfill] = -1;
    }
  }

  if (a->diag_flags) a->diag_flags[r] = flags;
  if (a->diag_gumbel_gap) a->diag_gumbel_gap[r] = gumbel_gap;
  if (a->diag_topp_margin) a->diag_topp_margin[r] = info->topp_margin;
  if (a->diag_kept) a->diag_kept[r] = n_kept;
  if (a->diag_token_alt) a->diag_token_alt[r] = token_alt;
}

/* The outputs of a row whose status is not 0 (no finite value, or +inf). */
static void orc_row_bad(const orc_args *a, int32_t r, int status) {
  const int32_t V = a->vocab;
  if (a->row_status) a->row_status[r] = status;
  a->token_ids[r] = -1;
  for (int32_t i = 0; i < V; ++i) {
    if (a->probs) a->probs[(int64_t)r * V + i] = 0.0f;
    if (a->logprobs) a->logprobs[(int64_t)r * V + i] = -INFINITY;
  }
  if (a->top_logprobs > 0 && a->top_logprob_vals && a->top_logprob_ids)
    for (int32_t j = 0; j < a->top_logprobs; ++j) {
      a->top_logprob_vals[(int64_t)r * a->top_logprobs + j] = -INFINITY;
      a->top_logprob_ids[(int64_t)r * a->top_logprobs + j] = -1;
    }
  if (a->diag_flags) a->diag_flags[r] = 0;
  if (a->diag_gumbel_gap) a->diag_gumbel_gap[r] = INFINITY;
  if (a->diag_topp_margin) a->diag_topp_margin[r] = INFINITY;
  if (a->diag_kept) a->diag_kept[r] = 0;
  if (a->diag_token_alt) a->diag_token_alt[r] = -1;
}

static void orc_row(const orc_args *a, int32_t r, orc_work *w) {
  orc_rowinfo info;
  orc_row_values(a, r, w, &info);
  if (info.status != 0) {
    orc_row_bad(a, r, info.status);
    return;
  }
  if (a->row_status) a->row_status[r] = 0;
  orc_row_truncate(a, r, w, &info);
  orc_row_emit(a, r, w, &info);
}

static int orc_work_alloc(orc_work *w, int32_t V) {
  w->z = (float *)malloc(sizeof(float) * (size_t)V);
  w->xp = (float *)malloc(sizeof(float) * (size_t)V);
  w->ord = (orc_zi *)malloc(sizeof(orc_zi) * (size_t)V);
  w->q = (double *)malloc(sizeof(double) * (size_t)V);
  w->cnt = (int32_t *)malloc(sizeof(int32_t) * (size_t)V);
  w->kept = (unsigned char *)malloc((size_t)V);
  return (w->z && w->xp && w->ord && w->q && w->cnt && w->kept) ? 0 : -2;
}

static void orc_work_free(orc_work *w) {
  free(w->z);
  free(w->xp);
  free(w->ord);
  free(w->q);
  free(w->cnt);
  free(w->kept);
}

typedef struct {
  const orc_args *a;
  int32_t r0, r1;
  int status;
} orc_job;

static void *orc_worker(void *p) {
  orc_job *job = (orc_job *)p;
  orc_work w;
  job->status = orc_work_alloc(&w, job->a->vocab);
  if (job->status == 0)
    for (int32_t r = job->r0; r < job->r1; ++r) orc_row(job->a, r, &w);
  orc_work_free(&w);
  return NULL;
}

static int orc_args_ok(const orc_args *a) {
  return a && a->n_rows > 0 && a->vocab > 0 && a->row_stride >= a->vocab && a->logits && a->token_ids &&
         a->logprob_mode >= 0 && a->logprob_mode <= 2 && !(a->vocab_mask && a->mask_stride < (a->vocab + 31) / 32);
}

/* Runs every row; returns 0, -1 for invalid sizes, -2 for allocation failure. */
int orc_step(const orc_args *a) {
  if (!orc_args_ok(a)) return -1;
  int nt = a->n_threads > 0 ? a->n_threads : 1;
  if (nt > a->n_rows) nt = a->n_rows;
  if (nt > 256) nt = 256;
  orc_job jobs[256];
  pthread_t th[256];
  int32_t per = (a->n_rows + nt - 1) / nt;
  for (int t = 0; t < nt; ++t) {
    jobs[t].a = a;
    jobs[t].r0 = t * per;
    jobs[t].r1 = (t + 1) * per < a->n_rows ? (t + 1) * per : a->n_rows;
    jobs[t].status = 0;
    if (jobs[t].r0 >= jobs[t].r1) continue;
    if (nt == 1) orc_worker(&jobs[t]);
    else pthread_create(&th[t], NULL, orc_worker, &jobs[t]);
  }
  int rc = 0;
  for (int t = 0; t < nt; ++t) {
    if (jobs[t].r0 >= jobs[t].r1) continue;
    if (nt > 1) pthread_join(th[t], NULL);
    if (jobs[t].status != 0) rc = jobs[t].status;
  }
  return rc;
}

/* ------------------------------------------------------------------ */
/* Kept sets a flagged row allows, and a row's outputs for a given     */
/* kept set (for checking rows whose boundary lies within a flag       */
/* margin: such a row must match the outputs of one allowed set).      */
/* ------------------------------------------------------------------ */

/* Alternative `which` of row r's kept set, written to kept_out[V]:
 *   which = c + 3 s, with c the top-p choice (0: the row's own crossing,
 *   1: one tie group earlier, 2: one group later; only where the margin
 *   reaches it) and s a subset of the near-boundary min-p values whose
 *   decision is flipped (bit t flips near value t).
 * Returns 1 when the alternative exists, 0 when it does not, -1 when
 * `which` is past the last one (or r is invalid), -2 on allocation failure.
 * Alternative 0 is the oracle's own kept set. */
int orc_row_alternative(const orc_args *a, int32_t r, int32_t which, unsigned char *kept_out) {
  if (!orc_args_ok(a) || r < 0 || r >= a->n_rows || which < 0 || which >= 3 << ORC_MAX_NEAR) return -1;
  orc_work w;
  int rc = orc_work_alloc(&w, a->vocab);
  if (rc != 0) {
    orc_work_free(&w);
    return rc;
  }
  orc_rowinfo info;
  orc_row_values(a, r, &w, &info);
  rc = 0;
  if (info.status == 0) {
    orc_row_truncate(a, r, &w, &info);
    const int c = which % 3, s = which / 3;
    const int32_t n_pre = c == 0 ? info.n_p : info.n_p_alt[c - 1];
    if (s >= (1 << info.n_near)) {
      rc = c == 0 ? -1 : 0;
    } else if (n_pre >= 0 && !info.greedy) {
      const float min_p = a->min_p ? a->min_p[r] : 0.0f;
      const int32_t V = a->vocab;
      for (int32_t i = 0; i < V; ++i) kept_out[i] = 0;
      for (int32_t j = 0; j < n_pre; ++j) {
        const int32_t i = w.ord[j].idx;
        int keep = !(min_p > 0.0f) || exp((double)w.z[i] - (double)info.m) >= (double)min_p;
        for (int32_t t = 0; t < info.n_near; ++t)
          if (((s >> t) & 1) && info.near_z[t] == w.z[i]) keep = !keep;
        kept_out[i] = (unsigned char)keep;
      }
      rc = 1;
    } else if (which == 0) {
      memcpy(kept_out, w.kept, (size_t)a->vocab);
      rc = 1;
    }
  } else {
    rc = which == 0 ? 0 : -1;
  }
  orc_work_free(&w);
  return rc;
}

/* Row r's outputs (token, probs, logprobs, top logprobs, diagnostics) for
 * the kept set kept_in[V] instead of the row's own truncation.  Returns 0,
 * -1 for invalid arguments or a row whose status is not 0, -2 on allocation
 * failure. */
int orc_row_with_kept(const orc_args *a, int32_t r, const unsigned char *kept_in) {
  if (!orc_args_ok(a) || r < 0 || r >= a->n_rows || !kept_in) return -1;
  orc_work w;
  int rc = orc_work_alloc(&w, a->vocab);
  if (rc == 0) {
    orc_rowinfo info;
    orc_row_values(a, r, &w, &info);
    if (info.status != 0) {
      rc = -1;
    } else {
      orc_row_truncate(a, r, &w, &info);
      memcpy(w.kept, kept_in, (size_t)a->vocab);
      info.flags = 0;
      if (a->row_status) a->row_status[r] = 0;
      orc_row_emit(a, r, &w, &info);
    }
  }
  orc_work_free(&w);
  return rc;
}
