// sampler_runtime.cpp -- host side of the decode-step sampler's C ABI.
//
// Validation, per-row normalisation, the batch predicate, the per-row
// records (in the kernel arguments for batches of up to kArgRows rows, so a
// step is one launch and no copy; otherwise through a pinned staging ring
// and one copy), launch planning (workgroups per row) and the cooperative
// launch.
//
// Sources (page titles; sections named where used):
//   [A] "SGLang's +75% sampler speedup skips Qwen3 chat requests"
//   [B] the SGLang 101 operations manual
//   [C] "采样参数对解码开销的影响：temperature、top_p 与采样核路径"
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/sampler.h"
#include "sampler_internal.h"

using namespace dsts;

namespace {

constexpr int kRing = 4;
// [A] "One request with top_p takes the whole batch off the fast path":
// temperatures in [0, 1e-6) are greedy.
constexpr double kGreedyEps = 1e-6;
// [B] "What the flag switches": requests without a seed use 42.
constexpr uint64_t kDeterministicSeed = 42;

thread_local std::string g_create_error;

void set_msg(std::string &dst, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  dst = buf;
}

}  // namespace

struct sampler_handle {
  sampler_config cfg{};
  int device = 0;
  int n_cu = 0;
  int resident = 0;  // workgroups of the row kernel that fit at once
  int slice_cap = 0;  // largest slice a workgroup holds in LDS
  int hash_slots = 0; // LDS hash slots for history counts
  int bias_slots = 0; // LDS hash slots for logit_bias / stop entries (0: none)
  RowParam *host_ring = nullptr;   // pinned, kRing slots of max_rows records
  RowParam *dev_ring = nullptr;    // device, kRing slots
  KernelArgs *args = nullptr;      // host: the launch's argument block
  RowParam *graph_rows = nullptr;  // device, max_rows records written by sampler_step_graph's first kernel
  std::vector<RowParam> recs;      // host scratch: a step's records in row order (max_rows)
  std::vector<int> rank, order;    // host scratch: group start order, rows by cost (max_rows)
  hipEvent_t slot_done[kRing] = {};
  bool slot_used[kRing] = {};
  int next_slot = 0;
  GroupSync *sync = nullptr;
  WgSlots *slots = nullptr;
  uint32_t *abort_word = nullptr;  // device word: epoch of an aborted launch
  uint32_t epoch = 0;
  std::vector<hipEvent_t> prof;  // 2 per recorded step
  int prof_cap = 0;
  int prof_n = 0;
  std::string err;
};

namespace {

bool row_is_greedy(float t) { return t >= 0.0f && (double)t < kGreedyEps; }

sampler_status validate_params(const sampler_config *cfg, const sampler_step_args *a, std::string &msg);

// Checks that need no device; fills msg and returns a status.
sampler_status validate(const sampler_config *cfg, const sampler_step_args *a, std::string &msg) {
  if (!a) {
    msg = "args is NULL";
    return SAMPLER_EINVAL;
  }
  if (a->n_rows <= 0) {
    // [A] path_for_batch: a batch needs at least one request
    set_msg(msg, "n_rows must be >= 1 (got %d): an empty batch has no sampling path", a->n_rows);
    return SAMPLER_EINVAL;
  }
  if (cfg && a->n_rows > cfg->max_rows) {
    set_msg(msg, "n_rows %d exceeds max_rows %d", a->n_rows, cfg->max_rows);
    return SAMPLER_ECAPACITY;
  }
  if (a->vocab <= 0) {
    set_msg(msg, "vocab must be >= 1 (got %d)", a->vocab);
    return SAMPLER_EINVAL;
  }
  if (cfg && a->vocab > cfg->max_vocab) {
    set_msg(msg, "vocab %d exceeds max_vocab %d", a->vocab, cfg->max_vocab);
    return SAMPLER_ECAPACITY;
  }
  if (a->row_stride < a->vocab) {
    set_msg(msg, "row_stride %lld is smaller than vocab %d", (long long)a->row_stride, a->vocab);
    return SAMPLER_EINVAL;
  }
  if (a->dtype != SAMPLER_DTYPE_F32 && a->dtype != SAMPLER_DTYPE_BF16) {
    set_msg(msg, "unknown dtype %d", a->dtype);
    return SAMPLER_EINVAL;
  }
  if (!a->logits) {
    msg = "logits is NULL";
    return SAMPLER_EINVAL;
  }
  if (!a->token_ids) {
    msg = "token_ids is NULL";
    return SAMPLER_EINVAL;
  }
  if (a->top_logprobs < 0 || (cfg && a->top_logprobs > cfg->max_top_logprobs) ||
      a->top_logprobs > kMaxTopLogprobs) {
    set_msg(msg, "top_logprobs %d outside [0, %d]", a->top_logprobs,
            cfg ? cfg->max_top_logprobs : kMaxTopLogprobs);
    return (a->top_logprobs < 0) ? SAMPLER_EINVAL : SAMPLER_ECAPACITY;
  }
  if (a->top_logprobs > 0 && (!a->top_logprob_vals || !a->top_logprob_ids)) {
    msg = "top_logprobs > 0 needs top_logprob_vals and top_logprob_ids";
    return SAMPLER_EINVAL;
  }
  if (a->vocab_mask && a->mask_stride < ((int64_t)a->vocab + 31) / 32) {
    set_msg(msg, "mask_stride %lld is smaller than ceil(vocab / 32) = %d words", (long long)a->mask_stride,
            (a->vocab + 31) / 32);
    return SAMPLER_EINVAL;
  }
  if (a->logprob_mode < SAMPLER_LOGPROB_PROCESSED || a->logprob_mode > SAMPLER_LOGPROB_RAW) {
    set_msg(msg, "unknown logprob_mode %d", a->logprob_mode);
    return SAMPLER_EINVAL;
  }
  if (a->logprob_mode == SAMPLER_LOGPROB_RAW) {
    for (int r = 0; r < a->n_rows; ++r) {
      const float t = a->temperature ? a->temperature[r] : 1.0f;
      if (!(row_is_greedy(t) || t == 1.0f)) {
        set_msg(msg, "row %d: the raw logprob mode is supported only at effective temperature 1 (got %g)", r,
                (double)t);
        return SAMPLER_ENOTSUP;
      }
    }
  }
  if ((a->min_tokens != nullptr) != (a->output_len != nullptr)) {
    msg = "min_tokens and output_len go together";
    return SAMPLER_EINVAL;
  }
  const int32_t bias_cap = cfg ? cfg->max_bias_per_row : kMaxBiasPerRow;
  for (int r = 0; r < a->n_rows; ++r) {
    const int32_t bl = a->bias_len ? a->bias_len[r] : 0;
    const bool stop_on = a->min_tokens && a->output_len[r] < a->min_tokens[r];
    const int32_t sl = (stop_on && a->stop_len) ? a->stop_len[r] : 0;
    if (bl < 0 || sl < 0) {
      set_msg(msg, "row %d: bias_len and stop_len must be >= 0", r);
      return SAMPLER_EINVAL;
    }
    if (bl > 0 && (!a->bias_ids || !a->bias_vals || !a->bias_start || a->bias_start[r] < 0)) {
      set_msg(msg, "row %d: bias_len > 0 needs bias_ids, bias_vals and a bias_start >= 0", r);
      return SAMPLER_EINVAL;
    }
    if (sl > 0 && (!a->stop_ids || !a->stop_start || a->stop_start[r] < 0)) {
      set_msg(msg, "row %d: an active stop list needs stop_ids and a stop_start >= 0", r);
      return SAMPLER_EINVAL;
    }
    if ((int64_t)bl + sl > bias_cap) {
      set_msg(msg, "row %d: %d bias and %d active stop entries exceed max_bias_per_row %d", r, bl, sl, bias_cap);
      return SAMPLER_ECAPACITY;
    }
  }
  return validate_params(cfg, a, msg);
}

// Per-row parameter checks (also used by the predicate alone).
sampler_status validate_params(const sampler_config *cfg, const sampler_step_args *a, std::string &msg) {
  bool any_hist = false;
  for (int r = 0; r < a->n_rows; ++r) {
    const float t = a->temperature ? a->temperature[r] : 1.0f;
    if (!(t >= 0.0f) || !std::isfinite(t)) {
      set_msg(msg, "row %d: temperature must be finite and >= 0 (got %g)", r, (double)t);
      return SAMPLER_EINVAL;
    }
    const float p = a->top_p ? a->top_p[r] : 1.0f;
    if (!(p > 0.0f && p <= 1.0f)) {
      set_msg(msg, "row %d: top_p must be in (0, 1] (got %g)", r, (double)p);
      return SAMPLER_EINVAL;
    }
    const int32_t k = a->top_k ? a->top_k[r] : -1;
    if (!(k == -1 || k >= 1)) {
      set_msg(msg, "row %d: top_k must be -1 or >= 1 (got %d)", r, k);
      return SAMPLER_EINVAL;
    }
    const float mp = a->min_p ? a->min_p[r] : 0.0f;
    if (!(mp >= 0.0f && mp <= 1.0f)) {
      set_msg(msg, "row %d: min_p must be in [0, 1] (got %g)", r, (double)mp);
      return SAMPLER_EINVAL;
    }
    const float rp = a->repetition_penalty ? a->repetition_penalty[r] : 1.0f;
    if (!(rp > 0.0f) || !std::isfinite(rp)) {
      set_msg(msg, "row %d: repetition_penalty must be finite and > 0 (got %g)", r, (double)rp);
      return SAMPLER_EINVAL;
    }
    const float pp = a->presence_penalty ? a->presence_penalty[r] : 0.0f;
    const float fp = a->frequency_penalty ? a->frequency_penalty[r] : 0.0f;
    if (!std::isfinite(pp) || !std::isfinite(fp)) {
      set_msg(msg, "row %d: presence and frequency penalties must be finite", r);
      return SAMPLER_EINVAL;
    }
    if (a->history_len) {
      const int32_t hl = a->history_len[r];
      const int32_t cap = cfg ? cfg->max_history_per_row : kMaxHistPerRow;
      if (hl < 0) {
        set_msg(msg, "row %d: history_len must be >= 0 (got %d)", r, hl);
        return SAMPLER_EINVAL;
      }
      if (hl > cap) {
        set_msg(msg, "row %d: history_len %d exceeds max_history_per_row %d", r, hl, cap);
        return SAMPLER_ECAPACITY;
      }
      if (hl > 0) {
        any_hist = true;
        if (!a->history_start) {
          msg = "history_len given without history_start";
          return SAMPLER_EINVAL;
        }
        if (a->history_start[r] < 0) {
          set_msg(msg, "row %d: history_start must be >= 0", r);
          return SAMPLER_EINVAL;
        }
      }
    }
  }
  if (any_hist && !a->history_ids) {
    msg = "history_ids is NULL but a row has history";
    return SAMPLER_EINVAL;
  }
  return SAMPLER_OK;
}

// [A] "One request with top_p takes the whole batch off the fast path":
// normalize each row, then is_all_greedy / need_top_p / need_top_k /
// need_min_p decide the path.
int choose_path(const sampler_step_args *a, uint32_t flags) {
  bool all_greedy = true, need_p = false, need_k = false, need_minp = false;
  for (int r = 0; r < a->n_rows; ++r) {
    const float t = a->temperature ? a->temperature[r] : 1.0f;
    int32_t k = a->top_k ? a->top_k[r] : -1;
    if (row_is_greedy(t)) k = 1;
    else if (k == -1) k = kTopKAll;
    const float p = a->top_p ? a->top_p[r] : 1.0f;
    const float mp = a->min_p ? a->min_p[r] : 0.0f;
    if (!(k <= 1)) all_greedy = false;
    if (p != 1.0f) need_p = true;
    if (k != kTopKAll) need_k = true;
    if (mp > 0.0f) need_minp = true;
  }
  if (all_greedy) return PATH_GREEDY;
  if (!(need_p || need_k || need_minp)) return (flags & SAMPLER_DETERMINISTIC) ? PATH_DETERMINISTIC : PATH_GUMBEL;
  return PATH_FILTERED;
}

sampler_status hip_fail(sampler_handle *h, hipError_t e, const char *what) {
  set_msg(h->err, "%s failed: %s", what, hipGetErrorString(e));
  return SAMPLER_EHIP;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(dev) == hipSuccess) ok = true;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

void free_profile(sampler_handle *h) {
  for (hipEvent_t e : h->prof) (void)hipEventDestroy(e);
  h->prof.clear();
  h->prof_cap = h->prof_n = 0;
}

void free_handle(sampler_handle *h) {
  if (!h) return;
  free_profile(h);
  for (int s = 0; s < kRing; ++s)
    if (h->slot_done[s]) {
      (void)hipEventSynchronize(h->slot_done[s]);
      (void)hipEventDestroy(h->slot_done[s]);
    }
  if (h->host_ring) (void)hipHostFree(h->host_ring);
  if (h->dev_ring) (void)hipFree(h->dev_ring);
  if (h->graph_rows) (void)hipFree(h->graph_rows);
  delete h->args;
  if (h->sync) (void)hipFree(h->sync);
  if (h->slots) (void)hipFree(h->slots);
  if (h->abort_word) (void)hipFree(h->abort_word);
  delete h;
}

}  // namespace

namespace {

// Launch plan (G workgroups per row, rows strided over groups), the kernel
// parameters and the launch, shared by both step entry points.  `dp`: the
// device records, or null (records in ka.rows); `dev`: per-row arrays in
// device memory that the kernel normalises itself (sampler_step_graph).
// The launch plan: G workgroups of `slice` values per row, `groups` row
// groups (rows strided over them).
sampler_status plan_groups(sampler_handle *h, int n, int V, int *G_out, int *slice_out, int *groups_out) {
  const bool det = (h->cfg.flags & SAMPLER_DETERMINISTIC) != 0;
  const int g_min = (V + h->slice_cap - 1) / h->slice_cap;
  if (g_min > kMaxG || g_min > h->resident) {
    set_msg(h->err, "vocab %d needs %d workgroups per row (max %d)", V, g_min,
            kMaxG < h->resident ? kMaxG : h->resident);
    return SAMPLER_ECAPACITY;
  }
  int G;
  if (det) {
    G = g_min;  // depends on V only: a row's reduction order is batch invariant
  } else {
    const int fill = h->resident / n;
    // at least ~32 values per thread: a row's steps are latency-bound, and
    // fewer workgroups per row exchange faster (measured on MI355X at N=8,
    // V=151,936: 10 workgroups per row 34.7 us, 32 workgroups 41.9 us)
    const int by_work = (V + 32 * kBlock - 1) / (32 * kBlock);
    G = fill < by_work ? fill : by_work;
    if (G > kMaxG) G = kMaxG;
    if (G > h->resident) G = h->resident;
    if (G < g_min) G = g_min;
  }
  int slice = (V + G - 1) / G;
  slice = (slice + 3) & ~3;
  G = (V + slice - 1) / slice;  // every workgroup gets a non-empty slice
  const int groups = h->resident / G;
  *G_out = G;
  *slice_out = slice;
  *groups_out = groups < n ? groups : n;
  return SAMPLER_OK;
}

// The order in which the kernel's row groups start: block b of the grid is
// dealt to XCD b % 8 and the kernel gives group x * gpx + j (gpx = groups /
// 8) the blocks 8 (j G + gid) + x, so groups start in (j, x) order; groups
// past 8 gpx take the last blocks.  rank[k] = the k-th group to start.
void group_start_order(int groups, int *rank) {
  const int gpx = groups / 8;
  int k = 0;
  for (int j = 0; j < gpx; ++j)
    for (int x = 0; x < 8; ++x) rank[k++] = x * gpx + j;
  for (int g = 8 * gpx; g < groups; ++g) rank[k++] = g;
}

// Expected cost class of a row (larger: longer): top-p without top-k keeps
// the most candidates and values; rows that keep everything run Philox on
// the whole slice; top-k rows decide from short lists; greedy rows draw
// nothing.  Penalties and biases add a pass.
int row_cost(const RowParam &p) {
  int c;
  if (p.flags & RF_GREEDY) c = 0;
  else if (p.flags & RF_TOP1) c = 1;
  else if ((p.flags & RF_TOPP) && !(p.flags & RF_TOPK)) c = 5;
  else if (!(p.flags & (RF_TOPK | RF_TOPP | RF_MINP))) c = 4;
  else if (p.flags & RF_TOPK) c = 3;
  else c = 2;
  return 2 * c + ((p.flags & (RF_PEN | RF_SPEC)) ? 1 : 0);
}

sampler_status plan_and_launch(sampler_handle *h, const sampler_step_args *a, KernelArgs &ka, const RowParam *dp,
                               bool any_pen, int path, hipStream_t stream, const DevRowArrays *dev = nullptr) {
  const int n = a->n_rows, V = a->vocab;
  const bool det = (h->cfg.flags & SAMPLER_DETERMINISTIC) != 0;
  hipError_t e;
  int G, slice, groups;
  sampler_status st = plan_groups(h, n, V, &G, &slice, &groups);
  if (st != SAMPLER_OK) return st;
  KernelParams &kp = ka.kp;
  kp = KernelParams{};
  kp.logits = a->logits;
  kp.row_stride = a->row_stride;
  kp.n_rows = n;
  kp.vocab = V;
  kp.rows = dp;
  kp.history_ids = a->history_ids;
  kp.token_ids = a->token_ids;
  kp.probs = a->probs;
  kp.logprobs = a->logprobs;
  kp.top_lp = a->top_logprobs;
  kp.top_lp_vals = a->top_logprob_vals;
  kp.top_lp_ids = a->top_logprob_ids;
  kp.row_status = a->row_status;
  kp.G = G;
  kp.n_groups = groups;
  kp.slice = slice;
  kp.hash_slots = h->hash_slots;
  kp.bias_slots = h->bias_slots;
  kp.vocab_mask = a->vocab_mask;
  kp.mask_stride = a->mask_stride;
  kp.bias_ids = a->bias_ids;
  kp.bias_vals = a->bias_vals;
  kp.stop_ids = a->stop_ids;
  kp.lp_mode = a->logprob_mode != SAMPLER_LOGPROB_PROCESSED ? 1 : 0;
  kp.icdf = (h->cfg.flags & SAMPLER_INVERSE_CDF) ? 1 : 0;
  if (dev) {
    kp.dev = *dev;
    kp.rows = h->graph_rows;
  }
  kp.det = det ? 1 : 0;
  kp.max_hist = h->cfg.max_history_per_row;
  kp.max_bias = h->cfg.max_bias_per_row;
  kp.seed = a->seed;
  kp.offset = a->offset;
  const size_t esz = a->dtype == SAMPLER_DTYPE_F32 ? 4 : 2;
  const bool lvec = ((uintptr_t)a->logits % (4 * esz) == 0) && (a->row_stride % 4 == 0);
  const bool ovec = ((V & 3) == 0) && ((uintptr_t)a->probs % 16 == 0) && ((uintptr_t)a->logprobs % 16 == 0);
  kp.vec_ok = (lvec ? 1 : 0) | (ovec ? 2 : 0);
  kp.path = path;
  kp.sync = h->sync;
  kp.slots = h->slots;
  kp.abort_word = h->abort_word;
  if (++h->epoch == 0) h->epoch = 1;
  kp.epoch = h->epoch;
  if (dev && (e = launch_rows(kp, h->graph_rows, stream)) != hipSuccess) return hip_fail(h, e, "rows kernel launch");
  const bool prof = h->prof_n < h->prof_cap;
  e = launch_step(ka, a->dtype, any_pen, (h->cfg.flags & SAMPLER_COOPERATIVE_LAUNCH) != 0, stream,
                  prof ? h->prof[2 * h->prof_n] : nullptr, prof ? h->prof[2 * h->prof_n + 1] : nullptr);
  if (e != hipSuccess) return hip_fail(h, e, "kernel launch");
  if (prof) ++h->prof_n;
  return SAMPLER_OK;
}

}  // namespace

extern "C" {

sampler_status sampler_create(const sampler_config *cfg, sampler_handle **out) {
  if (!out) {
    g_create_error = "out is NULL";
    return SAMPLER_EINVAL;
  }
  *out = nullptr;
  if (!cfg) {
    g_create_error = "cfg is NULL";
    return SAMPLER_EINVAL;
  }
  if (cfg->max_rows < 1 || cfg->max_vocab < 1 || cfg->max_vocab > kMaxVocab || cfg->max_history_per_row < 0 ||
      cfg->max_history_per_row > kMaxHistPerRow || cfg->max_top_logprobs < 0 ||
      cfg->max_top_logprobs > kMaxTopLogprobs || cfg->max_bias_per_row < 0 ||
      cfg->max_bias_per_row > kMaxBiasPerRow ||
      (cfg->flags &
       ~(SAMPLER_DETERMINISTIC | SAMPLER_FORCE_FILTERED | SAMPLER_COOPERATIVE_LAUNCH | SAMPLER_INVERSE_CDF))) {
    set_msg(g_create_error,
            "bad config: need max_rows >= 1, 1 <= max_vocab <= %d, 0 <= max_history_per_row <= %d, "
            "0 <= max_top_logprobs <= %d, 0 <= max_bias_per_row <= %d and known flags",
            kMaxVocab, kMaxHistPerRow, kMaxTopLogprobs, kMaxBiasPerRow);
    return SAMPLER_EINVAL;
  }
  int n_dev = 0;
  hipError_t e = hipGetDeviceCount(&n_dev);
  if (e != hipSuccess || n_dev <= 0) {
    set_msg(g_create_error, "no usable HIP device (%s)", e == hipSuccess ? "none found" : hipGetErrorString(e));
    (void)hipGetLastError();
    return SAMPLER_EHIP;
  }
  if (cfg->device < 0 || cfg->device >= n_dev) {
    set_msg(g_create_error, "device %d out of range (0..%d)", cfg->device, n_dev - 1);
    return SAMPLER_EINVAL;
  }
  DeviceGuard guard(cfg->device);
  if (!guard.ok) {
    g_create_error = "hipSetDevice failed";
    return SAMPLER_EHIP;
  }
  sampler_handle *h = new (std::nothrow) sampler_handle();
  if (!h) {
    g_create_error = "out of host memory";
    return SAMPLER_EHIP;
  }
  h->cfg = *cfg;
  h->device = cfg->device;
  hipDeviceProp_t prop;
  if ((e = hipGetDeviceProperties(&prop, cfg->device)) != hipSuccess) goto fail;
  h->n_cu = prop.multiProcessorCount;
  {
    // LDS plan: fixed part + slice of fp32 values + hash of history counts
    int slots = 64;
    while (slots < 2 * cfg->max_history_per_row) slots *= 2;
    h->hash_slots = slots;
    int bslots = 0;
    if (cfg->max_bias_per_row > 0) {
      bslots = 64;
      while (bslots < 2 * cfg->max_bias_per_row) bslots *= 2;
    }
    h->bias_slots = bslots;
    const size_t lds_max = prop.sharedMemPerBlock;
    const size_t fixed = kernel_lds_fixed() + kernel_lds_region(kMaxSlice, slots, bslots, true);
    if (lds_max <= fixed + 16 * kBlock) {
      set_msg(g_create_error, "device LDS per workgroup (%zu B) too small", lds_max);
      free_handle(h);
      return SAMPLER_EHIP;
    }
    size_t cap = (lds_max - fixed) / sizeof(float);
    if (cap > (size_t)kMaxSlice) cap = kMaxSlice;
    h->slice_cap = (int)(cap & ~(size_t)3);
    if ((int64_t)h->slice_cap * kMaxG < cfg->max_vocab) {
      set_msg(g_create_error, "max_vocab %d exceeds %d (%d workgroups x %d values; lower max_history_per_row "
              "to free LDS)", cfg->max_vocab, h->slice_cap * kMaxG, kMaxG, h->slice_cap);
      free_handle(h);
      return SAMPLER_ECAPACITY;
    }
  }
  if ((e = resident_blocks(cfg->device, kernel_lds_bytes(h->slice_cap, h->hash_slots, h->bias_slots, true),
                           &h->resident)) !=
      hipSuccess)
    goto fail;
  if (h->resident < 1) {
    g_create_error = "the row kernel does not fit on this device";
    free_handle(h);
    return SAMPLER_EHIP;
  }
  {
    const size_t ring_bytes = sizeof(RowParam) * (size_t)cfg->max_rows * kRing;
    if ((e = hipHostMalloc((void **)&h->host_ring, ring_bytes, hipHostMallocDefault)) != hipSuccess) goto fail;
    if ((e = hipMalloc((void **)&h->dev_ring, ring_bytes)) != hipSuccess) goto fail;
    if ((e = hipMalloc((void **)&h->graph_rows, sizeof(RowParam) * (size_t)cfg->max_rows)) != hipSuccess) goto fail;
    try {
      h->recs.resize((size_t)cfg->max_rows);
      h->rank.resize((size_t)cfg->max_rows);
      h->order.resize((size_t)cfg->max_rows);
    } catch (...) {
      g_create_error = "out of host memory";
      free_handle(h);
      return SAMPLER_EHIP;
    }
    h->args = new (std::nothrow) KernelArgs();
    if (!h->args) {
      g_create_error = "out of host memory";
      free_handle(h);
      return SAMPLER_EHIP;
    }
    const size_t n_groups_max = (size_t)h->resident;  // one group per resident workgroup at most
    if ((e = hipMalloc((void **)&h->sync, sizeof(GroupSync) * n_groups_max)) != hipSuccess) goto fail;
    if ((e = hipMemset(h->sync, 0, sizeof(GroupSync) * n_groups_max)) != hipSuccess) goto fail;
    if ((e = hipMalloc((void **)&h->slots, sizeof(WgSlots) * (size_t)h->resident)) != hipSuccess) goto fail;
    if ((e = hipMemset(h->slots, 0, sizeof(WgSlots) * (size_t)h->resident)) != hipSuccess) goto fail;
    if ((e = hipMalloc((void **)&h->abort_word, 256)) != hipSuccess) goto fail;
    if ((e = hipMemset(h->abort_word, 0, 256)) != hipSuccess) goto fail;
    for (int s = 0; s < kRing; ++s)
      if ((e = hipEventCreateWithFlags(&h->slot_done[s], hipEventDisableTiming)) != hipSuccess) goto fail;
    if ((e = hipDeviceSynchronize()) != hipSuccess) goto fail;
  }
  *out = h;
  return SAMPLER_OK;
fail:
  set_msg(g_create_error, "HIP error during create: %s", hipGetErrorString(e));
  free_handle(h);
  return SAMPLER_EHIP;
}

sampler_status sampler_validate(const sampler_config *cfg, const sampler_step_args *args, char *msg,
                                int32_t msg_len) {
  std::string m;
  sampler_status st = validate(cfg, args, m);
  if (msg && msg_len > 0) {
    std::snprintf(msg, (size_t)msg_len, "%s", m.c_str());
  }
  return st;
}

sampler_status sampler_select_path(const sampler_step_args *args, uint32_t flags, int32_t *path_out) {
  std::string m;
  if (!path_out || !args) return SAMPLER_EINVAL;
  if (args->n_rows <= 0) return SAMPLER_EINVAL;  // [A]: an empty batch has no path
  sampler_status st = validate_params(nullptr, args, m);
  if (st != SAMPLER_OK) return st;
  *path_out = choose_path(args, flags);
  return SAMPLER_OK;
}

sampler_status sampler_step(sampler_handle *h, const sampler_step_args *a, void *stream_ptr) {
  if (!h) return SAMPLER_EINVAL;
  h->err.clear();
  sampler_status st = validate(&h->cfg, a, h->err);
  if (st != SAMPLER_OK) return st;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  DeviceGuard guard(h->device);
  if (!guard.ok) {
    h->err = "hipSetDevice failed";
    return SAMPLER_EHIP;
  }

  const int n = a->n_rows, V = a->vocab;
  const bool det = (h->cfg.flags & SAMPLER_DETERMINISTIC) != 0;
  int path = choose_path(a, h->cfg.flags);
  if (a->path_out) *a->path_out = path;
  if (h->cfg.flags & SAMPLER_FORCE_FILTERED) path = PATH_FILTERED;

  // ---- per-row records: in the kernel arguments, or in a staging slot
  // (waits only when the ring wraps onto a slot whose copy is in flight)
  const bool inline_rows = n <= kArgRows;
  KernelArgs &ka = *h->args;
  int slot = -1;
  RowParam *rp = ka.rows, *dp = nullptr;
  if (!inline_rows) {
    slot = h->next_slot;
    h->next_slot = (slot + 1) % kRing;
    if (h->slot_used[slot]) {
      hipError_t e = hipEventSynchronize(h->slot_done[slot]);
      if (e != hipSuccess) return hip_fail(h, e, "hipEventSynchronize");
    }
    rp = h->host_ring + (size_t)slot * h->cfg.max_rows;
    dp = h->dev_ring + (size_t)slot * h->cfg.max_rows;
  }
  int G, slice, groups;
  {
    sampler_status pst = plan_groups(h, n, V, &G, &slice, &groups);
    if (pst != SAMPLER_OK) return pst;
  }
  RowParam *recs = h->recs.data();  // records in row order, placed below
  bool any_pen = false;
  for (int r = 0; r < n; ++r) {
    RowParam &p = recs[r];
    const float t = a->temperature ? a->temperature[r] : 1.0f;
    const bool greedy = row_is_greedy(t);
    int32_t k = a->top_k ? a->top_k[r] : -1;
    if (greedy) k = 1;
    p.temperature = greedy ? 1.0f : t;
    p.top_p = a->top_p ? a->top_p[r] : 1.0f;
    p.min_p = a->min_p ? a->min_p[r] : 0.0f;
    p.rep = a->repetition_penalty ? a->repetition_penalty[r] : 1.0f;
    p.pres = a->presence_penalty ? a->presence_penalty[r] : 0.0f;
    p.freq = a->frequency_penalty ? a->frequency_penalty[r] : 0.0f;
    p.top_k = (k == -1 || k >= V) ? V : k;
    uint32_t f = 0;
    if (greedy) f |= RF_GREEDY | RF_TOP1;
    else {
      if (k == 1) f |= RF_TOP1 | RF_TOPK;
      else if (k != -1 && k < V) f |= RF_TOPK;
      if (p.top_p < 1.0f) f |= RF_TOPP;
      if (p.min_p > 0.0f) f |= RF_MINP;
    }
    p.hist_start = 0;
    p.hist_len = 0;
    const bool pen_params = p.rep != 1.0f || p.pres != 0.0f || p.freq != 0.0f;
    if (pen_params && a->history_len && a->history_len[r] > 0) {
      f |= RF_PEN;
      p.hist_start = a->history_start[r];
      p.hist_len = a->history_len[r];
      any_pen = true;
    }
    p.bias_start = 0;
    p.bias_len = 0;
    p.stop_start = 0;
    p.stop_len = 0;
    if (a->bias_len && a->bias_len[r] > 0) {
      p.bias_start = a->bias_start[r];
      p.bias_len = a->bias_len[r];
    }
    if (a->min_tokens && a->output_len[r] < a->min_tokens[r] && a->stop_len && a->stop_len[r] > 0) {
      p.stop_start = a->stop_start[r];
      p.stop_len = a->stop_len[r];
    }
    if (p.bias_len + p.stop_len > 0) {
      f |= RF_SPEC;
      any_pen = true;  // the launch needs the hash machinery
    }
    p.flags = f;
    p.row = r;
    p.pad = 0;
    p.seed = a->row_seed ? a->row_seed[r] : (det ? kDeterministicSeed : a->seed);
    p.stream = a->row_stream ? a->row_stream[r] : (det ? 0u : (uint32_t)r);
    p.offset = a->row_offset ? a->row_offset[r] : a->offset;
  }
  // Place the records: the rows expected to take longest on the groups
  // whose workgroups start first (a stable counting sort by cost class);
  // rows past the first pass keep their order.
  {
    int *rank = h->rank.data(), *ord = h->order.data();
    group_start_order(groups, rank);
    constexpr int kClasses = 12;
    int start[kClasses] = {};
    for (int r = 0; r < n; ++r) ++start[row_cost(recs[r])];
    for (int c = kClasses - 1, acc = 0; c >= 0; --c) {
      const int cnt = start[c];
      start[c] = acc;
      acc += cnt;
    }
    for (int r = 0; r < n; ++r) ord[start[row_cost(recs[r])]++] = r;
    for (int k = 0; k < n; ++k) rp[k < groups ? rank[k] : k] = recs[ord[k]];
  }
  hipError_t e;
  if (!inline_rows) {
    e = hipMemcpyAsync(dp, rp, sizeof(RowParam) * (size_t)n, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(h, e, "hipMemcpyAsync");
    e = hipEventRecord(h->slot_done[slot], stream);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord");
    h->slot_used[slot] = true;
  }

  return plan_and_launch(h, a, ka, dp, any_pen, path, stream);
}

sampler_status sampler_step_graph(sampler_handle *h, const sampler_step_args *a, const sampler_device_params *dp,
                                  void *stream_ptr) {
  if (!h) return SAMPLER_EINVAL;
  h->err.clear();
  if (!a || !dp) {
    h->err = !a ? "args is NULL" : "device params are NULL";
    return SAMPLER_EINVAL;
  }
  if (a->temperature || a->top_p || a->min_p || a->repetition_penalty || a->presence_penalty ||
      a->frequency_penalty || a->top_k || a->history_start || a->history_len || a->row_seed || a->row_offset ||
      a->row_stream || a->bias_start || a->bias_len || a->stop_start || a->stop_len || a->min_tokens ||
      a->output_len) {
    h->err = "sampler_step_graph takes its per-row parameters from the device params: the host arrays of args "
             "must be NULL";
    return SAMPLER_EINVAL;
  }
  if ((dp->min_tokens != nullptr) != (dp->output_len != nullptr)) {
    h->err = "min_tokens and output_len go together";
    return SAMPLER_EINVAL;
  }
  if (a->logprob_mode == SAMPLER_LOGPROB_RAW) {
    h->err = "the raw logprob mode needs host temperatures (sampler_step)";
    return SAMPLER_ENOTSUP;
  }
  // the host checks of sizes, pointers and modes (per-row values are
  // checked on the device)
  sampler_status st = validate(&h->cfg, a, h->err);
  if (st != SAMPLER_OK) return st;
  DeviceGuard guard(h->device);
  if (!guard.ok) {
    h->err = "hipSetDevice failed";
    return SAMPLER_EHIP;
  }
  if (a->path_out) *a->path_out = PATH_FILTERED;
  DevRowArrays dev;
  dev.temperature = dp->temperature;
  dev.top_p = dp->top_p;
  dev.min_p = dp->min_p;
  dev.rep = dp->repetition_penalty;
  dev.pres = dp->presence_penalty;
  dev.freq = dp->frequency_penalty;
  dev.top_k = dp->top_k;
  dev.hist_start = dp->history_start;
  dev.hist_len = dp->history_len;
  dev.seed = dp->row_seed;
  dev.offset = dp->row_offset;
  dev.stream = dp->row_stream;
  dev.bias_start = dp->bias_start;
  dev.bias_len = dp->bias_len;
  dev.stop_start = dp->stop_start;
  dev.stop_len = dp->stop_len;
  dev.min_tokens = dp->min_tokens;
  dev.output_len = dp->output_len;
  // the penalty / bias machinery whenever a row could use it
  const bool any_pen = (dp->history_len && a->history_ids) || dp->bias_len || (dp->min_tokens && dp->stop_len);
  return plan_and_launch(h, a, *h->args, nullptr, any_pen, PATH_FILTERED, reinterpret_cast<hipStream_t>(stream_ptr),
                         &dev);
}

sampler_status sampler_profile_start(sampler_handle *h, int32_t capacity) {
  if (!h || capacity < 1) return SAMPLER_EINVAL;
  DeviceGuard guard(h->device);
  free_profile(h);
  h->prof.resize(2 * (size_t)capacity);
  for (auto &ev : h->prof) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      ev = nullptr;
      free_profile(h);
      return hip_fail(h, e, "hipEventCreate");
    }
  }
  h->prof_cap = capacity;
  h->prof_n = 0;
  return SAMPLER_OK;
}

sampler_status sampler_profile_stop(sampler_handle *h, float *ms, int32_t cap, int32_t *n) {
  if (!h || !n || (cap > 0 && !ms)) return SAMPLER_EINVAL;
  DeviceGuard guard(h->device);
  int k = 0;
  for (int i = 0; i < h->prof_n && i < cap; ++i) {
    hipError_t e = hipEventSynchronize(h->prof[2 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[k], h->prof[2 * i], h->prof[2 * i + 1]);
    if (e != hipSuccess) {
      free_profile(h);
      return hip_fail(h, e, "hipEventElapsedTime");
    }
    ++k;
  }
  *n = k;
  free_profile(h);
  return SAMPLER_OK;
}

void sampler_destroy(sampler_handle *h) {
  if (!h) return;
  DeviceGuard guard(h->device);
  free_handle(h);
}

const char *sampler_last_error(const sampler_handle *h) {
  if (!h) return g_create_error.c_str();
  return h->err.c_str();
}

}  // extern "C"
