// sampler_runtime.cpp -- host side of the decode-step sampler's C ABI.
//
// Validation, per-row normalisation, the batch predicate, the per-row
// records (in the kernel arguments for batches of up to kArgRows rows, so a
// step is one launch and no copy; otherwise through a pinned staging ring
// and one copy), launch planning (workgroups per row) and the launch.  A
// step's exchange workspace is a handle's allocation, or, for
// sampler_step_noalloc, the library's fixed scratch array.
//
// Sources (page titles; sections named where used):
//   [A] "SGLang's +75% sampler speedup skips Qwen3 chat requests"
//   [B] the SGLang 101 operations manual
//   [C] "采样参数对解码开销的影响：temperature、top_p 与采样核路径"
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
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
// Values per thread of a launch whose rows exchange only at the end (see
// launch_is_light).  Measured on MI355X, batch-1 Gumbel at V=151,936 (ids
// only), kernel time: 16 values per thread (19 workgroups) 18.0 us, 8 (38
// workgroups) 16.1 us, 4 (64, the cap for such launches) 15.0 us.
constexpr int kLightValuesPerThread = 4;
// [B] "What the flag switches": requests without a seed use 42.
constexpr uint64_t kDeterministicSeed = 42;
// Steps whose rows outnumber the row kernel's row groups by more than this
// factor run on the streaming kernel (measured on MI355X: see the design
// notes' streaming section).
constexpr int kStreamRowsPerGroup = 1;
// chunked rows: the chunks a launch aims at, above which chunks grow
constexpr int64_t kChunkBatchGroups = 4096;

thread_local std::string g_create_error;

void set_msg(std::string &dst, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  dst = buf;
}

// What a launch needs besides its arguments: the row kernel's limits on the
// device (resident workgroups, LDS plan) and the exchange workspace (group
// words, per-workgroup exchange slots, the abort word), which holds
// `resident` workgroups.
struct Workspace {
  int device = 0;
  int resident = 0;       // workgroups of the row kernel that fit at once (and slots of the workspace)
  int slice_cap = 0;      // largest slice a workgroup holds in LDS
  int det_slice_cap = 0;  // the slice cap of the largest history and bias hashes (deterministic launches)
  int hash_slots = 0;     // LDS hash slots for history counts
  int bias_slots = 0;     // LDS hash slots for logit_bias / stop entries (0: none)
  GroupSync *sync = nullptr;       // [resident]
  WgSlots *slots = nullptr;        // [resident]
  uint32_t *abort_word = nullptr;  // device word: epoch of an aborted launch
  uint32_t *epoch_dev = nullptr;   // device word: epoch of graph-path launches (advanced on the device), or null
  uint32_t epoch = 0;              // epoch of the last host-path launch (1 .. 2^31 - 1)
  // counted histories longer than kMaxHistPerRow (handles planned for them)
  uint32_t *hist_list = nullptr;  // [max_rows * hist_list_row] entries
  int32_t *hist_list_n = nullptr; // [max_rows * kMaxLightG]
  int64_t hist_list_row = 0;      // entries per row: min(kMaxLightG max_history, max_vocab + kMaxSlice)
  // the streaming kernel: workgroups that fit at once, and the rows it
  // leaves to the row kernel (records and the epoch-tagged count word)
  int stream_resident = 0;
  RowParam *defer_rows = nullptr;           // [max_rows]
  unsigned long long *defer_word = nullptr;
  // chunked rows: per record chunk_cap chunk results and one arrival word
  ChunkRec *chunk_recs = nullptr;           // [min(max_rows, kChunkMaxRows) * chunk_cap]
  unsigned long long *chunk_words = nullptr;  // [min(max_rows, kChunkMaxRows) * kChunkWordStride]
  int chunk_cap = 0;
  // limits the workspace was planned for
  int32_t max_history_per_row = 0, max_bias_per_row = 0, max_top_logprobs = 0, max_vocab = 0;
};

}  // namespace

struct sampler_handle {
  sampler_config cfg{};
  Workspace ws;
  RowParam *host_ring = nullptr;   // pinned, kRing slots of max_rows records
  RowParam *dev_ring = nullptr;    // device, kRing slots
  KernelArgs *args = nullptr;      // host: the launch's argument block
  RowParam *graph_rows = nullptr;  // device, max_rows records written by sampler_step_graph's first kernel
  std::vector<RowParam> recs;      // host scratch: a step's records in row order (max_rows)
  std::vector<int> rank, order;    // host scratch: group start order, rows by cost (max_rows)
  hipEvent_t slot_done[kRing] = {};
  bool slot_used[kRing] = {};
  int next_slot = 0;
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

// The path table of [A] "One request with top_p takes the whole batch off
// the fast path", as two properties of the batch: whether any row samples
// (top_k > 1 after normalisation; otherwise the batch is greedy), and
// whether any row truncates (top-k below the whole vocabulary -- greedy rows
// included, their top_k is 1 -- top-p or min-p), which makes it filtered.
int choose_path(const sampler_step_args *a, uint32_t flags) {
  bool samples = false, truncates = false;
  for (int r = 0; r < a->n_rows; ++r) {
    const float t = a->temperature ? a->temperature[r] : 1.0f;
    const int32_t raw = a->top_k ? a->top_k[r] : -1;
    const int32_t k = row_is_greedy(t) ? 1 : (raw == -1 ? kTopKAll : raw);
    samples = samples || k > 1;
    truncates = truncates || k != kTopKAll || (a->top_p && a->top_p[r] != 1.0f) || (a->min_p && a->min_p[r] > 0.0f);
  }
  if (!samples) return PATH_GREEDY;
  if (truncates) return PATH_FILTERED;
  return (flags & SAMPLER_DETERMINISTIC) ? PATH_DETERMINISTIC : PATH_GUMBEL;
}

sampler_status hip_fail(std::string &err, hipError_t e, const char *what) {
  set_msg(err, "%s failed: %s", what, hipGetErrorString(e));
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
  if (h->ws.sync) (void)hipFree(h->ws.sync);
  if (h->ws.slots) (void)hipFree(h->ws.slots);
  if (h->ws.abort_word) (void)hipFree(h->ws.abort_word);
  if (h->ws.epoch_dev) (void)hipFree(h->ws.epoch_dev);
  if (h->ws.hist_list) (void)hipFree(h->ws.hist_list);
  if (h->ws.hist_list_n) (void)hipFree(h->ws.hist_list_n);
  if (h->ws.defer_rows) (void)hipFree(h->ws.defer_rows);
  if (h->ws.defer_word) (void)hipFree(h->ws.defer_word);
  if (h->ws.chunk_recs) (void)hipFree(h->ws.chunk_recs);
  if (h->ws.chunk_words) (void)hipFree(h->ws.chunk_words);
  delete h;
}

int next_pow2_at_least(int v, int lo) {
  int s = lo;
  while (s < v) s *= 2;
  return s;
}

// The LDS plan of the row kernel for a history and bias limit, and the
// workgroups that fit on the device at once.  Returns SAMPLER_OK, or a
// status with a message in err.
sampler_status plan_workspace(Workspace &ws, int device, int32_t max_hist, int32_t max_bias, int32_t max_vocab,
                              int32_t max_top_lp, std::string &err) {
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(err, e, "hipGetDeviceProperties");
  ws.device = device;
  ws.max_history_per_row = max_hist;
  ws.max_bias_per_row = max_bias;
  ws.max_vocab = max_vocab;
  ws.max_top_logprobs = max_top_lp;
  // LDS plan: fixed part + slice of fp32 values + hash of history counts
  // (longer histories than the hash holds arrive counted: the hash area
  // then serves as a bitmap over the slice)
  ws.hash_slots = next_pow2_at_least(2 * (max_hist < kMaxHistPerRow ? max_hist : kMaxHistPerRow), 64);
  ws.bias_slots = max_bias > 0 ? next_pow2_at_least(2 * max_bias, 64) : 0;
  // the dynamic request may use what the kernel's own static LDS leaves
  size_t lds_static = 0;
  if ((e = kernel_lds_static(&lds_static)) != hipSuccess) return hip_fail(err, e, "hipFuncGetAttributes");
  const size_t lds_max = prop.sharedMemPerBlock > lds_static ? prop.sharedMemPerBlock - lds_static : 0;
  const size_t fixed = kernel_lds_fixed() + kernel_lds_region(kMaxSlice, ws.hash_slots, ws.bias_slots, true);
  if (lds_max <= fixed + 16 * kBlock) {
    set_msg(err, "device LDS per workgroup (%zu B) too small", lds_max);
    return SAMPLER_EHIP;
  }
  size_t cap = (lds_max - fixed) / sizeof(float);
  if (cap > (size_t)kMaxSlice) cap = kMaxSlice;
  ws.slice_cap = (int)(cap & ~(size_t)3);
  const size_t fixed_max = kernel_lds_fixed() + kernel_lds_region(kMaxSlice, kMaxHashSlots, 2 * kMaxBiasPerRow, true);
  size_t dcap = lds_max > fixed_max ? (lds_max - fixed_max) / sizeof(float) : 0;
  if (dcap > (size_t)kMaxSlice) dcap = kMaxSlice;
  ws.det_slice_cap = (int)(dcap & ~(size_t)3);
  if (ws.det_slice_cap < 4) ws.det_slice_cap = ws.slice_cap;
  if ((int64_t)ws.slice_cap * kMaxG < max_vocab) {
    set_msg(err, "max_vocab %d exceeds %d (%d workgroups x %d values; lower max_history_per_row to free LDS)",
            max_vocab, ws.slice_cap * kMaxG, kMaxG, ws.slice_cap);
    return SAMPLER_ECAPACITY;
  }
  e = resident_blocks(device, kernel_lds_bytes(ws.slice_cap, ws.hash_slots, ws.bias_slots, true), &ws.resident);
  if (e != hipSuccess) return hip_fail(err, e, "the row kernel's occupancy query");
  if (ws.resident < 1) {
    err = "the row kernel does not fit on this device";
    return SAMPLER_EHIP;
  }
  return SAMPLER_OK;
}

// The launch plan: G workgroups of `slice` values per row, `groups` row
// groups (rows strided over them).
sampler_status plan_groups(const Workspace &ws, bool det, bool light, int n, int V, int *G_out, int *slice_out,
                           int *groups_out, std::string &err) {
  // deterministic launches cut every row by the slice cap of the largest
  // hashes any handle may have, so that the cut -- and with it each row's
  // reduction order -- depends on V alone, not on the handle's limits
  const int cap = det ? ws.det_slice_cap : ws.slice_cap;
  const int g_min = (V + cap - 1) / cap;
  if (g_min > kMaxG || g_min > ws.resident) {
    set_msg(err, "vocab %d needs %d workgroups per row (max %d)", V, g_min, kMaxG < ws.resident ? kMaxG : ws.resident);
    return SAMPLER_ECAPACITY;
  }
  int G;
  if (det) {
    G = g_min;  // depends on V only: a row's reduction order is batch invariant
  } else {
    const int fill = ws.resident / n;
    // at least ~32 values per thread: a row's steps are latency-bound, and
    // fewer workgroups per row exchange faster (measured on MI355X at N=8,
    // V=151,936: 10 workgroups per row 34.7 us, 32 workgroups 41.9 us).
    // Light launches exchange once, at the end, and spend their time in
    // Philox and the loads: kLightValuesPerThread.
    const int vpt = light ? kLightValuesPerThread : 32;
    const int by_work = (V + vpt * kBlock - 1) / (vpt * kBlock);
    G = fill < by_work ? fill : by_work;
    const int gcap = light ? kMaxLightG : kMaxG;
    if (G > gcap) G = gcap;
    if (G > ws.resident) G = ws.resident;
    if (G < g_min) G = g_min;
  }
  int slice = (V + G - 1) / G;
  slice = (slice + 3) & ~3;
  G = (V + slice - 1) / slice;  // every workgroup gets a non-empty slice
  const int groups = ws.resident / G;
  *G_out = G;
  *slice_out = slice;
  *groups_out = groups < n ? groups : n;
  return SAMPLER_OK;
}

// Whether no row of a step needs its row's merged max: no outputs besides
// the token, no top-k / top-p / min-p, no inverse-CDF selection (rows that
// keep every token, and greedy rows).  Such rows meet their peers only in
// the final exchange, so the launch spreads them over more workgroups.
bool launch_is_light(const sampler_step_args *a, uint32_t flags) {
  if ((flags & SAMPLER_INVERSE_CDF) || a->probs || a->logprobs || a->top_logprobs > 0) return false;
  for (int r = 0; r < a->n_rows; ++r) {
    if (row_is_greedy(a->temperature ? a->temperature[r] : 1.0f)) continue;
    const int32_t k = a->top_k ? a->top_k[r] : -1;
    if ((k != -1 && k < a->vocab) || (a->top_p && a->top_p[r] < 1.0f) || (a->min_p && a->min_p[r] > 0.0f))
      return false;
  }
  return true;
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

// The normalised records of rows [r0, r0 + n) of a step, in row order
// ([A] "One request with top_p ...": 0 <= T < 1e-6 is greedy, T := 1 and
// top_k := 1; -1 means the whole vocabulary).  Returns whether any row needs
// the history / bias machinery.
bool build_records(const sampler_step_args *a, bool det, int r0, int n, RowParam *recs) {
  const int V = a->vocab;
  bool any_pen = false;
  for (int i = 0; i < n; ++i) {
    const int r = r0 + i;
    RowParam &p = recs[i];
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
  return any_pen;
}

// Place n records: the rows expected to take longest on the groups whose
// workgroups start first (a stable counting sort by cost class); rows past
// the first pass keep their order.  rank and ord hold n ints each.
void place_records(const RowParam *recs, int n, int groups, int *rank, int *ord, RowParam *out) {
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
  for (int k = 0; k < n; ++k) out[k < groups ? rank[k] : k] = recs[ord[k]];
}

// Whether a step may run on the streaming kernel: ids and top logprobs of
// the sampled distribution only, no logits processors, Gumbel-max (or
// argmax) selection, histories the hash holds, rows short enough for its
// hash packing.  recs: the step's records.
bool stream_eligible(const Workspace &ws, uint32_t flags, const sampler_step_args *a, const RowParam *recs, int n) {
  if (flags & (SAMPLER_NO_STREAM | SAMPLER_DETERMINISTIC | SAMPLER_INVERSE_CDF)) return false;
  if (a->probs || a->logprobs || a->vocab_mask) return false;
  if (a->top_logprobs > 0 && a->logprob_mode != SAMPLER_LOGPROB_PROCESSED) return false;
  if (a->vocab > kStreamMaxVocab || ws.stream_resident < 1) return false;
  for (int r = 0; r < n; ++r) {
    if (recs[r].flags & RF_SPEC) return false;
    if ((recs[r].flags & RF_PEN) && recs[r].hist_len > kMaxHistPerRow) return false;
  }
  return true;
}

// Whether a step may run on the small-row kernel: at most kSmallV values per
// row, every row keeping every value (Gumbel-max or greedy), no penalties,
// processors or top-logprob list, logprobs of the sampled distribution
// (the raw mode differs at T != 1).  The forced-filtered A/B switch and the
// deterministic and inverse-CDF modes keep the row kernel.
bool small_eligible(uint32_t flags, const sampler_step_args *a, const RowParam *recs, int n) {
  if (flags & (SAMPLER_DETERMINISTIC | SAMPLER_INVERSE_CDF | SAMPLER_FORCE_FILTERED)) return false;
  if (a->vocab > kSmallV || a->top_logprobs > 0 || a->vocab_mask) return false;
  if (a->logprobs && a->logprob_mode == SAMPLER_LOGPROB_RAW) return false;
  for (int r = 0; r < n; ++r)
    if (recs[r].flags & (RF_TOPK | RF_TOPP | RF_MINP | RF_PEN | RF_SPEC)) return false;
  return true;
}

// Whether a step may run on the chunked-row kernel: rows longer than kSmallV
// of the small-row kernel's kind, in a step that wants token ids (and row
// status) only.  *U: groups of four per thread, *C: chunks per row (more
// values per thread for batches of many chunks).
bool chunk_eligible(const Workspace &ws, uint32_t flags, const sampler_step_args *a, const RowParam *recs, int n,
                    int *U, int *C) {
  if (flags & (SAMPLER_DETERMINISTIC | SAMPLER_INVERSE_CDF | SAMPLER_FORCE_FILTERED | SAMPLER_FORCE_STREAM))
    return false;
  if (!ws.chunk_recs || a->vocab <= kSmallV || a->vocab > kChunkMaxV || n > kChunkMaxRows) return false;
  if (a->probs || a->logprobs || a->top_logprobs > 0 || a->vocab_mask) return false;
  for (int r = 0; r < n; ++r)
    if (recs[r].flags & (RF_TOPK | RF_TOPP | RF_MINP | RF_PEN | RF_SPEC)) return false;
  const int64_t V = a->vocab;
  auto chunks = [&](int uu) { return (V + 4 * kChunkBlock * uu - 1) / (4 * kChunkBlock * uu); };
  // one group per thread up to 64 chunks a row, else at least two (the
  // merge reads fewer records; measured on batch-1 rows of 151,936 values)
  int u = chunks(1) > 64 ? 2 : 1;
  while (u < kChunkMaxU && (chunks(u) > ws.chunk_cap || (int64_t)n * chunks(u) > kChunkBatchGroups)) u *= 2;
  if (chunks(u) > ws.chunk_cap) return false;
  *U = u;
  *C = (int)chunks(u);
  return true;
}

// Cost class of a row on the streaming kernel (larger: longer): rows that
// keep every value run Philox over the whole row; top-p without top-k keeps
// the most values; argmax rows read the row once.
int stream_cost(const RowParam &p) {
  if (p.flags & (RF_GREEDY | RF_TOP1)) return 0;
  if (!(p.flags & (RF_TOPK | RF_TOPP | RF_MINP))) return 4;
  if ((p.flags & RF_TOPP) && !(p.flags & RF_TOPK)) return 3;
  if (p.flags & RF_TOPK) return 1;
  return 2;
}

// The streaming kernel's order: costlier rows first (workgroup b starts on
// row b), a stable counting sort.  ord holds n ints.
void stream_records(const RowParam *recs, int n, int *ord, RowParam *out) {
  constexpr int kClasses = 5;
  int start[kClasses] = {};
  for (int r = 0; r < n; ++r) ++start[stream_cost(recs[r])];
  for (int c = kClasses - 1, acc = 0; c >= 0; --c) {
    const int cnt = start[c];
    start[c] = acc;
    acc += cnt;
  }
  for (int r = 0; r < n; ++r) ord[start[stream_cost(recs[r])]++] = r;
  for (int k = 0; k < n; ++k) out[k] = recs[ord[k]];
}

// Kernel parameters for n rows of a step and the launch.  `dp`: the device
// records, or null (records in ka.rows); `dev`: per-row arrays in device
// memory that rows_kernel normalises into `graph_rows` first
// (sampler_step_graph).
sampler_status plan_and_launch(Workspace &ws, uint32_t flags, int32_t wait_spin_limit, const sampler_step_args *a,
                               int n, KernelArgs &ka, const RowParam *dp, bool any_pen, int path, hipStream_t stream,
                               std::string &err, const DevRowArrays *dev = nullptr, RowParam *graph_rows = nullptr,
                               hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr, bool streamed = false,
                               bool small = false, int chunk_u = 0, int chunk_c = 0) {
  const int V = a->vocab;
  const bool det = (flags & SAMPLER_DETERMINISTIC) != 0;
  hipError_t e;
  int G, slice, groups;
  sampler_status st = plan_groups(ws, det, !dev && launch_is_light(a, flags), n, V, &G, &slice, &groups, err);
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
  kp.hash_slots = ws.hash_slots;
  kp.bias_slots = ws.bias_slots;
  kp.vocab_mask = a->vocab_mask;
  kp.mask_stride = a->mask_stride;
  kp.bias_ids = a->bias_ids;
  kp.bias_vals = a->bias_vals;
  kp.stop_ids = a->stop_ids;
  kp.lp_mode = a->logprob_mode != SAMPLER_LOGPROB_PROCESSED ? 1 : 0;
  kp.icdf = (flags & SAMPLER_INVERSE_CDF) ? 1 : 0;
  if (dev) {
    kp.dev = *dev;
    kp.rows = graph_rows;
  }
  kp.det = det ? 1 : 0;
  kp.max_hist = ws.max_history_per_row;
  kp.max_bias = ws.max_bias_per_row;
  kp.seed = a->seed;
  kp.offset = a->offset;
  // a history longer than the row kernel's hash holds is counted first
  bool long_hist = false;
  if (ws.hist_list) {
    long_hist = dev != nullptr;  // device-side lengths: the list kernel checks each row
    for (int r = 0; r < a->n_rows && !long_hist && a->history_len; ++r) long_hist = a->history_len[r] > kMaxHistPerRow;
  }
  if (long_hist) {
    kp.hist_list = ws.hist_list;
    kp.hist_list_n = ws.hist_list_n;
    kp.hist_list_cap = ws.max_history_per_row < slice ? ws.max_history_per_row : slice;
  }
  const size_t esz = a->dtype == SAMPLER_DTYPE_F32 ? 4 : 2;
  const bool lvec = ((uintptr_t)a->logits % (4 * esz) == 0) && (a->row_stride % 4 == 0);
  const bool ovec = ((V & 3) == 0) && ((uintptr_t)a->probs % 16 == 0) && ((uintptr_t)a->logprobs % 16 == 0);
  const bool lvec16 = ((uintptr_t)a->logits % 16 == 0) && ((a->row_stride * (int64_t)esz) % 16 == 0);
  kp.vec_ok = (lvec ? 1 : 0) | (ovec ? 2 : 0) | (lvec16 ? 4 : 0);
  kp.path = path;
  kp.sync = ws.sync;
  kp.slots = ws.slots;
  kp.abort_word = ws.abort_word;
  // every launch has its own epoch: host launches count up through
  // 1 .. 2^31 - 1; graph-path launches read theirs from a device word that
  // rows_kernel advances (bit 31 set), so each replay of a captured graph is
  // a launch of its own
  ws.epoch = (ws.epoch & 0x7FFFFFFFu) + 1u;
  if (ws.epoch == 0x80000000u) ws.epoch = 1;
  kp.epoch = ws.epoch;
  kp.epoch_dev = dev ? ws.epoch_dev : nullptr;
  kp.spin_limit = (uint32_t)wait_spin_limit;
  if (dev && (e = launch_rows(kp, graph_rows, stream)) != hipSuccess) return hip_fail(err, e, "rows kernel launch");
  if (long_hist && (e = launch_hist_list(ka, stream)) != hipSuccess)
    return hip_fail(err, e, "history count kernel launch");
  if (small) {
    e = launch_small(ka, a->dtype, stream, ev0, ev1);
    if (e != hipSuccess) return hip_fail(err, e, "small-row kernel launch");
    return SAMPLER_OK;
  }
  if (chunk_u > 0) {
    kp.chunk_recs = ws.chunk_recs;
    kp.chunk_words = ws.chunk_words;
    kp.chunk_u = chunk_u;
    kp.chunk_n = chunk_c;
    kp.chunk_stride = ws.chunk_cap;
    e = launch_chunk(ka, a->dtype, stream, ev0, ev1);
    if (e != hipSuccess) return hip_fail(err, e, "chunked-row kernel launch");
    return SAMPLER_OK;
  }
  if (streamed) {
    // the streaming kernel, then the row kernel on the rows it left (their
    // count read on the device; nothing to do when it left none)
    kp.defer_rows = ws.defer_rows;
    kp.defer_word = ws.defer_word;
    // one workgroup per row: the dispatcher starts each as a slot frees, so
    // the costlier rows (placed first) do not hold up a fixed set of others
    e = launch_stream(ka, a->dtype, any_pen, n, stream, ev0, nullptr);
    if (e != hipSuccess) return hip_fail(err, e, "streaming kernel launch");
    kp.n_rows_epoch = kp.epoch;
    kp.n_rows_word = ws.defer_word;
    kp.rows = ws.defer_rows;
    ws.epoch = (ws.epoch & 0x7FFFFFFFu) + 1u;
    if (ws.epoch == 0x80000000u) ws.epoch = 1;
    kp.epoch = ws.epoch;
    e = launch_step(ka, a->dtype, any_pen, (flags & SAMPLER_COOPERATIVE_LAUNCH) != 0, stream, nullptr, ev1);
    if (e != hipSuccess) return hip_fail(err, e, "kernel launch");
    return SAMPLER_OK;
  }
  e = launch_step(ka, a->dtype, any_pen, (flags & SAMPLER_COOPERATIVE_LAUNCH) != 0, stream, ev0, ev1);
  if (e != hipSuccess) return hip_fail(err, e, "kernel launch");
  // [B] "Logprobs are temperature-scaled", the original-logprob switch: the
  // rows whose effective temperature is not 1 get log_softmax of their
  // processed logits from a second kernel (on device-side parameters the
  // kernel itself skips the rows at temperature 1)
  bool raw = a->logprob_mode == SAMPLER_LOGPROB_RAW && (a->logprobs || a->top_logprobs > 0);
  if (raw && !dev) {
    raw = false;
    for (int r = 0; r < a->n_rows && !raw; ++r) {
      const float t = a->temperature ? a->temperature[r] : 1.0f;
      raw = !row_is_greedy(t) && t != 1.0f;
    }
  }
  if (raw) {
    ws.epoch = (ws.epoch & 0x7FFFFFFFu) + 1u;
    if (ws.epoch == 0x80000000u) ws.epoch = 1;
    kp.epoch = ws.epoch;
    kp.epoch_dev_add = 1;
    e = launch_raw_lp(ka, a->dtype, stream);
    kp.epoch_dev_add = 0;
    if (e != hipSuccess) return hip_fail(err, e, "raw-logprob kernel launch");
  }
  return SAMPLER_OK;
}

// The path a step runs under: the predicate's, unless a SAMPLER_FORCE_*
// flag names another.
int run_path(int predicate_path, uint32_t flags) {
  if (flags & SAMPLER_FORCE_FILTERED) return PATH_FILTERED;
  if (flags & SAMPLER_FORCE_PATH_GUMBEL) return PATH_GUMBEL;
  if (flags & SAMPLER_FORCE_PATH_GREEDY) return PATH_GREEDY;
  return predicate_path;
}

bool flags_ok(uint32_t flags) {
  return !(flags & ~(SAMPLER_DETERMINISTIC | SAMPLER_FORCE_FILTERED | SAMPLER_COOPERATIVE_LAUNCH |
                     SAMPLER_INVERSE_CDF | SAMPLER_FORCE_PATH_GREEDY | SAMPLER_FORCE_PATH_GUMBEL |
                     SAMPLER_FORCE_STREAM | SAMPLER_NO_STREAM)) &&
         __builtin_popcount(flags & (SAMPLER_FORCE_FILTERED | SAMPLER_FORCE_PATH_GREEDY | SAMPLER_FORCE_PATH_GUMBEL)) <= 1 &&
         __builtin_popcount(flags & (SAMPLER_FORCE_STREAM | SAMPLER_NO_STREAM)) <= 1;
}

// ---------------------------------------------------------------- no-alloc scratch
// The exchange workspace of sampler_step_noalloc, for callers that cannot
// allocate: group words, exchange slots and the abort word of kScratchWgs
// workgroups (one per compute unit of an MI355X), in one file-scope device
// array.  Every GPU the library runs on holds its own copy until the process
// ends; host code reaches a device's copy only through the address that
// hipGetSymbolAddress gave for that device, never through the array's name.
constexpr int kScratchWgs = 256;
constexpr size_t kScratchSync = 0;
constexpr size_t kScratchSlots = ((sizeof(GroupSync) * kScratchWgs + 255) / 256) * 256;
constexpr size_t kScratchAbort = kScratchSlots + ((sizeof(WgSlots) * kScratchWgs + 255) / 256) * 256;
constexpr size_t kScratchBytes = kScratchAbort + 256;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
struct StaticDevice {
  bool ready = false;
  Workspace ws;
  sampler_status st = SAMPLER_OK;
  std::string err;  // the set-up failure, if any
};
std::mutex g_static_mu;
StaticDevice g_static[kMaxDevices];
thread_local std::string g_static_error;
thread_local KernelArgs g_static_args;  // the launch's argument block (copied at launch)

// Set up device `dev` for sampler_step_noalloc once: its scratch address and
// the row kernel's plan for the largest history, bias and top-logprob
// limits.  Called with g_static_mu held and `dev` current.
sampler_status static_setup(int dev) {
  StaticDevice &sd = g_static[dev];
  if (sd.ready) return sd.st;
  sd.ready = true;
  unsigned char *ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(reinterpret_cast<void **>(&ptr), HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    set_msg(sd.err, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    return sd.st = SAMPLER_EHIP;
  }
  Workspace &ws = sd.ws;
  sd.st = plan_workspace(ws, dev, kMaxHistPerRow, kMaxBiasPerRow, kMaxVocab, kMaxTopLogprobs, sd.err);
  if (sd.st == SAMPLER_ECAPACITY) {
    // the largest vocabulary the plan allows
    const int V = ws.slice_cap * kMaxG;
    sd.st = plan_workspace(ws, dev, kMaxHistPerRow, kMaxBiasPerRow, V, kMaxTopLogprobs, sd.err);
  }
  if (sd.st != SAMPLER_OK) return sd.st;
  if (ws.resident > kScratchWgs) ws.resident = kScratchWgs;
  ws.sync = reinterpret_cast<GroupSync *>(ptr + kScratchSync);
  ws.slots = reinterpret_cast<WgSlots *>(ptr + kScratchSlots);
  ws.abort_word = reinterpret_cast<uint32_t *>(ptr + kScratchAbort);
  ws.epoch_dev = nullptr;
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
      cfg->max_history_per_row > kMaxHistLong || cfg->max_top_logprobs < 0 ||
      cfg->max_top_logprobs > kMaxTopLogprobs || cfg->max_bias_per_row < 0 ||
      cfg->max_bias_per_row > kMaxBiasPerRow || cfg->wait_spin_limit < 0 || !flags_ok(cfg->flags)) {
    set_msg(g_create_error,
            "bad config: need max_rows >= 1, 1 <= max_vocab <= %d, 0 <= max_history_per_row <= %d, "
            "0 <= max_top_logprobs <= %d, 0 <= max_bias_per_row <= %d, wait_spin_limit >= 0, known flags and "
            "at most one SAMPLER_FORCE_* flag",
            kMaxVocab, kMaxHistLong, kMaxTopLogprobs, kMaxBiasPerRow);
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
  {
    const sampler_status st = plan_workspace(h->ws, cfg->device, cfg->max_history_per_row, cfg->max_bias_per_row,
                                             cfg->max_vocab, cfg->max_top_logprobs, g_create_error);
    if (st != SAMPLER_OK) {
      free_handle(h);
      return st;
    }
  }
  {
    Workspace &ws = h->ws;
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
    const size_t n_groups_max = (size_t)ws.resident;  // one group per resident workgroup at most
    if ((e = hipMalloc((void **)&ws.sync, sizeof(GroupSync) * n_groups_max)) != hipSuccess) goto fail;
    if ((e = hipMemset(ws.sync, 0, sizeof(GroupSync) * n_groups_max)) != hipSuccess) goto fail;
    if ((e = hipMalloc((void **)&ws.slots, sizeof(WgSlots) * (size_t)ws.resident)) != hipSuccess) goto fail;
    if ((e = hipMemset(ws.slots, 0, sizeof(WgSlots) * (size_t)ws.resident)) != hipSuccess) goto fail;
    if ((e = hipMalloc((void **)&ws.abort_word, 256)) != hipSuccess) goto fail;
    if ((e = hipMemset(ws.abort_word, 0, 256)) != hipSuccess) goto fail;
    if ((e = hipMalloc((void **)&ws.epoch_dev, 256)) != hipSuccess) goto fail;
    if ((e = hipMemset(ws.epoch_dev, 0, 256)) != hipSuccess) goto fail;
    if (cfg->max_history_per_row > kMaxHistPerRow) {
      // list (row, slice) of a launch of G slices of `slice` values holds at
      // most min(max_history, slice) entries, and G min(max_history, slice)
      // <= min(kMaxLightG max_history, V + slice) (G never exceeds kMaxLightG)
      const int64_t by_hist = (int64_t)kMaxLightG * cfg->max_history_per_row;
      const int64_t by_vocab = (int64_t)cfg->max_vocab + kMaxSlice;
      ws.hist_list_row = by_hist < by_vocab ? by_hist : by_vocab;
      if ((e = hipMalloc((void **)&ws.hist_list, sizeof(uint32_t) * (size_t)ws.hist_list_row * cfg->max_rows)) !=
          hipSuccess)
        goto fail;
      if ((e = hipMalloc((void **)&ws.hist_list_n, sizeof(int32_t) * (size_t)kMaxLightG * cfg->max_rows)) !=
          hipSuccess)
        goto fail;
    }
    if ((e = hipMalloc((void **)&ws.defer_rows, sizeof(RowParam) * (size_t)cfg->max_rows)) != hipSuccess) goto fail;
    if ((e = hipMalloc((void **)&ws.defer_word, 256)) != hipSuccess) goto fail;
    if ((e = hipMemset(ws.defer_word, 0, 256)) != hipSuccess) goto fail;
    if (cfg->max_vocab > kSmallV) {
      // at most min(kChunkMax, ceil(V / (4 kChunkBlock))) chunks per row
      const int64_t by_vocab = ((int64_t)cfg->max_vocab + 4 * kChunkBlock - 1) / (4 * kChunkBlock);
      ws.chunk_cap = (int)(by_vocab < kChunkMax ? by_vocab : kChunkMax);
      const size_t crows = (size_t)(cfg->max_rows < kChunkMaxRows ? cfg->max_rows : kChunkMaxRows);
      if ((e = hipMalloc((void **)&ws.chunk_recs, sizeof(ChunkRec) * (size_t)ws.chunk_cap * crows)) != hipSuccess)
        goto fail;
      const size_t wbytes = sizeof(unsigned long long) * kChunkWordStride * crows;
      if ((e = hipMalloc((void **)&ws.chunk_words, wbytes)) != hipSuccess) goto fail;
      if ((e = hipMemset(ws.chunk_words, 0, wbytes)) != hipSuccess) goto fail;
    }
    if ((e = stream_resident(cfg->device,
                             stream_lds_bytes(ws.hash_slots, true,
                                              cfg->max_vocab < kStreamMaxVocab ? cfg->max_vocab : kStreamMaxVocab),
                             &ws.stream_resident)) != hipSuccess)
      goto fail;
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
  DeviceGuard guard(h->ws.device);
  if (!guard.ok) {
    h->err = "hipSetDevice failed";
    return SAMPLER_EHIP;
  }

  const int n = a->n_rows, V = a->vocab;
  const bool det = (h->cfg.flags & SAMPLER_DETERMINISTIC) != 0;
  const int pred = choose_path(a, h->cfg.flags);
  if (a->path_out) *a->path_out = pred;
  const int path = run_path(pred, h->cfg.flags);

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
      if (e != hipSuccess) return hip_fail(h->err, e, "hipEventSynchronize");
    }
    rp = h->host_ring + (size_t)slot * h->cfg.max_rows;
    dp = h->dev_ring + (size_t)slot * h->cfg.max_rows;
  }
  int G, slice, groups;
  st = plan_groups(h->ws, det, launch_is_light(a, h->cfg.flags), n, V, &G, &slice, &groups, h->err);
  if (st != SAMPLER_OK) return st;
  const bool any_pen = build_records(a, det, 0, n, h->recs.data());
  // the streaming kernel when forced, or when the row kernel would walk its
  // row groups through several rows each
  const bool small = small_eligible(h->cfg.flags, a, h->recs.data(), n);
  int chunk_u = 0, chunk_c = 0;
  const bool chunked = !small && chunk_eligible(h->ws, h->cfg.flags, a, h->recs.data(), n, &chunk_u, &chunk_c);
  const bool streamed = !small && !chunked && stream_eligible(h->ws, h->cfg.flags, a, h->recs.data(), n) &&
                        ((h->cfg.flags & SAMPLER_FORCE_STREAM) || n > kStreamRowsPerGroup * groups);
  if (a->kernel_out) *a->kernel_out = small ? 2 : chunked ? 3 : streamed ? 1 : 0;
  if (streamed) stream_records(h->recs.data(), n, h->order.data(), rp);
  else if (small || chunked) std::copy(h->recs.data(), h->recs.data() + n, rp);
  else place_records(h->recs.data(), n, groups, h->rank.data(), h->order.data(), rp);
  hipError_t e;
  if (!inline_rows) {
    e = hipMemcpyAsync(dp, rp, sizeof(RowParam) * (size_t)n, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(h->err, e, "hipMemcpyAsync");
    e = hipEventRecord(h->slot_done[slot], stream);
    if (e != hipSuccess) return hip_fail(h->err, e, "hipEventRecord");
    h->slot_used[slot] = true;
  }
  const bool prof = h->prof_n < h->prof_cap;
  st = plan_and_launch(h->ws, h->cfg.flags, h->cfg.wait_spin_limit, a, n, ka, dp, any_pen, path, stream, h->err,
                       nullptr, nullptr, prof ? h->prof[2 * h->prof_n] : nullptr,
                       prof ? h->prof[2 * h->prof_n + 1] : nullptr, streamed, small, chunk_u, chunk_c);
  if (st == SAMPLER_OK && prof) ++h->prof_n;
  return st;
}

sampler_status sampler_step_noalloc(const sampler_step_args *a, uint32_t flags, int32_t device, void *stream_ptr) {
  g_static_error.clear();
  if (!flags_ok(flags) || (flags & SAMPLER_COOPERATIVE_LAUNCH)) {
    g_static_error = "flags: SAMPLER_DETERMINISTIC, SAMPLER_INVERSE_CDF and at most one SAMPLER_FORCE_* flag";
    return SAMPLER_EINVAL;
  }
  int n_dev = 0;
  hipError_t e = hipGetDeviceCount(&n_dev);
  if (e != hipSuccess || n_dev <= 0) {
    set_msg(g_static_error, "no usable HIP device (%s)", e == hipSuccess ? "none found" : hipGetErrorString(e));
    (void)hipGetLastError();
    return SAMPLER_EHIP;
  }
  if (device < 0 || device >= n_dev || device >= kMaxDevices) {
    set_msg(g_static_error, "device %d out of range (0..%d)", device, (n_dev < kMaxDevices ? n_dev : kMaxDevices) - 1);
    return SAMPLER_EINVAL;
  }
  DeviceGuard guard(device);
  if (!guard.ok) {
    g_static_error = "hipSetDevice failed";
    return SAMPLER_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_static_mu);
  sampler_status st = static_setup(device);
  if (st != SAMPLER_OK) {
    g_static_error = g_static[device].err;
    return st;
  }
  Workspace &ws = g_static[device].ws;
  // the limits of the scratch plan; any number of rows (launched in pieces)
  sampler_config cfg{};
  cfg.max_rows = a ? (a->n_rows > 0 ? a->n_rows : 1) : 1;
  cfg.max_vocab = ws.max_vocab;
  cfg.max_history_per_row = ws.max_history_per_row;
  cfg.max_top_logprobs = ws.max_top_logprobs;
  cfg.max_bias_per_row = ws.max_bias_per_row;
  cfg.device = device;
  cfg.flags = flags;
  st = validate(&cfg, a, g_static_error);
  if (st != SAMPLER_OK) return st;
  // the raw logprobs of rows whose temperature is not 1 come from a second
  // kernel that carries a small private (scratch) segment, which the runtime
  // may back with memory at its first launch: not offered here
  if (a->logprob_mode == SAMPLER_LOGPROB_RAW)
    for (int r = 0; r < a->n_rows; ++r) {
      const float t = a->temperature ? a->temperature[r] : 1.0f;
      if (!row_is_greedy(t) && t != 1.0f) {
        set_msg(g_static_error, "row %d: the raw logprob mode at temperature %g needs a handle (sampler_step)", r,
                (double)t);
        return SAMPLER_ENOTSUP;
      }
    }
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  const bool det = (flags & SAMPLER_DETERMINISTIC) != 0;
  const int pred = choose_path(a, flags);
  if (a->path_out) *a->path_out = pred;
  if (a->kernel_out) *a->kernel_out = 0;
  const int path = run_path(pred, flags);
  // rows in pieces of up to kArgRows, each one launch with its records in
  // the kernel arguments; the pieces share the scratch in stream order
  for (int r0 = 0; r0 < a->n_rows; r0 += kArgRows) {
    const int n = a->n_rows - r0 < kArgRows ? a->n_rows - r0 : kArgRows;
    int G, slice, groups;
    st = plan_groups(ws, det, launch_is_light(a, flags), n, a->vocab, &G, &slice, &groups, g_static_error);
    if (st != SAMPLER_OK) return st;
    RowParam recs[kArgRows];
    int rank[kArgRows], ord[kArgRows];
    KernelArgs &ka = g_static_args;
    const bool any_pen = build_records(a, det, r0, n, recs);
    place_records(recs, n, groups, rank, ord, ka.rows);
    st = plan_and_launch(ws, flags, 0, a, n, ka, nullptr, any_pen, path, stream, g_static_error);
    if (st != SAMPLER_OK) return st;
  }
  return SAMPLER_OK;
}

const char *sampler_noalloc_last_error(void) { return g_static_error.c_str(); }

sampler_status sampler_phase_stamps(uint64_t *host_out, int32_t cap, int32_t *blocks_out, int32_t *slots_out,
                                    int32_t *clock_khz_out) {
  if (blocks_out) *blocks_out = kStampBlocks;
  if (slots_out) *slots_out = kStampSlots;
  if (!host_out || cap < 0) return SAMPLER_EINVAL;
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return SAMPLER_EHIP;
  if (clock_khz_out) *clock_khz_out = khz;
  e = phase_stamps_take(reinterpret_cast<unsigned long long *>(host_out), (size_t)cap);
  if (e == hipErrorNotSupported) return SAMPLER_ENOTSUP;
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
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
  // the host checks of sizes, pointers and modes (per-row values are
  // checked on the device)
  sampler_status st = validate(&h->cfg, a, h->err);
  if (st != SAMPLER_OK) return st;
  DeviceGuard guard(h->ws.device);
  if (!guard.ok) {
    h->err = "hipSetDevice failed";
    return SAMPLER_EHIP;
  }
  if (a->path_out) *a->path_out = PATH_FILTERED;
  if (a->kernel_out) *a->kernel_out = 0;
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
  const bool prof = h->prof_n < h->prof_cap;
  sampler_status lst = plan_and_launch(h->ws, h->cfg.flags, h->cfg.wait_spin_limit, a, a->n_rows, *h->args, nullptr,
                                       any_pen, PATH_FILTERED, reinterpret_cast<hipStream_t>(stream_ptr), h->err, &dev,
                                       h->graph_rows, prof ? h->prof[2 * h->prof_n] : nullptr,
                                       prof ? h->prof[2 * h->prof_n + 1] : nullptr);
  if (lst == SAMPLER_OK && prof) ++h->prof_n;
  return lst;
}

sampler_status sampler_set_wait_spin_limit(sampler_handle *h, int32_t limit) {
  if (!h || limit < 0) return SAMPLER_EINVAL;
  h->cfg.wait_spin_limit = limit;
  return SAMPLER_OK;
}

sampler_status sampler_profile_start(sampler_handle *h, int32_t capacity) {
  if (!h || capacity < 1) return SAMPLER_EINVAL;
  DeviceGuard guard(h->ws.device);
  free_profile(h);
  h->prof.resize(2 * (size_t)capacity);
  for (auto &ev : h->prof) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      ev = nullptr;
      free_profile(h);
      return hip_fail(h->err, e, "hipEventCreate");
    }
  }
  h->prof_cap = capacity;
  h->prof_n = 0;
  return SAMPLER_OK;
}

sampler_status sampler_profile_stop(sampler_handle *h, float *ms, int32_t cap, int32_t *n) {
  if (!h || !n || (cap > 0 && !ms)) return SAMPLER_EINVAL;
  DeviceGuard guard(h->ws.device);
  int k = 0;
  for (int i = 0; i < h->prof_n && i < cap; ++i) {
    hipError_t e = hipEventSynchronize(h->prof[2 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[k], h->prof[2 * i], h->prof[2 * i + 1]);
    if (e != hipSuccess) {
      free_profile(h);
      return hip_fail(h->err, e, "hipEventElapsedTime");
    }
    ++k;
  }
  *n = k;
  free_profile(h);
  return SAMPLER_OK;
}

void sampler_destroy(sampler_handle *h) {
  if (!h) return;
  DeviceGuard guard(h->ws.device);
  free_handle(h);
}

const char *sampler_last_error(const sampler_handle *h) {
  if (!h) return g_create_error.c_str();
  return h->err.c_str();
}

}  // extern "C"
