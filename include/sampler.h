/*
 * sampler.h -- C ABI of the MI355X (gfx950) per-decode-step token sampler.
 *
 * One call samples one decode step for a batch of N rows over a V-entry
 * vocabulary: penalties from each row's token history, temperature,
 * top-k / top-p / min-p truncation, fp32 softmax and log_softmax of the
 * distribution sampled from, and token selection by greedy argmax or by
 * Gumbel-max (probabilities divided by Exp(1) draws, then argmax).  A batch
 * predicate picks the greedy, Gumbel or filtered kernel.  Everything runs in
 * HIP kernels on the caller's stream; nothing is read back to the host.
 *
 * Pages the behaviour follows (cited by title and section below):
 *   [A] "SGLang's +75% sampler speedup skips Qwen3 chat requests"
 *   [B] the SGLang 101 operations manual ("Logprobs are temperature-scaled",
 *       "What the flag switches")
 *   [C] "采样参数对解码开销的影响：temperature、top_p 与采样核路径"
 *       (vLLM 0.5.0 sampling-parameter decode-cost note)
 *
 * Conventions for every entry point:
 *   - No C++ exception crosses this ABI; errors are negative status codes
 *     and a per-handle message (sampler_last_error).
 *   - Pointers documented "device" must point to device memory of the
 *     handle's GPU; "host" pointers are read before the call returns, so
 *     the caller may reuse them immediately.
 *   - The caller owns every buffer it passes.  The handle owns only its
 *     device workspace and its pinned host staging ring.
 *   - A handle serves one stream at a time and is not thread-safe.
 */
#ifndef DSTS_SAMPLER_H
#define DSTS_SAMPLER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sampler_status {
  SAMPLER_OK = 0,
  SAMPLER_EINVAL = -1,    /* an argument breaks the contract below */
  SAMPLER_ECAPACITY = -2, /* a size exceeds what the handle was created for */
  SAMPLER_EHIP = -3,      /* a HIP runtime call failed (no device, launch error) */
  SAMPLER_ENOTSUP = -4    /* a valid request this build does not support */
} sampler_status;

/* [A] "One request with top_p takes the whole batch off the fast path":
 * the four outcomes of the batch predicate. */
typedef enum sampler_path {
  SAMPLER_PATH_GREEDY = 0,       /* every row greedy (top_k <= 1 after normalisation) */
  SAMPLER_PATH_GUMBEL = 1,       /* no row truncates: Gumbel-max over the whole vocabulary */
  SAMPLER_PATH_FILTERED = 2,     /* some row uses top_k, top_p or min_p */
  SAMPLER_PATH_DETERMINISTIC = 3 /* as GUMBEL, on a handle created with SAMPLER_DETERMINISTIC */
} sampler_path;

typedef enum sampler_dtype {
  SAMPLER_DTYPE_F32 = 0,
  SAMPLER_DTYPE_BF16 = 1
} sampler_dtype;

/* sampler_config.flags */
/* [B] "What the flag switches": deterministic inference.  Rows without a
 * row_seed use seed 42 and (without row_stream) stream 0, so a row's draw
 * depends only on its own parameters; each row's reduction order depends
 * only on V, so a row gives bit-identical results at any batch position and
 * batch size. */
#define SAMPLER_DETERMINISTIC (1u << 0)
/* Run the general (filtered) kernel whatever the predicate says.  The
 * outputs are identical by construction; this is the A/B switch for the
 * specialised kernels. */
#define SAMPLER_FORCE_FILTERED (1u << 1)
/* Launch through hipLaunchCooperativeKernel, so the runtime itself checks
 * that every workgroup of a step is resident at once (the workgroups of a
 * row wait on one another).  Without the flag the step is a plain launch
 * whose grid never exceeds what the device holds at once, which makes all
 * workgroups resident whenever no other kernel occupies the compute units
 * at the same time (cooperative launches cost ~12 us more per step on
 * MI355X).  Either way every wait is bounded: a wait that expires marks the
 * step's rows with row_status 3. */
#define SAMPLER_COOPERATIVE_LAUNCH (1u << 2)
/* Select tokens by the seeded inverse CDF instead of Gumbel-max (the
 * "seeded multinomial" of [A] "One request with top_p takes the whole batch
 * off the fast path", used by the deterministic path of [B] "What the flag
 * switches"): row r draws one uniform u in [0, 1) (53 bits of the Philox
 * block at counter (0xFFFFFFFF, stream_r, offset_r lo, offset_r hi) under
 * key seed_r, words 0 and 1) and takes the first kept token, in index
 * order, whose running kept mass exceeds u times the kept total.  Rows with
 * top_k == 1 still take the first argmax; probs and logprobs are
 * unchanged.  With SAMPLER_DETERMINISTIC the result of a row does not
 * depend on its batch. */
#define SAMPLER_INVERSE_CDF (1u << 3)
/* A/B switches of the selection path (the role of the page's
 * SGLANG_OPT_USE_GUMBEL_SAMPLE switch, [A] "Nine lines, and exactly one call
 * site"), at most one SAMPLER_FORCE_* flag per handle; path_out still
 * reports the predicate's choice:
 *   SAMPLER_FORCE_PATH_GREEDY: every row takes the first argmax, the greedy
 *     path's selection, whatever its parameters; probs, logprobs and top
 *     logprobs still follow each row's own parameters.
 *   SAMPLER_FORCE_PATH_GUMBEL: the step runs under the Gumbel label; the
 *     kernel selects per row (argmax for top_k == 1, Gumbel-max over the
 *     kept set otherwise), so the outputs equal the unforced step's. */
#define SAMPLER_FORCE_PATH_GREEDY (1u << 4)
#define SAMPLER_FORCE_PATH_GUMBEL (1u << 5)
/* Kernel choice for steps that want only token ids and top logprobs of the
 * sampled distribution (no probs, logprobs or logits processors, no
 * SAMPLER_DETERMINISTIC or SAMPLER_INVERSE_CDF, vocab <= 524,288,
 * histories of at most 4096 ids).  Such a step runs
 * on a streaming kernel -- one workgroup per row, the row read from memory
 * in passes instead of held in LDS, every row of the batch in flight at
 * once -- when its rows outnumber the row kernel's row groups, which then
 * would walk several rows each ([C] "best_of 与 n 的放大": forks multiply a
 * step's rows).  A row that kernel cannot settle exactly is sampled by the
 * row kernel in a second launch on the same stream.  The outputs follow the
 * same definitions either way (the fp64 sums may round differently).
 *   SAMPLER_FORCE_STREAM: use the streaming kernel for every such step.
 *   SAMPLER_NO_STREAM: never use it.
 * At most one of the two per handle.  A handle whose largest vocabulary and
 * history need more LDS than a workgroup has (max_vocab near 2^19 with
 * histories over 2,048 ids) never streams, forced or not. */
#define SAMPLER_FORCE_STREAM (1u << 6)
#define SAMPLER_NO_STREAM (1u << 7)

typedef struct sampler_config {
  int32_t max_rows;            /* largest n_rows a step may pass (>= 1) */
  int32_t max_vocab;           /* largest vocab (>= 1, <= 1,048,576) */
  int32_t max_history_per_row; /* largest history_len of one row (0..131,071).  Up to
                                  4096 the row kernel counts a history itself; a
                                  handle planned for more holds a count list of
                                  4 * max_rows * min(64 * max_history_per_row,
                                  max_vocab + 32768) bytes, which a short kernel
                                  fills ahead of the row kernel in steps where a
                                  row's history is longer than 4096 */
  int32_t max_top_logprobs;    /* largest top_logprobs (0..32) */
  int32_t device;              /* HIP device ordinal */
  uint32_t flags;              /* SAMPLER_DETERMINISTIC | SAMPLER_COOPERATIVE_LAUNCH | SAMPLER_INVERSE_CDF |
                                  one of SAMPLER_FORCE_FILTERED, SAMPLER_FORCE_PATH_GREEDY,
                                  SAMPLER_FORCE_PATH_GUMBEL | one of SAMPLER_FORCE_STREAM,
                                  SAMPLER_NO_STREAM */
  int32_t max_bias_per_row;    /* largest bias_len + active stop_len of one row (0..512) */
  /* Bound of every wait of one workgroup for another, in polls of the group
   * word: 0 (the default) is ~2 s.  A wait that expires marks the step
   * aborted: its rows get row_status 3 (outputs not valid) and every later
   * wait of that step returns at once; later steps are unaffected.  Values
   * of 1 force that path (tests of the failure handling). */
  int32_t wait_spin_limit;
} sampler_config;

typedef struct sampler_handle sampler_handle;

typedef struct sampler_step_args {
  /* Logits: device, [n_rows, row_stride] elements of `dtype`, row-major.
   * Never written.  row_stride >= vocab. */
  const void *logits;
  int32_t dtype;               /* sampler_dtype */
  int32_t n_rows;              /* 1 .. max_rows; 0 is an error ([A]: an empty batch has no path) */
  int32_t vocab;               /* 1 .. max_vocab */
  int64_t row_stride;          /* in elements */

  /* Per-row sampling parameters: host arrays of n_rows entries.  NULL means
   * the default for every row, as in [C] "哪些参数会额外打开一趟全词表计算":
   * temperature 1, top_p 1, top_k -1, min_p 0, repetition 1, presence 0,
   * frequency 0.
   *   temperature >= 0 (0 <= T < 1e-6 is a greedy row: T := 1, top_k := 1,
   *                     [A] normalisation);
   *   top_p in (0, 1];  top_k = -1 (whole vocabulary) or >= 1;
   *   min_p in [0, 1];  repetition_penalty > 0;  presence/frequency finite. */
  const float *temperature;
  const float *top_p;
  const float *min_p;
  const float *repetition_penalty;
  const float *presence_penalty;
  const float *frequency_penalty;
  const int32_t *top_k;

  /* Token history for the penalties ([C] "解码一步里采样做什么",
   * _apply_penalties): history_ids is device memory; row r's history is
   * history_ids[history_start[r] .. history_start[r] + history_len[r]).
   * history_start / history_len are host arrays of n_rows entries.  Spans
   * may overlap or alias (forked rows share their parent's history).  Ids
   * outside [0, vocab) are ignored.  All three may be NULL when no row uses
   * a penalty.  history_len[r] <= max_history_per_row. */
  const int32_t *history_ids;
  const int64_t *history_start;
  const int32_t *history_len;

  /* Randomness (Philox4x32-10, Salmon et al. SC'11).  Vocabulary entry i of
   * row r draws word (i & 3) of the block at counter
   * (i >> 2, stream_r, offset_r lo, offset_r hi) under key (seed_r lo, seed_r hi);
   * E = -ln(1 - (x + 1/2) 2^-32), clamped below at FLT_MIN ([A] "Nine lines,
   * and exactly one call site").  Defaults: seed_r = seed, offset_r = offset,
   * stream_r = r; on a deterministic handle seed_r = 42 and stream_r = 0.
   * The library keeps no random state: replaying the same arguments
   * replays the same tokens. */
  uint64_t seed;
  uint64_t offset;
  const uint64_t *row_seed;    /* host, n_rows entries, or NULL */
  const uint64_t *row_offset;  /* host, n_rows entries, or NULL */
  const uint32_t *row_stream;  /* host, n_rows entries, or NULL */

  /* Outputs (device).  token_ids is required: int32 [n_rows]; -1 for a row
   * with row_status != 0.  probs / logprobs: fp32 [n_rows, vocab] (stride
   * vocab) or NULL; they are the distribution sampled from ([B] "Logprobs
   * are temperature-scaled"): after temperature and truncation, 0 and -inf
   * outside the kept set; greedy rows report the untruncated distribution
   * at temperature 1.  top_logprobs (0 .. max_top_logprobs) largest kept
   * logprobs per row with their ids, ordered by (logit desc, id asc), padded
   * with (-inf, -1): fp32 / int32 [n_rows, top_logprobs].  row_status: int32
   * [n_rows] or NULL; 0 ok, 1 no finite logit (all -inf/NaN after
   * sanitising NaN to -inf), 2 a +inf value after temperature, 3 the
   * step's cross-workgroup wait timed out (an internal error; the row's
   * outputs are not valid), 4 the row's device-side parameters broke the
   * rules (sampler_step_graph only). */
  int32_t *token_ids;
  float *probs;
  float *logprobs;
  int32_t top_logprobs;
  float *top_logprob_vals;
  int32_t *top_logprob_ids;
  int32_t *row_status;

  /* Output (host, may be NULL): the path the predicate chose. */
  int32_t *path_out;

  /* Logits processors, applied to the logits before the penalties, in this
   * order (each may be absent: NULL pointers):
   *   1. grammar bitmask ([B] "Constrained decoding", step 4 "Mask": the
   *      grammar fills a vocabulary bitmask that is applied to the logits
   *      before sampling).  vocab_mask is device memory, uint32
   *      [n_rows, mask_stride] (mask_stride >= ceil(vocab / 32) words); bit
   *      (i & 31) of word (i >> 5) set = token i allowed, cleared = its
   *      logit becomes -inf.
   *   2. logit_bias (a sampler option in [B] "On Apple silicon"): row r's
   *      entries are bias_ids / bias_vals[bias_start[r] .. + bias_len[r])
   *      (ids and values in device memory, spans host arrays); entries of
   *      one token are summed (order unspecified beyond two), then added to
   *      its logit once; a NaN result becomes -inf.  Ids outside [0, vocab)
   *      are ignored.
   *   3. min_tokens ([C] "解码一步里采样做什么", _apply_min_tokens_penalty):
   *      while output_len[r] < min_tokens[r] (host arrays), every id of row
   *      r's stop list stop_ids[stop_start[r] .. + stop_len[r]) (ids in
   *      device memory, spans host arrays) gets logit -inf.
   * bias_len[r] plus stop_len[r] (counted only while the row's min_tokens
   * is active) must not exceed max_bias_per_row. */
  const uint32_t *vocab_mask;
  int64_t mask_stride;
  const int32_t *bias_ids;
  const float *bias_vals;
  const int64_t *bias_start;
  const int32_t *bias_len;
  const int32_t *stop_ids;
  const int64_t *stop_start;
  const int32_t *stop_len;
  const int32_t *min_tokens;
  const int32_t *output_len;

  /* Which logprobs (and top logprobs) are returned ([B] "Logprobs are
   * temperature-scaled"):
   *   SAMPLER_LOGPROB_PROCESSED (0, default): the distribution sampled
   *     from, after truncation (0 / -inf outside the kept set);
   *   SAMPLER_LOGPROB_TEMPERATURE (1): log_softmax(logits / temperature)
   *     of the processed logits, untruncated: every token gets a value and
   *     top logprobs list the largest over all tokens;
   *   SAMPLER_LOGPROB_RAW (2): log_softmax of the processed logits without
   *     temperature (the page's original-logprob switch); top logprobs list
   *     the largest over all tokens, ordered as in mode 1.  Where a row's
   *     effective temperature is 1 (greedy rows, T = 1) it equals mode 1;
   *     the other rows take a second kernel after the sampling kernel,
   *     which reads their logits again and rewrites their logprobs.
   * probs and the sampled tokens do not depend on the mode. */
  int32_t logprob_mode;

  /* Output (host, may be NULL): the kernel the step ran on: 0 the row
   * kernel, 1 the streaming kernel, followed on the same stream by the row
   * kernel for the rows it left (SAMPLER_FORCE_STREAM above), 2 the
   * small-row kernel: steps of at most 4096 values per row whose every row
   * keeps every value (Gumbel-max or greedy; no penalties, logits
   * processors or top_logprobs; not the raw logprob mode, not
   * SAMPLER_DETERMINISTIC, SAMPLER_INVERSE_CDF or SAMPLER_FORCE_FILTERED)
   * take one small workgroup per row, 3 the chunked-row kernel: steps of
   * up to 4,096 longer rows of that kind that want only token_ids and
   * row_status (no probs, logprobs or top_logprobs; not
   * SAMPLER_FORCE_STREAM either) take
   * one workgroup per chunk of 1024 to 4096 values, and the last chunk of a
   * row to finish merges the row.  sampler_step only: the graph and
   * no-allocation entry points always report 0. */
  int32_t *kernel_out;
} sampler_step_args;

#define SAMPLER_LOGPROB_PROCESSED 0
#define SAMPLER_LOGPROB_TEMPERATURE 1
#define SAMPLER_LOGPROB_RAW 2

/* Create a handle on cfg->device: checks the device, allocates the device
 * workspace (exchange areas, barrier words, parameter ring) and a pinned
 * host staging ring of depth 4.  Returns SAMPLER_EHIP when no usable HIP
 * device exists (and *out = NULL), SAMPLER_EINVAL for a bad config.
 * Ownership: the caller owns *out and must call sampler_destroy. */
sampler_status sampler_create(const sampler_config *cfg, sampler_handle **out);

/* Enqueue one decode step on `stream` (a hipStream_t; NULL is the default
 * stream).  Validates every host-side argument before any launch and returns
 * a negative status without launching if one is wrong.  Allocates nothing,
 * never synchronises the device and never reads device memory back; waits on
 * the host only when the 4-slot staging ring wraps onto a slot whose copy is
 * still in flight (batches of up to 72 rows pass their per-row records in
 * the kernel arguments and use no staging slot).  The step is the row
 * kernel, preceded by a history-count kernel when a row's history is longer
 * than 4096 ids and followed by the raw-logprob kernel in the raw mode when a
 * row's effective temperature is not 1.  Outputs are valid when the stream
 * reaches this point. */
sampler_status sampler_step(sampler_handle *h, const sampler_step_args *args, void *stream);

/* Per-row parameters in device memory, for sampler_step_graph.  Each array
 * has n_rows entries in device memory of the handle's GPU, or is NULL (the
 * default for every row, as in sampler_step_args).  Their meaning is that of
 * the host arrays of the same names in sampler_step_args. */
typedef struct sampler_device_params {
  const float *temperature;
  const float *top_p;
  const float *min_p;
  const float *repetition_penalty;
  const float *presence_penalty;
  const float *frequency_penalty;
  const int32_t *top_k;
  const int64_t *history_start;
  const int32_t *history_len;
  const uint64_t *row_seed;
  const uint64_t *row_offset;
  const uint32_t *row_stream;
  const int64_t *bias_start;
  const int32_t *bias_len;
  const int64_t *stop_start;
  const int32_t *stop_len;
  const int32_t *min_tokens;
  const int32_t *output_len;
} sampler_device_params;

/* One decode step whose per-row parameters live in device memory, so that a
 * caller can capture the call into a HIP graph once per (n_rows, vocab)
 * bucket and replay it after updating those arrays (offsets, temperatures,
 * histories...) in place -- the launch-bound batch-1 decode loop ([A] "What
 * a free T4 can and cannot tell you": the sampler's host overhead is the
 * cost at batch 1).  The call enqueues two kernels and nothing else (one
 * normalises the rows' parameters into a record buffer of the handle, the
 * other samples; no copy, no memset, no event unless profiling is on); it
 * allocates nothing; the workspace addresses are fixed by the handle.
 *   args: as for sampler_step, except that its per-row host arrays
 *     (temperature .. top_k, history_start / history_len, row_seed /
 *     row_offset / row_stream, bias_start / bias_len, stop_start / stop_len,
 *     min_tokens / output_len) must be NULL: dp carries them.  args->seed
 *     and args->offset are the defaults of rows without row_seed /
 *     row_offset (and are frozen into a captured graph).  path_out, when
 *     given, receives SAMPLER_PATH_FILTERED: the kernel decides each row's
 *     treatment from its parameters on the device.
 *   dp: device pointers (the struct itself is read before the call
 *     returns).
 * Each row's parameters are normalised and checked on the device with the
 * rules of sampler_step; a row that breaks them gets row_status 4, token -1,
 * probs 0 and logprobs -inf, and the other rows are unaffected.  Results
 * equal those of sampler_step with the same values.  Replays of one
 * captured step must not overlap each other or other steps of the handle. */
sampler_status sampler_step_graph(sampler_handle *h, const sampler_step_args *args, const sampler_device_params *dp,
                                  void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: one decode
 * step without a handle.  Arguments, outputs and results are those of
 * sampler_step on a handle created with the same flags and the largest
 * limits the row kernel serves alone (max_history_per_row 4096,
 * max_bias_per_row 512,
 * max_top_logprobs 32); n_rows may be any positive number (batches above
 * 72 rows run as several launches on `stream`).  `flags` takes
 * SAMPLER_DETERMINISTIC, SAMPLER_INVERSE_CDF and at most one
 * SAMPLER_FORCE_* flag.  The raw logprob mode is offered where every row's
 * effective temperature is 1 (SAMPLER_ENOTSUP otherwise: the kernel that
 * serves the other rows carries a private segment, which the runtime may
 * back with memory at its first launch).
 *   Workspace: a fixed array of the library in device memory, about 8 MB
 *   (group words and exchange slots of 256 workgroups), one copy per GPU,
 *   held until the process ends.  The call allocates nothing: no hipMalloc,
 *   no hipFree, no allocating library routine; the first call on a device
 *   looks up that device's copy (hipGetSymbolAddress) and plans the row
 *   kernel for it.
 *   Every call on a GPU shares that GPU's array: calls that overlap on one
 *   GPU (other streams, other host threads) race and give wrong results.
 *   Calls in stream order on one GPU are safe, as are calls on different
 *   GPUs.
 *   Errors: SAMPLER_EINVAL / SAMPLER_ECAPACITY for arguments beyond those
 *   limits (vocab beyond what 32 workgroups hold at those limits, about
 *   950,000), SAMPLER_EHIP for device errors; the message of the calling
 *   thread's last failure is sampler_noalloc_last_error(). */
sampler_status sampler_step_noalloc(const sampler_step_args *args, uint32_t flags, int32_t device, void *stream);

/* Message of the calling thread's last failed sampler_step_noalloc ("" when
 * none). */
const char *sampler_noalloc_last_error(void);

/* The batch predicate alone ([A] "One request with top_p takes the whole
 * batch off the fast path": normalize, then is_all_greedy / need_top_p /
 * need_top_k / need_min_p).  Pure host code: works without a GPU.  `flags`
 * takes SAMPLER_DETERMINISTIC.  Reads only n_rows and the parameter arrays
 * of args.  SAMPLER_EINVAL for an empty batch or invalid parameters. */
sampler_status sampler_select_path(const sampler_step_args *args, uint32_t flags, int32_t *path_out);

/* Check a step's host-side arguments against a config without a device
 * (the same checks sampler_step performs before launching).  Writes a
 * message into msg (when non-NULL, msg_len > 0). */
sampler_status sampler_validate(const sampler_config *cfg, const sampler_step_args *args, char *msg,
                                int32_t msg_len);

/* Change the handle's wait bound (sampler_config.wait_spin_limit; 0 is the
 * default ~2 s) for the steps enqueued from now on.  A captured graph keeps
 * the bound it was captured with.  SAMPLER_EINVAL for limit < 0. */
sampler_status sampler_set_wait_spin_limit(sampler_handle *h, int32_t limit);

/* Profiling: from now on each step records a HIP event pair that brackets
 * its sampling kernel's execution on the step's stream (hipExtLaunchKernel's
 * start and stop events; around the launch for cooperative launches), for
 * up to `capacity` steps.  This call creates the events (it may allocate); the
 * steps themselves allocate nothing.  SAMPLER_EINVAL for capacity < 1. */
sampler_status sampler_profile_start(sampler_handle *h, int32_t capacity);

/* Stop recording, wait for the recorded kernels, and write the kernel
 * durations in milliseconds (one per recorded step, in launch order) to
 * ms[0 .. min(n_recorded, cap)); *n receives the number written.  Releases
 * the events. */
sampler_status sampler_profile_stop(sampler_handle *h, float *ms, int32_t cap, int32_t *n);

/* Free the handle's device workspace and pinned ring after waiting for its
 * in-flight staging copies.  NULL is a no-op. */
void sampler_destroy(sampler_handle *h);

/* Message of the last failed call on h ("" when none); with h == NULL, the
 * message of the last sampler_create failure on this thread.  The string
 * stays valid until the next call on the handle. */
const char *sampler_last_error(const sampler_handle *h);

/* Phase timeline of the row kernel, for performance work.  A library built
 * with -DDSTS_PHASE_STAMPS (build option `stamps`) records the device's
 * real-time clock at the phase boundaries of the first row each workgroup
 * walks, in a device array of *blocks_out x *slots_out words (workgroup
 * b's stamps at [b * slots ..], one slot per phase, 0 where a phase did not
 * run; the phases are those of the row kernel's description).  This call
 * copies the first `cap` words of the current device's array to host_out,
 * synchronously, then clears the array; *clock_khz_out receives the
 * clock's rate.  Other builds return SAMPLER_ENOTSUP (after setting
 * *blocks_out and *slots_out). */
sampler_status sampler_phase_stamps(uint64_t *host_out, int32_t cap, int32_t *blocks_out, int32_t *slots_out,
                                    int32_t *clock_khz_out);

#ifdef __cplusplus
}
#endif

#endif /* DSTS_SAMPLER_H */
