// sampler_internal.h -- records shared by the host runtime and the HIP
// kernels of the decode-step sampler (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsts {

// [A] "One request with top_p takes the whole batch off the fast path":
// top_k = -1 (whole vocabulary) is carried as 1 << 30.
constexpr int32_t kTopKAll = 1 << 30;
// Largest number of workgroups that cooperate on one row.
constexpr int kMaxG = 32;
// The same for a launch whose rows exchange only in the final merge (no
// merged max, thresholds or sums): that merge reads one record per lane of
// one wave, and no per-workgroup LDS array is involved.
constexpr int kMaxLightG = 64;
// Largest top-logprob list per row.
constexpr int kMaxTopLogprobs = 32;
// Largest history the row kernel counts by itself.  Its counts live in an
// LDS hash table of next_pow2(2 * max_history_per_row) slots (at most
// kMaxHashSlots), each packing a slice-local index (15 bits) and a count
// (13 bits) into one word.
constexpr int kMaxHistPerRow = 4096;
constexpr int kMaxHashSlots = 8192;
// Largest history of one row.  A longer history than kMaxHistPerRow is
// counted ahead of the row kernel by hist_list_kernel: one workgroup per
// (row, slice) counts the slice's ids in a dense LDS array and writes the
// nonzero ones in index order as slice-local index << 17 | count.
constexpr int32_t kMaxHistLong = (1 << 17) - 1;
// Largest list of logit_bias plus active stop entries of one row: one per
// thread.  They live in a second LDS hash of next_pow2(2 * max) 8-byte
// slots (slice-local index, summed bias).
constexpr int kMaxBiasPerRow = 512;
// Largest vocabulary (masses are summed as 2^-44 fixed point in 64 bits).
constexpr int32_t kMaxVocab = 1 << 20;
// The streaming kernel packs a token and a count into one hash word (19 + 13
// bits), so it takes vocabularies up to 2^19; its bitmap of the tokens that
// have history holds one bit per token, in whole 16-byte units.
constexpr int32_t kStreamMaxVocab = 1 << 19;
__host__ __device__ inline int stream_bitmap_words(int vocab) { return (((vocab + 31) / 32) + 3) & ~3; }

// Workgroup shape of the row kernel: 512 threads (8 wave64s; LDS allows one
// workgroup per CU, so each thread may use 256 VGPRs).  Each
// workgroup keeps its slice of the processed logits in LDS; the slice is at
// most 32768 values (the hash packs 15-bit slice-local indices) and is also
// bounded by the LDS left after the fixed part and the shared region.
constexpr int kBlock = 512;
constexpr int kMaxSlice = 32768;

// Threshold window: values are binned on an absolute grid, bin(z) =
// floor(z min(1, T) 32), counted down from the bin of the row max (so the
// window spans 16 nats of z / max(1, 1/T)); kWinBins bins hold counts and
// masses exp(z - max) in 2^-31 units, the deeper values only a mass total.
// kWinBins equals kBlock: the merge gives each thread one bin.
constexpr int kWinBins = 512;
constexpr float kBinsPerNat = 32.0f;
// Candidates (values in the bins that hold a threshold or the top logprobs)
// gathered per row for exact selection; more sends the row to the general
// radix-select path.
constexpr int kCandCap = 1024;

// Per-row flags, decided on the host from the row's parameters.
enum : uint32_t {
  RF_GREEDY = 1u << 0,  // greedy row: keep every token at T = 1; token = first argmax
  RF_TOP1 = 1u << 1,    // top_k == 1 after normalisation: token = first argmax
  RF_PEN = 1u << 2,     // a penalty differs from its default and the row has history
  RF_TOPK = 1u << 3,    // 1 <= top_k < vocab (set for non-greedy top_k == 1 rows too)
  RF_TOPP = 1u << 4,    // top_p < 1
  RF_MINP = 1u << 5,    // min_p > 0
  RF_SPEC = 1u << 6,    // the row has logit_bias entries or active stop ids
  RF_BAD = 1u << 7,     // device-side parameters broke the rules (status 4); no other flag
};

// One row's parameters as the kernel reads them (96 bytes).
struct alignas(16) RowParam {
  float temperature;  // effective temperature (1 for greedy rows)
  float top_p;
  float min_p;
  float rep;
  float pres;
  float freq;
  int32_t top_k;      // meaningful with RF_TOPK
  uint32_t flags;
  uint64_t seed;
  uint64_t offset;
  int64_t hist_start;
  int32_t hist_len;
  uint32_t stream;
  int64_t bias_start;  // logit_bias span (RF_SPEC)
  int64_t stop_start;  // stop-id span, counted only while min_tokens is active
  int32_t bias_len;
  int32_t stop_len;    // 0 when min_tokens is not active
  int32_t row;         // the batch row this record describes (records may be reordered)
  uint32_t pad;
};
static_assert(sizeof(RowParam) == 96, "RowParam layout");

// Group words of one row group, each on its own 128-byte line: the barrier
// word (epoch << 32 | generation << 8 | arrival count) and the
// final-exchange word (epoch << 32 | arrival count); the epoch is that of
// the launch that last used the word.
struct alignas(128) GroupSync {
  unsigned long long word;
  unsigned long long pad0[15];
  unsigned long long fin;
  unsigned long long pad1[15];
};


// Exchange slots owned by one workgroup (indexed by its block id); every
// array starts on a 16-byte boundary, since readers fetch 16-byte pieces.
struct alignas(128) WgSlots {
  // Arrays read by every workgroup of the row after a group barrier are
  // double buffered by the group's exchange count, so a workgroup rewrites
  // one only after all readers have passed the next barrier.
  // exchange 2: the order key of this slice's max, the slice's bin anchor
  // (float bits), and relative to the slice's max the mass of the values
  // deeper than the window and the exact sum (fp64 bits)
  unsigned long long x1[2][4];
  // final exchange, by row parity: best Gumbel score (fp64 bits), its
  // index, this slice's max order key
  unsigned long long fin[2][4];
  uint32_t cand_n[2][4];                          // candidates gathered by this workgroup (word 0)
  uint32_t pad0[24];
  unsigned long long whist[2][kWinBins];          // window bins: count << 48 | mass (2^-31 units)
  unsigned long long cand[2][kCandCap];           // candidate keys: order key << 32 | ~index
  uint32_t hcnt[2][256];                          // general path: radix counts
  unsigned long long hmass[2][256];               // general path: radix masses
  unsigned long long toplist[2][kMaxTopLogprobs]; // general path: local top-logprob candidates
  double ssum[2];                                 // general path: kept-set sum
};
static_assert(offsetof(WgSlots, x1) % 16 == 0 && offsetof(WgSlots, fin) % 16 == 0 && offsetof(WgSlots, whist) % 16 == 0 &&
                  offsetof(WgSlots, cand) % 16 == 0,
              "WgSlots layout");

enum : int { PATH_GREEDY = 0, PATH_GUMBEL = 1, PATH_FILTERED = 2, PATH_DETERMINISTIC = 3 };

// Phase stamps (builds with DSTS_PHASE_STAMPS): slot k of a workgroup's
// record holds the real-time clock at the end of phase k of its first row
// (0 where the row skipped the phase).
constexpr int kStampBlocks = 2048;
constexpr int kStampSlots = 32;
enum : int {
  kStampStart = 0,       // the kernel starts
  kStampRow = 1,         // the row's record is read
  kStampLoaded = 2,      // the slice is in LDS (loads, temperature, penalties, processors)
  kStampMax = 3,         // the slice's max and first argmax
  kStampHist = 4,        // the window histogram and the exchange-2 record are stored
  kStampX2 = 5,          // the exchange-2 barrier is passed
  kStampDecided = 6,     // exchange 2 is merged: row max, threshold bins
  kStampGathered = 7,    // the candidates are gathered and stored
  kStampX3 = 8,          // the exchange-3 barrier is passed
  kStampThresholds = 9,  // thresholds and the kept-set sum are exact
  kStampSelect = 10,     // selection and output stores start (after the general path)
  kStampToken = 11,      // the last workgroup to arrive has written the token
  kStampEnd = 12,        // the row's outputs are issued
  kStampGumbel = 13,     // this workgroup's Gumbel-max winner is known (thread 0's wave)
  kStampReleased = 14,   // final exchange: this workgroup's record is stored
  kStampArrived = 15,    // final exchange: this workgroup has arrived
  kStampGumbelBound = 16,   // Gumbel-max: the argmax's draw and the listing cut are known
  kStampGumbelListed = 17,  // Gumbel-max: the candidate groups are listed
  kStampGumbelListedCount = 18,  // not a time: groups thread 0's wave listed
  kStampRowIndex = 19,   // not a time: 1 + the index of the row the stamps describe
  kStampGumbelBatched = 20,  // Gumbel-max: thread 0's wave has scored its listed groups
  kStampGumbelRounds = 21,   // not a time: fp64 scoring rounds of thread 0's wave
  kStampTable = 22,          // the kernel's fp64 exp table is built (before the first row)
  kStampX3Read = 23,         // exchange 3: wave 0 has read and placed the candidates
  kStampX3Ranked = 24,       // exchange 3: the candidates are sorted
  kStampX3Decided = 25,      // exchange 3: wave 0 has decided (short lists)
  kStampHalf = 26,           // load phase: the first half of the slice is transformed (vector loads)
  kStampHashed = 27,         // load phase: the history and bias hashes are built
  kStampTransformed = 28,    // load phase: the whole slice is transformed
  kStampStreamStart = 29,    // the streaming kernel starts (its other stamps reuse the row kernel's
                             // slots: row read 1, history hashed 27, pass A 3, pass B 4, ranges 6,
                             // pass C 7, list sorted 24, decisions 9, end 12, row index 19)
};

// Per-row parameters in device memory (one entry per row, or null for the
// default), normalised by the kernel itself.
struct DevRowArrays {
  const float *temperature, *top_p, *min_p, *rep, *pres, *freq;
  const int32_t *top_k;
  const int64_t *hist_start;
  const int32_t *hist_len;
  const uint64_t *seed, *offset;
  const uint32_t *stream;
  const int64_t *bias_start;
  const int32_t *bias_len;
  const int64_t *stop_start;
  const int32_t *stop_len;
  const int32_t *min_tokens, *output_len;
};

struct ChunkRec;
struct KernelParams {
  const void *logits;
  int64_t row_stride;
  int32_t n_rows;
  int32_t vocab;
  const RowParam *rows;  // device records, or null: KernelArgs::rows
  const int32_t *history_ids;
  int32_t *token_ids;
  float *probs;
  float *logprobs;
  float *top_lp_vals;
  int32_t *top_lp_ids;
  int32_t *row_status;
  int32_t top_lp;
  int32_t G;          // workgroups per row
  int32_t n_groups;   // row groups (rows are strided over groups)
  int32_t slice;      // elements per workgroup slice (multiple of 4)
  int32_t hash_slots; // LDS hash slots (power of two) when penalties are on
  int32_t vec_ok;     // bit 0: logits rows aligned for vector loads of four values; bit 1: outputs for
                      // vector stores; bit 2: logits rows aligned for 16-byte loads
  int32_t path;
  GroupSync *sync;    // [n_groups]
  WgSlots *slots;     // [n_groups * G]
  uint32_t *abort_word;  // equals the epoch once a barrier wait of this launch expired
  uint32_t epoch;        // the launch's epoch (host launches: 1 .. 2^31 - 1)
  uint32_t *epoch_dev;   // or null; else the launch's epoch is *epoch_dev + epoch_dev_add (rows_kernel
                         // advances the word by 2 per step: the row kernel adds 0, the raw-logprob kernel 1)
  uint32_t epoch_dev_add;
  uint32_t spin_limit;   // bound of every cross-workgroup wait in spins (0: the default, ~2 s)
  // logits processors
  const uint32_t *vocab_mask;  // [n_rows, mask_stride] allowed bits, or null
  int64_t mask_stride;         // words
  const int32_t *bias_ids;
  const float *bias_vals;
  const int32_t *stop_ids;
  int32_t bias_slots;          // LDS bias-hash slots (power of two), 0 without bias
  int32_t lp_mode;             // 0: logprobs of the sampled distribution; 1: untruncated at the row's temperature
  int32_t icdf;                // select by the seeded inverse CDF instead of Gumbel-max
  // rows from device arrays (rows_kernel): the defaults and the limits they
  // are checked against
  int32_t det;                 // deterministic handle: default seed 42, stream 0
  int32_t max_hist, max_bias;
  uint64_t seed, offset;
  DevRowArrays dev;
  // counts of the histories longer than kMaxHistPerRow (hist_list_kernel):
  // the (row, slice) list starts at hist_list + (row G + gid) hist_list_cap
  // and holds hist_list_n[row G + gid] entries; null when no row is that long
  uint32_t *hist_list;
  int32_t *hist_list_n;
  int64_t hist_list_cap;
  // rows the streaming kernel leaves to the row kernel: their records and
  // a word epoch << 32 | count (arrivals of the streaming kernel's epoch)
  RowParam *defer_rows;
  unsigned long long *defer_word;
  // the row kernel launched after it reads its row count from that word
  // (count of epoch n_rows_epoch, else 0) instead of n_rows
  const unsigned long long *n_rows_word;
  uint32_t n_rows_epoch;
  // chunked rows (chunk_kernel): chunk_n chunks of 4 kChunkBlock chunk_u
  // values per row; record r's chunk c result at chunk_recs[r chunk_stride +
  // c], its arrival word at chunk_words[kChunkWordStride r]
  ChunkRec *chunk_recs;
  unsigned long long *chunk_words;
  int32_t chunk_n, chunk_u, chunk_stride;
};

// Batches of up to kArgRows rows carry their per-row records in the kernel
// arguments (no copy ahead of the launch); larger ones are copied to a
// device ring first and KernelParams::rows points there.
constexpr int kArgRows = 72;
struct KernelArgs {
  KernelParams kp;
  RowParam rows[kArgRows];  // used when kp.rows is null
};
// measured on MI355X: kernel argument blocks up to 8 KB launch correctly
static_assert(sizeof(KernelArgs) <= 8192, "kernel argument block");

// Normalise the per-row device arrays of kp.dev into records at `out`
// (one thread per row).
hipError_t launch_rows(const KernelParams &kp, RowParam *out, hipStream_t stream);
// The raw logprobs of the rows whose effective temperature is not 1, after
// the row kernel of the same step (same arguments, its own epoch).
hipError_t launch_raw_lp(const KernelArgs &ka, int dtype, hipStream_t stream);
// Count the histories longer than kMaxHistPerRow into kp.hist_list (one
// workgroup per record and slice), ahead of the row kernel of the same step.
hipError_t launch_hist_list(const KernelArgs &ka, hipStream_t stream);
// Builds with DSTS_PHASE_STAMPS: copy the first n stamp words of the
// current device to host (synchronously), then clear them; other builds
// return hipErrorNotSupported.
hipError_t phase_stamps_take(unsigned long long *host, size_t n);
// Dynamic LDS bytes of hist_list_kernel for a slice.
size_t hist_list_lds_bytes(int slice);
// Launch one step.  The grid never exceeds the workgroups the device holds at
// once; `cooperative` launches through hipLaunchCooperativeKernel, which
// also has the runtime check that they are all resident.
// ev0 / ev1 (or null): an event pair that brackets the kernel's execution.
hipError_t launch_step(const KernelArgs &ka, int dtype, bool penalties, bool cooperative, hipStream_t stream,
                       hipEvent_t ev0, hipEvent_t ev1);
// The streaming kernel (batches of many rows that want only tokens and top
// logprobs): one workgroup per row, `grid` workgroups walking the rows; rows
// it cannot settle go to kp.defer_rows for a row-kernel launch after it.
hipError_t launch_stream(const KernelArgs &ka, int dtype, bool penalties, int grid, hipStream_t stream, hipEvent_t ev0,
                         hipEvent_t ev1);
// Its dynamic LDS bytes for a vocabulary, and the workgroups of it that fit on
// the device at once (0 when those bytes exceed a workgroup's LDS: such a
// handle never streams).
size_t stream_lds_bytes(int hash_slots, bool penalties, int vocab);
hipError_t stream_resident(int device, size_t lds_bytes, int *out);
// Rows of at most kSmallV values that keep every value (no truncation,
// penalties, processors or top-logprob list): one small workgroup per row.
constexpr int kSmallV = 4096;
hipError_t launch_small(const KernelArgs &ka, int dtype, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
// Longer rows of that kind in a step that wants only token ids: one
// workgroup of kChunkBlock threads per chunk of 4 kChunkBlock U values
// (U = 1, 2 or 4), at most kChunkMax chunks per row; the last chunk of a row
// to arrive merges the chunks' results.
constexpr int kChunkBlock = 256;
constexpr int kChunkMaxU = 4;
constexpr int kChunkMax = 256;
constexpr int kChunkMaxV = 4 * kChunkBlock * kChunkMaxU * kChunkMax;
constexpr int kChunkWordStride = 16;  // arrival words 128 bytes apart
constexpr int kChunkMaxRows = 4096;   // rows of a chunked step (the grid's y extent; workspace)
// One chunk's result.  Gumbel-max rows: b = the winner's fp32 score bits
// << 32 | flags << 28 | the winner's index (flags bits 0-1: status, 1 no
// finite value in the chunk, 2 a +inf value; bit 2: exact), a = the
// winner's z bits << 32 | its Philox word, or with the exact flag its fp64
// score (several values were near the chunk's best fp32 score).  Greedy
// rows: a = the order key of its max (order key << 32 | ~first index).
struct alignas(16) ChunkRec {
  unsigned long long a;
  unsigned long long b;
};
hipError_t launch_chunk(const KernelArgs &ka, int dtype, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
// Workgroups of the row kernel that fit on the device at once for a given
// dynamic LDS size.
hipError_t resident_blocks(int device, size_t lds_bytes, int *out);
// Static LDS bytes of the row kernel (the compiler's own, besides the
// dynamic request).
hipError_t kernel_lds_static(size_t *out);
// Fixed LDS bytes of one workgroup.
size_t kernel_lds_fixed();
// LDS bytes of the shared region (history hash and bias hash; merged prefix
// arrays with the local histogram, candidate staging or sorting after them;
// general-path histograms: used one at a time).
size_t kernel_lds_region(int slice, int hash_slots, int bias_slots, bool penalties);
// Dynamic LDS bytes of one workgroup for a slice and hash sizes.
size_t kernel_lds_bytes(int slice, int hash_slots, int bias_slots, bool penalties);

}  // namespace dsts
