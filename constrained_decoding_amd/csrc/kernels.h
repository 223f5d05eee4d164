// kernels.h -- launch interface between the host ABI code (sampler_abi.cpp)
// and the HIP kernels (kernels.hip) of libcd_sampler.so.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.h"

namespace cds {

struct SampleArgs {
  const RowParams* rows;
  const RowSlots* slots;       // per row: where its lists, records and histograms live
  const int32_t* task_row;     // task k: row index | kPass2 (pass-2 task), -1: none
  int32_t n_groups;            // task groups of kXcds tasks (grid: n_groups * kXcds * P)
  const void* logits;
  int64_t ld;
  int32_t B, V;
  const int32_t* mask;  // bitmask words or nullptr
  int64_t mask_ld;
  const uint8_t* row_has_mask;
  int32_t* out_ids;
  float* out_lp;
  int32_t* out_st;
  float* out_cut;       // per sampled row the smallest kept value, or nullptr
  RowSync* sync;
  Plan* plans;
  SliceHead* heads;
  unsigned long long* hist;  // slice histograms [NBINS]: count << kCountShift | mass
  SliceBest* bests; // list records (RowSlots::rec)
  uint64_t* ulist;  // list entries (RowSlots::list64, cap): okey(z) << 32 | ~t
  int32_t P;
  int64_t S;
  uint64_t spin_limit;  // wall-clock ticks a race task waits for its row's plan
  uint32_t gen;         // call generation (nonzero, differs from the previous call's)
  unsigned long long* trace;  // 8 words per workgroup of phase timestamps, or nullptr
};

// Per row and slice of the further outputs' slice pass: the slice's max
// (lowest id), finite count, flags (1: a NaN or +inf; 2: candidate list
// overflow), exp-sum against its max in the requested basis, and how many
// top-N keys it kept.
struct alignas(16) OutSliceStat {
  float zm;
  int32_t am;
  int32_t nf;
  uint32_t flags;
  double se;
  int32_t nc;
  int32_t pad;
};
static_assert(sizeof(OutSliceStat) == 32, "OutSliceStat layout");
// tokens per slice of the further outputs' slice pass (whole mask words)
constexpr int kOutSlice = 16384;

// Record of one slice of a support row (support sets from the sampling
// call's thresholds, by slices): the slice's largest finite z and the lowest
// id holding it, its finite and kept (z >= threshold) token counts, the kept
// tokens' sum of exp((z - zm) / T), and whether a NaN or +inf was seen.
struct alignas(16) SupSliceStat {
  float zm;
  int32_t am;
  int32_t nf;
  int32_t cnt;
  double st;
  uint32_t nonfin;
  uint32_t pad;
};
static_assert(sizeof(SupSliceStat) == 32, "SupSliceStat layout");
// tokens per support slice (whole mask words)
constexpr int kSupSlice = 4096;

// Further per-row outputs (logprob-outputs kernel, outputs.hip).  Row blocks:
// one workgroup per row for the chosen token's logprob, the top-N logprobs
// and the logprobs of named tokens; support blocks: one workgroup per entry
// of sup_rows for that row's support set.
struct OutputArgs {
  int32_t basis;          // 0: the row's sampling distribution, 1: before the temperature
  int32_t top_n_max;      // columns of top_ids / top_vals (0: none)
  const int32_t* top_n;   // [B] per-row N (clamped to [0, top_n_max]) or nullptr
  const int64_t* tok_off; // [B+1] CSR offsets of named tokens or nullptr
  const int32_t* tok_ids;
  const int32_t* sel_ids; // [B] the drawn tokens, or nullptr (scoring: no draw)
  const float* cuts;      // [B] the sampling call's kept-set thresholds, or nullptr
  const int32_t* sup_rows;
  int32_t n_sup;
  int32_t sup_cap;
  int32_t n_row_blocks;   // B, or 0 when no per-row output is asked for
  float* next_lp;         // [B] or nullptr
  int32_t* top_ids;       // [B, top_n_max]
  float* top_vals;
  float* tok_vals;        // [tok_off[B]]
  int32_t* sup_ids;       // [n_sup, sup_cap]
  float* sup_lp;          // [n_sup, sup_cap] or nullptr
  int32_t* sup_len;       // [n_sup]
  float* sup_sel;         // [n_sup] or nullptr
  int32_t* sup_st;        // [n_sup]
  // slice records (workspace) for the row blocks, or nullptr: the row blocks
  // then stream their rows themselves
  OutSliceStat* sl_stat;    // [B][n_slices]
  unsigned long long* sl_keys;   // [B][n_slices][top_n_max]
  int32_t n_slices;
  // support slice records (workspace; needs cuts), or nullptr: one
  // workgroup per support row then streams the row itself
  int32_t n_sup_slices;
  SupSliceStat* sup_stat;   // [n_sup][n_sup_slices]
};


// ---- vocabulary-parallel protocol (shard.hip) ----------------------------------
// Phases, run in order: the row statistics, four radix rounds of the top-k
// threshold, the top-p mass sums, four radix rounds of the top-p threshold,
// the race.  Each phase is a pass over every shard (partials) and a merge of
// the shards' partials into the row state.
enum ShardPhase : int32_t {
  SHARD_STATS = 0,
  SHARD_TOPK0 = 1,       // 1..4: digits at shifts 24, 16, 8, 0
  SHARD_TOPP_SUMS = 5,
  SHARD_TOPP0 = 6,       // 6..9
  SHARD_RACE = 10,
  SHARD_PHASES = 11,
};

// Per-row state of the protocol, written by the merges (device).
struct alignas(16) ShardState {
  float zm;               // row max z
  int32_t am;             // its lowest global id
  int32_t nf;             // finite allowed tokens
  int32_t active;         // sampled row with status OK: later phases run
  double m;               // zm / T
  double log_z;           // log sum exp(s - m)
  float zcut;             // kept-set threshold so far
  float zk;               // top-k threshold (-inf: none)
  uint32_t prefix, pmask; // radix select digits so far
  unsigned long long krem; // top-k: tokens still to take at the current prefix
  unsigned long long base; // top-p: mass above the current prefix
  double need;            // top-p: the mass the cut must reach
  int32_t topk_on, topp_on;
};
static_assert(sizeof(ShardState) == 80, "ShardState layout");

// One shard's contribution to one phase, per row (device).
struct alignas(16) ShardPartial {
  float zm;             // stats: shard max, its lowest global id, finite
  int32_t am;           // count, non-finite flag, exp-sum against the
  int32_t nf;           // shard max
  uint32_t nonfin;
  double se;
  unsigned long long s0, s1;  // top-p sums: kept mass, normalising mass
  double key;           // race: best key, its global id and z
  int32_t t;
  float z;
  unsigned long long hist[256];  // radix rounds: counts or fixed-point masses
};
static_assert(sizeof(ShardPartial) == 2112, "ShardPartial layout");

// A shard's pass splits each row into sub-slices of kShardSub tokens (a
// multiple of 32, so that a sub-slice starts on a mask word), one workgroup
// and one record each: a shard of width w makes ceil(w / kShardSub) records
// per row, laid out [sub-slice][B].
constexpr int kShardSub = 4096;

struct ShardArgs {
  const RowParams* rows;
  const void* logits;   // the shard: [B, ld], tokens v0 .. v0 + width - 1
  int64_t ld;
  int32_t B, V;         // V: the whole vocabulary
  int32_t v0, width;
  const int32_t* mask;  // the shard's bitmask words (bit j: token v0 + j), or nullptr
  int64_t mask_ld;
  const uint8_t* row_has_mask;
  ShardState* state;
  ShardPartial* part;   // pass: this shard's [subs][B]; merge: [n_parts][B]
  int32_t n_parts;      // merge: records per row over every shard
  int32_t phase;
  int32_t* out_ids;
  float* out_lp;
  int32_t* out_st;
};

hipError_t launch_shard_pass(const ShardArgs& a, bool bf16, bool vec, hipStream_t stream);
hipError_t launch_shard_merge(const ShardArgs& a, hipStream_t stream);

// ---- speculative verification (spec.hip) -----------------------------------------
struct SpecArgs {
  int32_t n_req, k;         // requests, drafts per request (k+1 rows each)
  const int32_t* sampled;   // [n_req, k+1] the rows' drawn tokens
  const int32_t* status;    // [n_req, k+1] or nullptr
  const int32_t* draft;     // [n_req, k]
  const int32_t* eos;       // [n_req] terminator per request (-1: none) or nullptr
  int32_t* tokens;          // [n_req, k+1] emitted tokens, then -1
  int32_t* count;           // [n_req] tokens emitted
  int32_t* rollback;        // [n_req] positions to roll back, or nullptr
};

hipError_t launch_spec_accept(const SpecArgs& a, hipStream_t stream);

// Optional timing events recorded around the sampling kernel.
struct KernelEvents {
  hipEvent_t start;
  hipEvent_t stop;
};

hipError_t launch_transforms(const RowParams* rows, const int32_t* hist_raw, const PenEntry* pen,
                             const BiasEntry* bias, float* logits, int64_t ld, int32_t B,
                             hipStream_t stream);
hipError_t launch_bitmask(void* logits, bool bf16, int64_t ld, int32_t B, int32_t V,
                          const int32_t* mask, int64_t mask_ld, const uint8_t* row_has_mask,
                          hipStream_t stream);
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream);
// Device address of the library's own workspace (kStaticWorkspaceBytes) on
// the current device; the first call on a device clears its row counters on
// `stream`.
hipError_t static_workspace(void** ptr, hipStream_t stream);

// algo 0: the fused fast path; algo 1: the row-serial exact path.
hipError_t launch_sample(const SampleArgs& a, bool bf16, bool vec, int algo,
                         const KernelEvents* ev, hipStream_t stream);

// The logprob-outputs kernels: with slice records, the slice pass (B *
// n_slices workgroups) first; then n_row_blocks + n_sup workgroups.
hipError_t launch_outputs(const SampleArgs& a, const OutputArgs& o, bool bf16, bool vec,
                          const KernelEvents* ev, hipStream_t stream);

}  // namespace cds
