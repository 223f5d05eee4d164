// layout.h -- device-memory layouts shared by the host code and the kernels
// of libcd_sampler.so: the packed per-row parameter records and the
// workspace the sampling kernel's workgroups share.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace cds {

// ---- packed parameters (written by sampler_pack_params) -------------------
enum RowFlag : uint32_t {
  ROW_GREEDY = 1u << 0,  // argmax row: T < 1e-5 or top_k == 1
  ROW_TOPK = 1u << 1,    // 1 < top_k < V on a non-greedy row
  ROW_TOPP = 1u << 2,    // top_p < 1 on a non-greedy row
  ROW_MINP = 1u << 3,    // min_p > 0 on a non-greedy row
  ROW_PEN = 1u << 4,     // has penalty entries
  ROW_PEN_RAW = 1u << 6, // its history is raw int32 ids (repeats not merged):
                         // the transforms kernel counts them
  ROW_BIAS = 1u << 5,    // has bias entries
  // filter order (neither bit: min-p, then top-k, then top-p); set only on
  // rows where the order changes the kept set (top-p with top-k or min-p)
  ROW_ORDER_JOINT = 1u << 8,      // top-k and top-p cut one distribution jointly
  ROW_ORDER_MINP_LAST = 1u << 9,  // top-k, then top-p, then min-p
};
constexpr uint32_t kRowOrderBits = ROW_ORDER_JOINT | ROW_ORDER_MINP_LAST;

struct alignas(16) RowParams {
  float temperature;
  float top_p;
  float min_p;
  int32_t top_k;  // effective: 0 when off
  float rep, freq, pres;
  uint32_t flags;  // RowFlag
  int32_t pen_lo, pen_hi;    // [lo, hi) into the raw history ids (ROW_PEN_RAW)
                             // or into the counted penalty entries
  int32_t bias_lo, bias_hi;  // [lo, hi) into the bias entries
  uint64_t seed;
  uint64_t offset;
};
static_assert(sizeof(RowParams) == 64, "RowParams layout");

// Task rows of the sampling kernel: a pass-2 task (the race of a row whose
// slices needed the row's plan first) carries kPass2 on its row index.  In a
// split batch (kSplit) a pass-2 task covers one half of its slice (kHalf: the
// second half), so that twice as many workgroups share a row's race.
constexpr int32_t kPass2 = 1 << 30;
constexpr int32_t kHalf = 1 << 29;
constexpr int32_t kSplit = 1 << 28;
constexpr int32_t kTaskRow = kSplit - 1;  // the row index bits

// Where a row's data lives in the workspace (written by the host pack, one
// per row): the rows that list candidates (LIST rows: a list per slice; HOLD
// rows: a boundary list per pass-2 task) get lists of row_list_cap() entries
// each, contiguous from entry 64*list64 of the list area, and one SliceBest
// record per list (RACE rows: records only).  HOLD rows come first in the
// record area with 2P records each, so a HOLD row's P slice histograms start
// at histogram slot (rec / 2P) * P.  Rows get only what their class uses, so
// a workspace can be sized for the batch it serves.
struct RowSlots {
  uint32_t list64;  // first entry of the row's lists, in units of 64 entries
  uint32_t rec;     // first SliceBest record of the row
};
static_assert(sizeof(RowSlots) == 8, "RowSlots layout");

struct PenEntry {
  int32_t id;
  int32_t count;
};
struct BiasEntry {
  int32_t id;
  float val;
};

// ---- sampling geometry ------------------------------------------------------
// A row is split into P slices (S tokens each, S a multiple of 4), one
// workgroup of kScanThreads per slice, each thread holding up to kMaxChunks
// chunks of four tokens in registers.
//
// Histogram bins are aligned to a power-of-two grid in z: width
// delta = 2^floor(log2(T/16)), i.e. between 1/32 and 1/16 in s = z/T.  Bin
// index floor(z/delta) and the offset inside the bin are exact fp32
// operations, bins of different slices line up, and the value range of a bin
// is exactly [k*delta, (k+1)*delta).  The window holds the NBINS bins below the
// row maximum (at least 35 units of s); tokens further down can neither win
// the race (the exponential-race key is bounded, see device_common.h) nor carry
// mass that matters at the 1e-10 level.
constexpr int NBINS = 1120;
#ifndef CDS_SCAN_THREADS
#define CDS_SCAN_THREADS 256
#endif
#ifndef CDS_MAX_CHUNKS
#define CDS_MAX_CHUNKS 15
#endif
constexpr int kScanThreads = CDS_SCAN_THREADS;
constexpr int kMaxChunks = CDS_MAX_CHUNKS;
constexpr int64_t kSliceMax = (int64_t)kScanThreads * 4 * kMaxChunks;  // 15360 tokens
constexpr int kCountShift = 48;   // histogram word: count << 48 | fixed-point mass
constexpr int UCAP = 4096;        // listed tokens of a row the finisher holds on chip
constexpr int SCAP = 2048;        // listed tokens one slice can hand over
constexpr int kHistDevice = 4096;  // history tokens per row counted on the device
constexpr int kMaxSlices = 64;
constexpr int kShortList = 256;   // a row's listed tokens one wave of the finisher resolves
constexpr int kXcds = 8;          // XCDs of an MI355X (workgroups go round-robin over them)
constexpr int kMaxRows = 65535;
// Size of the library's own workspace (sampler_sample_static), per device.
constexpr size_t kStaticWorkspaceBytes = (size_t)64 << 20;

// How a row's slices work in the sampling kernel.  The host dispatches the rows
// in the order HOLD, then top-k LIST rows by the length of their lists, then
// the other RACE and LIST rows, then GREEDY.
enum RowClass : uint32_t {
  CLS_GREEDY = 0,  // argmax: the planner answers from the slice summaries
  CLS_RACE = 1,    // no cut: each slice races all its tokens
  CLS_LIST = 2,    // top-k whose lists fit (list_q), or min-p without top-k:
                   // each slice lists a superset of its candidates; the
                   // planner resolves the row from the lists
  CLS_HOLD = 3,    // top-p as the only cut, or a larger top-k: the row's plan
                   // (histogram cuts) comes first, then a second pass races
};

// Tokens a slice of a top-k row lists: its own top-q, q = min(k, ceil(2 k/P)
// + 64), enough for its share of the row's top-k unless that share is far
// above the average k/P (the row's finisher checks, and falls back).
// (constexpr: callable from host and device code alike)
// A slice finds its list cut from its waves' ceil(q/W)-th largest of four
// group maxima per lane (W waves); past q = 3/8 of the 4*kScanThreads group
// maxima that cut lets too many tokens through, and the row takes HOLD.  The
// cut passes up to ~1.5 q tokens of a slice, so a LIST row also needs
// 1.5 q P <= UCAP (the finisher's capacity).
constexpr int32_t kListQMax = 3 * kScanThreads / 2;
constexpr int32_t list_q(int32_t top_k, int32_t P) {
  return top_k < (2 * top_k + P - 1) / P + 64 ? top_k : (2 * top_k + P - 1) / P + 64;
}
constexpr RowClass row_class_of(uint32_t flags, int32_t top_k, int32_t P) {
  return (flags & ROW_GREEDY)  ? CLS_GREEDY
         : (flags & ROW_TOPK)  ? (3 * (int64_t)list_q(top_k, P) * P <= 2 * UCAP &&
                                          list_q(top_k, P) <= kListQMax
                                      ? CLS_LIST : CLS_HOLD)
         : (flags & ROW_MINP)  ? CLS_LIST
         : (flags & ROW_TOPP)  ? CLS_HOLD
                               : CLS_RACE;
}

// Entries per list of a row: top-k rows that list candidates hold twice their
// share and a margin (list_cap_topk), min-p rows and second-pass boundary
// lists SCAP, rows that list nothing 0.
constexpr uint32_t list_cap_topk(int32_t q);
constexpr uint32_t row_list_cap(uint32_t flags, int32_t top_k, int32_t P);

// ---- workspace ------------------------------------------------------------
// Per-row meeting point of the row's workgroups.  Counters count the slices
// of the current call that passed them; the last one resets the counter to
// zero (so they are zero between calls).  Flags hold the call generation that
// set them.
struct RowSync {
  unsigned long long arrive;  // slices that published their summary
  unsigned long long done;    // HOLD slices that finished their race
  uint32_t ready;             // generation whose plan is published
  uint32_t failed;            // generation in which a race task gave up waiting
  uint32_t pad[2];
};
static_assert(sizeof(RowSync) == 32, "RowSync layout");

enum SliceFlag : uint32_t {
  SLICE_NONFINITE = 1u,   // a NaN or +inf among the slice's allowed tokens
  SLICE_BINS_LOST = 2u,   // |zmax / delta| too large for exact fp32 bin indices
};

struct SliceHead {
  float zmax;           // max allowed finite z of the slice (-inf if none)
  int32_t arg;          // its lowest index (-1 if none)
  uint32_t flags;       // SliceFlag
  float kmax;           // floor(zmax / delta) (histogram rows)
  double sumexp;        // sum exp((z - zmax) / T_eff): rows without a histogram
                        // sum the tokens, HOLD rows their histogram bins
  uint32_t pad[2];
};
static_assert(sizeof(SliceHead) == 32, "SliceHead layout");

struct SliceBest {  // fp32 race keys: the slice's best two, and its listed tokens
  float k1;         // best key (-inf if the slice had no candidate)
  int32_t t1;       // its token
  float z1;         // its logit
  float k2;         // second-best key
  uint32_t ucnt;    // tokens in the slice's list (> SCAP: overflowed)
  uint32_t pad[3];  // pad[0] = 1: keys are relative to the slice maximum,
                    // whose fp32 bits are pad[1]
};
static_assert(sizeof(SliceBest) == 32, "SliceBest layout");

enum PlanMode : int32_t { PLAN_NONE = 0, PLAN_DONE = 1, PLAN_FAST = 2, PLAN_SLOW = 3 };

struct alignas(16) Plan {
  int32_t mode;      // PlanMode
  int32_t arg;       // row argmax (lowest index)
  float zmax;
  float zcut1;       // min-p value cut, -inf when inactive
  double m;          // zmax / T
  double log_z;      // log sum exp(s - m) over allowed finite tokens
  float z_sure;      // tokens >= max(z_sure, zcut1) are raced by the slices
  float a_lo, a_hi;  // top-p boundary value range [a_lo, a_hi)
  float k_lo, k_hi;  // top-k / min-p boundary bin [k_lo, k_hi)
  int32_t k_rank;    // > 0: zcut2 is the k_rank-th largest U value in [k_lo,k_hi)
  int32_t topp;      // top-p cut lies in [a_lo, a_hi)
  uint32_t u_expected;
  double m_sure;     // mass (relative to exp(m)) of tokens >= z_sure
  double m_mid;      // mass of tokens below a_lo and at or above k_hi
  double p;          // top_p
  int32_t path;      // how the row's finisher resolved the row (FinishPath)
  int32_t list_mode; // 1: the slices' lists hold every candidate (no sure region)
};
static_assert(sizeof(Plan) == 96, "Plan layout");

// Written back into Plan::path by the workgroup that resolved the row
// (diagnostics and tests).
enum FinishPath : int32_t {
  PATH_NONE = 0,
  PATH_FAST = 1,       // fp32 race margin decided the winner
  PATH_RERACE = 2,     // fp32 top two within the error bound: fp64 re-race
  PATH_EXACT = 3,      // row-serial exact path (plan SLOW, list overflow, cut outside range)
};

struct WorkspaceLayout {
  size_t sync_off, plan_off, head_off, hist_off, best_off, ulist_off, total;
  int P;
  int64_t S;
};

// Entries per list of a top-k row that lists candidates: room for twice its
// per-slice share q plus a margin, in whole 64-entry blocks (a slice whose
// list would pass it overflows, and the row takes the exact path).
constexpr uint32_t list_cap_topk(int32_t q) {
  return (uint32_t)((2 * q + 64 + 63) / 64 * 64) < (uint32_t)SCAP
             ? (uint32_t)((2 * q + 64 + 63) / 64 * 64)
             : (uint32_t)SCAP;
}
constexpr uint32_t row_list_cap(uint32_t flags, int32_t top_k, int32_t P) {
  return row_class_of(flags, top_k, P) == CLS_HOLD ? (uint32_t)SCAP
         : row_class_of(flags, top_k, P) == CLS_LIST
             ? ((flags & ROW_TOPK) ? list_cap_topk(list_q(top_k, P)) : (uint32_t)SCAP)
             : 0u;
}

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Slices per row: the fewest that keep a slice register-resident.
inline int choose_slices(int32_t V) {
  int64_t p = (V + kSliceMax - 1) / kSliceMax;
  if (p < 1) p = 1;
  if (p > kMaxSlices) p = kMaxSlices;
  return (int)p;
}

// Pass-2 tasks per row slice: two halves when the pass-2 rows are few (at
// most a quarter of the batch: their latency then matters more than the
// workgroups' count) and the row's 2P lists fit one wave of the finisher
// (P <= 32); else one.
constexpr int pass2_halves(int P, int32_t n_hold, int32_t B) {
  return (2 * P <= 64 && 4 * n_hold <= B) ? 2 : 1;
}

// Workspace layout for B rows of V tokens whose rows take n_hist slice
// histograms, n_rec list records and n_entries list entries in all (see
// RowSlots).
inline WorkspaceLayout workspace_layout(int32_t B, int32_t V, uint64_t n_hist, uint64_t n_rec,
                                        uint64_t n_entries) {
  WorkspaceLayout L;
  L.P = choose_slices(V);
  L.S = round_up((V + L.P - 1) / L.P, 4);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = (size_t)round_up((int64_t)(off + bytes), 256);
    return o;
  };
  // The counters sit at a fixed place sized for the largest batch, so a
  // workspace stays valid across calls with different B (they are the only
  // bytes that must be zero on entry; everything else is written before it is
  // read within a call).
  L.sync_off = take(sizeof(RowSync) * (size_t)kMaxRows);
  L.plan_off = take(sizeof(Plan) * (size_t)B);
  L.head_off = take(sizeof(SliceHead) * (size_t)B * L.P);
  L.hist_off = take(sizeof(uint64_t) * NBINS * (size_t)n_hist);
  L.best_off = take(sizeof(SliceBest) * (size_t)n_rec);
  L.ulist_off = take(sizeof(uint64_t) * (size_t)n_entries);
  L.total = off;
  return L;
}

// The largest layout any batch of B rows of V tokens can need: every row with
// P histograms and 2P lists of SCAP entries.
inline WorkspaceLayout workspace_layout(int32_t B, int32_t V) {
  const int P = choose_slices(V);
  return workspace_layout(B, V, (uint64_t)B * P, (uint64_t)B * 2 * P,
                          (uint64_t)B * 2 * P * SCAP);
}

}  // namespace cds
