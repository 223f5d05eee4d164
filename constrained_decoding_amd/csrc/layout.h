// layout.h -- device-memory layouts shared by the host code and the kernels
// of libcd_sampler.so: the packed per-row parameter records and the
// workspace used between the two sampling kernels.
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
  ROW_BIAS = 1u << 5,    // has bias entries
};

struct alignas(16) RowParams {
  float temperature;
  float top_p;
  float min_p;
  int32_t top_k;  // effective: 0 when off
  float rep, freq, pres;
  uint32_t flags;  // RowFlag
  int32_t pen_lo, pen_hi;    // [lo, hi) into the penalty entries
  int32_t bias_lo, bias_hi;  // [lo, hi) into the bias entries
  uint64_t seed;
  uint64_t offset;
};
static_assert(sizeof(RowParams) == 64, "RowParams layout");

struct PenEntry {
  int32_t id;
  int32_t count;
};
struct BiasEntry {
  int32_t id;
  float val;
};

// ---- sampling geometry ------------------------------------------------------
// A row is split into P slices of S tokens (S a multiple of 4); one workgroup
// per slice.  The histogram window covers s = z/T within NBINS/16 of the row
// maximum in bins of width 1/16; tokens further below can neither win the race
// (the exponential race key is bounded, see kernels.hip) nor carry mass that
// matters at the 1e-9 level.
constexpr int kBinsPerUnit = 16;
constexpr int NBINS = 560;        // 35 units of s
constexpr int UCAP = 4096;        // boundary tokens the refinement holds on chip
constexpr int kMaxSlices = 64;
constexpr int kMaxRows = 65535;

// ---- workspace ------------------------------------------------------------
struct RowSync {        // zero between calls; restored by the last arrivers
  uint32_t scan_ticket;
  uint32_t race_ticket;
  uint32_t ucount;
  uint32_t pad;
};

struct SliceHead {
  float zmax;           // max finite allowed z of the slice (-inf if none)
  int32_t arg;          // its lowest index (-1 if none)
  uint32_t nonfinite;   // any NaN / +inf among allowed tokens
  int32_t nfin;         // finite allowed tokens
  double sumexp;        // sum exp((z - zmax) * invT_eff)
  double jmax;          // floor(zmax * invT * 16) (histogram rows)
  uint32_t under;       // tokens below the slice window
  uint32_t pad[3];
};
static_assert(sizeof(SliceHead) == 48, "SliceHead layout");

struct SliceBest {
  double key;  // race key of the slice's winner (-inf if it had no candidate)
  int32_t t;   // its token (INT_MAX if none)
  float z;     // its logit
};

enum PlanMode : int32_t { PLAN_NONE = 0, PLAN_DONE = 1, PLAN_FAST = 2, PLAN_SLOW = 3 };

struct alignas(16) Plan {
  int32_t mode;      // PlanMode
  int32_t arg;       // row argmax (lowest index)
  float zmax;
  float zcut1;       // min-p value cut, -inf when inactive
  double m;          // zmax / T
  double log_z;      // log sum exp(s - m) over allowed finite tokens
  float z_win;       // tokens below lie outside the histogram window
  float z_sure;      // tokens >= max(z_sure, zcut1) are raced by the slices
  float a_lo, a_hi;  // top-p boundary value range [a_lo, a_hi)
  float k_lo, k_hi;  // top-k / min-p boundary bin [k_lo, k_hi)
  int32_t k_rank;    // > 0: zcut2 is the k_rank-th largest U value in [k_lo,k_hi)
  int32_t topp;      // top-p cut lies in [a_lo, a_hi)
  uint32_t u_expected;
  uint32_t pad;
  double m_sure;     // mass (relative to exp(m)) of tokens >= z_sure
  double m_mid;      // mass of tokens between a_lo (excl.) and k_hi (excl.)
  double p;          // top_p
};

struct WorkspaceLayout {
  size_t sync_off, plan_off, head_off, hist_off, best_off, ulist_off, total;
  int P;
  int64_t S;
};

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Slices per row: as many as keep a slice <= 16384 tokens, at most kMaxSlices.
inline int choose_slices(int32_t V) {
  int64_t p = (V + 16383) / 16384;
  if (p < 1) p = 1;
  if (p > kMaxSlices) p = kMaxSlices;
  return (int)p;
}

inline WorkspaceLayout workspace_layout(int32_t B, int32_t V) {
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
  L.hist_off = take((sizeof(uint32_t) + sizeof(uint64_t)) * NBINS * (size_t)B * L.P);
  L.best_off = take(sizeof(SliceBest) * (size_t)B * L.P);
  L.ulist_off = take(sizeof(uint64_t) * UCAP * (size_t)B);
  L.total = off;
  return L;
}

}  // namespace cds
