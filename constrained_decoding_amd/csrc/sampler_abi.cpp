// sampler_abi.cpp -- the C ABI of libcd_sampler.so (declared and documented in
// include/cd_sampler.h): parameter validation and packing on the host, and the
// kernel launches of the sampling step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <utility>
#include <vector>

#include "cd_sampler.h"
#include "kernels.h"
#include "layout.h"

using namespace cds;

namespace {

constexpr int32_t kMaxV = 1 << 24;
constexpr int32_t kMaxB = kMaxRows;

std::atomic<uint32_t> g_gen{0u};  // call generations (see sampler_sample_ex)

// Wall-clock rate (kHz) of each device, read once per device: a property of
// the device, so concurrent first calls store the same value.
constexpr int kMaxDevices = 64;
std::atomic<int> g_rate_khz[kMaxDevices];

int wall_clock_khz() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 100000;
  int r = g_rate_khz[dev].load(std::memory_order_relaxed);
  if (r > 0) return r;
  if (hipDeviceGetAttribute(&r, hipDeviceAttributeWallClockRate, dev) != hipSuccess || r <= 0)
    r = 100000;
  g_rate_khz[dev].store(r, std::memory_order_relaxed);
  return r;
}

inline bool finite_f(float x) { return std::isfinite(x); }

// Device parameter block: RowParams[B] | int32 row order [B] (the dispatch order
// of sampler_sample) | int32 task rows [tasks_max(B)] (the sampling kernel's
// tasks, see below) | RowSlots[B] (workspace places) | PenEntry[n_pen]
// (counted histories) | BiasEntry[n_bias] | int32 raw history ids
// [n_hist_raw]; the int32 arrays are padded to 16 bytes.  (The block stays
// small: it is copied every step.)
//
// Tasks: the sampling kernel runs groups of 8 tasks (one per XCD), each task
// a row's P slices.  Task k is row task_row[k] & ~(kPass2 | kHalf) (-1:
// none).  Pass-1 task groups take the ordered rows 8 at a time;
// rows whose cut needs the whole row's histogram (the first n_hold of the
// order) also get pass-2 groups (bit kPass2; one per slice half, the second
// with kHalf), a lag of groups after their pass-1 group, whose workgroups race
// once the row's plan is out.
size_t list_bytes(int32_t B) { return ((size_t)B * sizeof(int32_t) + 15) / 16 * 16; }
int32_t tasks_max(int32_t B) { return 24 * ((B + 7) / 8); }  // pass 1 + two pass-2 halves
// the task table a batch uses: pass-1 groups, and pass-2 groups of its n_hold
// rows (two per group of rows when their tasks take half slices)
int32_t tasks_used(int32_t B, int32_t n_hold, bool split) {
  return 8 * ((B + 7) / 8 + (split ? 2 : 1) * ((n_hold + 7) / 8));
}

size_t slots_bytes(int32_t B) { return sizeof(RowSlots) * (size_t)B; }

size_t params_bytes_exact(int32_t B, int32_t n_tasks, int64_t n_pen, int64_t n_bias,
                          int64_t n_raw) {
  return sizeof(RowParams) * (size_t)B + list_bytes(B) + list_bytes(n_tasks) + slots_bytes(B) +
         sizeof(PenEntry) * (size_t)n_pen + sizeof(BiasEntry) * (size_t)n_bias +
         list_bytes((int32_t)n_raw);
}

// Pass-2 groups follow their pass-1 group after about one generation of
// resident workgroups (4 per CU on 256 CUs), when the row's plan is likely out;
// a quarter generation later when the pass-2 tasks take whole slices (many
// such rows: their plans come out later, as their slices load together).
#ifndef CDS_PASS2_LAG_SLOTS
#define CDS_PASS2_LAG_SLOTS 1024
#endif
#ifndef CDS_PASS2_LAG_SLOTS_WHOLE
#define CDS_PASS2_LAG_SLOTS_WHOLE 1280
#endif
int pass2_lag(int P, int halves) {
  const int slots = halves == 2 ? CDS_PASS2_LAG_SLOTS : CDS_PASS2_LAG_SLOTS_WHOLE;
  return std::max(1, (slots + 8 * P - 1) / (8 * P));
}

// Validate and pack into host memory: `dst` (cap bytes), or when dst is null
// into `tmp`.  Everything is validated and sized first, then written once into
// the destination.  Returns a SAMPLER_* code (ENOSPC: cap too small).
int pack_into(const sampler_host_params* h, unsigned char* dst, size_t cap,
              std::vector<unsigned char>* tmp, sampler_batch* out) {
  if (!h || !out) return SAMPLER_EINVAL;
  const int32_t B = h->B, V = h->V;
  if (B <= 0 || V <= 0) return SAMPLER_EINVAL;
  if (B > kMaxB || V > kMaxV) return SAMPLER_ERANGE;
  if (!h->temperature) return SAMPLER_EINVAL;
  if (h->filter_order < SAMPLER_ORDER_MINP_FIRST || h->filter_order > SAMPLER_ORDER_MINP_LAST)
    return SAMPLER_EINVAL;
  const uint32_t order_bits = h->filter_order == SAMPLER_ORDER_JOINT       ? ROW_ORDER_JOINT
                              : h->filter_order == SAMPLER_ORDER_MINP_LAST ? ROW_ORDER_MINP_LAST
                                                                           : 0u;
  if ((h->hist_indptr == nullptr) != (h->hist_ids == nullptr)) return SAMPLER_EINVAL;
  if ((h->bias_indptr == nullptr) != (h->bias_ids == nullptr) ||
      (h->bias_ids == nullptr) != (h->bias_vals == nullptr))
    return SAMPLER_EINVAL;

  // CSR structure (the ids themselves are range-checked where they are
  // copied or counted below, before anything reaches the device)
  if (h->hist_indptr) {
    if (h->hist_indptr[0] != 0) return SAMPLER_EINVAL;
    for (int32_t r = 0; r < B; ++r)
      if (h->hist_indptr[r + 1] < h->hist_indptr[r]) return SAMPLER_EINVAL;
    if (h->hist_indptr[B] > (int64_t)INT32_MAX) return SAMPLER_ERANGE;
  }
  if (h->bias_indptr) {
    if (h->bias_indptr[0] != 0) return SAMPLER_EINVAL;
    for (int32_t r = 0; r < B; ++r)
      if (h->bias_indptr[r + 1] < h->bias_indptr[r]) return SAMPLER_EINVAL;
    const int64_t nb = h->bias_indptr[B];
    const int32_t* ids = h->bias_ids;
    const float* vals = h->bias_vals;
    int bad = 0;
    for (int64_t i = 0; i < nb; ++i)  // (branch-free: vectorised)
      bad |= (ids[i] < 0) | (ids[i] >= V) | !(vals[i] < INFINITY);  // NaN or +inf
    if (bad) return SAMPLER_EINVAL;
  }

  std::vector<RowParams> rows((size_t)B);
  std::vector<int32_t> sampled, greedy_rows;
  // Penalties: rows of up to kHistDevice history tokens go to the device as
  // raw ids (copied later straight from hist_ids, n_raw in all; the transforms
  // kernel counts them); only longer rows are counted here, into `pen`.
  std::vector<PenEntry> pen;
  int64_t n_raw = 0;
  // bias entries, written by index into room for all of them (a push_back per
  // entry reloads the vector's end from memory around every other store)
  std::vector<BiasEntry> bias(h->bias_indptr ? (size_t)h->bias_indptr[B] : 0u);
  BiasEntry* const bout = bias.data();
  size_t n_bias_out = 0;
  uint32_t flags = SAMPLER_FLAG_ALL_GREEDY;
  bool all_nongreedy_have_k = true;
  int32_t max_k = 0;
  std::vector<int32_t> scratch_ids;
  std::vector<std::pair<int32_t, int64_t>> scratch_bias;

  for (int32_t r = 0; r < B; ++r) {
    RowParams rp;
    std::memset(&rp, 0, sizeof rp);
    const float T = h->temperature[r];
    if (!finite_f(T) || T < 0.0f) return SAMPLER_EINVAL;
    const int32_t k = h->top_k ? h->top_k[r] : 0;
    const float p = h->top_p ? h->top_p[r] : 1.0f;
    const float mp = h->min_p ? h->min_p[r] : 0.0f;
    const float rep = h->repetition_penalty ? h->repetition_penalty[r] : 1.0f;
    const float fr = h->frequency_penalty ? h->frequency_penalty[r] : 0.0f;
    const float pr = h->presence_penalty ? h->presence_penalty[r] : 0.0f;
    if (!(p > 0.0f && p <= 1.0f)) return SAMPLER_EINVAL;   // also rejects NaN
    if (!(mp >= 0.0f && mp <= 1.0f)) return SAMPLER_EINVAL;
    if (!finite_f(rep) || !(rep > 0.0f)) return SAMPLER_EINVAL;
    if (!finite_f(fr) || !finite_f(pr)) return SAMPLER_EINVAL;

    rp.temperature = T;
    rp.top_p = p;
    rp.min_p = mp;
    rp.rep = rep;
    rp.freq = fr;
    rp.pres = pr;
    rp.seed = h->seed ? h->seed[r] : 0ull;
    rp.offset = h->offset ? h->offset[r] : (uint64_t)r;
    const bool greedy = (T < 1e-5f) || (k == 1);
    if (greedy) {
      greedy_rows.push_back(r);
      rp.flags |= ROW_GREEDY;
      flags |= SAMPLER_FLAG_ANY_GREEDY;
    } else {
      flags &= ~SAMPLER_FLAG_ALL_GREEDY;
      sampled.push_back(r);
      if (k > 1 && k < V) {
        rp.flags |= ROW_TOPK;
        rp.top_k = k;
        flags |= SAMPLER_FLAG_NEED_TOP_K;
        max_k = std::max(max_k, k);
      } else {
        all_nongreedy_have_k = false;
      }
      if (p < 1.0f) {
        rp.flags |= ROW_TOPP;
        flags |= SAMPLER_FLAG_NEED_TOP_P;
      }
      if (mp > 0.0f) {
        rp.flags |= ROW_MINP;
        flags |= SAMPLER_FLAG_NEED_MIN_P;
      }
      // the order matters only where top-p meets another cut
      if ((rp.flags & ROW_TOPP) && (rp.flags & (ROW_TOPK | ROW_MINP))) rp.flags |= order_bits;
    }

    // penalties: the row's history, raw (counted on the device) or as
    // (token, count) entries; pen_lo / pen_hi index the raw ids or the entries
    const bool pen_active = (rep != 1.0f) || (fr != 0.0f) || (pr != 0.0f);
    if (h->hist_indptr && !pen_active) {
      // an unused history is still checked: any id outside [0, V) is rejected
      const int64_t lo = h->hist_indptr[r], hi = h->hist_indptr[r + 1];
      const int32_t* ids = h->hist_ids;
      int bad = 0;
      for (int64_t i = lo; i < hi; ++i) bad |= (ids[i] < 0) | (ids[i] >= V);
      if (bad) return SAMPLER_EINVAL;
    }
    if (h->hist_indptr && pen_active) {
      const int64_t lo = h->hist_indptr[r], hi = h->hist_indptr[r + 1];
      if (hi > lo) {
        if (hi - lo <= kHistDevice) {
          // as they come: the transforms kernel merges repeats
          rp.pen_lo = (int32_t)n_raw;
          n_raw += hi - lo;
          rp.pen_hi = (int32_t)n_raw;
          rp.flags |= ROW_PEN_RAW;
        } else {
          rp.pen_lo = (int32_t)pen.size();
          scratch_ids.assign(h->hist_ids + lo, h->hist_ids + hi);
          for (const int32_t id : scratch_ids)
            if (id < 0 || id >= V) return SAMPLER_EINVAL;
          std::sort(scratch_ids.begin(), scratch_ids.end());
          for (size_t i = 0; i < scratch_ids.size();) {
            size_t j = i;
            while (j < scratch_ids.size() && scratch_ids[j] == scratch_ids[i]) ++j;
            pen.push_back(PenEntry{scratch_ids[i], (int32_t)(j - i)});
            i = j;
          }
          rp.pen_hi = (int32_t)pen.size();
        }
        rp.flags |= ROW_PEN;
        flags |= SAMPLER_FLAG_NEED_PENALTY;
      }
    }
    // bias: duplicates of a token keep the later entry
    rp.bias_lo = rp.bias_hi = (int32_t)n_bias_out;
    if (h->bias_indptr) {
      const int64_t lo = h->bias_indptr[r], hi = h->bias_indptr[r + 1];
      if (hi > lo) {
        if (hi - lo <= 32) {
          // short rows (the usual case): an entry survives unless a later one
          // names the same token; survivors keep their order
          // (from the last entry back: a token seen before, i.e. later in the
          // row, drops the entry; one pass over the row's few entries each)
          const int32_t* ids = h->bias_ids + lo;
          const float* vals = h->bias_vals + lo;
          const int n = (int)(hi - lo);
          uint32_t keep = 0u;
          for (int i = n - 1; i >= 0; --i) {
            const int32_t id = ids[i];
            int seen = 0;
            for (int j = i + 1; j < n; ++j) seen |= ids[j] == id;
            keep |= seen ? 0u : (1u << i);
          }
          for (int i = 0; i < n; ++i)
            if ((keep >> i) & 1u) bout[n_bias_out++] = BiasEntry{ids[i], vals[i]};
        } else {
          scratch_bias.clear();
          for (int64_t i = lo; i < hi; ++i) scratch_bias.emplace_back(h->bias_ids[i], i);
          std::sort(scratch_bias.begin(), scratch_bias.end());
          for (size_t i = 0; i < scratch_bias.size(); ++i) {
            if (i + 1 < scratch_bias.size() && scratch_bias[i + 1].first == scratch_bias[i].first)
              continue;  // a later duplicate follows
            bout[n_bias_out++] =
                BiasEntry{scratch_bias[i].first, h->bias_vals[scratch_bias[i].second]};
          }
        }
        rp.bias_hi = (int32_t)n_bias_out;
        rp.flags |= ROW_BIAS;
        flags |= SAMPLER_FLAG_HAS_BIAS;
      }
    }
    rows[(size_t)r] = rp;
  }
  bias.resize(n_bias_out);
  if (bias.size() > (size_t)INT32_MAX) return SAMPLER_ERANGE;

  // dispatch order: the rows whose last slice has the longest way to go
  // first -- rows whose slices wait for the row's plan, then top-k rows with
  // long candidate lists, then top-k rows whose lists are too long for the
  // finisher's one-wave path -- then the other sampled rows, then the greedy
  // rows
  std::vector<int32_t> order;
  const int P = choose_slices(V);
  auto rank = [&](int32_t r) {
    const RowParams& q = rows[(size_t)r];
    const RowClass c = row_class_of(q.flags, q.top_k, P);
    if (c == CLS_HOLD) return 0;
    if (c == CLS_LIST && (q.flags & ROW_TOPK)) {
      const int64_t n = (int64_t)list_q(q.top_k, P) * P;  // the lists' nominal length
      if (!(q.flags & ROW_MINP) && n > 1024) return 1;
      if (n > kShortList) return 2;
    }
    return 3;
  };
  // within a group, hotter rows first: a flatter distribution lists and races
  // more tokens at the end
  order = sampled;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    const int rx = rank(x), ry = rank(y);
    if (rx != ry) return rx < ry;
    return rows[(size_t)x].temperature > rows[(size_t)y].temperature;
  });
  int32_t n_hold = 0;
  while (n_hold < (int32_t)order.size() && rank(order[(size_t)n_hold]) == 0) ++n_hold;
  order.insert(order.end(), greedy_rows.begin(), greedy_rows.end());
  const int halves = pass2_halves(P, n_hold, B);
  if (halves == 2) flags |= SAMPLER_FLAG_SPLIT_PASS2;
  const int32_t n_tasks = tasks_used(B, n_hold, halves == 2);

  const int64_t n_pen = (int64_t)pen.size();
  const size_t bytes = params_bytes_exact(B, n_tasks, n_pen, (int64_t)bias.size(), n_raw);
  unsigned char* p = dst;
  if (!p) {
    tmp->resize(bytes);
    p = tmp->data();
  } else if (cap < bytes) {
    return SAMPLER_ENOSPC;
  }
  const size_t off_list = sizeof(RowParams) * (size_t)B;
  const size_t off_task = off_list + list_bytes(B);
  const size_t off_slots = off_task + list_bytes(n_tasks);
  const size_t off_pen = off_slots + slots_bytes(B);
  std::memcpy(p, rows.data(), sizeof(RowParams) * rows.size());
  if (!order.empty()) std::memcpy(p + off_list, order.data(), sizeof(int32_t) * order.size());
  std::memset(p + off_list + sizeof(int32_t) * order.size(), 0,
              list_bytes(B) - sizeof(int32_t) * order.size());
  // the task groups: pass-1 group g, and pass-2 group g - lag after it
  const int32_t G1 = (B + 7) / 8, GH = (n_hold + 7) / 8, lag = pass2_lag(P, halves);
  std::vector<std::pair<int, int32_t>> seq;  // (pass: 1, or 2 + half, group)
  auto pass2 = [&](int32_t g) {
    for (int h = 0; h < halves; ++h) seq.push_back({2 + h, g});
  };
  for (int32_t g = 0; g < G1; ++g) {
    seq.push_back({1, g});
    if (g - lag >= 0 && g - lag < GH) pass2(g - lag);
  }
  for (int32_t g = std::max(0, G1 - lag); g < GH; ++g) pass2(g);
  int32_t* trow = reinterpret_cast<int32_t*>(p + off_task);
  std::memset(p + off_task, 0, list_bytes(n_tasks));
  for (int32_t k = 0; k < n_tasks; ++k) trow[k] = -1;
  for (size_t q = 0; q < seq.size(); ++q)
    for (int32_t x = 0; x < 8; ++x) {
      const int32_t o = seq[q].second * 8 + x;
      if (o >= (seq[q].first == 1 ? B : n_hold)) continue;
      const int32_t r = order[(size_t)o];
      trow[q * 8 + (size_t)x] = r | (seq[q].first >= 2 ? kPass2 : 0) |
                                (seq[q].first >= 2 && halves == 2 ? kSplit : 0) |
                                (seq[q].first == 3 ? kHalf : 0);
    }
  // workspace places: lists, records and histograms for the rows that use
  // them (see RowSlots), in dispatch order: the HOLD rows (the first n_hold)
  // take 2P records each from record 0, so their histogram slot follows
  uint64_t ws_entries = 0, ws_rec = 0;
  const uint64_t ws_hist = (uint64_t)n_hold * P;
  {
    RowSlots* sl = reinterpret_cast<RowSlots*>(p + off_slots);
    std::memset(sl, 0, slots_bytes(B));
    for (size_t q = 0; q < order.size(); ++q) {
      const int32_t r = order[(size_t)q];
      const RowParams& rp = rows[(size_t)r];
      const RowClass c = row_class_of(rp.flags, rp.top_k, P);
      const uint32_t lcap = row_list_cap(rp.flags, rp.top_k, P);
      const int lists = c == CLS_HOLD ? 2 * P : (c == CLS_LIST || c == CLS_RACE) ? P : 0;
      sl[r].rec = (uint32_t)ws_rec;
      sl[r].list64 = (uint32_t)(ws_entries / 64);
      ws_rec += (uint64_t)lists;
      ws_entries += (uint64_t)(c == CLS_HOLD ? halves * P : lists) * lcap;
    }
  }

  // counted penalty entries, the bias, then the raw history ids in row order
  // (runs of consecutive raw rows are one copy each: their CSR ranges adjoin)
  // (memcpy from an empty vector's null data() is undefined even for 0 bytes)
  if (!pen.empty()) std::memcpy(p + off_pen, pen.data(), sizeof(PenEntry) * pen.size());
  if (!bias.empty())
    std::memcpy(p + off_pen + sizeof(PenEntry) * (size_t)n_pen, bias.data(),
                sizeof(BiasEntry) * bias.size());
  const size_t off_raw = off_pen + sizeof(PenEntry) * (size_t)n_pen +
                         sizeof(BiasEntry) * bias.size();
  int32_t* raw = reinterpret_cast<int32_t*>(p + off_raw);
  for (int32_t r = 0; r < B;) {
    if (!(rows[(size_t)r].flags & ROW_PEN_RAW)) {
      ++r;
      continue;
    }
    int32_t e = r + 1;
    while (e < B && (rows[(size_t)e].flags & ROW_PEN_RAW) &&
           rows[(size_t)e].pen_lo == rows[(size_t)(e - 1)].pen_hi &&
           h->hist_indptr[e] == h->hist_indptr[e - 1] + (rows[(size_t)(e - 1)].pen_hi -
                                                         rows[(size_t)(e - 1)].pen_lo))
      ++e;
    // one block copy (the destination may be pinned staging memory, where
    // the library copy writes fastest), then the range check on the source
    const int32_t n = rows[(size_t)(e - 1)].pen_hi - rows[(size_t)r].pen_lo;
    const int32_t* src = h->hist_ids + h->hist_indptr[r];
    int32_t* dstp = raw + rows[(size_t)r].pen_lo;
    std::memcpy(dstp, src, sizeof(int32_t) * (size_t)n);
    int bad = 0;
    for (int32_t i = 0; i < n; ++i) bad |= (src[i] < 0) | (src[i] >= V);
    if (bad) return SAMPLER_EINVAL;
    r = e;
  }
  std::memset(reinterpret_cast<unsigned char*>(raw + n_raw), 0,
              list_bytes((int32_t)n_raw) - sizeof(int32_t) * (size_t)n_raw);

  std::memset(out, 0, sizeof *out);
  out->B = B;
  out->V = V;
  out->flags = flags;
  out->max_top_k = ((flags & SAMPLER_FLAG_ALL_GREEDY) || !all_nongreedy_have_k) ? 0 : max_k;
  out->n_pen = n_pen;
  out->n_bias = (int64_t)bias.size();
  out->n_hist_raw = n_raw;
  out->bytes = bytes;
  out->n_sampled = (int32_t)sampled.size();
  out->n_hold = n_hold;
  out->ws_list_entries = ws_entries;
  out->ws_records = ws_rec;
  out->ws_hist_slices = ws_hist;
  return SAMPLER_OK;
}

void set_pointers(sampler_batch* out, const void* base) {
  const unsigned char* b = static_cast<const unsigned char*>(base);
  const size_t off_list = sizeof(RowParams) * (size_t)out->B;
  const size_t off_slots =
      off_list + list_bytes(out->B) +
      list_bytes(tasks_used(out->B, out->n_hold, (out->flags & SAMPLER_FLAG_SPLIT_PASS2) != 0));
  const size_t off_pen = off_slots + slots_bytes(out->B);
  out->d_rows = b;
  out->d_sampled = b + off_list;
  out->d_slots = b + off_slots;
  out->d_pen = b + off_pen;
  out->d_bias = b + off_pen + sizeof(PenEntry) * (size_t)out->n_pen;
  out->d_hist_raw = b + off_pen + sizeof(PenEntry) * (size_t)out->n_pen +
                    sizeof(BiasEntry) * (size_t)out->n_bias;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The workspace a packed batch needs (its rows' lists, records, histograms).
WorkspaceLayout batch_layout(const sampler_batch* b) {
  return workspace_layout(b->B, b->V, b->ws_hist_slices, b->ws_records, b->ws_list_entries);
}

}  // namespace

extern "C" {

const char* sampler_strerror(int code) {
  switch (code) {
    case SAMPLER_OK: return "ok";
    case SAMPLER_EINVAL: return "invalid argument or parameter value";
    case SAMPLER_ERANGE: return "size outside the supported range";
    case SAMPLER_ENOSPC: return "buffer or workspace too small";
    case SAMPLER_EUNSUPPORTED: return "unsupported request";
    case SAMPLER_EHIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

const char* sampler_version(void) { return "cd_sampler 0.1 (gfx950)"; }

size_t sampler_params_bytes(int32_t B, int64_t n_hist, int64_t n_bias) {
  if (B < 0 || n_hist < 0 || n_bias < 0) return 0;
  // a history id takes 8 bytes at most (a counted entry) and 4 at least
  return params_bytes_exact(B, tasks_max(B), n_hist, n_bias, 0) + 16;
}

int sampler_pack_host(const sampler_host_params* h, void* host_buf, size_t bytes,
                      sampler_batch* out) {
  if (!host_buf) return SAMPLER_ENOSPC;
  sampler_batch tmp;
  const int rc = pack_into(h, static_cast<unsigned char*>(host_buf), bytes, nullptr, &tmp);
  if (rc != SAMPLER_OK) return rc;
  set_pointers(&tmp, host_buf);
  *out = tmp;
  return SAMPLER_OK;
}

int sampler_pack_params(const sampler_host_params* h, void* d_buf, size_t d_bytes,
                        void* h_staging, void* stream, sampler_batch* out) {
  if (!d_buf) return SAMPLER_ENOSPC;
  std::vector<unsigned char> buf;
  sampler_batch tmp;
  // with a staging buffer (>= d_bytes) the block is packed straight into it
  const int rc = pack_into(h, static_cast<unsigned char*>(h_staging), d_bytes, &buf, &tmp);
  if (rc != SAMPLER_OK) return rc;
  if (d_bytes < tmp.bytes) return SAMPLER_ENOSPC;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (h_staging) {
    if (hipMemcpyAsync(d_buf, h_staging, tmp.bytes, hipMemcpyHostToDevice, s) != hipSuccess)
      return SAMPLER_EHIP;
  } else {
    if (hipMemcpyAsync(d_buf, buf.data(), buf.size(), hipMemcpyHostToDevice, s) != hipSuccess)
      return SAMPLER_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SAMPLER_EHIP;
  }
  set_pointers(&tmp, d_buf);
  *out = tmp;
  return SAMPLER_OK;
}

int sampler_apply_transforms(const sampler_batch* b, float* logits, int64_t ld, void* stream) {
  if (!b || !logits || ld < b->V || b->B <= 0) return SAMPLER_EINVAL;
  if (!aligned(logits, 4)) return SAMPLER_EINVAL;
  if (!(b->flags & (SAMPLER_FLAG_NEED_PENALTY | SAMPLER_FLAG_HAS_BIAS))) return SAMPLER_OK;
  const hipError_t e = launch_transforms(
      static_cast<const RowParams*>(b->d_rows), static_cast<const int32_t*>(b->d_hist_raw),
      static_cast<const PenEntry*>(b->d_pen),
      static_cast<const BiasEntry*>(b->d_bias), logits, ld, b->B,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
}

int sampler_apply_bitmask(void* logits, int dtype, int64_t ld, int32_t B, int32_t V,
                          const int32_t* bitmask, int64_t mask_ld, const uint8_t* row_has_mask,
                          void* stream) {
  if (!logits || !bitmask || B <= 0 || V <= 0 || ld < V) return SAMPLER_EINVAL;
  if (dtype != SAMPLER_DTYPE_F32 && dtype != SAMPLER_DTYPE_BF16) return SAMPLER_EINVAL;
  if (B > kMaxB || V > kMaxV) return SAMPLER_ERANGE;
  if (mask_ld < ((int64_t)V + 31) / 32) return SAMPLER_EINVAL;
  const hipError_t e = launch_bitmask(logits, dtype == SAMPLER_DTYPE_BF16, ld, B, V, bitmask,
                                      mask_ld, row_has_mask, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
}

size_t sampler_workspace_bytes(int32_t B, int32_t V) {
  if (B <= 0 || V <= 0 || B > kMaxB || V > kMaxV) return 0;
  return workspace_layout(B, V).total;
}

size_t sampler_workspace_bytes_batch(const sampler_batch* b) {
  if (!b || b->B <= 0 || b->V <= 0 || b->B > kMaxB || b->V > kMaxV) return 0;
  return batch_layout(b).total;
}

int sampler_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || ws_bytes % 4 != 0) return SAMPLER_EINVAL;
  const hipError_t e = launch_fill_zero(workspace, ws_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
}

int sampler_sample_ex(const sampler_batch* b, const void* logits, int dtype, int64_t ld,
                      const int32_t* bitmask, int64_t mask_ld, const uint8_t* row_has_mask,
                      int32_t* out_ids, float* out_logprobs, int32_t* out_status,
                      void* workspace, size_t ws_bytes, void* stream,
                      const sampler_options* opt) {
  sampler_options o;
  std::memset(&o, 0, sizeof o);
  if (opt) {
    if (opt->size != sizeof(sampler_options)) return SAMPLER_EINVAL;
    o = *opt;
  }
  if (o.algo != SAMPLER_ALGO_FAST && o.algo != SAMPLER_ALGO_EXACT) return SAMPLER_EINVAL;
  if (o.wait_ns < 0 && o.wait_ns != SAMPLER_WAIT_NONE) return SAMPLER_EINVAL;
  if (!b || !logits || !out_ids || !b->d_rows) return SAMPLER_EINVAL;
  const int32_t B = b->B, V = b->V;
  if (B <= 0 || V <= 0 || ld < V) return SAMPLER_EINVAL;
  if (B > kMaxB || V > kMaxV) return SAMPLER_ERANGE;
  if (dtype != SAMPLER_DTYPE_F32 && dtype != SAMPLER_DTYPE_BF16) return SAMPLER_EINVAL;
  const bool bf16 = dtype == SAMPLER_DTYPE_BF16;
  if (!aligned(logits, bf16 ? 2 : 4)) return SAMPLER_EINVAL;
  if (bitmask && mask_ld < ((int64_t)V + 31) / 32) return SAMPLER_EINVAL;
  if (!b->d_slots) return SAMPLER_EINVAL;
  const WorkspaceLayout L = batch_layout(b);
  if (!workspace || ws_bytes < L.total) return SAMPLER_ENOSPC;
  if (!aligned(workspace, 256)) return SAMPLER_EINVAL;

  unsigned char* ws = static_cast<unsigned char*>(workspace);
  SampleArgs a;
  if (b->n_sampled < 0 || b->n_sampled > B || !b->d_sampled) return SAMPLER_EINVAL;
  a.rows = static_cast<const RowParams*>(b->d_rows);
  a.slots = static_cast<const RowSlots*>(b->d_slots);
  if (b->n_hold < 0 || b->n_hold > b->n_sampled) return SAMPLER_EINVAL;
  {
    const unsigned char* t = static_cast<const unsigned char*>(b->d_sampled) + list_bytes(B);
    a.task_row = reinterpret_cast<const int32_t*>(t);
    a.n_groups = (B + 7) / 8 + ((b->flags & SAMPLER_FLAG_SPLIT_PASS2) ? 2 : 1) * ((b->n_hold + 7) / 8);
  }
  a.logits = logits;
  a.ld = ld;
  a.B = B;
  a.V = V;
  a.mask = bitmask;
  a.mask_ld = mask_ld;
  a.row_has_mask = row_has_mask;
  a.out_ids = out_ids;
  a.out_lp = out_logprobs;
  a.out_st = out_status;
  a.out_cut = static_cast<float*>(o.cut);
  a.sync = reinterpret_cast<RowSync*>(ws + L.sync_off);
  a.plans = reinterpret_cast<Plan*>(ws + L.plan_off);
  a.heads = reinterpret_cast<SliceHead*>(ws + L.head_off);
  a.hist = reinterpret_cast<unsigned long long*>(ws + L.hist_off);
  a.bests = reinterpret_cast<SliceBest*>(ws + L.best_off);
  a.ulist = reinterpret_cast<uint64_t*>(ws + L.ulist_off);
  a.P = L.P;
  a.S = L.S;

  // 16-byte vector loads need every row start (and the base) 16-byte aligned
  const size_t elem = bf16 ? 2 : 4;
  const bool vec = aligned(logits, 4 * elem) && (ld % 4 == 0) && (V % 4 == 0);
  int algo = o.algo;
  if (L.S > kSliceMax) algo = SAMPLER_ALGO_EXACT;  // slices beyond the register-resident size

  // A slice waits at most wait_ns (default 5 ms) of wall clock for its row's
  // plan, then the row takes the exact path; 0 ticks = no wait at all.
  const int64_t wait_ns = o.wait_ns == 0 ? 5000000 : (o.wait_ns < 0 ? 0 : o.wait_ns);
  a.spin_limit = wait_ns == 0 ? 0u
                              : std::max<uint64_t>(1u, (uint64_t)wait_ns * (uint64_t)wall_clock_khz() /
                                                           1000000u);
  // Generation of this call: the plan-ready and wait-failed flags hold the
  // generation that set them, so a flag left by an earlier call never reads
  // as set.  Never 0 (a zeroed workspace).  (The arrival / done tickets are
  // plain counters that the last slice of each row resets: a workspace must
  // be zero before its first call, sampler_workspace_init.)
  uint32_t gen = g_gen.fetch_add(1u) + 1u;
  if (gen == 0u) gen = g_gen.fetch_add(1u) + 1u;
  a.gen = gen;
  a.trace = static_cast<unsigned long long*>(o.trace);

  KernelEvents ev;
  ev.start = static_cast<hipEvent_t>(o.start_event);
  ev.stop = static_cast<hipEvent_t>(o.stop_event);
  const bool have_ev = ev.start || ev.stop;
  const hipError_t e = launch_sample(a, bf16, vec, algo, have_ev ? &ev : nullptr,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
}

int sampler_sample_static(const sampler_batch* b, const void* logits, int dtype, int64_t ld,
                          const int32_t* bitmask, int64_t mask_ld, const uint8_t* row_has_mask,
                          int32_t* out_ids, float* out_logprobs, int32_t* out_status,
                          void* stream) {
  if (!b || b->B <= 0 || b->V <= 0 || b->B > kMaxB || b->V > kMaxV) return SAMPLER_EINVAL;
  if (batch_layout(b).total > kStaticWorkspaceBytes) return SAMPLER_ENOSPC;
  void* ws = nullptr;
  if (static_workspace(&ws, static_cast<hipStream_t>(stream)) != hipSuccess) return SAMPLER_EHIP;
  return sampler_sample_ex(b, logits, dtype, ld, bitmask, mask_ld, row_has_mask, out_ids,
                           out_logprobs, out_status, ws, kStaticWorkspaceBytes, stream, nullptr);
}

int sampler_sample(const sampler_batch* b, const void* logits, int dtype, int64_t ld,
                   const int32_t* bitmask, int64_t mask_ld, const uint8_t* row_has_mask,
                   int32_t* out_ids, float* out_logprobs, int32_t* out_status, void* workspace,
                   size_t ws_bytes, void* stream) {
  return sampler_sample_ex(b, logits, dtype, ld, bitmask, mask_ld, row_has_mask, out_ids,
                           out_logprobs, out_status, workspace, ws_bytes, stream, nullptr);
}

namespace {
// sampler_logprobs workspace: the row slice records and keys, then (16-byte
// aligned) the support slice records
size_t logprobs_rows_bytes(int32_t B, int32_t V, int32_t top_n_max) {
  const size_t Q = ((size_t)V + kOutSlice - 1) / kOutSlice;
  const size_t n = (size_t)B * Q * (sizeof(OutSliceStat) + sizeof(uint64_t) * (size_t)top_n_max);
  return (n + 15) / 16 * 16;
}
int32_t support_slices(int32_t V) { return (int32_t)(((int64_t)V + kSupSlice - 1) / kSupSlice); }
}  // namespace

size_t sampler_logprobs_workspace_bytes(int32_t B, int32_t V, int32_t top_n_max,
                                        int32_t n_mask_rows) {
  if (B <= 0 || V <= 0 || B > kMaxB || V > kMaxV || top_n_max < 0 ||
      top_n_max > SAMPLER_MAX_TOP_N || n_mask_rows < 0 ||
      (int64_t)n_mask_rows * support_slices(V) > (int64_t)INT32_MAX)
    return 0;
  return logprobs_rows_bytes(B, V, top_n_max) +
         (size_t)n_mask_rows * (size_t)support_slices(V) * sizeof(SupSliceStat);
}

int sampler_logprobs(const sampler_batch* b, const void* logits, int dtype, int64_t ld,
                     const int32_t* bitmask, int64_t mask_ld, const uint8_t* row_has_mask,
                     const sampler_logprob_request* req, const sampler_logprob_outputs* out,
                     void* stream) {
  if (!req || !out || req->size != sizeof(sampler_logprob_request) ||
      out->size != sizeof(sampler_logprob_outputs))
    return SAMPLER_EINVAL;
  if (!b || !logits || !b->d_rows) return SAMPLER_EINVAL;
  const int32_t B = b->B, V = b->V;
  if (B <= 0 || V <= 0 || ld < V) return SAMPLER_EINVAL;
  if (B > kMaxB || V > kMaxV) return SAMPLER_ERANGE;
  if (dtype != SAMPLER_DTYPE_F32 && dtype != SAMPLER_DTYPE_BF16) return SAMPLER_EINVAL;
  const bool bf16 = dtype == SAMPLER_DTYPE_BF16;
  if (!aligned(logits, bf16 ? 2 : 4)) return SAMPLER_EINVAL;
  if (bitmask && mask_ld < ((int64_t)V + 31) / 32) return SAMPLER_EINVAL;
  if (req->basis != SAMPLER_LOGPROB_SAMPLED && req->basis != SAMPLER_LOGPROB_ORIGINAL)
    return SAMPLER_EINVAL;
  if (req->top_n_max < 0 || req->top_n_max > SAMPLER_MAX_TOP_N) return SAMPLER_EINVAL;
  // each output needs its input, each input its output
  if (out->next_token_logprobs && !req->selected) return SAMPLER_EINVAL;
  const bool top = req->top_n_max > 0;
  if (top != (out->top_logprobs_idx != nullptr) || top != (out->top_logprobs_val != nullptr))
    return SAMPLER_EINVAL;
  if (req->top_n && !top) return SAMPLER_EINVAL;
  const bool named = req->token_indptr != nullptr;
  if (named != (req->token_ids != nullptr) || named != (out->token_ids_logprobs != nullptr))
    return SAMPLER_EINVAL;
  if (req->n_mask_rows < 0 || req->mask_cap < 0) return SAMPLER_EINVAL;
  const bool mask = req->n_mask_rows > 0;
  if (mask && (!req->mask_rows || !out->mask_lengths || !out->mask_statuses ||
               (req->mask_cap > 0 && !out->mask_token_ids)))
    return SAMPLER_EINVAL;
  if (!mask && (out->mask_token_ids || out->mask_support_logprobs || out->mask_lengths ||
                out->mask_selected_logprobs || out->mask_statuses))
    return SAMPLER_EINVAL;
  if (out->mask_support_logprobs && !out->mask_token_ids) return SAMPLER_EINVAL;
  if ((int64_t)req->n_mask_rows * (int64_t)req->mask_cap > ((int64_t)1 << 40)) return SAMPLER_ERANGE;

  SampleArgs a;
  std::memset(&a, 0, sizeof a);
  a.rows = static_cast<const RowParams*>(b->d_rows);
  a.logits = logits;
  a.ld = ld;
  a.B = B;
  a.V = V;
  a.mask = bitmask;
  a.mask_ld = mask_ld;
  a.row_has_mask = row_has_mask;

  OutputArgs o;
  std::memset(&o, 0, sizeof o);
  o.basis = req->basis;
  o.top_n_max = req->top_n_max;
  o.top_n = req->top_n;
  o.tok_off = req->token_indptr;
  o.tok_ids = req->token_ids;
  o.sel_ids = req->selected;
  o.cuts = req->cuts;
  o.sup_rows = mask ? req->mask_rows : nullptr;
  o.n_sup = mask ? req->n_mask_rows : 0;
  o.sup_cap = req->mask_cap;
  o.next_lp = out->next_token_logprobs;
  o.top_ids = out->top_logprobs_idx;
  o.top_vals = out->top_logprobs_val;
  o.tok_vals = out->token_ids_logprobs;
  o.sup_ids = out->mask_token_ids;
  o.sup_lp = out->mask_support_logprobs;
  o.sup_len = out->mask_lengths;
  o.sup_sel = out->mask_selected_logprobs;
  o.sup_st = out->mask_statuses;
  o.n_row_blocks = (top || named || o.next_lp) ? B : 0;
  if (o.n_row_blocks == 0 && o.n_sup == 0) return SAMPLER_OK;
  if (req->workspace) {
    const size_t need =
        sampler_logprobs_workspace_bytes(B, V, req->top_n_max, mask ? req->n_mask_rows : 0);
    if (need == 0) return SAMPLER_ERANGE;
    if (req->workspace_bytes < need) return SAMPLER_ENOSPC;
    if (!aligned(req->workspace, 16)) return SAMPLER_EINVAL;
    o.n_slices = (int32_t)(((int64_t)V + kOutSlice - 1) / kOutSlice);
    o.sl_stat = static_cast<OutSliceStat*>(req->workspace);
    o.sl_keys = reinterpret_cast<unsigned long long*>(o.sl_stat + (size_t)B * o.n_slices);
    if (mask && req->cuts) {  // support sets by slices need the thresholds
      o.n_sup_slices = support_slices(V);
      o.sup_stat = reinterpret_cast<SupSliceStat*>(static_cast<unsigned char*>(req->workspace) +
                                                   logprobs_rows_bytes(B, V, req->top_n_max));
    }
  }

  const size_t elem = bf16 ? 2 : 4;
  const bool vec = aligned(logits, 4 * elem) && (ld % 4 == 0) && (V % 4 == 0);
  const hipError_t e = launch_outputs(a, o, bf16, vec, nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
}

size_t sampler_shard_state_bytes(int32_t B) {
  if (B <= 0 || B > kMaxB) return 0;
  return sizeof(ShardState) * (size_t)B;
}

int32_t sampler_shard_records(int32_t width) {
  if (width <= 0) return 0;
  return (int32_t)(((int64_t)width + kShardSub - 1) / kShardSub);
}

size_t sampler_shard_partial_bytes(int32_t B, int32_t width) {
  if (B <= 0 || B > kMaxB || width <= 0) return 0;
  return sizeof(ShardPartial) * (size_t)B * (size_t)sampler_shard_records(width);
}

uint32_t sampler_shard_phases(const sampler_batch* b) {
  if (!b || b->B <= 0) return 0u;
  uint32_t ph = 1u << SHARD_STATS;
  if (b->flags & SAMPLER_FLAG_NEED_TOP_K)
    for (int i = 0; i < 4; ++i) ph |= 1u << (SHARD_TOPK0 + i);
  if (b->flags & SAMPLER_FLAG_NEED_TOP_P) {
    ph |= 1u << SHARD_TOPP_SUMS;
    for (int i = 0; i < 4; ++i) ph |= 1u << (SHARD_TOPP0 + i);
  }
  if (b->n_sampled > 0) ph |= 1u << SHARD_RACE;
  return ph;
}

int sampler_shard_pass(const sampler_batch* b, int32_t phase, const void* logits, int dtype,
                       int64_t ld, int32_t v0, int32_t width, const int32_t* bitmask,
                       int64_t mask_ld, const uint8_t* row_has_mask, const void* state,
                       void* partial, void* stream) {
  if (!b || !logits || !b->d_rows || !partial) return SAMPLER_EINVAL;
  const int32_t B = b->B, V = b->V;
  if (B <= 0 || V <= 0) return SAMPLER_EINVAL;
  if (B > kMaxB || V > kMaxV) return SAMPLER_ERANGE;
  if (phase < 0 || phase >= SHARD_PHASES) return SAMPLER_EINVAL;
  if (phase > SHARD_STATS && !state) return SAMPLER_EINVAL;
  if (v0 < 0 || v0 % 4 != 0 || width <= 0 || (int64_t)v0 + width > V || ld < width)
    return SAMPLER_EINVAL;
  if (dtype != SAMPLER_DTYPE_F32 && dtype != SAMPLER_DTYPE_BF16) return SAMPLER_EINVAL;
  const bool bf16 = dtype == SAMPLER_DTYPE_BF16;
  if (!aligned(logits, bf16 ? 2 : 4)) return SAMPLER_EINVAL;
  if (bitmask && mask_ld < ((int64_t)width + 31) / 32) return SAMPLER_EINVAL;
  if (!aligned(partial, 16) || (state && !aligned(state, 16))) return SAMPLER_EINVAL;
  ShardArgs a;
  std::memset(&a, 0, sizeof a);
  a.rows = static_cast<const RowParams*>(b->d_rows);
  a.logits = logits;
  a.ld = ld;
  a.B = B;
  a.V = V;
  a.v0 = v0;
  a.width = width;
  a.mask = bitmask;
  a.mask_ld = mask_ld;
  a.row_has_mask = row_has_mask;
  a.state = static_cast<ShardState*>(const_cast<void*>(state));
  a.part = static_cast<ShardPartial*>(partial);
  a.n_parts = 1;
  a.phase = phase;
  const size_t elem = bf16 ? 2 : 4;
  const bool vec = aligned(logits, 4 * elem) && (ld % 4 == 0) && (width % 4 == 0);
  const hipError_t e = launch_shard_pass(a, bf16, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
}

int sampler_shard_merge(const sampler_batch* b, int32_t phase, void* state, const void* partials,
                        int32_t n_records, int32_t* out_ids, float* out_logprobs,
                        int32_t* out_status, void* stream) {
  if (!b || !b->d_rows || !state || !partials || !out_ids) return SAMPLER_EINVAL;
  const int32_t B = b->B, V = b->V;
  if (B <= 0 || V <= 0) return SAMPLER_EINVAL;
  if (B > kMaxB || V > kMaxV) return SAMPLER_ERANGE;
  if (phase < 0 || phase >= SHARD_PHASES) return SAMPLER_EINVAL;
  if (n_records < 1 || n_records > V / 4 + 1) return SAMPLER_EINVAL;
  if (!aligned(state, 16) || !aligned(partials, 16)) return SAMPLER_EINVAL;
  ShardArgs a;
  std::memset(&a, 0, sizeof a);
  a.rows = static_cast<const RowParams*>(b->d_rows);
  a.B = B;
  a.V = V;
  a.state = static_cast<ShardState*>(state);
  a.part = static_cast<ShardPartial*>(const_cast<void*>(partials));
  a.n_parts = n_records;
  a.phase = phase;
  a.out_ids = out_ids;
  a.out_lp = out_logprobs;
  a.out_st = out_status;
  const hipError_t e = launch_shard_merge(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
}

int sampler_spec_accept(int32_t n_req, int32_t k, const int32_t* sampled, const int32_t* status,
                        const int32_t* draft, const int32_t* eos, int32_t* tokens, int32_t* count,
                        int32_t* rollback, void* stream) {
  if (n_req < 0 || k < 0 || n_req > kMaxB) return SAMPLER_EINVAL;
  if (n_req == 0) return SAMPLER_OK;
  if (!sampled || !tokens || !count || (k > 0 && !draft)) return SAMPLER_EINVAL;
  if ((int64_t)n_req * (k + 1) > kMaxB) return SAMPLER_ERANGE;
  SpecArgs a;
  a.n_req = n_req;
  a.k = k;
  a.sampled = sampled;
  a.status = status;
  a.draft = draft;
  a.eos = eos;
  a.tokens = tokens;
  a.count = count;
  a.rollback = rollback;
  const hipError_t e = launch_spec_accept(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SAMPLER_OK : SAMPLER_EHIP;
}

}  // extern "C"
