// kernels.hip -- HIP kernels of libcd_sampler.so for gfx950 (MI355X).
//
// The sampling step is one kernel, sample_kernel: one workgroup per slice of a
// row (P slices of at most kMaxChunks * 4 * kScanThreads tokens).  Each slice
// streams its tokens from HBM once into registers (bf16 upcast and the grammar
// bitmask fused into the load), summarises them, does the work its row's
// class asks for (see slice_task), and publishes the result; the last slice of
// a row to arrive resolves the row.  Only rows whose cut needs the whole row's
// histogram (top-p as the only cut, large top-k) make their slices wait for a
// row plan, with their tokens still in registers.
//
// The row-serial exact path (row_exact) does everything with one workgroup
// and several passes over the row: radix select for the k-th largest value,
// a mass-weighted radix select for the top-p cut (fixed-point masses), then
// the race.  It is the fallback of rows the fast path cannot hold on chip, and
// selectable for all rows (SAMPLER_OPT_ALGO = 1).
//
// Definitions followed (sources cited by page title and section):
//  - transforms: "SGLang 源码完全拆解(十)", section 惩罚项的顺序语义 (additive
//    penalties, then repetition scaling, then the mask, then the bias);
//  - bitmask: same page, section 位掩码 (bit 0 -> -inf; -1 = all allowed);
//  - min-p / top-k / top-p sets: same page, section 概率裁剪的数学;
//  - order temperature -> min-p -> top-k/top-p, greedy below T = 1e-5 on the
//    logits before the temperature: "GLM-5.3 推理全链路(七)", section 采样;
//  - logprob = log_softmax of the scaled logits before truncation: SGLang
//    page, section logprobs 的数值一致性; greedy rows use T = 1 (section
//    贪心路径).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <mutex>

#include "device_common.h"
#include "exact_path.h"
#include "kernels.h"

namespace cds {

__device__ __forceinline__ void write_out(const SampleArgs& a, int r, int32_t id, float lp,
                                          int32_t st) {
  a.out_ids[r] = id;
  if (a.out_lp) a.out_lp[r] = lp;
  if (a.out_st) a.out_st[r] = st;
}


// ============================================================================
// transforms and bitmask (in place)
// ============================================================================
// One workgroup per row.  Raw history rows (ROW_PEN_RAW, at most kHistDevice
// int32 ids) are first merged into (token, count) pairs in an LDS hash table with
// at least twice as many slots as tokens (linear probing, atomicCAS on the
// key), so every penalised token is updated exactly once with its full count.
__device__ __forceinline__ void apply_penalty(float* z, int32_t id, int32_t count,
                                              const RowParams& rp) {
  float v = z[id];
  const float p = __fadd_rn(__fmul_rn(rp.freq, (float)count), rp.pres);
  v = __fsub_rn(v, p);
  if (rp.rep != 1.0f) v = (v > 0.0f) ? __fdiv_rn(v, rp.rep) : __fmul_rn(v, rp.rep);
  z[id] = v;
}

__global__ __launch_bounds__(256) void transforms_kernel(const RowParams* rows,
                                                         const int32_t* hist_raw,
                                                         const PenEntry* pen,
                                                         const BiasEntry* bias, float* logits,
                                                         int64_t ld) {
  constexpr uint32_t kEmpty = 0xFFFFFFFFu;
  __shared__ uint32_t keys[2 * kHistDevice];
  __shared__ int32_t cnts[2 * kHistDevice];
  const int r = blockIdx.x;
  const RowParams rp = rows[r];
  float* z = logits + (int64_t)r * ld;
  if ((rp.flags & ROW_PEN) && (rp.flags & ROW_PEN_RAW)) {
    const int n = rp.pen_hi - rp.pen_lo;
    int lg = 6;
    while ((1 << lg) < 2 * n) ++lg;  // <= log2(2 * kHistDevice)
    const uint32_t ht = 1u << lg;
    for (uint32_t k = threadIdx.x; k < ht; k += blockDim.x) {
      keys[k] = kEmpty;
      cnts[k] = 0;
    }
    __syncthreads();
    for (int i = rp.pen_lo + (int)threadIdx.x; i < rp.pen_hi; i += blockDim.x) {
      const uint32_t id = (uint32_t)hist_raw[i];
      uint32_t h = (id * 0x9E3779B1u) >> (32 - lg);
      while (true) {
        const uint32_t old = atomicCAS(&keys[h], kEmpty, id);
        if (old == kEmpty || old == id) {
          atomicAdd(&cnts[h], 1);
          break;
        }
        h = (h + 1u) & (ht - 1u);
      }
    }
    __syncthreads();
    for (uint32_t k = threadIdx.x; k < ht; k += blockDim.x)
      if (keys[k] != kEmpty) apply_penalty(z, (int32_t)keys[k], cnts[k], rp);
  } else if (rp.flags & ROW_PEN) {
    for (int i = rp.pen_lo + (int)threadIdx.x; i < rp.pen_hi; i += blockDim.x)
      apply_penalty(z, pen[i].id, pen[i].count, rp);
  }
  __syncthreads();  // a token may carry both a penalty and a bias
  if (rp.flags & ROW_BIAS) {
    for (int i = rp.bias_lo + (int)threadIdx.x; i < rp.bias_hi; i += blockDim.x) {
      const BiasEntry e = bias[i];
      z[e.id] = __fadd_rn(z[e.id], e.val);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void bitmask_kernel(void* logits, int64_t ld, int32_t V,
                                                      const int32_t* mask, int64_t mask_ld,
                                                      const uint8_t* row_has_mask) {
  const int r = blockIdx.y;
  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t W = ((int64_t)V + 31) / 32;
  if (w >= W) return;
  if (row_has_mask && !row_has_mask[r]) return;
  const uint32_t bits = (uint32_t)mask[(int64_t)r * mask_ld + w];
  if (bits == 0xFFFFFFFFu) return;
  for (int q = 0; q < 32; ++q) {
    const int64_t t = w * 32 + q;
    if (t >= V) break;
    if (!((bits >> q) & 1u)) {
      if (BF16)
        static_cast<uint16_t*>(logits)[(int64_t)r * ld + t] = 0xFF80u;  // bf16 -inf
      else
        static_cast<float*>(logits)[(int64_t)r * ld + t] = CDS_NEG_INF;
    }
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ============================================================================
// row-serial exact path: one workgroup, several passes over the row
// ============================================================================
template <int NT, bool BF16, bool VEC>
__device__ __forceinline__ void row_exact(const SampleArgs& a, int r, ExactShared<NT>& sh) {
  const RowParams rp = a.rows[r];
  const RowView rv = row_view<BF16>(a, r);
  const int64_t V = a.V;
  const bool greedy = (rp.flags & ROW_GREEDY) != 0;
  const RowStats st = row_stats<NT, BF16, VEC>(rv, V, sh);
  if (st.nf == 0) {
    if (threadIdx.x == 0) write_out(a, r, -1, CDS_NEG_INF, 2);
    return;
  }
  if (st.nonfin) {
    if (threadIdx.x == 0) write_out(a, r, -1, __builtin_nanf(""), 1);
    return;
  }
  const float zm = st.zm;
  const double se =
      row_expsum<NT, BF16, VEC>(rv, V, zm, (float)(greedy ? 1.0 : 1.0 / (double)rp.temperature), sh);
  if (greedy) {
    if (threadIdx.x == 0) write_out(a, r, st.am, (float)(-log(se)), 0);
    return;
  }
  const double Td = (double)rp.temperature;
  const double m = (double)zm / Td;
  const double log_z = log(se);
  const float zcut = row_cut<NT, BF16, VEC>(rv, V, rp, zm, st.nf, sh);

  // the race over {z >= zcut}
  uint32_t nonfin = 0;
  const RaceCtx c = make_race_ctx(rp, zm);
  Best b = best_init();
  const float zf = zcut;
  for_row4<NT, BF16, VEC>(rv, V, nonfin, [&](const float* x, int64_t t0) {
    bool need = false;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      need |= (x[q] != CDS_NEG_INF && x[q] >= zf && race_hopeful(b, x[q], c));
    if (!need) return;
    const uint4 blk = race_block(c, t0);
    const uint32_t xs[4] = {blk.x, blk.y, blk.z, blk.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (x[q] != CDS_NEG_INF && x[q] >= zf) race_consider(b, x[q], (int32_t)(t0 + q), xs[q], c);
  });
  block_best<NT>(b, sh.red);
  if (threadIdx.x == 0) {
    write_out(a, r, b.t, (float)((double)b.z / Td - m - log_z), 0);
    if (a.out_cut) a.out_cut[r] = zcut;
  }
}

template <int NT, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void exact_kernel(const SampleArgs a) {
  __shared__ ExactShared<NT> es;
  row_exact<NT, BF16, VEC>(a, blockIdx.x, es);
}

// ============================================================================
// fast path: one kernel, one workgroup per slice (see slice_task)
// ============================================================================

// ---- cross-workgroup data and counters ----------------------------------------
// Everything one workgroup hands to another goes through agent-coherent
// accesses (relaxed agent-scope atomic loads and stores: "sc1" on gfx950),
// never through plain stores that could sit in one XCD's L2.  A producer
// waits for its own stores to complete (vm_drain) before the ticket or flag
// that publishes them, and a consumer issues its loads only after it has seen
// that ticket or flag.  This avoids agent-scope release / acquire fences,
// which write back or invalidate a whole L2 each time.
__device__ __forceinline__ void st_u32(void* p, uint32_t v) {
  __hip_atomic_store(static_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u64(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const void* p) {
  return __hip_atomic_load(static_cast<const uint32_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_u64(const void* p) {
  return __hip_atomic_load(static_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_obj(T* dst, const T& v) {
  static_assert(sizeof(T) % 8 == 0, "8-byte words");
  uint64_t w[sizeof(T) / 8];
  __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 8); ++k) st_u64(reinterpret_cast<uint64_t*>(dst) + k, w[k]);
}
template <typename T>
__device__ __forceinline__ T ld_obj(const T* src) {
  static_assert(sizeof(T) % 8 == 0, "8-byte words");
  uint64_t w[sizeof(T) / 8];
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 8); ++k) w[k] = ld_u64(reinterpret_cast<const uint64_t*>(src) + k);
  T v;
  __builtin_memcpy(&v, w, sizeof(T));
  return v;
}
// Wait until this wave's memory operations have completed.
__device__ __forceinline__ void vm_drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Row ticket: every slice of the row adds 1 once per call and gets the count
// before its addition; the slice that gets P-1 is the last and resets the
// counter to zero for the next call (no slice of this call touches it again).
__device__ __forceinline__ uint32_t take_ticket(unsigned long long* w) {
  return (uint32_t)__hip_atomic_fetch_add(w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin until *p == gen, at most `limit` ticks of the constant-rate wall
// clock; false on timeout, and at once when limit is 0.
__device__ __forceinline__ bool gen_wait(const uint32_t* p, uint32_t gen, uint64_t limit) {
  if (limit == 0) return false;  // the caller asked for no wait at all
  const uint64_t t0 = wall_clock64();
  while (ld_u32(p) != gen) {
    if (wall_clock64() - t0 > limit) return false;
    __builtin_amdgcn_s_sleep(4);
  }
  return true;
}

// A value every lane of the wave holds, moved to a scalar register.
__device__ __forceinline__ float sgpr_f(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// ---- phase 2: the plan ----------------------------------------------------------
template <int NT>
struct PlanShared {
  SliceHead head[kMaxSlices];
  int32_t shift[kMaxSlices];        // row bin of slice j's bin 0 (-1: nothing allowed)
  double md[NBINS];                 // cumulative mass from the top, relative to exp(m)
  uint32_t cumc[NBINS];             // cumulative count from the top
  unsigned long long bm[NT];        // one block of NT merged row bins: fixed-point masses
  uint32_t bc[NT];                  //   and counts
  double wtot_d[NT / 64];
  uint32_t wtot_u[NT / 64];
  int mode, inK, k_rank, rb12;
  float zmax, zcut1;
  int32_t arg;
  double m, log_z, tlo, thi;
};

// Per-row phase marks (wall clock) in a.trace after the workgroup words.
#ifdef CDS_TRACE_DETAIL
#define CDS_TRACE_ROW(k)                                                                        \
  do {                                                                                          \
    if (a.trace && threadIdx.x == 0)                                                            \
      a.trace[(size_t)gridDim.x * 8 + (size_t)r * 8 + (k)] = wall_clock64();                   \
  } while (0)
#else
#define CDS_TRACE_ROW(k) do {} while (0)
#endif
// Per-workgroup sub-phase marks after the per-row marks (detail traces only).
#ifdef CDS_TRACE_DETAIL
#define CDS_TRACE_SUB(k)                                                                        \
  do {                                                                                          \
    if (a.trace && threadIdx.x == 0)                                                            \
      a.trace[(size_t)gridDim.x * 8 + (size_t)a.B * 8 + (size_t)blockIdx.x * 8 + (k)] =         \
          wall_clock64();                                                                       \
  } while (0)
#else
#define CDS_TRACE_SUB(k) do {} while (0)
#endif

// Merge the slice summaries of row r into its plan (all NT threads).  Writes
// the output of rows that end here (greedy, no finite token, non-finite
// token) and the plan to a.plans[r] and to *out (LDS).
//
// HOLD rows (hist): the row's histogram is merged from the slices' in blocks
// of NT bins from the top (row frame: bin b spans [(kmax-b)*delta,
// (kmax-b+1)*delta), kmax the row maximum's bin), with integer LDS atomics
// (exact in any order), and scanned; further blocks are merged only while
// the cuts lie below the part scanned so far.  Block 0 is loaded together
// with the slice heads: bins 0 .. NT-1 of every slice's own frame cover the
// row's top NT bins whatever the slice's offset.  The row's total mass comes
// from the slices' totals (heads), so the scan can stop at the cut.
template <int NT>
__device__ __forceinline__ void plan_row(const SampleArgs& a, int r, bool hist, PlanShared<NT>& ps,
                                         Plan* out) {
  const int tid = threadIdx.x, P = a.P;
  const RowParams rp = a.rows[r];
  const bool greedy = (rp.flags & ROW_GREEDY) != 0;
  const bool topk = (rp.flags & ROW_TOPK) != 0, topp = (rp.flags & ROW_TOPP) != 0;
  const double Td = (double)rp.temperature;
  constexpr int JC = 10;  // slices per round of histogram loads
  const unsigned long long* gh =
      a.hist + (int64_t)(a.slots[r].rec / (2u * (uint32_t)P)) * P * NBINS;
  unsigned long long hv[JC];
  // slice j's bins that land in row block blk (its bins 0 .. NT-1 for block 0)
  auto load_block = [&](int j0, int blk) {
#pragma unroll
    for (int jj = 0; jj < JC; ++jj) {
      const int j = j0 + jj;
      const int sb = blk == 0 ? tid : blk * NT - (j < P ? ps.shift[j] : 0) + tid;
      const bool ok = j < P && (blk == 0 || ps.shift[j] >= 0) && sb >= 0 && sb < NBINS;
      hv[jj] = ok ? ld_u64(gh + (int64_t)j * NBINS + sb) : 0ull;
    }
  };
  if (hist) load_block(0, 0);
  // merge the slice heads: wave 0, lane j holds slice j (P <= 64)
  if (tid < 64) {
    float zm = CDS_NEG_INF;
    int32_t am = INT_MAX;
    uint32_t fl = 0;
    double hs = 0.0;
    float hk = 0.0f;
    if (tid < P) {
      const SliceHead h = ld_obj(&a.heads[(int64_t)r * P + tid]);
      ps.head[tid] = h;
      zm = h.zmax;
      am = h.zmax == CDS_NEG_INF ? INT_MAX : h.arg;
      fl = h.flags;
      hs = h.sumexp;
      hk = h.kmax;
    }
    const float hz = zm;
    struct ZAF {
      float z;
      int32_t a;
      uint32_t f;
    };
    const ZAF hm = wave_allreduce(ZAF{zm, am, fl}, [](const ZAF& p, const ZAF& q) {
      ZAF o = (q.z > p.z || (q.z == p.z && q.a < p.a)) ? q : p;
      o.f = p.f | q.f;
      return o;
    });
    zm = hm.z;
    am = hm.a;
    fl = hm.f;
    // slice masses relative to the slice maxima, moved to the row maximum and
    // summed in a fixed order (deterministic): token sums, or for HOLD rows
    // the slices' histogram totals
    const double invTe = greedy ? 1.0 : 1.0 / Td;
    double Z = (hz != CDS_NEG_INF) ? hs * exp(((double)hz - (double)zm) * invTe) : 0.0;
    Z = wave_allreduce(Z, [](double x, double y) { return x + y; });
    if (hist && tid < P) {
      // row bin of the slice's bin 0 (both maxima's bins are exact integers)
      const float kmax_row = floorf(zm * bin_geom(rp.temperature).inv_delta);
      ps.shift[tid] = hz == CDS_NEG_INF ? -1 : (int32_t)(kmax_row - hk);
    }
    if (tid == 0) {
      int mode = PLAN_FAST;
      if (zm == CDS_NEG_INF) {
        write_out(a, r, -1, CDS_NEG_INF, 2);
        mode = PLAN_DONE;
      } else if (fl & SLICE_NONFINITE) {
        write_out(a, r, -1, __builtin_nanf(""), 1);
        mode = PLAN_DONE;
      } else if (greedy) {
        write_out(a, r, am, (float)(-log(Z)), 0);
        mode = PLAN_DONE;
      } else if (fl & SLICE_BINS_LOST) {
        mode = PLAN_SLOW;
      } else if (hist && (rp.flags & kRowOrderBits)) {
        mode = PLAN_SLOW;  // a large top-k with top-p in another filter order
      }
      ps.mode = mode;
      ps.zmax = zm;
      ps.arg = am;
      ps.m = (double)zm / Td;
      ps.log_z = log(Z);
    }
  }
  __syncthreads();
  // min-p: the smallest fp32 value whose weight reaches min_p (wave 0)
  if (tid < 64) {
    float zc = CDS_NEG_INF;
    if (ps.mode == PLAN_FAST && (rp.flags & ROW_MINP)) {
      const double m = ps.m, mp = (double)rp.min_p;
      auto pred = [&](uint32_t k) { return exp((double)from_okey(k) / Td - m) >= mp; };
      if (!pred(okey(-FLT_MAX))) zc = from_okey(wave_first_true(okey(-FLT_MAX), okey(ps.zmax), pred));
    }
    if (tid == 0) ps.zcut1 = zc;
  }
  __syncthreads();

  auto base_plan = [&](int mode) {
    Plan pl = {};
    pl.mode = mode;
    pl.arg = ps.arg;
    pl.zmax = ps.zmax;
    pl.zcut1 = ps.zcut1;
    pl.m = ps.m;
    pl.log_z = ps.log_z;
    pl.z_sure = CDS_NEG_INF;
    pl.a_lo = pl.a_hi = pl.k_lo = pl.k_hi = CDS_POS_INF;
    pl.p = (double)rp.top_p;
    return pl;
  };
  if (ps.mode != PLAN_FAST || !hist) {
    if (tid == 0) {
      const Plan pl = base_plan(ps.mode);
      st_obj(&a.plans[r], pl);
      *out = pl;
    }
    return;
  }

  CDS_TRACE_ROW(5);
  const BinGeom g = bin_geom(rp.temperature);
  const float kmax = floorf(ps.zmax * g.inv_delta);
  const double m = ps.m, mtot = exp(ps.log_z);
  // the scan must reach the row's cuts: the top_k-th token, the min-p bin,
  // and (top-p over every token) the bin where the mass reaches top_p of it
  int rb1_need = -1;
  if (ps.zcut1 != CDS_NEG_INF) {
    const float rbf = kmax - floorf(ps.zcut1 * g.inv_delta);
    rb1_need = rbf >= (float)NBINS ? NBINS : (int)rbf;
  }
  const bool p_over_all = topp && !topk && ps.zcut1 == CDS_NEG_INF;
  const double p_need = (double)rp.top_p * mtot * (1.0 + 1e-9);
  const int lane = tid & 63, wv = tid >> 6;
  uint32_t run_c = 0u;
  double run_m = 0.0;
  int blk = 0;
  for (;;) {
    ps.bc[tid] = 0u;
    ps.bm[tid] = 0ull;
    __syncthreads();
    for (int j0 = 0; j0 < P; j0 += JC) {
      if (blk > 0 || j0 > 0) load_block(j0, blk);
#pragma unroll
      for (int jj = 0; jj < JC; ++jj) {
        const int j = j0 + jj;
        if (j >= P) break;
        const int sh = ps.shift[j];
        const unsigned long long v = hv[jj];
        // row bin of this value, relative to the block
        const int sb = blk == 0 ? tid : blk * NT - sh + tid;
        const int rb = sb + sh - blk * NT;
        if (v && sh >= 0 && rb >= 0 && rb < NT) {
          atomicAdd(&ps.bc[rb], (uint32_t)(v >> kCountShift));
          atomicAdd(&ps.bm[rb], v & ((1ull << kCountShift) - 1ull));
        }
      }
    }
    __syncthreads();
    const int B = blk * NT + tid;
    uint32_t cb = 0u;
    double mb = 0.0;
    if (B < NBINS) {
      cb = ps.bc[tid];
      const double top = ((double)kmax + 1.0 - (double)B) * (double)g.delta;
      mb = ps.bm[tid] ? (double)ps.bm[tid] * 0x1p-31 * exp(top / Td - m) : 0.0;
    }
    // inclusive scan of the block in bin order, then the running totals
    const uint32_t ic = wave_incl_sum(cb);
    const double im = wave_incl_sum(mb);
    if (lane == 63) {
      ps.wtot_u[wv] = ic;
      ps.wtot_d[wv] = im;
    }
    __syncthreads();
    uint32_t bc0 = 0u, tc = 0u;
    double bm0 = 0.0, tm = 0.0;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) {
      const uint32_t u = ps.wtot_u[k];
      const double d = ps.wtot_d[k];
      bc0 += k < wv ? u : 0u;
      bm0 += k < wv ? d : 0.0;
      tc += u;
      tm += d;
    }
    if (B < NBINS) {
      ps.cumc[B] = run_c + bc0 + ic;
      ps.md[B] = run_m + (bm0 + im);
    }
    run_c += tc;
    run_m += tm;
    ++blk;
    if (blk * NT >= NBINS) break;
    bool more = false;
    if (topk && run_c < (uint32_t)rp.top_k) more = true;   // the k-th token lies below
    if (rb1_need >= blk * NT) more = true;                  // the min-p bin lies below
    if (p_over_all && run_m < p_need) more = true;          // the top-p mass is not reached
    if (!more) break;
  }
  // bins below the scanned part: the totals (their own values are never
  // searched; the last bin's mass is the row's)
  for (int B = blk * NT + tid; B < NBINS; B += NT) {
    ps.cumc[B] = run_c;
    ps.md[B] = run_m > mtot ? run_m : mtot;
  }
  __syncthreads();
  CDS_TRACE_ROW(6);
  // the rest is searches over the monotone cumulative arrays: wave 0 only
  if (tid >= 64) return;
  constexpr int KB = (NBINS + 63) / 64;
  const int rb2 = topk ? wave0_first_ge<KB>(ps.cumc, NBINS, (uint32_t)rp.top_k) : NBINS;
  if (tid == 0) {
    int rb1 = NBINS;
    if (ps.zcut1 != CDS_NEG_INF) rb1 = rb1_need;
    int inK = -1, k_rank = 0;
    if (rb2 < NBINS && rb2 <= rb1) {
      inK = rb2;
      k_rank = rp.top_k - (int)(rb2 > 0 ? ps.cumc[rb2 - 1] : 0u);
    } else if (topp && rb1 < NBINS) {
      inK = rb1;
    }
    const int rb12 = min(rb1, rb2);
    const double M_lo = rb12 > 0 ? ps.md[min(rb12, NBINS) - 1] : 0.0;
    const double M_hi = rb12 < NBINS ? ps.md[rb12] : M_lo;
    ps.inK = inK;
    ps.k_rank = k_rank;
    ps.rb12 = rb12;
    ps.tlo = (double)rp.top_p * M_lo * (1.0 - 1e-9);
    ps.thi = (double)rp.top_p * M_hi * (1.0 + 1e-9);
  }
  __builtin_amdgcn_wave_barrier();
  const int i_lo = topp ? wave0_first_ge<KB>(ps.md, NBINS, ps.tlo) : NBINS;
  const int i_hi = topp ? wave0_first_ge<KB>(ps.md, NBINS, ps.thi) : NBINS;
  if (tid == 0) {
    const int cap = ps.rb12 < NBINS ? ps.rb12 : NBINS - 1;
    const int rb3_hi = min(i_hi, cap);
    const int rb3_lo = min(i_lo, rb3_hi);
    const int inK = ps.inK;
    int umin = NBINS;
    if (topp) umin = rb3_lo;
    if (inK >= 0) umin = min(umin, inK);
    auto cnt_range = [&](int lo_b, int hi_b) -> uint32_t {
      return ps.cumc[hi_b] - (lo_b > 0 ? ps.cumc[lo_b - 1] : 0u);
    };
    uint32_t uexp = topp ? cnt_range(rb3_lo, rb3_hi) : 0u;
    if (inK >= 0 && !(topp && inK >= rb3_lo && inK <= rb3_hi)) uexp += cnt_range(inK, inK);
    auto edge = [&](int b) { return (kmax - (float)b) * g.delta; };  // bottom of bin b (exact)
    Plan pl = base_plan(uexp > (uint32_t)UCAP ? PLAN_SLOW : PLAN_FAST);
    pl.z_sure = umin < NBINS ? edge(umin - 1) : edge(NBINS - 1);
    if (topp) {
      pl.a_lo = edge(rb3_hi);
      pl.a_hi = edge(rb3_lo - 1);
    }
    if (inK >= 0) {
      pl.k_lo = edge(inK);
      pl.k_hi = edge(inK - 1);
    }
    pl.k_rank = ps.k_rank;
    pl.topp = topp ? 1 : 0;
    pl.u_expected = uexp;
    pl.m_sure = (topp && umin > 0) ? ps.md[umin - 1] : 0.0;
    const int end = inK >= 0 ? inK - 1 : NBINS - 1;
    pl.m_mid = (topp && end > rb3_hi) ? ps.md[end] - ps.md[rb3_hi] : 0.0;
    pl.log_z = ps.log_z;
    CDS_TRACE_ROW(7);
    st_obj(&a.plans[r], pl);
    *out = pl;
  }
}

// Two u64 sums and the range [lo, hi] of a u32 over the block in one exchange
// (all NT threads; every thread gets the results).  Nothing: lo > hi.
template <int NT>
__device__ __forceinline__ void block_sums_range(unsigned long long& s0, unsigned long long& s1,
                                                 uint32_t& lo, uint32_t& hi, RedScratch<NT>& red) {
  // (~min, max) as two 32-bit maxima
  auto mm = [](unsigned long long a, unsigned long long b) {
    const uint32_t ah = (uint32_t)(a >> 32), bh = (uint32_t)(b >> 32);
    const uint32_t al = (uint32_t)a, bl = (uint32_t)b;
    return ((unsigned long long)(ah > bh ? ah : bh) << 32) | (unsigned long long)(al > bl ? al : bl);
  };
  auto add = [](unsigned long long a, unsigned long long b) { return a + b; };
  const unsigned long long pr = wave_allreduce(((unsigned long long)(~lo) << 32) | hi, mm);
  const unsigned long long t0 = wave_allreduce(s0, add), t1 = wave_allreduce(s1, add);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red.u[w] = t0;
    red.d[w] = __longlong_as_double((long long)t1);
    red.i[w] = (int32_t)(uint32_t)(pr >> 32);
    red.f[w] = __uint_as_float((uint32_t)pr);
  }
  __syncthreads();
  unsigned long long r = 0ull;
  s0 = s1 = 0ull;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    s0 += red.u[k];
    s1 += (unsigned long long)__double_as_longlong(red.d[k]);
    r = mm(r, ((unsigned long long)(uint32_t)red.i[k] << 32) | __float_as_uint(red.f[k]));
  }
  lo = ~(uint32_t)(r >> 32);
  hi = (uint32_t)r;
}

// LDS of the finisher's selections.
struct alignas(16) SelShared {
  unsigned long long hist[512];   // one radix round: weight per digit
  unsigned long long cw[64];      // the bin holding the answer, compacted
  uint32_t ck[64];
  unsigned long long above;       // weight above the picked digit
  int32_t pick;
  int32_t cnt;
  uint32_t result;
  uint32_t wt[16];                // block prefix sums (NT <= 1024)
};

// Weighted selection over the finisher's list ul[0, n): the largest order key
// v such that base + (sum of wt(e) over entries e with sel(e), wt(e) > 0 and
// key(e) >= v) reaches `need`.  The caller guarantees that the selected keys
// lie in [lo, hi] and that their whole weight reaches need - base > 0.  The
// bits in which lo and hi differ are resolved top-down in radix rounds of up
// to 9 bits; as soon as the bin holding v has at most 64 entries, they are
// compacted and wave 0 finishes the select from one entry per lane.  Weights
// are integers (counts, or fixed-point masses), so sums are exact in any
// order.  All NT threads call it; all get v.
template <int NT, typename Sel, typename Wt>
__device__ __forceinline__ uint32_t list_select(const uint64_t* ul, int n, Sel sel, Wt wt,
                                                double need, unsigned long long base,
                                                uint32_t lo, uint32_t hi, SelShared& s) {
  const int tid = threadIdx.x;
  if (lo == hi) return lo;
  int h = 31 - (int)__clz(lo ^ hi);  // the highest differing bit
  uint32_t pmask = h == 31 ? 0u : ~0u << (h + 1);
  uint32_t prefix = lo & pmask;
  while (true) {
    const int shift = h > 8 ? h - 8 : 0;
    const uint32_t dmask = (2u << (h - shift)) - 1u;
    {
      ulonglong2* h2 = reinterpret_cast<ulonglong2*>(s.hist);
      for (int i = tid; i < 256; i += NT) h2[i] = make_ulonglong2(0ull, 0ull);
    }
    __syncthreads();
#pragma unroll 1
    for (int i = tid; i < n; i += NT) {
      const unsigned long long e = ul[i];
      const uint32_t u = (uint32_t)(e >> 32);
      if ((u & pmask) == prefix && sel(e)) {
        const unsigned long long w = wt(e);
        if (w) atomicAdd(&s.hist[(u >> shift) & dmask], w);
      }
    }
    __syncthreads();
    // wave 0 picks the digit: lane l sums bins 511-8l down to 504-8l, the
    // first lane whose running total reaches need holds the digit's bin
    if (tid < 64) {
      const int l = tid;
      const ulonglong2* hp = reinterpret_cast<const ulonglong2*>(s.hist + 504 - 8 * l);
      unsigned long long sum = 0ull;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const ulonglong2 v = hp[q];
        sum += v.x + v.y;
      }
      const unsigned long long incl = wave_incl_sum(sum);
      const unsigned long long hit = __ballot((double)(base + incl) >= need);
      const int f = hit ? __ffsll((long long)hit) - 1 : 63;
      const unsigned long long ex = readlane_obj(incl - sum, f);
      const unsigned long long hb = l < 8 ? s.hist[511 - 8 * f - l] : 0ull;
      const unsigned long long incl2 = wave_incl_sum(hb);
      const unsigned long long hit2 = __ballot(l < 8 && (double)(base + ex + incl2) >= need);
      const int g = hit2 ? __ffsll((long long)hit2) - 1 : 7;
      if (l == g) {
        s.pick = 511 - 8 * f - g;
        s.above = base + ex + incl2 - hb;
        s.cnt = 0;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s.pick << shift;
    pmask |= dmask << shift;
    base = s.above;
    if (shift == 0) return prefix;  // every bit resolved
    h = shift - 1;
    // compact the bin's entries (the count goes on past 64: then another round)
#pragma unroll 1
    for (int i = tid; i < n; i += NT) {
      const unsigned long long e = ul[i];
      const uint32_t u = (uint32_t)(e >> 32);
      if ((u & pmask) == prefix && sel(e)) {
        const unsigned long long w = wt(e);
        if (w) {
          const int j = atomicAdd(&s.cnt, 1);
          if (j < 64) {
            s.ck[j] = u;
            s.cw[j] = w;
          }
        }
      }
    }
    __syncthreads();
    const int cnt = s.cnt;
    if (cnt <= 64) {
      if (tid < 64) {
        const bool valid = tid < cnt;
        const uint32_t uj = valid ? s.ck[tid] : 0u;
        const unsigned long long wj = valid ? s.cw[tid] : 0ull;
        unsigned long long cum = base;  // weight at keys >= uj
#pragma unroll 1
        for (int i = 0; i < cnt; ++i) {
          const uint32_t ui = (uint32_t)__builtin_amdgcn_readlane((int)uj, i);
          const unsigned long long wi = readlane_obj(wj, i);
          cum += ui >= uj ? wi : 0ull;
        }
        uint32_t v = valid && (double)cum >= need ? uj : 0u;
        v = wave_allreduce(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
        if (tid == 0) s.result = v;
      }
      __syncthreads();
      return s.result;
    }
  }
}

// ---- phase 4: the boundary list --------------------------------------------------
__device__ __forceinline__ float ukey_z(unsigned long long k) { return from_okey((uint32_t)(k >> 32)); }
__device__ __forceinline__ int32_t ukey_t(unsigned long long k) {
  return (int32_t)(0xFFFFFFFFu - (uint32_t)k);
}

// The race over n listed tokens (get(i, z, t) reads entry i), thread tid
// taking entries tid, tid + NT, ...: a draw only for tokens that can still
// enter the thread's top two.  draw(t0) gives the four 32-bit draws of tokens
// t0..t0+3.
template <int NT, typename Get, typename Draw>
__device__ __forceinline__ void race_list(Top2& b, int n, float zmax, float invT32, Get get,
                                          Draw draw) {
#pragma unroll 1
  for (int i = threadIdx.x; i < n; i += NT) {
    float z;
    int32_t t;
    get(i, z, t);
    if (!race32_hopeful(b, z, zmax, invT32)) continue;
    const uint4 blk = draw(t & ~3);
    const int w = t & 3;
    const uint32_t xw = w == 0 ? blk.x : (w == 1 ? blk.y : (w == 2 ? blk.z : blk.w));
    race32(b, z, t, xw, zmax, invT32);
  }
}

// One-wave selections over up to 64*KW list entries held KW per lane (lane l
// holds entries l + 64k): the largest order key v with (number, or summed
// integer weight, of the selected entries with key >= v) reaching need.  The
// selected keys lie in [lo, hi]; the bits below their common prefix are set
// greedily from the top.  Same definition as list_select, no barrier.
template <int KW>
__device__ __forceinline__ uint32_t wave_select_count(const uint32_t (&u)[KW], const bool (&sel)[KW],
                                                      uint32_t need, uint32_t lo, uint32_t hi) {
  if (lo == hi) return lo;
  const int h = 31 - (int)__clz(lo ^ hi);
  uint32_t prefix = h == 31 ? 0u : lo & ~((2u << h) - 1u);
  for (int bit = h; bit >= 0; --bit) {
    const uint32_t t = prefix | (1u << bit);
    uint32_t c = 0u;
#pragma unroll
    for (int k = 0; k < KW; ++k) c += (uint32_t)__popcll(__ballot(sel[k] && u[k] >= t));
    if (c >= need) prefix = t;
  }
  return prefix;
}
template <int KW>
__device__ __forceinline__ uint32_t wave_select_mass(const uint32_t (&u)[KW],
                                                     const unsigned long long (&w)[KW],
                                                     double need, uint32_t lo, uint32_t hi) {
  if (lo == hi) return lo;
  const int h = 31 - (int)__clz(lo ^ hi);
  uint32_t prefix = h == 31 ? 0u : lo & ~((2u << h) - 1u);
  auto add = [](unsigned long long a, unsigned long long b) { return a + b; };
  for (int bit = h; bit >= 0; --bit) {
    const uint32_t t = prefix | (1u << bit);
    unsigned long long m = 0ull;
#pragma unroll
    for (int k = 0; k < KW; ++k) m += u[k] >= t ? w[k] : 0ull;
    if ((double)wave_allreduce(m, add) >= need) prefix = t;
  }
  return prefix;
}

// fp64 race over {z >= zfinal} for tokens whose fp32 key reaches k_floor: the
// tie-breaker when the fp32 top two are within the fp32 error.
template <int NT, bool BF16, bool VEC>
__device__ __forceinline__ Best exact_rerace(const SampleArgs& a, int r, const Plan& pl, float zfinal,
                             float k_floor, RedScratch<NT>& red) {
  const RowParams rp = a.rows[r];
  const RowView rv = row_view<BF16>(a, r);
  const RaceCtx c = make_race_ctx(rp, pl.zmax);
  Best b = best_init();
  uint32_t nonfin = 0;
  for_row4<NT, BF16, VEC>(rv, a.V, nonfin, [&](const float* x, int64_t t0) {
    bool need = false;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      need |= (x[q] != CDS_NEG_INF && x[q] >= zfinal &&
               (x[q] - c.zmax) * c.invT32 + 16.7f >= k_floor);
    if (!need) return;
    const uint4 blk = race_block(c, t0);
    const uint32_t xs[4] = {blk.x, blk.y, blk.z, blk.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (x[q] == CDS_NEG_INF || x[q] < zfinal) continue;
      const float k32 = (x[q] - c.zmax) * c.invT32 + gumbel_fast(xs[q]);
      if (k32 < k_floor) continue;
      const double k64 = race_key64(x[q], c, xs[q]);
      const int32_t t = (int32_t)(t0 + q);
      if (better(k64, t, b.key, b.t)) {
        b.key = k64;
        b.t = t;
        b.z = x[q];
      }
    }
  });
  block_best<NT>(b, red);
  return b;
}

// Resolve the boundary list of row r and write its output (all NT threads of
// the finisher).  The row's list is gathered from the slices' lists into LDS.
// Returns false when the row must take the exact path.

// Lists of at most kShortList tokens are resolved by one wave.
template <int NT, bool BF16, bool VEC>
__device__ __forceinline__ bool finish_row(const SampleArgs& a, int r, int nl, const Plan& pl,
                                           ExactShared<NT>& sh, uint64_t* ul, int32_t* off,
                                           SelShared& sel, RedScratch<NT>& red) {
  // the row's nl <= 64 lists: list j is number r * 2P + j
  const int tid = threadIdx.x;
  const RowSlots rs = a.slots[r];
  const RowParams rp = a.rows[r];
  const int64_t l0 = rs.rec;                                    // record of list 0
  const uint64_t* ulr = a.ulist + (int64_t)rs.list64 * 64;      // list 0
  const int64_t lcap = row_list_cap(rp.flags, rp.top_k, a.P);   // entries per list
  const double Td = (double)rp.temperature;
  // A top-k row whose k-th token lies below the histogram window (no boundary
  // bin inside it, and min-p cuts nothing above the window's bottom): the
  // draw is exact (tokens below the window cannot win the race), but the kept
  // set reaches below the window's bottom, which the sure region stops at.  A
  // caller that asks for the kept-set threshold gets it from the exact path,
  // which selects the k-th value over the whole row.
  if (a.out_cut && !pl.list_mode && (rp.flags & ROW_TOPK) && !pl.topp && pl.k_rank == 0 &&
      pl.z_sure > pl.zcut1)
    return false;
  // One round of loads brings the records and a window of the first W
  // entries of every list (thread t reads list t % nl at positions
  // t / nl + M*k, M = NT / nl threads per list): most lists fit their window,
  // and only the entries past it are loaded once the lengths are known.
  constexpr int KP = 8;
  const int M = NT / nl;
  const int wj = tid % nl, wm = tid / nl;
  const int W = (int)min((int64_t)M * KP, lcap);  // window entries per list
  SliceBest sb{};
  if (tid < nl) sb = ld_obj(&a.bests[l0 + tid]);
  unsigned long long pre[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int pos = wm + M * k;
    pre[k] = (wm < M && pos < W) ? ld_u64(ulr + wj * lcap + pos) : 0ull;
  }
  // the slices' top two and list lengths; list offsets by a prefix sum
  Top2 b = top2_init();
  if (tid < 64) {  // nl <= 64: one wave
    uint32_t cnt = 0;
    float lcut = CDS_NEG_INF;  // list mode: the highest slice list cut
    if (tid < nl) {
      b.k1 = sb.k1;
      b.t1 = sb.t1;
      b.z1 = sb.z1;
      b.k2 = sb.k2;
      if (sb.pad[0]) {  // keys relative to the slice maximum: shift to the row's
        const float sh_k = (__uint_as_float(sb.pad[1]) - pl.zmax) *
                           (float)(1.0 / (double)rp.temperature);
        b.k1 += sh_k;
        b.k2 += sh_k;
      }
      // a list past its capacity was not written: the row takes the exact path
      cnt = sb.ucnt > (uint32_t)lcap ? (uint32_t)(lcap * 64 + 1) : sb.ucnt;
      if (pl.list_mode) lcut = __uint_as_float(sb.pad[2]);
    }
    lcut = wave_allreduce(lcut, [](float u, float v) { return fmaxf(u, v); });
    const bool over = __ballot(cnt > (uint32_t)W) != 0ull;
    if (tid == 0) {
      sh.fshare = lcut;
      sh.wrest = over ? 1 : 0;
    }
    const uint32_t incl = wave_incl_sum(cnt);
    off[tid + 1] = (int32_t)incl;
    if (tid == 0) off[0] = 0;
  }
  __syncthreads();
  CDS_TRACE_ROW(0);
  const int n_all = off[nl];
  if ((int64_t)n_all > lcap * nl) return false;
  // gather the slices' lists into LDS: every load of a round is issued before
  // any result is stored; element i = tid + k*NT of a round increases with k
  // (and over rounds), so its slice j (with off[j] <= i < off[j+1]) is found
  // by a forward scan.  Lists longer than the finisher holds are gathered in
  // rounds keeping only the tokens at or above the row's min-p cut (none below
  // it can be drawn); the row takes the exact path if even those overflow.
  int n = n_all;
  constexpr int KG = UCAP / NT;
  if (__builtin_expect(n_all <= UCAP, 1)) {
    // the windows, then whatever lies past them
    if (wm < M) {
      const int cj = off[wj + 1] - off[wj], oj = off[wj];
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int pos = wm + M * k;
        if (pos < W && pos < cj) ul[oj + pos] = pre[k];
      }
    }
    if (sh.wrest) {
      unsigned long long v[KG];
      bool got[KG];
      int j = 0;
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        const int i = tid + k * NT;
        while (j + 1 < nl && off[j + 1] <= i) ++j;
        got[k] = i < n && i - off[j] >= W;
        v[k] = got[k] ? ld_u64(ulr + j * lcap + (i - off[j])) : 0ull;
      }
#pragma unroll
      for (int k = 0; k < KG; ++k)
        if (got[k]) ul[tid + k * NT] = v[k];
    }
  } else {
    if (!(pl.zcut1 > CDS_NEG_INF)) return false;  // nothing to filter by
    const float zf = pl.zcut1;
    int j = 0, kept = 0;
#pragma unroll 1
    for (int base = 0; base < n_all; base += UCAP) {
      unsigned long long v[KG];
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        const int i = base + tid + k * NT;
        while (j + 1 < nl && off[j + 1] <= i) ++j;
        v[k] = i < n_all ? ld_u64(ulr + j * lcap + (i - off[j])) : 0ull;
      }
      uint32_t c = 0u;
#pragma unroll
      for (int k = 0; k < KG; ++k) c += (base + tid + k * NT < n_all && ukey_z(v[k]) >= zf) ? 1u : 0u;
      uint32_t tot;
      uint32_t pos = block_excl<NT>(c, sel.wt, tot);
      if (kept + (int)tot > UCAP) return false;  // (uniform)
#pragma unroll
      for (int k = 0; k < KG; ++k)
        if (base + tid + k * NT < n_all && ukey_z(v[k]) >= zf) ul[kept + (int)pos++] = v[k];
      kept += (int)tot;
      __syncthreads();  // sel.wt is read again by the next round
    }
    n = kept;
  }
  __syncthreads();

  CDS_TRACE_ROW(1);
  float zfin;
  if (n <= kShortList) {
    // short lists: wave 0 alone resolves the row (no workgroup barrier until
    // the result is shared): the same cuts and race as below
    if (tid < 64) {
      constexpr int KW = kShortList / 64;
      uint32_t u[KW], tl[KW];  // entry halves: order key, ~token
      float z[KW];
      bool v[KW];
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const int i = tid + 64 * k;
        v[k] = i < n;
        const unsigned long long e = v[k] ? ul[i] : 0ull;
        u[k] = (uint32_t)(e >> 32);
        tl[k] = (uint32_t)e;
        z[k] = v[k] ? ukey_z(e) : CDS_NEG_INF;
      }
      auto mn = [](uint32_t x, uint32_t y) { return x < y ? x : y; };
      auto mx = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
      int status = 0;  // 1: the row takes the exact path
      float zc12 = pl.zcut1;
      float zk = CDS_NEG_INF;  // the k-th largest value
      if (pl.k_rank > 0) {
        bool inK[KW];
        uint32_t c = 0u, lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
          inK[k] = v[k] && z[k] >= pl.k_lo && z[k] < pl.k_hi;
          c += (uint32_t)__popcll(__ballot(inK[k]));
          if (inK[k]) {
            lo = mn(lo, u[k]);
            hi = mx(hi, u[k]);
          }
        }
        lo = wave_allreduce(lo, mn);
        hi = wave_allreduce(hi, mx);
        if (c < (uint32_t)pl.k_rank && !pl.list_mode) status = 1;
        else if (c >= (uint32_t)pl.k_rank) {
          zk = from_okey(wave_select_count<KW>(u, inK, (uint32_t)pl.k_rank, lo, hi));
          zc12 = fmaxf(zc12, zk);
        }
      }
      if (pl.list_mode && zc12 < sh.fshare) status = 1;
      const uint32_t ord = rp.flags & kRowOrderBits;
      // min-p last: every token of the top-k set must be listed (its mass
      // normalises the top-p cut)
      if ((ord & ROW_ORDER_MINP_LAST) && pl.k_rank > 0 && pl.list_mode && zk < sh.fshare)
        status = 1;
      float zf = zc12;
      if (status == 0 && pl.topp) {
        const float zref = pl.a_hi, a_lo = pl.a_lo, zc = zc12;
        const float c32 = (float)(1.4426950408889634 / Td);
        const double F = exp((double)zref / Td - pl.m);
        constexpr double kFix = 0x1p46;
        unsigned long long w[KW], wi[KW], mu = 0ull, m_in = 0ull, mk = 0ull;
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int k = 0; k < KW; ++k) {
          const unsigned long long wz =
              v[k] ? (unsigned long long)((double)__builtin_amdgcn_exp2f((z[k] - zref) * c32) * kFix)
                   : 0ull;
          w[k] = z[k] >= zc ? wz : 0ull;
          mk += z[k] >= zk ? wz : 0ull;  // the top-k set (min-p last)
          mu += w[k];
          wi[k] = (z[k] >= a_lo) ? w[k] : 0ull;
          m_in += wi[k];
          if (wi[k]) {
            lo = mn(lo, u[k]);
            hi = mx(hi, u[k]);
          }
        }
        auto add = [](unsigned long long a, unsigned long long b) { return a + b; };
        mu = wave_allreduce(mu, add);
        m_in = wave_allreduce(m_in, add);
        lo = wave_allreduce(lo, mn);
        hi = wave_allreduce(hi, mx);
        // the mass top-p is normalised by: what min-p and top-k left (min-p
        // first), the top-k set (min-p last), every token (joint)
        double M2 = pl.m_sure + pl.m_mid + F * ((double)mu / kFix);
        if (ord & ROW_ORDER_JOINT) {
          M2 = exp(pl.log_z);
        } else if (ord & ROW_ORDER_MINP_LAST) {
          mk = wave_allreduce(mk, add);
          M2 = pl.k_rank > 0 ? F * ((double)mk / kFix) : exp(pl.log_z);
        }
        const double need = (pl.p * M2 - pl.m_sure) / F * kFix;
        // (other orders: a target above the mass of what min-p and top-k left
        // keeps all of it)
        const bool keep_all = ord != 0u && need > 0.0 && (double)m_in < need;
        if (!(need > 0.0) || ((double)m_in < need && !keep_all)) {
          status = 1;
        } else if (!keep_all) {
          // the cut is the key of a boundary entry (wi > 0): with at most 64
          // such entries, one per lane, each lane sums the weight at or above
          // its own key and the largest key whose sum reaches need wins (the
          // same value as the bitwise select, without a cross-lane sum per bit)
          uint32_t nb = 0u;
#pragma unroll
          for (int k = 0; k < KW; ++k) nb += (uint32_t)__popcll(__ballot(wi[k] != 0ull));
          uint32_t v;
          if (nb <= 64u) {
            uint32_t slot0 = 0u;
#pragma unroll
            for (int k = 0; k < KW; ++k) {
              const unsigned long long bm = __ballot(wi[k] != 0ull);
              if (wi[k]) {
                const uint32_t s = slot0 + (uint32_t)__popcll(bm & ((1ull << tid) - 1ull));
                sel.ck[s] = u[k];
                sel.cw[s] = wi[k];
              }
              slot0 += (uint32_t)__popcll(bm);
            }
            __builtin_amdgcn_wave_barrier();
            const bool valid = (uint32_t)tid < nb;
            const uint32_t uj = valid ? sel.ck[tid] : 0u;
            const unsigned long long wj = valid ? sel.cw[tid] : 0ull;
            unsigned long long cum = 0ull;
#pragma unroll 1
            for (uint32_t i = 0; i < nb; ++i) {
              const uint32_t ui = (uint32_t)__builtin_amdgcn_readlane((int)uj, (int)i);
              const unsigned long long wq = readlane_obj(wj, (int)i);
              cum += ui >= uj ? wq : 0ull;
            }
            v = valid && (double)cum >= need ? uj : 0u;
            v = wave_allreduce(v, mx);
            __builtin_amdgcn_wave_barrier();
          } else {
            v = wave_select_mass<KW>(u, wi, need, lo, hi);
          }
          zf = fmaxf(zf, from_okey(v));
        }
      }
      if (status == 0) {
        // the race over the survivors, merged with the slices' top two (lanes
        // below the list count hold those in b)
        const RaceCtx c = make_race_ctx(rp, pl.zmax);
#pragma unroll
        for (int k = 0; k < KW; ++k) {
          const bool in = v[k] && z[k] >= zf;
          if (in && race32_hopeful(b, z[k], c.zmax, c.invT32)) {
            const int32_t t = (int32_t)(0xFFFFFFFFu - tl[k]);
            const uint4 blk = race_block(c, (int64_t)(t & ~3));
            const int q = t & 3;
            const uint32_t xw = q == 0 ? blk.x : (q == 1 ? blk.y : (q == 2 ? blk.z : blk.w));
            race32(b, z[k], t, xw, c.zmax, c.invT32);
          }
        }
        b = wave_allreduce(b, [](Top2 x, const Top2& y) {
          top2_merge(x, y);
          return x;
        });
      }
      if (tid == 0) {
        sel.cw[0] = ((unsigned long long)__float_as_uint(b.k1) << 32) | (uint32_t)b.t1;
        sel.cw[1] = ((unsigned long long)__float_as_uint(b.z1) << 32) | __float_as_uint(b.k2);
        sel.cw[2] = ((unsigned long long)__float_as_uint(zf) << 32) | (uint32_t)status;
      }
    }
    __syncthreads();
    if ((uint32_t)sel.cw[2] != 0u) return false;
    b.k1 = __uint_as_float((uint32_t)(sel.cw[0] >> 32));
    b.t1 = (int32_t)(uint32_t)sel.cw[0];
    b.z1 = __uint_as_float((uint32_t)(sel.cw[1] >> 32));
    b.k2 = __uint_as_float((uint32_t)sel.cw[1]);
    zfin = __uint_as_float((uint32_t)(sel.cw[2] >> 32));
  } else {
  // exact top-k value: the k_rank-th largest list value inside [k_lo, k_hi)
  float zc12 = pl.zcut1;
  float zk = CDS_NEG_INF;
  if (pl.k_rank > 0) {
    const float k_lo = pl.k_lo, k_hi = pl.k_hi;
    auto inK = [&](unsigned long long e) {
      const float z = ukey_z(e);
      return z >= k_lo && z < k_hi;
    };
    unsigned long long cnt = 0ull, none = 0ull;
    uint32_t klo = 0xFFFFFFFFu, khi = 0u;
#pragma unroll 1
    for (int i = tid; i < n; i += NT) {
      const unsigned long long e = ul[i];
      if (inK(e)) {
        const uint32_t u = (uint32_t)(e >> 32);
        ++cnt;
        klo = min(klo, u);
        khi = max(khi, u);
      }
    }
    block_sums_range<NT>(cnt, none, klo, khi, red);
    // A boundary list short of k_rank contradicts the plan.  A candidate list
    // (list_mode) holds every token of the min-p set when that set has at most
    // k tokens; top-k then cuts nothing.
    if (cnt < (unsigned long long)pl.k_rank && !pl.list_mode) return false;
    if (cnt >= (unsigned long long)pl.k_rank) {
      const uint32_t v = list_select<NT>(
          ul, n, inK, [](unsigned long long) { return 1ull; }, (double)pl.k_rank, 0ull, klo, khi,
          sel);
      zk = from_okey(v);
      zc12 = fmaxf(zc12, zk);
    }
  }
  // list mode: the lists hold every token >= their slice's cut, so the set
  // {z >= zc12} is complete only if zc12 is at or above every cut (always so
  // when the slices listed their full top-k; truncated lists may miss it)
  if (pl.list_mode && zc12 < sh.fshare) return false;
  const uint32_t ord = rp.flags & kRowOrderBits;
  // min-p last: the whole top-k set must be listed (its mass normalises top-p)
  if ((ord & ROW_ORDER_MINP_LAST) && pl.k_rank > 0 && pl.list_mode && zk < sh.fshare) return false;
  CDS_TRACE_ROW(2);
  zfin = zc12;

  // exact top-p cut: the largest value v in [a_lo, a_hi) whose cumulative mass
  // (the sure region, plus every list token >= v that survived top-k) reaches
  // top_p * M2.  List masses are exp((z - a_hi)/T) (arguments <= 0, fp32)
  // times one fp64 factor, summed in fixed point (exact in any order).
  if (pl.topp) {
    const float zref = pl.a_hi, a_lo = pl.a_lo, zc = zc12;
    const float c32 = (float)(1.4426950408889634 / Td);
    const double F = exp((double)zref / Td - pl.m);
    constexpr double kFix = 0x1p46;  // <= 4096 weights <= 1 fit in 64 bits
    auto wfix = [=](float z) -> unsigned long long {
      return z >= zc ? (unsigned long long)((double)__builtin_amdgcn_exp2f((z - zref) * c32) * kFix)
                     : 0ull;
    };
    unsigned long long mu = 0ull, m_in = 0ull;
    uint32_t plo = 0xFFFFFFFFu, phi = 0u;
#pragma unroll 1
    for (int i = tid; i < n; i += NT) {
      const unsigned long long e = ul[i];
      const float z = ukey_z(e);
      const unsigned long long w = wfix(z);
      mu += w;
      if (z >= a_lo && w) {
        const uint32_t u = (uint32_t)(e >> 32);
        m_in += w;
        plo = min(plo, u);
        phi = max(phi, u);
      }
    }
    block_sums_range<NT>(mu, m_in, plo, phi, red);
    // the mass top-p is normalised by (see the one-wave path)
    double M2 = pl.m_sure + pl.m_mid + F * ((double)mu / kFix);
    if (ord & ROW_ORDER_JOINT) {
      M2 = exp(pl.log_z);
    } else if ((ord & ROW_ORDER_MINP_LAST) && pl.k_rank > 0) {
      unsigned long long mk = 0ull;
      const float zkk = zk;
#pragma unroll 1
      for (int i = tid; i < n; i += NT) {
        const float z = ukey_z(ul[i]);
        if (z >= zkk)
          mk += (unsigned long long)((double)__builtin_amdgcn_exp2f((z - zref) * c32) * kFix);
      }
      mk = block_sum_u64<NT>(mk, red);
      M2 = F * ((double)mk / kFix);
    } else if (ord & ROW_ORDER_MINP_LAST) {
      M2 = exp(pl.log_z);
    }
    // the list mass (in fixed units) the cut must reach above the sure region
    const double need = (pl.p * M2 - pl.m_sure) / F * kFix;
    if (!(need > 0.0)) return false;         // the cut lies above the range
    if ((double)m_in < need) {
      // ... or below it: for the joint and min-p-last orders all of what
      // min-p and top-k left is kept; otherwise the plan was wrong
      if (!ord) return false;
    } else {
      const uint32_t v = list_select<NT>(
          ul, n, [=](unsigned long long e) { return ukey_z(e) >= a_lo; },
          [=](unsigned long long e) { return wfix(ukey_z(e)); }, need, 0ull, plo, phi, sel);
      zfin = fmaxf(zfin, from_okey(v));
    }
  }

  CDS_TRACE_ROW(3);
  // race the list tokens that survive, merge with the slices' top two; the
  // survivors are first compacted (when they fit), so that a wave draws only
  // for tokens that race
  const RaceCtx c = make_race_ctx(rp, pl.zmax);
  auto draw = [&](int32_t t0) { return race_block(c, (int64_t)t0); };
  {
    // the survivors move to the front of the list, in place: every entry is
    // read into registers before the barrier inside block_excl
    constexpr int KG = UCAP / NT;
    unsigned long long e[KG];
    uint32_t cs = 0u;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int i = tid + k * NT;
      e[k] = i < n ? ul[i] : 0ull;
      cs += (i < n && ukey_z(e[k]) >= zfin) ? 1u : 0u;
    }
    uint32_t ns;
    uint32_t pos = block_excl<NT>(cs, sel.wt, ns);
#pragma unroll
    for (int k = 0; k < KG; ++k)
      if (tid + k * NT < n && ukey_z(e[k]) >= zfin) ul[pos++] = e[k];
    __syncthreads();
    race_list<NT>(
        b, (int)ns, c.zmax, c.invT32,
        [&](int i, float& z, int32_t& t) {
          const uint64_t v = ul[i];
          z = ukey_z(v);
          t = ukey_t(v);
        },
        draw);
  }
  block_top2<NT>(b, red);
  }
  CDS_TRACE_ROW(4);
  if (b.t1 == INT_MAX) return false;
  // the drawn-from set is {allowed z >= zfinal}
  const float zs = fmaxf(pl.z_sure, pl.zcut1);
  const float zfinal = (pl.topp || pl.k_rank > 0) ? zfin : zs;
  if (b.k1 - b.k2 > 2.0f * kRaceEps) {
    if (tid == 0) {
      write_out(a, r, b.t1, (float)((double)b.z1 / Td - pl.m - pl.log_z), 0);
      if (a.out_cut) a.out_cut[r] = zfinal;
      a.plans[r].path = PATH_FAST;
    }
    return true;
  }
  // fp32 top two too close: decide in fp64 over the final set
  const Best e = exact_rerace<NT, BF16, VEC>(a, r, pl, zfinal, b.k1 - 2.0f * kRaceEps, red);
  if (tid == 0) {
    write_out(a, r, e.t, (float)((double)e.z / Td - pl.m - pl.log_z), 0);
    if (a.out_cut) a.out_cut[r] = zfinal;
    a.plans[r].path = PATH_RERACE;
  }
  return true;
}

constexpr int kHistCopies = 4;

template <int NT>
union FusedLds {
  unsigned long long hist[kHistCopies * (NBINS + 32)];
  PlanShared<NT> plan;
  struct {
    ExactShared<NT> ex;
    uint64_t list[UCAP];
    int32_t off[kMaxSlices + 1];
    SelShared select;
  } fin;
  struct {
    uint32_t wt[2 * NT / 64];  // per-wave token counts (list_tokens, list_tokens2)
  } sel;
};


__device__ __forceinline__ int row_class(const RowParams& rp, int P) {
  return (int)row_class_of(rp.flags, rp.top_k, P);
}

// Lists the slice's tokens whose value passes keep(), in thread-major order:
// each thread counts its tokens, a wave prefix sum and one workgroup barrier
// give every thread its position, then emit(pos, v, t) stores token t (value
// v) at list position pos.  Returns the number of tokens that passed; when it
// exceeds cap the list is not written at all (every consumer then takes
// another path).  Blocks of four tokens that no lane of a wave keeps are
// skipped as a whole.  wt is LDS scratch of NT/64 words; all NT threads must
// call it.
template <int NT, int E4, typename Keep, typename Emit>
__device__ __forceinline__ uint32_t list_tokens(const float (&x)[E4][4], int32_t tbase,
                                                uint32_t cap, uint32_t* wt, Keep keep, Emit emit) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t c = 0u;
#pragma unroll
  for (int i = 0; i < E4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) c += keep(x[i][q]) ? 1u : 0u;
  const uint32_t incl = wave_incl_sum(c);
  if (lane == 63) wt[w] = incl;
  __syncthreads();
  uint32_t base = 0u, total = 0u;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const uint32_t tk = wt[k];
    base += k < w ? tk : 0u;
    total += tk;
  }
  if (total <= cap && c) {
    uint32_t pos = base + incl - c;
#pragma unroll
    for (int i = 0; i < E4; ++i) {
      // the predicates are evaluated again here (opaque copies): keeping the
      // counting pass's E4*4 masks alive across the barrier costs registers
      float v[4];
      bool kq[4];
      bool any = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = x[i][q];
        asm volatile("" : "+v"(v[q]));
        kq[q] = keep(v[q]);
        any |= kq[q];
      }
      if (any) {
        const int32_t t0 = tbase + 4 * NT * i;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (kq[q]) emit(pos++, v[q], t0 + q);
      }
    }
  }
  return total;
}

// list_tokens with one ballot per register instead of a counting pass: each
// wave appends the entries it keeps (entry(v, t)) to its own region of
// `stage` (LDS, NT/64 regions of UCAP/(NT/64) entries) in (register, lane)
// order, skipping registers no lane keeps; one barrier shares the wave counts,
// then each wave copies its region to list positions after the waves before
// it, through emit(pos, entry).  Returns the number of tokens kept; when that
// exceeds cap nothing is emitted.  If a wave keeps more than its region holds
// (and the total fits cap) nothing is emitted either and *spill is set: the
// caller lists with list_tokens instead.  wt: LDS scratch of NT/64 words.
template <int NT, int E4, typename Keep, typename Entry, typename Emit>
__device__ __forceinline__ uint32_t list_tokens_staged(const float (&x)[E4][4], int32_t tbase,
                                                       uint32_t cap, uint64_t* stage, uint32_t* wt,
                                                       bool* spill, Keep keep, Entry entry,
                                                       Emit emit) {
  constexpr uint32_t kRegion = (uint32_t)UCAP / (uint32_t)(NT / 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t* mine = stage + (size_t)w * kRegion;
  uint32_t n = 0u;  // wave-uniform
#pragma unroll
  for (int i = 0; i < E4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool k = keep(x[i][q]);
      const unsigned long long m = __ballot(k);
      if (m) {
        const uint32_t pos = n + lanes_below(m);
        if (k && pos < kRegion) mine[pos] = entry(x[i][q], tbase + 4 * NT * i + q);
        n += (uint32_t)__popcll(m);
      }
    }
  if (lane == 0) wt[w] = n;
  __syncthreads();
  uint32_t base = 0u, total = 0u, most = 0u;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const uint32_t tk = wt[k];
    base += k < w ? tk : 0u;
    total += tk;
    most = tk > most ? tk : most;
  }
  *spill = total <= cap && most > kRegion;
  if (total <= cap && most <= kRegion)
    for (uint32_t j = (uint32_t)lane; j < n; j += 64u) emit(base + j, mine[j]);
  return total;
}

// list_tokens for two disjoint predicates at once: one counting pass, one
// barrier, one writing pass; returns (number kept by keep1, by keep2).  wt is
// LDS scratch of 2*NT/64 words.
template <int NT, int E4, typename K1, typename E1, typename K2, typename E2>
__device__ __forceinline__ uint2 list_tokens2(const float (&x)[E4][4], int32_t tbase,
                                              uint32_t cap1, uint32_t cap2, uint32_t* wt,
                                              K1 keep1, E1 emit1, K2 keep2, E2 emit2) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t c1 = 0u, c2 = 0u;
#pragma unroll
  for (int i = 0; i < E4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c1 += keep1(x[i][q]) ? 1u : 0u;
      c2 += keep2(x[i][q]) ? 1u : 0u;
    }
  const uint32_t incl1 = wave_incl_sum(c1), incl2 = wave_incl_sum(c2);
  if (lane == 63) {
    wt[w] = incl1;
    wt[NT / 64 + w] = incl2;
  }
  __syncthreads();
  uint32_t base1 = 0u, base2 = 0u, n1 = 0u, n2 = 0u;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const uint32_t t1 = wt[k], t2 = wt[NT / 64 + k];
    base1 += k < w ? t1 : 0u;
    base2 += k < w ? t2 : 0u;
    n1 += t1;
    n2 += t2;
  }
  const bool w1 = n1 <= cap1 && c1, w2 = n2 <= cap2 && c2;
  if (w1 || w2) {
    uint32_t pos1 = base1 + incl1 - c1, pos2 = base2 + incl2 - c2;
#pragma unroll
    for (int i = 0; i < E4; ++i) {
      float v[4];
      bool k1[4], k2[4];
      bool any = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = x[i][q];
        asm volatile("" : "+v"(v[q]));  // evaluated again, see list_tokens
        k1[q] = w1 && keep1(v[q]);
        k2[q] = w2 && keep2(v[q]);
        any |= k1[q] | k2[q];
      }
      if (any) {
        const int32_t t0 = tbase + 4 * NT * i;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (k1[q]) emit1(pos1++, v[q], t0 + q);
          if (k2[q]) emit2(pos2++, v[q], t0 + q);
        }
      }
    }
  }
  return make_uint2(n1, n2);
}

// List entry of the row's boundary and candidate lists: okey(v) << 32 | ~t
// (larger values first, then lower token ids, in unsigned order).
__device__ __forceinline__ uint64_t ulist_entry(float v, int32_t t) {
  return ((uint64_t)okey(v + 0.0f) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
}

// Smallest fp32 value v with exp(v/T - zmax/T) >= min_p (the min-p set
// relative to zmax is {z >= v}); -inf when every finite value qualifies.  Wave
// 0 only; every lane of it gets the result.
__device__ __forceinline__ float minp_cut_wave(float zmax, double Td, float min_p) {
  const double m = (double)zmax / Td, mp = (double)min_p;
  auto pred = [&](uint32_t k) { return exp((double)from_okey(k) / Td - m) >= mp; };
  if (pred(okey(-FLT_MAX))) return CDS_NEG_INF;
  return from_okey(wave_first_true(okey(-FLT_MAX), okey(zmax), pred));
}

// One workgroup per slice of a row.  The slice is streamed once into
// registers (bf16 upcast and the grammar bitmask fused into the load) and is
// never read again from memory.  Every slice reduces max, lowest argmax and the
// non-finite flag, then by row class:
//   GREEDY  sum exp((z - max)) for the logprob;
//   RACE    sum exp((z - max)/T), and the race over all its tokens (keys
//           relative to the slice maximum);
//   LIST    sum exp((z - max)/T), and a list of its tokens that may survive:
//           for top-k rows every token at or above the top_k-th largest of a
//           set of group maxima (which is at most the slice's own top_k-th
//           value), for min-p rows every token at or above the min-p cut
//           relative to the slice maximum (at most the row's cut);
//   HOLD    a histogram of s = z/T on a power-of-two grid (counts and masses).
// The slice publishes its summary and takes the row's arrival ticket; the last
// slice of the row (the planner) merges the summaries.  GREEDY, RACE and LIST
// rows are then resolved by the planner alone: the other slices have exited.
// HOLD rows need the row's top-p cut before the race: the planner publishes a
// plan (min-p cut, the value range of sure tokens, the top-p boundary bins),
// the other slices wait for it with their slice still in registers, race their
// sure tokens, list their boundary tokens and take the done ticket; the last
// one resolves the boundary list.  A wait that times out marks the row, whose
// finisher then takes the exact path, so results never depend on timing.
// STREAM: non-temporal loads, for rows whose slices are read once (every
// class but HOLD, whose second pass reads its slices again).
// Diagnostic phase timestamp k of this workgroup (SAMPLER_OPT_TRACE).
#define CDS_TRACE(k)                                                             \
  do {                                                                           \
    if (a.trace && threadIdx.x == 0) a.trace[(size_t)blockIdx.x * 8 + (k)] = wall_clock64(); \
  } while (0)

// CLS >= 0: the row's class, fixed at compile time (the instantiation then
// holds that class's code only).
template <int NT, int E4, bool BF16, bool VEC, bool STREAM, int CLS>
__device__ __forceinline__ void slice_task(const SampleArgs& a, int r, const RowParams& rp, int sl,
                                           FusedLds<NT>& sh, RedScratch<NT>& red,
                                           StatScratch<NT>& sst, Plan* s_plan, uint32_t* s_word) {
  const int tid = threadIdx.x, P = a.P;
  const int cls = CLS >= 0 ? CLS : row_class(rp, a.P);
  const bool greedy = cls == CLS_GREEDY;
  const int64_t lo = (int64_t)sl * a.S;
  const int64_t hi = min(lo + a.S, (int64_t)a.V);
  const int32_t tbase = (int32_t)lo + 4 * tid;  // token of chunk i: tbase + 4*NT*i
  const RowView rv = row_view<BF16>(a, r);
  const RowSlots rs = a.slots[r];
  const uint32_t lcap = row_list_cap(rp.flags, rp.top_k, P);
  const int64_t slot = (int64_t)r * P + sl;                              // head
  const int64_t hslot = (int64_t)(rs.rec / (2u * (uint32_t)P)) * P + sl;  // histogram (HOLD)
  const int64_t lslot = (int64_t)rs.rec + sl;      // record of list sl of the row
  CDS_TRACE(1);

  float x[E4][4];
  uint32_t nonfin = 0;
  load_chunks<NT, E4, BF16, VEC, STREAM, false>(rv, lo, hi, 0, x, nonfin);

  // ---- the slice summary: one pass over the registers, one merge ----
  // max, non-finite flag, sum exp((z - max)/T_eff) (rows that are not HOLD),
  // and for top-k rows the minimum of the thread maxima; then the lowest index
  // holding the max
  const bool topk_list = cls == CLS_LIST && (rp.flags & ROW_TOPK);
  const int kq = topk_list ? list_q(rp.top_k, P) : 0;  // <= 4 * NT for LIST rows
  const float cexp =
      cls == CLS_HOLD ? 0.0f : (greedy ? 1.0f : (float)(1.0 / (double)rp.temperature)) * kLog2e;
  SliceStat st;
  st.m = CDS_NEG_INF;
  st.a = INT_MAX;
  st.s = 0.0;
  st.nf = nonfin;
  st.lb = CDS_POS_INF;
  {
#pragma unroll
    for (int i = 0; i < E4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) st.m = fmaxf(st.m, x[i][q]);
    // top-k rows (q = list_q <= 3 NT / 2): each wave's ceil(q/W)-th largest of the
    // lanes' maxima (of the whole lane, or of four groups of its chunks when
    // one value per lane is not enough; W waves).  Every wave has that many tokens
    // at or above its own value, so at least q tokens of the slice lie at or
    // above the minimum over waves.
    if (topk_list) {
      const int qw = (kq + NT / 64 - 1) / (NT / 64);
      // one maximum per lane keeps the cut tight only while qw is a small
      // share of the 64 lanes (a low rank among lane maxima lets several
      // tokens of each lane through, and the row's lists overflow); past 16,
      // four group maxima per lane
      if (qw <= 16) {
        st.lb = wave_kth_largest(st.m, qw);
      } else {
        // the maxima of four groups of the lane's chunks: four distinct tokens
        float gm[4] = {CDS_NEG_INF, CDS_NEG_INF, CDS_NEG_INF, CDS_NEG_INF};
#pragma unroll
        for (int i = 0; i < E4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) gm[(i * 4) / E4] = fmaxf(gm[(i * 4) / E4], x[i][q]);
        st.lb = wave_kth_largest_n<4>(gm, qw);
      }
    }
    if (cexp != 0.0f && st.m != CDS_NEG_INF) {
      // exp2((x - max) * c): the difference first, so that the rounding of
      // max * c does not scale every term of the sum alike (that offset would
      // reach the logprob at low temperatures); a NaN or +inf token makes the
      // sum NaN (or the max +inf), which flags the slice
      const float mt = st.m;
#pragma unroll
      for (int i = 0; i < E4; ++i) {
        float part = __builtin_amdgcn_exp2f((x[i][0] - mt) * cexp);
#pragma unroll
        for (int q = 1; q < 4; ++q) part += __builtin_amdgcn_exp2f((x[i][q] - mt) * cexp);
        st.s += (double)part;
      }
    }
    if (cls == CLS_HOLD || st.m == CDS_NEG_INF) {
      // NaN / +inf check where the exp-sum does not run (HOLD rows, and threads
      // whose values are all -inf: fmaxf passes over a NaN, so a NaN among
      // masked tokens would otherwise go unseen): a plain sum propagates them
      float sx = 0.0f;
#pragma unroll
      for (int i = 0; i < E4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) sx += x[i][q];
      if (sx != sx || sx == CDS_POS_INF) st.nf = 1u;
    }
  }
  const float lmax = st.m;
  st = block_stat<NT>(st, cexp, sst);
  const float zm = st.m == CDS_POS_INF ? CDS_NEG_INF : st.m;
  if (st.m == CDS_POS_INF || st.s != st.s) st.nf = 1u;
  // the lowest index holding the maximum (searched only by threads holding it)
  int32_t am = INT_MAX;
  if (zm != CDS_NEG_INF && lmax == zm) {
#pragma unroll
    for (int i = E4 - 1; i >= 0; --i)
#pragma unroll
      for (int q = 3; q >= 0; --q)
        if (x[i][q] == zm) am = tbase + 4 * NT * i + q;
  }
  if (zm != CDS_NEG_INF) am = block_min_i32<NT>(am, red);
  nonfin = st.nf;
  CDS_TRACE(2);

  uint32_t flags = nonfin ? SLICE_NONFINITE : 0u;
  const double se = st.s;
  double hold_mass = 0.0;  // HOLD rows: the slice's mass relative to its maximum
  float kmax = 0.0f;
  if (cls == CLS_HOLD && zm != CDS_NEG_INF) {
    // histogram of the values below the slice maximum, bins aligned to delta
    const BinGeom g = bin_geom(rp.temperature);
    kmax = floorf(zm * g.inv_delta);
    if (!(fabsf(kmax) < 4194304.0f)) {
      flags |= SLICE_BINS_LOST;  // bin indices would not be exact: row takes the exact path
    } else {
      for (int b = tid; b < kHistCopies * (NBINS + 32); b += NT) sh.hist[b] = 0ull;
      __syncthreads();
      // tokens outside the window (and -inf) land in 32 per-lane sink bins:
      // no branch per token.  kHistCopies interleaved copies (lane % copies)
      // spread the atomics of one instruction over more addresses.
      const int sink = NBINS + (tid & 31);
      const int copy = tid & (kHistCopies - 1);
#pragma unroll
      for (int i = 0; i < E4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float y = x[i][q] * g.inv_delta;
          const float kf = floorf(y);
          const float rbf = kmax - kf;
          const int rb = (rbf >= 0.0f && rbf < (float)NBINS) ? (int)rbf : sink;
          const float w = __builtin_amdgcn_exp2f(fmaf(y - kf, g.c_bin, -g.c_bin));
          const uint32_t fix = (uint32_t)(w * 2147483648.0f);
          atomicAdd(&sh.hist[rb * kHistCopies + copy],
                    (1ull << kCountShift) | (unsigned long long)fix);
        }
      __syncthreads();
      // publish the bins, and the slice's total mass relative to its maximum
      // (the row's planner reads the slice totals first and only the top
      // bins of each histogram): bin b spans [(kmax-b)*delta,
      // (kmax-b+1)*delta) and holds fixed-point masses relative to its top
      unsigned long long* gh = a.hist + hslot * NBINS;
      const double Td = (double)rp.temperature, dd = (double)g.delta;
      double msum = 0.0;
      for (int b = tid; b < NBINS; b += NT) {
        unsigned long long v = 0ull;
#pragma unroll
        for (int c = 0; c < kHistCopies; ++c) v += sh.hist[b * kHistCopies + c];
        st_u64(gh + b, v);
        const unsigned long long mfix = v & ((1ull << kCountShift) - 1ull);
        if (mfix)
          msum += (double)mfix * 0x1p-31 *
                  exp((((double)kmax + 1.0 - (double)b) * dd - (double)zm) / Td);
      }
      hold_mass = block_sum_f64<NT>(msum, red);
    }
  }
  CDS_TRACE(3);
  if (cls == CLS_RACE && zm != CDS_NEG_INF && !nonfin) {
    // the race over every allowed token, keys relative to the slice maximum
    const float invT32 = sgpr_f((float)(1.0 / (double)rp.temperature));
    const uint32_t k0 = (uint32_t)rp.seed, k1 = (uint32_t)(rp.seed >> 32);
    const uint32_t off_lo = (uint32_t)rp.offset, off_hi = (uint32_t)(rp.offset >> 32);
    Top2 b = top2_init();
#pragma unroll
    for (int i = 0; i < E4; ++i) {
      int32_t tb = tbase;
      asm volatile("" : "+v"(tb));
      const int32_t t0 = tb + 4 * NT * i;
      bool need = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) need |= race32_hopeful(b, x[i][q], zm, invT32);
      if (need) {
        const uint4 blk =
            philox4x32_10(make_uint4((uint32_t)t0 >> 2, off_lo, off_hi, 0u), k0, k1);
        const uint32_t xs[4] = {blk.x, blk.y, blk.z, blk.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          race32_if(b, x[i][q] != CDS_NEG_INF, x[i][q], t0 + q, xs[q], zm, invT32);
      }
    }
    block_top2<NT>(b, red);
    if (tid == 0) {
      SliceBest sb;
      sb.k1 = b.k1;
      sb.t1 = b.t1;
      sb.z1 = b.z1;
      sb.k2 = b.k2;
      sb.ucnt = 0u;
      sb.pad[0] = 1u;
      sb.pad[1] = __float_as_uint(zm);
      sb.pad[2] = __float_as_uint(CDS_NEG_INF);  // no list
      st_obj(&a.bests[lslot], sb);
    }
  } else if (cls == CLS_LIST && zm != CDS_NEG_INF && !nonfin) {
    // a superset of the slice's candidates, listed: every token at or above a
    // cut that is at most the slice's top_k-th largest value (top-k rows) and
    // at most the min-p bound relative to the slice maximum (min-p rows; the
    // row's bound, relative to the row maximum, is at least as high)
    float cut = (topk_list && st.lb != CDS_POS_INF) ? st.lb : CDS_NEG_INF;
    // (min-p last: the top-p cut is normalised by the whole top-k set's
    // mass, so a top-k row lists it without the min-p bound)
    if ((rp.flags & ROW_MINP) && !(topk_list && (rp.flags & ROW_ORDER_MINP_LAST))) {
      const double b = (double)zm + (double)rp.temperature * log((double)rp.min_p);
      const float bm = (float)(b - 1e-5 * (1.0 + fabs(b) + fabs((double)zm)));
      cut = fmaxf(cut, bm);
    }
    const float cutv = sgpr_f(cut);
    const float cutk = fmaxf(cutv, -FLT_MAX);  // v >= cutk keeps no -inf
    uint64_t* gl = a.ulist + (int64_t)rs.list64 * 64 + (int64_t)sl * lcap;
    bool spill;
    uint32_t nst = list_tokens_staged<NT, E4>(
        x, tbase, lcap, sh.fin.list, sh.sel.wt, &spill, [&](float v) { return v >= cutk; },
        [](float v, int32_t t) { return ulist_entry(v, t); },
        [&](uint32_t pos, uint64_t e) { st_u64(gl + pos, e); });
    if (spill) {
      __syncthreads();  // sh.sel.wt is written again
      nst = list_tokens<NT, E4>(
          x, tbase, lcap, sh.sel.wt, [&](float v) { return v >= cutk; },
          [&](uint32_t pos, float v, int32_t t) { st_u64(gl + pos, ulist_entry(v, t)); });
    }
    if (tid == 0) {
      SliceBest sb;
      sb.k1 = CDS_NEG_INF;
      sb.t1 = INT_MAX;
      sb.z1 = CDS_NEG_INF;
      sb.k2 = CDS_NEG_INF;
      sb.ucnt = nst;
      sb.pad[0] = sb.pad[1] = 0u;
      sb.pad[2] = __float_as_uint(cutv);  // the list holds every token >= this
      st_obj(&a.bests[lslot], sb);
    }
  } else if ((cls == CLS_RACE || cls == CLS_LIST) && tid == 0) {
    // nothing allowed or a non-finite value: the planner answers the row
    SliceBest sb;
    sb.k1 = CDS_NEG_INF;
    sb.t1 = INT_MAX;
    sb.z1 = CDS_NEG_INF;
    sb.k2 = CDS_NEG_INF;
    sb.ucnt = 0u;
    sb.pad[0] = sb.pad[1] = 0u;
    sb.pad[2] = __float_as_uint(CDS_NEG_INF);  // lists nothing, holds nothing
    st_obj(&a.bests[lslot], sb);
  }

  CDS_TRACE(4);
  if (tid == 0) {
    SliceHead h;
    h.zmax = zm;
    h.arg = (zm == CDS_NEG_INF) ? -1 : am;
    h.flags = flags;
    h.kmax = kmax;
    h.sumexp = cls == CLS_HOLD ? hold_mass : se;
    h.pad[0] = h.pad[1] = 0u;
    st_obj(&a.heads[slot], h);
  }
  vm_drain();
  __syncthreads();
  RowSync* sy = &a.sync[r];
  if (tid == 0) {
    const uint32_t t = take_ticket(&sy->arrive);
    if (t == (uint32_t)(P - 1)) st_u64(&sy->arrive, 0ull);
    s_word[0] = t;
  }
  __syncthreads();
  const bool planner = s_word[0] == (uint32_t)(P - 1);
  if (a.trace && tid == 0)
    a.trace[(size_t)blockIdx.x * 8] = (unsigned long long)r | ((unsigned long long)sl << 20) |
                                      ((unsigned long long)cls << 28) |
                                      ((unsigned long long)planner << 31);
  CDS_TRACE(5);
  if (cls != CLS_HOLD) {
    if (!planner) {
      CDS_TRACE(7);
      return;
    }
    // the last slice of the row resolves it from the summaries and lists
    plan_row<NT>(a, r, false, sh.plan, s_plan);
    __syncthreads();
    CDS_TRACE(6);
    if (greedy) {
      CDS_TRACE(7);
      return;
    }
    Plan pl = *s_plan;
    if (pl.mode != PLAN_FAST) return;  // answered (no finite token, non-finite)
    pl.list_mode = 1;
    pl.z_sure = CDS_NEG_INF;
    pl.m_sure = pl.m_mid = 0.0;
    pl.p = (double)rp.top_p;
    pl.k_rank = 0;
    pl.topp = 0;
    pl.a_lo = pl.a_hi = pl.k_lo = pl.k_hi = CDS_POS_INF;
    if (rp.flags & ROW_TOPK) {
      pl.k_rank = rp.top_k;
      // the k-th largest within the min-p set, or over every token when
      // min-p comes last (the same value when the min-p set holds k tokens)
      pl.k_lo = (rp.flags & ROW_ORDER_MINP_LAST) ? -FLT_MAX : pl.zcut1;
      pl.k_hi = CDS_POS_INF;
    }
    if (rp.flags & ROW_TOPP) {
      pl.topp = 1;
      pl.a_lo = -FLT_MAX;
      pl.a_hi = pl.zmax;   // masses exp((z - zmax)/T) <= 1
    }
    if (!finish_row<NT, BF16, VEC>(a, r, P, pl, sh.fin.ex, sh.fin.list, sh.fin.off, sh.fin.select,
                                   red)) {
      __syncthreads();
      row_exact<NT, BF16, VEC>(a, r, sh.fin.ex);
      if (tid == 0) a.plans[r].path = PATH_EXACT;
    }
    CDS_TRACE(7);
    return;
  }

  // ---- HOLD rows: the last slice plans the row; the race is a pass-2 task ----
  if (planner) {
    plan_row<NT>(a, r, true, sh.plan, s_plan);
    if (tid == 0) {
      vm_drain();  // the plan (written by this thread) before its flag
      st_u32(&sy->ready, a.gen);
    }
    CDS_TRACE(6);
  }
  CDS_TRACE(7);
}

// Pass 2 of a HOLD row (slice sl): the slice is loaded again (the loads are
// issued before the wait), the row's plan awaited, then the sure tokens race,
// the boundary tokens are listed, and the last slice resolves the row.
// SPLIT: the task takes one half of the slice (EC = ceil(E4/2) chunks), and
// draws every token's Gumbel term while the plan is being made.
template <int NT, int E4, bool SPLIT, bool BF16, bool VEC>
__device__ __forceinline__ void hold_race_task(const SampleArgs& a, int r, const RowParams& rp,
                                               int sl, int half, FusedLds<NT>& sh,
                                               RedScratch<NT>& red, Plan* s_plan,
                                               uint32_t* s_word) {
  constexpr int EC = SPLIT ? (E4 + 1) / 2 : E4;  // chunks held
  constexpr int halves = SPLIT ? 2 : 1;
  const int tid = threadIdx.x, P = a.P;
  // the task's part of slice sl: all of it, or one of two halves (the first
  // holds chunks 0 .. ceil(E4/2)-1 of the slice)
  const int64_t s0 = (int64_t)sl * a.S, s1 = min(s0 + a.S, (int64_t)a.V);
  constexpr int64_t kHalfLen = (int64_t)((E4 + 1) / 2) * 4 * NT;
  const int64_t lo = halves == 1 ? s0 : min(s0 + half * kHalfLen, s1);
  const int64_t hi = halves == 1 ? s1 : (half ? s1 : min(s0 + kHalfLen, s1));
  const int32_t tbase = (int32_t)lo + 4 * tid;  // token of chunk i: tbase + 4*NT*i
  const RowView rv = row_view<BF16>(a, r);
  const int nl = halves * P;                                     // the row's lists
  const RowSlots rs = a.slots[r];
  const int64_t li = (int64_t)sl * halves + half;                // this task's list
  const int64_t slot = (int64_t)rs.rec + li;                     // ... and its record
  RowSync* sy = &a.sync[r];
  if (a.trace && tid == 0)
    a.trace[(size_t)blockIdx.x * 8] = (unsigned long long)r | ((unsigned long long)sl << 20) |
                                      (4ull << 28);
  CDS_TRACE(1);
  float x[EC][4];
  uint32_t nonfin = 0;
  load_chunks<NT, EC, BF16, VEC, true, false>(rv, lo, hi, 0, x, nonfin);
  // SPLIT: the draws do not depend on the plan: every token's Gumbel term is
  // computed now, while the row's plan is being made
  float g[SPLIT ? EC : 1][4];
  if (SPLIT) {
    const uint32_t k0 = (uint32_t)rp.seed, k1 = (uint32_t)(rp.seed >> 32);
    const uint32_t off_lo = (uint32_t)rp.offset, off_hi = (uint32_t)(rp.offset >> 32);
#pragma unroll
    for (int i = 0; i < (SPLIT ? EC : 0); ++i) {
      int32_t tb = tbase;
      asm volatile("" : "+v"(tb));
      const uint4 blk =
          philox4x32_10(make_uint4((uint32_t)(tb + 4 * NT * i) >> 2, off_lo, off_hi, 0u), k0, k1);
      g[i][0] = gumbel_fast(blk.x);
      g[i][1] = gumbel_fast(blk.y);
      g[i][2] = gumbel_fast(blk.z);
      g[i][3] = gumbel_fast(blk.w);
    }
  }
  if (tid == 0) {
    if (gen_wait(&sy->ready, a.gen, a.spin_limit)) {
      *s_plan = ld_obj(&a.plans[r]);
    } else {
      s_plan->mode = PLAN_NONE;
      st_u32(&sy->failed, a.gen);
    }
  }
  __syncthreads();
  CDS_TRACE(6);

  if (s_plan->mode == PLAN_FAST) {
    // plan values are uniform: keep them in scalar registers (the slice holds
    // 4*E4 vector registers)
    const float zmax = sgpr_f(s_plan->zmax);
    const float invT32 = sgpr_f((float)(1.0 / (double)rp.temperature));
    const uint32_t k0 = (uint32_t)rp.seed, k1 = (uint32_t)(rp.seed >> 32);
    const uint32_t off_lo = (uint32_t)rp.offset, off_hi = (uint32_t)(rp.offset >> 32);
    const float zc1 = sgpr_f(s_plan->zcut1);
    const float zs = fmaxf(fmaxf(sgpr_f(s_plan->z_sure), zc1), -FLT_MAX);
    const float a_lo = sgpr_f(s_plan->a_lo), a_hi = sgpr_f(s_plan->a_hi);
    const float k_lo = sgpr_f(s_plan->k_lo), k_hi = sgpr_f(s_plan->k_hi);
    const bool has_u = a_lo < a_hi || k_lo < k_hi;
    Top2 b = top2_init();
    // the race over the sure tokens: staged densely in LDS when they fit, so
    // that a wave draws only for tokens that race (not for every block in
    // which one of its lanes has one); else straight from registers
    // One listing pass for both lists: the sure tokens staged in LDS as (token,
    // value bits), and the boundary-bin tokens to the slice's global list.
    // Boundary: below zs, at or above zc1, inside [a_lo, a_hi) or [k_lo, k_hi).
    uint2* stage = reinterpret_cast<uint2*>(sh.fin.list);
    const uint32_t lcap = row_list_cap(rp.flags, rp.top_k, P);
    uint64_t* gl = a.ulist + (int64_t)rs.list64 * 64 + li * lcap;
    const float lo1 = fmaxf(a_lo, zc1), hi1 = fminf(a_hi, zs);
    const float lo2 = fmaxf(k_lo, zc1), hi2 = fminf(k_hi, zs);
    const uint2 nn = list_tokens2<NT, EC>(
        x, tbase, (uint32_t)UCAP, lcap, sh.sel.wt,
        [&](float v) { return !SPLIT && v >= zs; },
        [&](uint32_t pos, float v, int32_t t) {
          stage[pos] = make_uint2((uint32_t)t, __float_as_uint(v));
        },
        [&](float v) { return ((v >= lo1) & (v < hi1)) | ((v >= lo2) & (v < hi2)); },
        [&](uint32_t pos, float v, int32_t t) { st_u64(gl + pos, ulist_entry(v, t)); });
    const uint32_t nsure = nn.x, nst = has_u ? nn.y : 0u;
    __syncthreads();
    CDS_TRACE_SUB(0);
    if (SPLIT) {
      // the sure tokens race with the Gumbel terms drawn before the plan
#pragma unroll
      for (int i = 0; i < EC; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          race32_g_if(b, x[i][q] >= zs, x[i][q], tbase + 4 * NT * i + q, g[SPLIT ? i : 0][q],
                      zmax, invT32);
    } else if (nsure <= (uint32_t)UCAP) {
      race_list<NT>(
          b, (int)nsure, zmax, invT32,
          [&](int i, float& z, int32_t& t) {
            const uint2 e = stage[i];
            t = (int32_t)e.x;
            z = __uint_as_float(e.y);
          },
          [&](int32_t t0) {
            return philox4x32_10(make_uint4((uint32_t)t0 >> 2, off_lo, off_hi, 0u), k0, k1);
          });
    } else {
#pragma unroll
      for (int i = 0; i < EC; ++i) {
        int32_t tb = tbase;
        asm volatile("" : "+v"(tb));
        const int32_t t0 = tb + 4 * NT * i;
        bool need = false;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          need |= x[i][q] >= zs && race32_hopeful(b, x[i][q], zmax, invT32);
        if (need) {
          const uint4 blk =
              philox4x32_10(make_uint4((uint32_t)t0 >> 2, off_lo, off_hi, 0u), k0, k1);
          const uint32_t xs[4] = {blk.x, blk.y, blk.z, blk.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            race32_if(b, x[i][q] >= zs, x[i][q], t0 + q, xs[q], zmax, invT32);
        }
      }
    }
    CDS_TRACE_SUB(1);
    block_top2<NT>(b, red);
    if (tid == 0) {
      SliceBest sb;
      sb.k1 = b.k1;
      sb.t1 = b.t1;
      sb.z1 = b.z1;
      sb.k2 = b.k2;
      sb.ucnt = nst;
      sb.pad[0] = sb.pad[1] = sb.pad[2] = 0u;
      st_obj(&a.bests[slot], sb);
    }
  }

  CDS_TRACE_SUB(3);
  // the last slice of the row to finish its race resolves the row
  vm_drain();
  __syncthreads();
  CDS_TRACE_SUB(4);
  if (tid == 0) {
    const uint32_t t = take_ticket(&sy->done);
    if (t == (uint32_t)(nl - 1)) st_u64(&sy->done, 0ull);
    s_word[0] = t;
  }
  __syncthreads();
  CDS_TRACE_SUB(5);
  if (s_word[0] != (uint32_t)(nl - 1)) {
    CDS_TRACE(7);
    return;
  }
  if (tid == 0) s_word[0] = ld_u32(&sy->failed) == a.gen;
  __syncthreads();
  const bool failed = s_word[0] != 0u;
  const Plan pl = *s_plan;
  if (failed || pl.mode == PLAN_SLOW ||
      (pl.mode == PLAN_FAST &&
       !finish_row<NT, BF16, VEC>(a, r, nl, pl, sh.fin.ex, sh.fin.list, sh.fin.off, sh.fin.select,
                                  red))) {
    __syncthreads();
    row_exact<NT, BF16, VEC>(a, r, sh.fin.ex);
    if (tid == 0) a.plans[r].path = PATH_EXACT;
  }
  CDS_TRACE(7);
}

#ifndef CDS_WAVES_PER_EU
#define CDS_WAVES_PER_EU 4
#endif
// CDS_WAVES_PER_EU waves per SIMD (the slice takes 4*E4 vector registers).
template <int NT, int E4, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(CDS_WAVES_PER_EU))) void sample_kernel(
    const SampleArgs a) {
  __shared__ RedScratch<NT> red;
  __shared__ StatScratch<NT> sst;
  __shared__ FusedLds<NT> sh;
  __shared__ Plan s_plan;
  __shared__ uint32_t s_word[2];
  // Workgroups are dispatched round-robin over the kXcds XCDs.  Block b runs on
  // XCD x = b % kXcds as that XCD's j-th block (j = b / kXcds); it takes slice
  // j % P of the XCD's (j / P)-th task, task k = (j / P) * kXcds + x of the
  // packed task table.  All slices of a task then run on one XCD, next to each
  // other in its dispatch order; a pass-2 task comes after its row's pass-1
  // task in every XCD's order, so the pass-1 slices it waits for are running
  // or done.
  CDS_TRACE_SUB(6);
  const unsigned x = blockIdx.x % (unsigned)kXcds, j = blockIdx.x / (unsigned)kXcds;
  const int lr = (int)(j / (unsigned)a.P);
  const int sl = (int)(j - (unsigned)lr * (unsigned)a.P);
  const int k = lr * kXcds + (int)x;
  const int32_t tr = a.task_row[k];
  if (tr < 0) return;
  const int r = tr & kTaskRow;
  const RowParams rp = a.rows[r];
  if ((tr & kPass2) && (tr & kSplit))
    hold_race_task<NT, E4, true, BF16, VEC>(a, r, rp, sl, (tr & kHalf) ? 1 : 0, sh, red,
                                            &s_plan, s_word);
  else if (tr & kPass2)
    hold_race_task<NT, E4, false, BF16, VEC>(a, r, rp, sl, 0, sh, red, &s_plan, s_word);
  else if (rp.flags & ROW_GREEDY)  // read once: non-temporal loads
    slice_task<NT, E4, BF16, VEC, true, CLS_GREEDY>(a, r, rp, sl, sh, red, sst, &s_plan, s_word);
  else {
    const int c = row_class(rp, a.P);
    if (c == CLS_HOLD)  // its second pass reads the slice again
      slice_task<NT, E4, BF16, VEC, false, CLS_HOLD>(a, r, rp, sl, sh, red, sst, &s_plan, s_word);
    else if (c == CLS_LIST)  // LIST and RACE rows, read once
      slice_task<NT, E4, BF16, VEC, true, CLS_LIST>(a, r, rp, sl, sh, red, sst, &s_plan, s_word);
    else
      slice_task<NT, E4, BF16, VEC, true, CLS_RACE>(a, r, rp, sl, sh, red, sst, &s_plan, s_word);
  }
}

// ============================================================================
// launchers
// ============================================================================
hipError_t launch_transforms(const RowParams* rows, const int32_t* hist_raw, const PenEntry* pen,
                             const BiasEntry* bias, float* logits, int64_t ld, int32_t B,
                             hipStream_t stream) {
  hipLaunchKernelGGL(transforms_kernel, dim3(B), dim3(256), 0, stream, rows, hist_raw, pen, bias,
                     logits, ld);
  return hipGetLastError();
}

hipError_t launch_bitmask(void* logits, bool bf16, int64_t ld, int32_t B, int32_t V,
                          const int32_t* mask, int64_t mask_ld, const uint8_t* row_has_mask,
                          hipStream_t stream) {
  const int64_t W = ((int64_t)V + 31) / 32;
  const dim3 grid((unsigned)((W + 255) / 256), (unsigned)B);
  if (bf16)
    hipLaunchKernelGGL(bitmask_kernel<true>, grid, dim3(256), 0, stream, logits, ld, V, mask,
                       mask_ld, row_has_mask);
  else
    hipLaunchKernelGGL(bitmask_kernel<false>, grid, dim3(256), 0, stream, logits, ld, V, mask,
                       mask_ld, row_has_mask);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ptr), n);
  return hipGetLastError();
}

// ---- the library's own workspace (sampler_sample_static) ---------------------
// A file-scope device array, so that callers that cannot allocate (graph
// capture, allocation-free serving loops) need no workspace of their own.
// Each device the library runs on holds its copy until the process ends.  In
// host code `scratch` names a host-side stand-in: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kMaxStaticDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxStaticDevices];  // device address of `scratch` per device
}  // namespace

hipError_t static_workspace(void** ptr, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxStaticDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the row counters must start at zero (every call leaves them zero
    // again); a fill kernel, not a memset, so the call is capturable
    e = launch_fill_zero(p, workspace_layout(1, 1, 0, 0, 0).plan_off, stream);
    if (e != hipSuccess) return e;
    g_static_ptr[dev] = p;
  }
  *ptr = g_static_ptr[dev];
  return hipSuccess;
}

constexpr int kExactNT = 512;

static inline void rec(const KernelEvents* ev, bool start, hipStream_t s) {
  if (!ev) return;
  hipEvent_t e = start ? ev->start : ev->stop;
  if (e) (void)hipEventRecord(e, s);
}

template <bool BF16, bool VEC>
static hipError_t launch_fused(const SampleArgs& a, const KernelEvents* ev, hipStream_t s) {
  if (a.S > kSliceMax) return hipErrorInvalidValue;
  rec(ev, true, s);
  hipLaunchKernelGGL((sample_kernel<kScanThreads, kMaxChunks, BF16, VEC>),
                     dim3((unsigned)(a.n_groups * kXcds) * (unsigned)a.P),
                     dim3(kScanThreads), 0, s, a);
  rec(ev, false, s);
  return hipGetLastError();
}

template <bool BF16, bool VEC>
static hipError_t launch_any(const SampleArgs& a, int algo, const KernelEvents* ev,
                             hipStream_t s) {
  if (algo == 1) {
    rec(ev, true, s);
    hipLaunchKernelGGL((exact_kernel<kExactNT, BF16, VEC>), dim3((unsigned)a.B), dim3(kExactNT),
                       0, s, a);
    rec(ev, false, s);
    return hipGetLastError();
  }
  return launch_fused<BF16, VEC>(a, ev, s);
}

hipError_t launch_sample(const SampleArgs& a, bool bf16, bool vec, int algo,
                         const KernelEvents* ev, hipStream_t stream) {
  if (bf16)
    return vec ? launch_any<true, true>(a, algo, ev, stream)
               : launch_any<true, false>(a, algo, ev, stream);
  return vec ? launch_any<false, true>(a, algo, ev, stream)
             : launch_any<false, false>(a, algo, ev, stream);
}

}  // namespace cds
