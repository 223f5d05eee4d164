// kernels.hip -- HIP kernels of libcd_sampler.so for gfx950 (MI355X).
//
// The sampling step for rows that are not greedy runs as three kernels:
//
//   scan    grid (P, B): one workgroup per slice of S tokens.  Streams the
//           slice from HBM once into registers (bf16 upcast and the grammar
//           bitmask fused into the load), reduces max / argmax / finite count /
//           sum exp, and for rows with a top-k or top-p cut builds a histogram
//           of s = z/T over bins of width 1/16 aligned to an absolute grid
//           (counts, and fixed-point masses relative to each bin's upper edge,
//           so slices merge by integer addition).  The last slice of a row to
//           finish (atomic ticket) merges the slices, writes greedy / invalid
//           rows' outputs, and for the rest writes a plan: the exact min-p cut,
//           the value range of "sure" tokens (certainly inside the final
//           candidate set), and the value ranges of the bins that hold the top-k
//           and top-p boundaries.
//   race    grid (P, B): re-reads the slice; runs the exponential race over the
//           sure tokens and appends the boundary-bin tokens to a per-row list.
//   finish  grid (B): sorts the boundary list in LDS, finds the exact top-k
//           value, the exact top-p cut (fp64 cumulative mass in sorted order),
//           races the boundary tokens that survive, merges with the slices'
//           winners and writes the output.  Rows whose boundary list would not
//           fit in LDS, and rows whose plan the exact pass contradicts, run the
//           row-serial exact path instead.
//
// The row-serial exact path (row_exact) does everything with one workgroup
// and several passes over the row: radix select for the k-th largest value,
// a mass-weighted radix select for the top-p cut (fixed-point masses), then
// the race.  It is also selectable for all rows (SAMPLER_OPT_ALGO = 1).
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

#include "device_common.h"
#include "kernels.h"

namespace cds {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void write_out(const SampleArgs& a, int r, int32_t id, float lp,
                                          int32_t st) {
  a.out_ids[r] = id;
  if (a.out_lp) a.out_lp[r] = lp;
  if (a.out_st) a.out_st[r] = st;
}

template <bool BF16>
__device__ __forceinline__ RowView row_view(const SampleArgs& a, int r) {
  RowView v;
  if (BF16) {
    v.b16 = static_cast<const uint16_t*>(a.logits) + (int64_t)r * a.ld;
    v.f32 = nullptr;
  } else {
    v.f32 = static_cast<const float*>(a.logits) + (int64_t)r * a.ld;
    v.b16 = nullptr;
  }
  v.mrow = (a.mask && (!a.row_has_mask || a.row_has_mask[r])) ? a.mask + (int64_t)r * a.mask_ld
                                                              : nullptr;
  return v;
}

// Smallest fp32 value v with exp(v/T - m) >= min_p (the min-p set is then
// {z >= v}); -inf when every finite value qualifies.  Same expression as the
// set definition, evaluated on fp32 values by bisection over order keys.
__device__ float minp_cut(float zmax, double Td, double m, float min_p) {
  const double mp = (double)min_p;
  if (exp((double)(-FLT_MAX) / Td - m) >= mp) return CDS_NEG_INF;
  uint32_t lo = okey(-FLT_MAX), hi = okey(zmax);
  while (hi - lo > 1u) {
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (exp((double)from_okey(mid) / Td - m) >= mp)
      hi = mid;
    else
      lo = mid;
  }
  return from_okey(hi);
}

// ============================================================================
// transforms and bitmask (in place)
// ============================================================================
__global__ __launch_bounds__(256) void transforms_kernel(const RowParams* rows,
                                                         const PenEntry* pen,
                                                         const BiasEntry* bias, float* logits,
                                                         int64_t ld) {
  const int r = blockIdx.x;
  const RowParams rp = rows[r];
  float* z = logits + (int64_t)r * ld;
  if (rp.flags & ROW_PEN) {
    for (int i = rp.pen_lo + (int)threadIdx.x; i < rp.pen_hi; i += blockDim.x) {
      const PenEntry e = pen[i];
      float v = z[e.id];
      const float p = __fadd_rn(__fmul_rn(rp.freq, (float)e.count), rp.pres);
      v = __fsub_rn(v, p);
      if (rp.rep != 1.0f) v = (v > 0.0f) ? __fdiv_rn(v, rp.rep) : __fmul_rn(v, rp.rep);
      z[e.id] = v;
    }
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
template <int NT>
struct ExactShared {
  RedScratch<NT> red;
  unsigned long long hist[256];
  unsigned long long scan[256];
  unsigned long long wtot[NT / 64];
  int32_t pick;
  float fshare;
};

// Visit every token of the row in groups of four (t0 % 4 == 0).
template <int NT, bool BF16, bool VEC, typename F>
__device__ __forceinline__ void for_row4(const RowView& rv, int64_t V, uint32_t& nonfin, F f) {
  for (int64_t t0 = 4 * (int64_t)threadIdx.x; t0 < V; t0 += 4 * (int64_t)NT) {
    float x[4];
    load4<BF16, VEC>(rv, t0, V, x, nonfin);
    f(x, t0);
  }
}

// hist[256] holds per-digit totals (digit = bucket of values, larger digit =
// larger values).  Returns the largest digit d with base + (total over digits
// >= d) >= need, and sets *above = base + total over digits > d.
template <int NT>
__device__ int pick_digit(ExactShared<NT>& sh, double need, unsigned long long base,
                          unsigned long long* above) {
  if (threadIdx.x < 256) sh.scan[threadIdx.x] = sh.hist[255 - threadIdx.x];
  if (threadIdx.x == 0) sh.pick = 256;
  __syncthreads();
  block_scan_inplace<NT>(
      sh.scan, 256, 0ull, [](unsigned long long x, unsigned long long y) { return x + y; },
      sh.wtot);
  if (threadIdx.x < 256 && (double)(base + sh.scan[threadIdx.x]) >= need)
    atomicMin(&sh.pick, (int)threadIdx.x);
  __syncthreads();
  const int i = sh.pick < 256 ? sh.pick : 255;
  *above = base + (i > 0 ? sh.scan[i - 1] : 0ull);
  __syncthreads();
  return 255 - i;
}

template <int NT, bool BF16, bool VEC>
__device__ void row_exact(const SampleArgs& a, int r, ExactShared<NT>& sh) {
  const RowParams rp = a.rows[r];
  const RowView rv = row_view<BF16>(a, r);
  const int64_t V = a.V;
  const bool greedy = (rp.flags & ROW_GREEDY) != 0;
  uint32_t nonfin = 0;
  float zm = CDS_NEG_INF;
  int32_t am = INT_MAX;
  int32_t nf = 0;
  for_row4<NT, BF16, VEC>(rv, V, nonfin, [&](const float* x, int64_t t0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (x[q] > zm) {
        zm = x[q];
        am = (int32_t)(t0 + q);
      }
      nf += (x[q] != CDS_NEG_INF);
    }
  });
  block_argmax<NT>(zm, am, sh.red);
  nf = block_sum_i32<NT>(nf, sh.red);
  nonfin = block_or_u32<NT>(nonfin, sh.red);
  if (nf == 0) {
    if (threadIdx.x == 0) write_out(a, r, -1, CDS_NEG_INF, 2);
    return;
  }
  if (nonfin) {
    if (threadIdx.x == 0) write_out(a, r, -1, __builtin_nanf(""), 1);
    return;
  }
  const double invTe = greedy ? 1.0 : 1.0 / (double)rp.temperature;
  const float invTe32 = (float)invTe;
  double se = 0.0;
  for_row4<NT, BF16, VEC>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (x[q] != CDS_NEG_INF) se += (double)exp2f((x[q] - zm) * invTe32 * kLog2e);
  });
  se = block_sum_f64<NT>(se, sh.red);
  if (greedy) {
    if (threadIdx.x == 0) write_out(a, r, am, (float)(-log(se)), 0);
    return;
  }
  const double Td = (double)rp.temperature;
  const double m = (double)zm / Td;
  const double log_z = log(se);

  // min-p: exact value cut
  float zcut = CDS_NEG_INF;
  if (rp.flags & ROW_MINP) {
    if (threadIdx.x == 0) sh.fshare = minp_cut(zm, Td, m, rp.min_p);
    __syncthreads();
    zcut = sh.fshare;
    __syncthreads();
  }

  // top-k: radix select of the k-th largest value (8-bit digits of the order key)
  if ((rp.flags & ROW_TOPK) && rp.top_k < nf) {
    uint32_t prefix = 0, pmask = 0;
    unsigned long long krem = (unsigned long long)rp.top_k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0ull;
      __syncthreads();
      for_row4<NT, BF16, VEC>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (x[q] == CDS_NEG_INF) continue;
          const uint32_t u = okey(x[q]);
          if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], 1ull);
        }
      });
      __syncthreads();
      unsigned long long above;
      const int d = pick_digit<NT>(sh, (double)krem, 0ull, &above);
      krem -= above;
      prefix |= (uint32_t)d << shift;
      pmask |= 255u << shift;
    }
    zcut = fmaxf(zcut, from_okey(prefix));
  }

  // top-p: mass-weighted radix select on fixed-point masses exp(s - m) * 2^sc
  if (rp.flags & ROW_TOPP) {
    int lg = 0;
    while ((1ll << lg) < V) ++lg;
    const double scale = ldexp(1.0, 62 - lg);
    const float zc = zcut;
    auto wfix = [&](float v) -> unsigned long long {
      return (unsigned long long)(exp((double)v / Td - m) * scale + 0.5);
    };
    unsigned long long msum = 0;
    for_row4<NT, BF16, VEC>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (x[q] != CDS_NEG_INF && x[q] >= zc) msum += wfix(x[q]);
    });
    msum = block_sum_u64<NT>(msum, sh.red);
    const double need = (double)rp.top_p * (double)msum;
    uint32_t prefix = 0, pmask = 0;
    unsigned long long base = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0ull;
      __syncthreads();
      for_row4<NT, BF16, VEC>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (x[q] == CDS_NEG_INF || x[q] < zc) continue;
          const uint32_t u = okey(x[q]);
          if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], wfix(x[q]));
        }
      });
      __syncthreads();
      unsigned long long above;
      const int d = pick_digit<NT>(sh, need, base, &above);
      base = above;
      prefix |= (uint32_t)d << shift;
      pmask |= 255u << shift;
    }
    zcut = fmaxf(zcut, from_okey(prefix));
  }

  // the race over {z >= zcut}
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
  if (threadIdx.x == 0) write_out(a, r, b.t, (float)((double)b.z / Td - m - log_z), 0);
}

template <int NT, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void exact_kernel(const SampleArgs a) {
  __shared__ ExactShared<NT> es;
  row_exact<NT, BF16, VEC>(a, blockIdx.x, es);
}

// ============================================================================
// fast path, kernel 1: scan (one HBM pass per slice, register resident)
// ============================================================================
template <int NT, int E4, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void scan_kernel(const SampleArgs a) {
  __shared__ RedScratch<NT> red;
  __shared__ unsigned long long s_hist[NBINS + 32];
  const int r = blockIdx.y, sl = blockIdx.x, tid = threadIdx.x;
  const RowParams rp = a.rows[r];
  const bool greedy = (rp.flags & ROW_GREEDY) != 0;
  const bool hist = !greedy && (rp.flags & (ROW_TOPK | ROW_TOPP));
  const int64_t lo = (int64_t)sl * a.S;
  const int64_t hi = min(lo + a.S, (int64_t)a.V);
  const RowView rv = row_view<BF16>(a, r);

  float x[E4][4];
  uint32_t nonfin = 0;
  load_chunks<NT, E4, BF16, VEC>(rv, lo, hi, 0, x, nonfin);

  // max, then the lowest index holding it (searched only by threads that hold it)
  float lm = CDS_NEG_INF;
#pragma unroll
  for (int i = 0; i < E4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) lm = fmaxf(lm, x[i][q]);
  const float zm = block_max_f32<NT>(lm, red);
  int32_t am = INT_MAX;
  if (zm != CDS_NEG_INF && lm == zm) {
#pragma unroll
    for (int i = E4 - 1; i >= 0; --i)
#pragma unroll
      for (int q = 3; q >= 0; --q)
        if (x[i][q] == zm) am = (int32_t)(lo + 4 * ((int64_t)i * NT + tid) + q);
  }
  am = block_min_i32<NT>(am, red);
  nonfin = block_or_u32<NT>(nonfin, red);

  const int64_t slot = (int64_t)r * a.P + sl;
  uint32_t flags = nonfin ? SLICE_NONFINITE : 0u;
  double se = 0.0;
  float kmax = 0.0f;
  if (!hist) {
    // sum exp((z - zmax) / T_eff): the row's log-partition for the logprob
    const float c = (greedy ? 1.0f : (float)(1.0 / (double)rp.temperature)) * kLog2e;
    if (zm != CDS_NEG_INF) {
#pragma unroll
      for (int i = 0; i < E4; ++i) {
        float part = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) part += __builtin_amdgcn_exp2f((x[i][q] - zm) * c);
        se += (double)part;
      }
    }
    se = block_sum_f64<NT>(se, red);
  } else if (zm != CDS_NEG_INF) {
    // histogram of the values below the slice maximum, bins aligned to delta
    const BinGeom g = bin_geom(rp.temperature);
    kmax = floorf(zm * g.inv_delta);
    if (!(fabsf(kmax) < 4194304.0f)) {
      flags |= SLICE_BINS_LOST;  // bin indices would not be exact: row takes the exact path
    } else {
      for (int b = tid; b < NBINS + 32; b += NT) s_hist[b] = 0ull;
      __syncthreads();
      // tokens outside the window (and -inf) land in 32 per-lane sink bins:
      // no branch per token
      const int sink = NBINS + (tid & 31);
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
          atomicAdd(&s_hist[rb], (1ull << kCountShift) | (unsigned long long)fix);
        }
      __syncthreads();
      unsigned long long* gh = a.hist + slot * NBINS;
      for (int b = tid; b < NBINS; b += NT) gh[b] = s_hist[b];
    }
  }
  if (tid == 0) {
    SliceHead h;
    h.zmax = zm;
    h.arg = (zm == CDS_NEG_INF) ? -1 : am;
    h.flags = flags;
    h.kmax = kmax;
    h.sumexp = se;
    h.pad[0] = h.pad[1] = 0u;
    a.heads[slot] = h;
  }
}

// ============================================================================
// fast path, kernel 2: plan (one workgroup per row)
// ============================================================================
template <int NT>
struct PlanShared {
  SliceHead head[kMaxSlices];
  double md[NBINS];                 // per-bin mass relative to exp(m), then scanned
  uint32_t cumc[NBINS];             // per-bin count, then scanned
  unsigned long long accm[NBINS];   // merge accumulators
  uint32_t accc[NBINS];
  double wtot_d[NT / 64];
  uint32_t wtot_u[NT / 64];
  int idx[3];
  int mode, inK, k_rank, rb12;
  uint32_t lost;
  float zmax, zcut1, kmax;
  int32_t arg;
  double m, log_z, tlo, thi;
};

template <int NT>
__global__ __launch_bounds__(NT) void plan_kernel(const SampleArgs a) {
  __shared__ PlanShared<NT> ps;
  const int r = blockIdx.x, tid = threadIdx.x, P = a.P;
  const RowParams rp = a.rows[r];
  const bool greedy = (rp.flags & ROW_GREEDY) != 0;
  const bool topk = (rp.flags & ROW_TOPK) != 0, topp = (rp.flags & ROW_TOPP) != 0;
  const bool hist = !greedy && (topk || topp);
  const double Td = (double)rp.temperature;
  if (tid < P) ps.head[tid] = a.heads[(int64_t)r * P + tid];
  __syncthreads();
  if (tid == 0) {
    float zm = CDS_NEG_INF;
    int32_t am = INT_MAX;
    uint32_t fl = 0;
    for (int j = 0; j < P; ++j) {
      const SliceHead& h = ps.head[j];
      fl |= h.flags;
      if (h.zmax != CDS_NEG_INF && (h.zmax > zm || (h.zmax == zm && h.arg < am))) {
        zm = h.zmax;
        am = h.arg;
      }
    }
    const double invTe = greedy ? 1.0 : 1.0 / Td;
    double Z = 0.0;
    if (!hist)
      for (int j = 0; j < P; ++j)
        if (ps.head[j].zmax != CDS_NEG_INF)
          Z += ps.head[j].sumexp * exp(((double)ps.head[j].zmax - (double)zm) * invTe);
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
    }
    ps.mode = mode;
    ps.zmax = zm;
    ps.arg = am;
    ps.m = (double)zm / Td;
    ps.log_z = log(Z);
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

  auto write_plan = [&](int mode) {
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
    if (tid == 0) a.plans[r] = write_plan(ps.mode);
    return;
  }

  // merge the slices' histograms: row bin = slice bin + (row kmax - slice kmax)
  const BinGeom g = bin_geom(rp.temperature);
  const float kmax = floorf(ps.zmax * g.inv_delta);
  for (int b = tid; b < NBINS; b += NT) {
    ps.accm[b] = 0ull;
    ps.accc[b] = 0u;
  }
  __syncthreads();
#pragma unroll 4
  for (int e = tid; e < P * NBINS; e += NT) {
    const int j = e / NBINS, sb = e - j * NBINS;
    const unsigned long long v = a.hist[((int64_t)r * P + j) * NBINS + sb];
    if (v == 0ull || ps.head[j].zmax == CDS_NEG_INF) continue;
    const float rowbin = (kmax - ps.head[j].kmax) + (float)sb;
    if (rowbin >= (float)NBINS) continue;
    atomicAdd(&ps.accc[(int)rowbin], (uint32_t)(v >> kCountShift));
    atomicAdd(&ps.accm[(int)rowbin], v & ((1ull << kCountShift) - 1ull));
  }
  __syncthreads();
  const double m = ps.m;
  for (int b = tid; b < NBINS; b += NT) {
    ps.cumc[b] = ps.accc[b];
    // bin b spans [(kmax-b)*delta, (kmax-b+1)*delta); masses are relative to its top
    const double top = ((double)kmax + 1.0 - (double)b) * (double)g.delta;
    ps.md[b] = (double)ps.accm[b] * 0x1p-31 * exp(top / Td - m);
  }
  __syncthreads();
  block_scan_inplace<NT>(ps.cumc, NBINS, 0u, [](uint32_t x, uint32_t y) { return x + y; },
                         ps.wtot_u);
  block_scan_inplace<NT>(ps.md, NBINS, 0.0, [](double x, double y) { return x + y; },
                         ps.wtot_d);
  if (tid < 3) ps.idx[tid] = NBINS;
  __syncthreads();
  if (topk)
    for (int b = tid; b < NBINS; b += NT)
      if (ps.cumc[b] >= (uint32_t)rp.top_k) atomicMin(&ps.idx[0], b);
  __syncthreads();
  if (tid == 0) {
    ps.log_z = log(ps.md[NBINS - 1]);
    const int rb2 = ps.idx[0];
    int rb1 = NBINS;
    if (ps.zcut1 != CDS_NEG_INF) {
      const float rbf = kmax - floorf(ps.zcut1 * g.inv_delta);
      rb1 = rbf >= (float)NBINS ? NBINS : (int)rbf;
    }
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
  __syncthreads();
  if (topp)
    for (int b = tid; b < NBINS; b += NT) {
      if (ps.md[b] >= ps.tlo) atomicMin(&ps.idx[1], b);
      if (ps.md[b] >= ps.thi) atomicMin(&ps.idx[2], b);
    }
  __syncthreads();
  if (tid == 0) {
    const int cap = ps.rb12 < NBINS ? ps.rb12 : NBINS - 1;
    const int rb3_hi = min(ps.idx[2], cap);
    const int rb3_lo = min(ps.idx[1], rb3_hi);
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
    Plan pl = write_plan(uexp > (uint32_t)UCAP ? PLAN_SLOW : PLAN_FAST);
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
    a.plans[r] = pl;
  }
}

// ============================================================================
// fast path, kernel 3: race over the sure tokens, compact the boundary tokens
// ============================================================================
template <int NT, int E4, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void race_kernel(const SampleArgs a) {
  __shared__ RedScratch<NT> red;
  const int r = blockIdx.y, sl = blockIdx.x, tid = threadIdx.x;
  const Plan pl = a.plans[r];
  if (pl.mode != PLAN_FAST) return;
  const RowParams rp = a.rows[r];
  const int64_t lo = (int64_t)sl * a.S;
  const int64_t hi = min(lo + a.S, (int64_t)a.V);
  const RowView rv = row_view<BF16>(a, r);
  const RaceCtx c = make_race_ctx(rp, pl.zmax);
  const float zs = fmaxf(pl.z_sure, pl.zcut1);
  const bool has_u = pl.a_lo < pl.a_hi || pl.k_lo < pl.k_hi;
  Top2 b = top2_init();
  uint64_t* ul = a.ulist + (int64_t)r * UCAP;
  uint32_t* ucount = &a.sync[r].ucount;
  const int lane = tid & 63;
  uint32_t nonfin = 0;
  constexpr int G = E4 < 4 ? E4 : 4;
#pragma unroll 1
  for (int g = 0; g < E4; g += G) {
    float x[G][4];
    load_chunks<NT, G, BF16, VEC>(rv, lo, hi, g, x, nonfin);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int64_t t0 = lo + 4 * ((int64_t)(g + i) * NT + tid);
      bool need = false;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        need |= (x[i][q] >= zs && x[i][q] != CDS_NEG_INF &&
                 race32_hopeful(b, x[i][q], c.zmax, c.invT32));
      if (need) {
        const uint4 blk = race_block(c, t0);
        const uint32_t xs[4] = {blk.x, blk.y, blk.z, blk.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (x[i][q] >= zs && x[i][q] != CDS_NEG_INF)
            race32(b, x[i][q], (int32_t)(t0 + q), xs[q], c.zmax, c.invT32);
      }
      if (has_u) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = x[i][q];
          const bool isU = v < zs && v >= pl.zcut1 &&
                           ((v >= pl.a_lo && v < pl.a_hi) || (v >= pl.k_lo && v < pl.k_hi));
          const unsigned long long msk = __ballot(isU);
          if (msk) {
            const int leader = __ffsll((long long)msk) - 1;
            uint32_t base = 0;
            if (lane == leader) base = atomicAdd(ucount, (uint32_t)__popcll(msk));
            base = __shfl(base, leader, 64);
            if (isU) {
              const uint32_t pos = base + (uint32_t)__popcll(msk & __lanemask_lt());
              if (pos < (uint32_t)UCAP)
                ul[pos] = ((uint64_t)okey(v + 0.0f) << 32) |
                          (uint64_t)(0xFFFFFFFFu - (uint32_t)(t0 + q));
            }
          }
        }
      }
    }
  }
  block_top2<NT>(b, red);
  if (tid == 0) {
    SliceBest sb;
    sb.k1 = b.k1;
    sb.t1 = b.t1;
    sb.z1 = b.z1;
    sb.k2 = b.k2;
    a.bests[(int64_t)r * a.P + sl] = sb;
  }
}

// ============================================================================
// fast path, kernel 4: exact cuts on the boundary list, race it, merge, output
// ============================================================================
template <int NT>
struct FinishShared {
  unsigned long long key[UCAP];
  double w[UCAP];
  int32_t g[UCAP];
  double wtot_d[NT / 64];
  int32_t wtot_i[NT / 64];
  RedScratch<NT> red;
  uint32_t z3key;
  int32_t lastA;
  int32_t has3;
  int32_t fail;
  int32_t ambiguous;
  float zfinal;
  float k1;
};

__device__ __forceinline__ float ukey_z(unsigned long long k) { return from_okey((uint32_t)(k >> 32)); }
__device__ __forceinline__ int32_t ukey_t(unsigned long long k) {
  return (int32_t)(0xFFFFFFFFu - (uint32_t)k);
}

// fp64 race over {z >= zfinal} for tokens whose fp32 key reaches k_floor: the
// tie-breaker when the fp32 top two are within the fp32 error.
template <int NT, bool BF16, bool VEC>
__device__ Best exact_rerace(const SampleArgs& a, int r, float zfinal, float k_floor,
                             RedScratch<NT>& red) {
  const RowParams rp = a.rows[r];
  const RowView rv = row_view<BF16>(a, r);
  const Plan pl = a.plans[r];
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

template <int NT, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void finish_kernel(const SampleArgs a) {
  __shared__ FinishShared<NT> fs;
  __shared__ ExactShared<NT> es;
  const int r = blockIdx.x, tid = threadIdx.x;
  const Plan pl = a.plans[r];
  if (pl.mode != PLAN_FAST && pl.mode != PLAN_SLOW) return;
  const uint32_t n_raw = a.sync[r].ucount;
  __syncthreads();
  if (tid == 0) a.sync[r].ucount = 0u;  // ready for the next call
  if (pl.mode == PLAN_SLOW || n_raw > (uint32_t)UCAP) {
    row_exact<NT, BF16, VEC>(a, r, es);
    if (tid == 0) a.plans[r].path = PATH_EXACT;
    return;
  }
  const RowParams rp = a.rows[r];
  const double Td = (double)rp.temperature;
  const int n = (int)n_raw;
  int N = 1;
  while (N < n) N <<= 1;
  for (int i = tid; i < N; i += NT) fs.key[i] = i < n ? a.ulist[(int64_t)r * UCAP + i] : 0ull;
  if (tid == 0) {
    fs.z3key = 0xFFFFFFFFu;
    fs.lastA = -1;
    fs.has3 = 0;
    fs.fail = 0;
    fs.ambiguous = 0;
  }
  __syncthreads();
  // bitonic sort, descending: larger value first, then lower token index
  for (int k = 2; k <= N; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < N; i += NT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long p = fs.key[i], q = fs.key[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (p < q) : (p > q)) {
            fs.key[i] = q;
            fs.key[ixj] = p;
          }
        }
      }
      __syncthreads();
    }

  // exact top-k value: the k_rank-th largest token of the boundary bin
  float zc12 = pl.zcut1;
  if (pl.k_rank > 0) {
    int ch = 0, cl = 0;
    for (int i = tid; i < n; i += NT) {
      const float z = ukey_z(fs.key[i]);
      ch += (z >= pl.k_hi);
      cl += (z >= pl.k_lo);
    }
    ch = block_sum_i32<NT>(ch, fs.red);
    cl = block_sum_i32<NT>(cl, fs.red);
    const int idx = ch + pl.k_rank - 1;
    if (idx < cl) zc12 = fmaxf(zc12, ukey_z(fs.key[idx]));
  }
  float zfin = zc12;

  // exact top-p cut: fp64 masses in sorted order, tie groups all in or out
  if (pl.topp) {
    for (int i = tid; i < n; i += NT) {
      const float z = ukey_z(fs.key[i]);
      fs.w[i] = (z >= zc12) ? exp((double)z / Td - pl.m) : 0.0;
      fs.g[i] = (i == 0 || z != ukey_z(fs.key[i - 1])) ? i : 0;
    }
    __syncthreads();
    block_scan_inplace<NT>(fs.w, n, 0.0, [](double x, double y) { return x + y; }, fs.wtot_d);
    block_scan_inplace<NT>(fs.g, n, 0, [](int32_t x, int32_t y) { return max(x, y); },
                           fs.wtot_i);
    const double M2 = pl.m_sure + pl.m_mid + (n > 0 ? fs.w[n - 1] : 0.0);
    const double target = pl.p * M2;
    for (int i = tid; i < n; i += NT) {
      const float z = ukey_z(fs.key[i]);
      if (!(z >= pl.a_lo && z < pl.a_hi && z >= zc12)) continue;
      atomicMax(&fs.lastA, i);
      const int g = fs.g[i];
      const double above = pl.m_sure + (g > 0 ? fs.w[g - 1] : 0.0);
      if (above < target) {
        atomicMin(&fs.z3key, okey(z));
        fs.has3 = 1;
      }
    }
    __syncthreads();
    if (tid == 0) {
      if (!fs.has3) {
        fs.fail = 1;  // the cut lies above the boundary range
      } else if (fs.lastA >= 0) {
        const float zl = ukey_z(fs.key[fs.lastA]);
        if (zl >= from_okey(fs.z3key) && pl.m_sure + fs.w[fs.lastA] < target)
          fs.fail = 1;  // ... or below it
      }
    }
    __syncthreads();
    if (!fs.fail) zfin = fmaxf(zfin, from_okey(fs.z3key));
  }
  if (fs.fail) {
    row_exact<NT, BF16, VEC>(a, r, es);
    if (tid == 0) a.plans[r].path = PATH_EXACT;
    return;
  }

  // race the boundary tokens that survive, merge with the slices' top two
  const RaceCtx c = make_race_ctx(rp, pl.zmax);
  Top2 b = top2_init();
  for (int i = tid; i < n; i += NT) {
    const float z = ukey_z(fs.key[i]);
    if (!(z >= zfin)) continue;
    const int32_t t = ukey_t(fs.key[i]);
    if (!race32_hopeful(b, z, c.zmax, c.invT32)) continue;
    const uint4 blk = race_block(c, (int64_t)(t & ~3));
    const int w = t & 3;
    const uint32_t xw = w == 0 ? blk.x : (w == 1 ? blk.y : (w == 2 ? blk.z : blk.w));
    race32(b, z, t, xw, c.zmax, c.invT32);
  }
  block_top2<NT>(b, fs.red);
  if (tid == 0) {
    for (int j = 0; j < a.P; ++j) {
      const SliceBest sb = a.bests[(int64_t)r * a.P + j];
      Top2 o;
      o.k1 = sb.k1;
      o.t1 = sb.t1;
      o.z1 = sb.z1;
      o.k2 = sb.k2;
      top2_merge(b, o);
    }
    const float zs = fmaxf(pl.z_sure, pl.zcut1);
    fs.zfinal = (pl.topp || pl.k_rank > 0) ? zfin : zs;
    fs.k1 = b.k1;
    if (b.t1 == INT_MAX) {
      fs.fail = 1;
    } else if (!(b.k1 - b.k2 > 2.0f * kRaceEps)) {
      fs.ambiguous = 1;
    } else {
      write_out(a, r, b.t1, (float)((double)b.z1 / Td - pl.m - pl.log_z), 0);
      a.plans[r].path = PATH_FAST;
    }
  }
  __syncthreads();
  if (fs.fail) {
    row_exact<NT, BF16, VEC>(a, r, es);
    if (tid == 0) a.plans[r].path = PATH_EXACT;
  } else if (fs.ambiguous) {
    const Best e = exact_rerace<NT, BF16, VEC>(a, r, fs.zfinal, fs.k1 - 2.0f * kRaceEps, fs.red);
    if (tid == 0) {
      write_out(a, r, e.t, (float)((double)e.z / Td - pl.m - pl.log_z), 0);
      a.plans[r].path = PATH_RERACE;
    }
  }
}

// ============================================================================
// launchers
// ============================================================================
hipError_t launch_transforms(const RowParams* rows, const PenEntry* pen, const BiasEntry* bias,
                             float* logits, int64_t ld, int32_t B, hipStream_t stream) {
  hipLaunchKernelGGL(transforms_kernel, dim3(B), dim3(256), 0, stream, rows, pen, bias, logits,
                     ld);
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

constexpr int kPlanNT = 256;
constexpr int kFinishNT = 512;

static inline void rec(const KernelEvents* ev, bool start, int k, hipStream_t s) {
  if (!ev) return;
  hipEvent_t e = start ? ev->start[k] : ev->stop[k];
  if (e) (void)hipEventRecord(e, s);
}

template <int E4, bool BF16, bool VEC>
static hipError_t launch_fast(const SampleArgs& a, bool need_race, const KernelEvents* ev,
                              hipStream_t s) {
  const dim3 grid((unsigned)a.P, (unsigned)a.B);
  rec(ev, true, 0, s);
  hipLaunchKernelGGL((scan_kernel<kScanThreads, E4, BF16, VEC>), grid, dim3(kScanThreads), 0, s,
                     a);
  rec(ev, false, 0, s);
  rec(ev, true, 3, s);
  hipLaunchKernelGGL((plan_kernel<kPlanNT>), dim3((unsigned)a.B), dim3(kPlanNT), 0, s, a);
  rec(ev, false, 3, s);
  if (need_race) {
    rec(ev, true, 1, s);
    hipLaunchKernelGGL((race_kernel<kScanThreads, E4, BF16, VEC>), grid, dim3(kScanThreads), 0,
                       s, a);
    rec(ev, false, 1, s);
    rec(ev, true, 2, s);
    hipLaunchKernelGGL((finish_kernel<kFinishNT, BF16, VEC>), dim3((unsigned)a.B),
                       dim3(kFinishNT), 0, s, a);
    rec(ev, false, 2, s);
  }
  return hipGetLastError();
}

template <bool BF16, bool VEC>
static hipError_t launch_fast_e4(const SampleArgs& a, bool need_race, const KernelEvents* ev,
                                 hipStream_t s) {
  const int64_t e4 = (a.S + 4 * kScanThreads - 1) / (4 * kScanThreads);
  if (e4 <= 1) return launch_fast<1, BF16, VEC>(a, need_race, ev, s);
  if (e4 <= 2) return launch_fast<2, BF16, VEC>(a, need_race, ev, s);
  if (e4 <= 4) return launch_fast<4, BF16, VEC>(a, need_race, ev, s);
  if (e4 <= 8) return launch_fast<8, BF16, VEC>(a, need_race, ev, s);
  if (e4 <= 12) return launch_fast<12, BF16, VEC>(a, need_race, ev, s);
  if (e4 <= 16) return launch_fast<16, BF16, VEC>(a, need_race, ev, s);
  if (e4 <= 20) return launch_fast<20, BF16, VEC>(a, need_race, ev, s);
  return hipErrorInvalidValue;
}

template <bool BF16, bool VEC>
static hipError_t launch_any(const SampleArgs& a, int algo, bool need_race,
                             const KernelEvents* ev, hipStream_t s) {
  if (algo == 1) {
    rec(ev, true, 0, s);
    hipLaunchKernelGGL((exact_kernel<kFinishNT, BF16, VEC>), dim3((unsigned)a.B),
                       dim3(kFinishNT), 0, s, a);
    rec(ev, false, 0, s);
    return hipGetLastError();
  }
  return launch_fast_e4<BF16, VEC>(a, need_race, ev, s);
}

hipError_t launch_sample(const SampleArgs& a, bool bf16, bool vec, int algo, bool need_race,
                         const KernelEvents* ev, hipStream_t stream) {
  if (bf16)
    return vec ? launch_any<true, true>(a, algo, need_race, ev, stream)
               : launch_any<true, false>(a, algo, need_race, ev, stream);
  return vec ? launch_any<false, true>(a, algo, need_race, ev, stream)
             : launch_any<false, false>(a, algo, need_race, ev, stream);
}

}  // namespace cds
