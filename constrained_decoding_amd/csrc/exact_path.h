// exact_path.h -- building blocks of the row-serial exact path: one
// workgroup per row and several passes over it, each pass streaming the row
// (the row stays in L2 / the last-level cache between passes).  Used by the
// sampling kernel's exact fallback and by the logprob-outputs kernel.
//
// Set definitions ("SGLang 源码完全拆解(十)", section 概率裁剪的数学; order
// min-p -> top-k -> top-p, "GLM-5.3 推理全链路(七)", section 采样; the other
// filter orders, SGLang page section 后端分支): the kept set is
// {allowed z >= zcut} for one value threshold zcut, found by exact selection
// on fp32 values (no sort).
#pragma once
#include <cfloat>

#include "device_common.h"
#include "kernels.h"
#include "layout.h"

namespace cds {

// Row r of the logits (and of the bitmask, if the row has one).
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

constexpr float kLog2e = 1.4426950408889634f;

// Smallest fp32 value v with exp(v/T - m) >= min_p (the min-p set is then
// {z >= v}); -inf when every finite value qualifies.  Same expression as the
// set definition, evaluated on fp32 values by bisection over order keys.
__device__ __forceinline__ float minp_cut(float zmax, double Td, double m, float min_p) {
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

template <int NT>
struct ExactShared {
  RedScratch<NT> red;
  unsigned long long hist[256];
  unsigned long long pick_above;
  int32_t pick;
  float fshare;
  int32_t wrest;  // finish_row: some list is longer than its window
};

// Visit every token of the row in groups of four (t0 % 4 == 0).
// K chunks per thread are loaded per round, all loads in flight at once (one
// workgroup per row: the bytes in flight set the pass's speed).
template <int NT, bool BF16, bool VEC, int K = 4, typename F>
__device__ __forceinline__ void for_row4(const RowView& rv, int64_t V, uint32_t& nonfin, F f) {
#pragma unroll 1
  for (int g = 0; (int64_t)g * 4 * NT < V; g += K) {
    float x[K][4];
    load_chunks<NT, K, BF16, VEC>(rv, 0, V, g, x, nonfin);
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int64_t t0 = 4 * ((int64_t)(g + i) * NT + threadIdx.x);
      if (t0 < V) f(x[i], t0);
    }
  }
}

// hist[256] holds per-digit totals (digit = bucket of values, larger digit =
// larger values).  Returns the largest digit d with base + (total over digits
// >= d) >= need (digit 0 if there is none), and sets *above = base + total
// over digits > d.  Wave 0 scans by DPP; lane l owns digits 255-4l .. 252-4l.
// Called by all NT threads after the histogram is complete.
template <int NT>
__device__ __forceinline__ int pick_digit(ExactShared<NT>& sh, double need,
                                          unsigned long long base,
                                          unsigned long long* above) {
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const unsigned long long c1 = sh.hist[255 - 4 * l];
    const unsigned long long c2 = c1 + sh.hist[254 - 4 * l];
    const unsigned long long c3 = c2 + sh.hist[253 - 4 * l];
    const unsigned long long c4 = c3 + sh.hist[252 - 4 * l];
    const unsigned long long incl = wave_incl_sum(c4);
    const unsigned long long ex = base + (incl - c4);
    const unsigned long long hit = __ballot((double)(base + incl) >= need);
    const int first = hit ? __ffsll((long long)hit) - 1 : 63;
    if (l == first) {
      int j;
      unsigned long long ab;
      if ((double)(ex + c1) >= need) { j = 0; ab = ex; }
      else if ((double)(ex + c2) >= need) { j = 1; ab = ex + c1; }
      else if ((double)(ex + c3) >= need) { j = 2; ab = ex + c2; }
      else { j = 3; ab = ex + c3; }
      sh.pick = 255 - 4 * l - j;
      sh.pick_above = ab;
    }
  }
  __syncthreads();
  const int d = sh.pick;
  *above = sh.pick_above;
  __syncthreads();
  return d;
}

// Row summary of the first pass: max z (lowest index on ties), number of
// finite allowed tokens, and whether a NaN or +inf lies among the allowed ones.
struct RowStats {
  float zm;
  int32_t am;
  int32_t nf;
  uint32_t nonfin;
};

template <int NT, bool BF16, bool VEC, int K = 4>
__device__ __forceinline__ RowStats row_stats(const RowView& rv, int64_t V, ExactShared<NT>& sh) {
  uint32_t nonfin = 0;
  float zm = CDS_NEG_INF;
  int32_t am = INT_MAX;
  int32_t nf = 0;
  for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t t0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (x[q] > zm) {
        zm = x[q];
        am = (int32_t)(t0 + q);
      }
      // finite values only: the vector loads leave NaN and +inf in place
      nf += (x[q] > CDS_NEG_INF && x[q] < CDS_POS_INF);
    }
  });
  block_argmax<NT>(zm, am, sh.red);
  RowStats st;
  st.zm = zm;
  st.am = am;
  st.nf = block_sum_i32<NT>(nf, sh.red);
  st.nonfin = block_or_u32<NT>(nonfin, sh.red);
  return st;
}

// sum over the finite allowed tokens of exp((z - zm) * invT), accumulated in
// fp64 (each term an fp32 exp2 of an fp32 exponent)
template <int NT, bool BF16, bool VEC, int K = 4>
__device__ __forceinline__ double row_expsum(const RowView& rv, int64_t V, float zm, float invT32,
                                             ExactShared<NT>& sh) {
  uint32_t nonfin = 0;
  double se = 0.0;
  for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (x[q] != CDS_NEG_INF) se += (double)exp2f((x[q] - zm) * invT32 * kLog2e);
  });
  return block_sum_f64<NT>(se, sh.red);
}

// The value threshold of a sampled row (finite allowed values, nonempty): the
// kept set is {allowed z >= returned value} (-inf: no cut).  zm: the row's
// max z; nf: its number of finite allowed tokens.
template <int NT, bool BF16, bool VEC, int K = 4>
__device__ __forceinline__ float row_cut(const RowView& rv, int64_t V, const RowParams& rp, float zm,
                                         int32_t nf, ExactShared<NT>& sh) {
  uint32_t nonfin = 0;
  const double Td = (double)rp.temperature;
  const double m = (double)zm / Td;
  // min-p: exact value cut
  float zcut = CDS_NEG_INF;
  if (rp.flags & ROW_MINP) {
    if (threadIdx.x == 0) sh.fshare = minp_cut(zm, Td, m, rp.min_p);
    __syncthreads();
    zcut = sh.fshare;
    __syncthreads();
  }

  // top-k: radix select of the k-th largest value (8-bit digits of the order key)
  float zk = CDS_NEG_INF;
  if ((rp.flags & ROW_TOPK) && rp.top_k < nf) {
    uint32_t prefix = 0, pmask = 0;
    unsigned long long krem = (unsigned long long)rp.top_k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0ull;
      __syncthreads();
      for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t) {
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
    zk = from_okey(prefix);
    zcut = fmaxf(zcut, zk);
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
    for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (x[q] != CDS_NEG_INF && x[q] >= zc) msum += wfix(x[q]);
    });
    msum = block_sum_u64<NT>(msum, sh.red);
    // the mass the cut is normalised by: what min-p and top-k left (min-p
    // first), the top-k set (min-p last), every token (joint)
    const uint32_t ord = rp.flags & kRowOrderBits;
    unsigned long long mnorm = msum;
    if (ord) {
      const float zn = (ord & ROW_ORDER_MINP_LAST) ? zk : CDS_NEG_INF;
      mnorm = 0ull;
      for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (x[q] != CDS_NEG_INF && x[q] >= zn) mnorm += wfix(x[q]);
      });
      mnorm = block_sum_u64<NT>(mnorm, sh.red);
    }
    const double need = (double)rp.top_p * (double)mnorm;
    // a target above what min-p and top-k left keeps all of it
    const bool keep_all = (double)msum < need;
    uint32_t prefix = 0, pmask = 0;
    unsigned long long base = 0;
    for (int shift = 24; shift >= 0 && !keep_all; shift -= 8) {
      if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0ull;
      __syncthreads();
      for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t) {
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
    if (!keep_all) zcut = fmaxf(zcut, from_okey(prefix));
  }

  return zcut;
}

}  // namespace cds
