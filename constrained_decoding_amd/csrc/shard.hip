// shard.hip -- one rank's share of vocabulary-parallel sampling, for gfx950.
//
// Under tensor parallelism the LM head's output is split along the
// vocabulary: each rank holds [B, V/TP] logits ("GLM-5.3 推理全链路(七)",
// section 从最后一层 hidden 到 token id: 输出边界在哪里).  Instead of
// gathering the full logits before sampling, each rank works on its shard
// and the ranks exchange per-row partial results (same page, section
// 输出侧的通信与开销账本, sampling after a gather of per-shard candidates;
// the grammar bitmask split by vocabulary shard, section 结构化输出).
//
// The protocol is the exact path's sequence of passes (exact_path.h), each
// split over the shards:
//   stats      shard max (lowest global id), finite count, non-finite flag,
//              exp-sum against the shard max -> row max, status, normaliser,
//              the min-p threshold;
//   top-k      four radix rounds on the fp32 order key: per-shard 256-bin
//              counts, summed -> the next digit;
//   top-p      the kept and normalising fixed-point masses, then four radix
//              rounds of fixed-point masses, summed -> the next digit;
//   race       the shard's best race key over the kept set, with global token
//              ids in the Philox counter -> the row's winner is the best of
//              the shards' winners.
// Every shard uses the row's global maximum and the same fixed-point scale,
// so the sums are exact integers and the thresholds, hence the drawn ids, are
// those of the exact path on the whole row.
//
// On several GPUs each rank runs the pass over its shard, the partials are
// all-gathered, and every rank runs the same merge (so every rank holds the
// same state).  On one GPU the passes of all shards write their slots of one
// partials buffer and one merge follows.
#include <hip/hip_runtime.h>

#include <cfloat>

#include "device_common.h"
#include "exact_path.h"
#include "kernels.h"

namespace cds {

constexpr int kShardNT = 256;
constexpr int kShardK = 4;
constexpr int kMergeNT = 1024;

// Sub-slice s of row r of the shard: tokens s * kShardSub .. (whole mask
// words: kShardSub is a multiple of 32).
template <bool BF16>
__device__ __forceinline__ RowView shard_view(const ShardArgs& a, int r, int s) {
  RowView v;
  const int64_t o = (int64_t)r * a.ld + (int64_t)s * kShardSub;
  if (BF16) {
    v.b16 = static_cast<const uint16_t*>(a.logits) + o;
    v.f32 = nullptr;
  } else {
    v.f32 = static_cast<const float*>(a.logits) + o;
    v.b16 = nullptr;
  }
  v.mrow = (a.mask && (!a.row_has_mask || a.row_has_mask[r]))
               ? a.mask + (int64_t)r * a.mask_ld + (int64_t)s * (kShardSub / 32)
               : nullptr;
  return v;
}

// fixed-point scale of the top-p masses: 2^(62 - ceil(log2 V)) for the whole
// vocabulary, so that no sum over the row overflows
__device__ __forceinline__ double mass_scale(int64_t V) {
  int lg = 0;
  while ((1ll << lg) < V) ++lg;
  return ldexp(1.0, 62 - lg);
}

template <int NT, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void shard_pass_kernel(const ShardArgs a) {
  constexpr int K = kShardK;
  __shared__ ExactShared<NT> sh;
  // workgroup k: row k % B, sub-slice k / B (its record sits at k)
  const int r = (int)(blockIdx.x % (unsigned)a.B);
  const int sub = (int)(blockIdx.x / (unsigned)a.B);
  const RowParams rp = a.rows[r];
  const RowView rv = shard_view<BF16>(a, r, sub);
  const int64_t W = min((int64_t)kShardSub, (int64_t)a.width - (int64_t)sub * kShardSub);
  const int64_t v0 = (int64_t)a.v0 + (int64_t)sub * kShardSub;
  ShardPartial* P = a.part + blockIdx.x;
  const int tid = threadIdx.x;
  uint32_t nonfin = 0;

  if (a.phase == SHARD_STATS) {
    const bool greedy = (rp.flags & ROW_GREEDY) != 0;
    const RowStats st = row_stats<NT, BF16, VEC, K>(rv, W, sh);
    double se = 0.0;
    if (st.nf > 0 && !st.nonfin)
      se = row_expsum<NT, BF16, VEC, K>(
          rv, W, st.zm, (float)(greedy ? 1.0 : 1.0 / (double)rp.temperature), sh);
    if (tid == 0) {
      P->zm = st.zm;
      P->am = st.nf > 0 ? (int32_t)(v0 + st.am) : INT_MAX;
      P->nf = st.nf;
      P->nonfin = st.nonfin;
      P->se = se;
    }
    return;
  }

  const ShardState S = a.state[r];
  if (!S.active) return;  // greedy, INVALID and OVERFLOW rows end with the stats
  const double Td = (double)rp.temperature;

  if (a.phase >= SHARD_TOPK0 && a.phase < SHARD_TOPK0 + 4) {
    if (!S.topk_on) return;
    const int shift = 24 - 8 * (a.phase - SHARD_TOPK0);
    if (tid < 256) sh.hist[tid] = 0ull;
    __syncthreads();
    for_row4<NT, BF16, VEC, K>(rv, W, nonfin, [&](const float* x, int64_t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (x[q] == CDS_NEG_INF) continue;
        const uint32_t u = okey(x[q]);
        if ((u & S.pmask) == S.prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], 1ull);
      }
    });
    __syncthreads();
    if (tid < 256) P->hist[tid] = sh.hist[tid];
    return;
  }

  if (rp.flags & ROW_TOPP) {
    const double scale = mass_scale(a.V);
    const double m = S.m;
    auto wfix = [&](float v) -> unsigned long long {
      return (unsigned long long)(exp((double)v / Td - m) * scale + 0.5);
    };
    const float zc = S.zcut;
    if (a.phase == SHARD_TOPP_SUMS) {
      // the mass of what min-p and top-k left, and the mass the cut is
      // normalised by (the top-k set for min-p last, every token for joint)
      const uint32_t ord = rp.flags & kRowOrderBits;
      const float zn = (ord & ROW_ORDER_MINP_LAST) ? S.zk : CDS_NEG_INF;
      unsigned long long s0 = 0, s1 = 0;
      for_row4<NT, BF16, VEC, K>(rv, W, nonfin, [&](const float* x, int64_t) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (x[q] == CDS_NEG_INF) continue;
          if (x[q] >= zc) s0 += wfix(x[q]);
          if (ord && x[q] >= zn) s1 += wfix(x[q]);
        }
      });
      s0 = block_sum_u64<NT>(s0, sh.red);
      s1 = block_sum_u64<NT>(s1, sh.red);
      if (tid == 0) {
        P->s0 = s0;
        P->s1 = s1;
      }
      return;
    }
    if (a.phase >= SHARD_TOPP0 && a.phase < SHARD_TOPP0 + 4) {
      if (!S.topp_on) return;
      const int shift = 24 - 8 * (a.phase - SHARD_TOPP0);
      if (tid < 256) sh.hist[tid] = 0ull;
      __syncthreads();
      for_row4<NT, BF16, VEC, K>(rv, W, nonfin, [&](const float* x, int64_t) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (x[q] == CDS_NEG_INF || x[q] < zc) continue;
          const uint32_t u = okey(x[q]);
          if ((u & S.pmask) == S.prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], wfix(x[q]));
        }
      });
      __syncthreads();
      if (tid < 256) P->hist[tid] = sh.hist[tid];
      return;
    }
  }

  if (a.phase == SHARD_RACE) {
    // the race over {z >= zcut} with global ids: t0 + v0 is a multiple of
    // four (the host checks the shard's v0), so one Philox block serves
    // each group.  Keys are ranked in fp32 first (within 1e-5 of the exact
    // key for any token that can win): each thread keeps its best two tokens
    // and its third-best key; only tokens within kNear of the sub-slice's
    // best fp32 key can hold the exact best, and those get fp64 keys.  A
    // thread with three such tokens sends the sub-slice to the fp64 race
    // over every token.
    const RaceCtx c = make_race_ctx(rp, S.zm);
    const float zf = S.zcut;
    constexpr float kNear = 1e-4f;
    float k1 = CDS_NEG_INF, k2 = CDS_NEG_INF, k3 = CDS_NEG_INF;
    float z1 = CDS_NEG_INF, z2 = CDS_NEG_INF;
    int32_t t1 = INT_MAX, t2 = INT_MAX;
    uint32_t x1 = 0u, x2 = 0u;
    for_row4<NT, BF16, VEC, K>(rv, W, nonfin, [&](const float* x, int64_t t0) {
      bool need = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sd = (x[q] - c.zmax) * c.invT32;
        need |= x[q] != CDS_NEG_INF && x[q] >= zf && sd >= -19.5f && sd + 16.7f >= k3;
      }
      if (!need) return;
      const uint4 blk = race_block(c, v0 + t0);
      const uint32_t xs[4] = {blk.x, blk.y, blk.z, blk.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sd = (x[q] - c.zmax) * c.invT32;
        if (!(x[q] != CDS_NEG_INF && x[q] >= zf && sd >= -19.5f)) continue;
        const float k = sd + gumbel_fast(xs[q]);
        const int32_t t = (int32_t)(v0 + t0 + q);
        if (k > k1) {
          k3 = k2;
          k2 = k1, t2 = t1, z2 = z1, x2 = x1;
          k1 = k, t1 = t, z1 = x[q], x1 = xs[q];
        } else if (k > k2) {
          k3 = k2;
          k2 = k, t2 = t, z2 = x[q], x2 = xs[q];
        } else {
          k3 = fmaxf(k3, k);
        }
      }
    });
    const float kb = block_max_f32<NT>(k1, sh.red);  // -inf: nothing kept here
    const bool crowded =
        block_or_u32<NT>(kb != CDS_NEG_INF && k3 >= kb - kNear ? 1u : 0u, sh.red) != 0u;
    Best b = best_init();
    if (kb == CDS_NEG_INF) {
      // no candidate in this sub-slice
    } else if (!crowded) {
      if (k1 >= kb - kNear) {
        b.key = race_key64(z1, c, x1);
        b.t = t1;
        b.z = z1;
      }
      if (k2 >= kb - kNear) {
        const double key = race_key64(z2, c, x2);
        if (better(key, t2, b.key, b.t)) {
          b.key = key;
          b.t = t2;
          b.z = z2;
        }
      }
    } else {
      for_row4<NT, BF16, VEC, K>(rv, W, nonfin, [&](const float* x, int64_t t0) {
        bool need = false;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          need |= (x[q] != CDS_NEG_INF && x[q] >= zf && race_hopeful(b, x[q], c));
        if (!need) return;
        const uint4 blk = race_block(c, v0 + t0);
        const uint32_t xs[4] = {blk.x, blk.y, blk.z, blk.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (x[q] != CDS_NEG_INF && x[q] >= zf)
            race_consider(b, x[q], (int32_t)(v0 + t0 + q), xs[q], c);
      });
    }
    block_best<NT>(b, sh.red);
    if (tid == 0) {
      P->key = b.key;
      P->t = b.t;
      P->z = b.z;
    }
  }
}

// One workgroup per row: fold the shards' partials of one phase into the
// row state (and write the row's outputs when the phase ends it).
template <int NT>
__global__ __launch_bounds__(NT) void shard_merge_kernel(const ShardArgs a) {
  static_assert(NT % 256 == 0, "whole groups of 256 histogram bins");
  __shared__ ExactShared<NT> sh;
  __shared__ unsigned long long hgrp[NT / 256 > 1 ? NT / 256 - 1 : 1][256];
  const int r = blockIdx.x;
  const int B = a.B;
  const int tid = threadIdx.x;
  const RowParams rp = a.rows[r];
  ShardState* S = a.state + r;
  const ShardPartial* part = a.part;
  const int np = a.n_parts;
  auto out = [&](int32_t id, float lp, int32_t st) {
    a.out_ids[r] = id;
    if (a.out_lp) a.out_lp[r] = lp;
    if (a.out_st) a.out_st[r] = st;
  };

  if (a.phase == SHARD_STATS) {
    if (tid >= 64) return;  // one wave: lane p folds records p, p + 64, ...
    const bool greedy = (rp.flags & ROW_GREEDY) != 0;
    float zm = CDS_NEG_INF;
    int32_t am = INT_MAX, nf = 0;
    uint32_t nonfin = 0;
    for (int p = tid; p < np; p += 64) {
      const ShardPartial& q = part[(int64_t)p * B + r];
      nf += q.nf;
      nonfin |= q.nonfin;
      if (q.nf > 0 && (q.zm > zm || (q.zm == zm && q.am < am))) {
        zm = q.zm;
        am = q.am;
      }
    }
    struct ZA {
      float z;
      int32_t t;
    };
    const ZA za = wave_allreduce(ZA{zm, am}, [](const ZA& x, const ZA& y) {
      return (y.z > x.z || (y.z == x.z && y.t < x.t)) ? y : x;
    });
    zm = za.z;
    am = za.t;
    nf = wave_allreduce(nf, [](int32_t x, int32_t y) { return x + y; });
    nonfin = wave_allreduce(nonfin, [](uint32_t x, uint32_t y) { return x | y; });
    const double invTe = greedy ? 1.0 : 1.0 / (double)rp.temperature;
    double se = 0.0;
    if (nf > 0 && !nonfin)
      for (int p = tid; p < np; p += 64) {
        const ShardPartial& q = part[(int64_t)p * B + r];
        if (q.nf > 0) se += q.se * exp(((double)q.zm - (double)zm) * (double)(float)invTe);
      }
    se = wave_allreduce(se, [](double x, double y) { return x + y; });
    if (tid != 0) return;
    S->active = 0;
    if (nf == 0) {
      out(-1, CDS_NEG_INF, 2);
      return;
    }
    if (nonfin) {
      out(-1, __builtin_nanf(""), 1);
      return;
    }
    if (greedy) {
      out(am, (float)(-log(se)), 0);
      return;
    }
    const double Td = (double)rp.temperature;
    ShardState st;
    st.zm = zm;
    st.am = am;
    st.nf = nf;
    st.active = 1;
    st.m = (double)zm / Td;
    st.log_z = log(se);
    st.zcut = (rp.flags & ROW_MINP) ? minp_cut(zm, Td, st.m, rp.min_p) : CDS_NEG_INF;
    st.zk = CDS_NEG_INF;
    st.prefix = st.pmask = 0u;
    st.krem = (unsigned long long)rp.top_k;
    st.base = 0ull;
    st.need = 0.0;
    st.topk_on = (rp.flags & ROW_TOPK) && rp.top_k < nf;
    st.topp_on = 0;
    *S = st;
    return;
  }

  const ShardState s = *S;  // every thread: the branches below are uniform
  if (!s.active) return;

  const bool topk_round = a.phase >= SHARD_TOPK0 && a.phase < SHARD_TOPK0 + 4;
  const bool topp_round = a.phase >= SHARD_TOPP0 && a.phase < SHARD_TOPP0 + 4;
  if ((topk_round && s.topk_on) || (topp_round && s.topp_on)) {
    // the shards' histograms summed, then the digit: as the exact path's
    // radix rounds on the whole row
    const int i = a.phase - (topk_round ? SHARD_TOPK0 : SHARD_TOPP0);
    const int shift = 24 - 8 * i;
    // NT / 256 groups of 256 threads, group g summing records g, g + NT/256,
    // ...: a row's records (up to 64 per group) are loaded in one round;
    // integer sums, exact in any order
    constexpr int NG = NT / 256;
    const int bin = tid & 255, g = tid >> 8;
    unsigned long long h = 0;
#pragma unroll 16
    for (int p = g; p < np; p += NG) h += part[(int64_t)p * B + r].hist[bin];
    if (g > 0) hgrp[g - 1][bin] = h;
    __syncthreads();
    if (g == 0) {
#pragma unroll
      for (int k = 0; k < NG - 1; ++k) h += hgrp[k][bin];
      sh.hist[bin] = h;
    }
    __syncthreads();
    unsigned long long above;
    const int d = topk_round ? pick_digit<NT>(sh, (double)s.krem, 0ull, &above)
                             : pick_digit<NT>(sh, s.need, s.base, &above);
    if (tid == 0) {
      ShardState n = s;
      if (topk_round)
        n.krem -= above;
      else
        n.base = above;
      n.prefix |= (uint32_t)d << shift;
      n.pmask |= 255u << shift;
      if (i == 3) {
        const float v = from_okey(n.prefix);
        if (topk_round) n.zk = v;
        n.zcut = fmaxf(n.zcut, v);
        n.prefix = n.pmask = 0u;
      }
      *S = n;
    }
    return;
  }

  if (tid >= 64) return;  // one wave: lane p folds records p, p + 64, ...
  if (a.phase == SHARD_TOPP_SUMS && (rp.flags & ROW_TOPP)) {
    unsigned long long msum = 0, mnorm = 0;
    for (int p = tid; p < np; p += 64) {
      msum += part[(int64_t)p * B + r].s0;
      mnorm += part[(int64_t)p * B + r].s1;
    }
    auto add = [](unsigned long long x, unsigned long long y) { return x + y; };
    msum = wave_allreduce(msum, add);
    mnorm = wave_allreduce(mnorm, add);
    if (tid != 0) return;
    if (!(rp.flags & kRowOrderBits)) mnorm = msum;
    ShardState n = s;
    n.need = (double)rp.top_p * (double)mnorm;
    // a target above what min-p and top-k left keeps all of it
    n.topp_on = !((double)msum < n.need);
    n.prefix = n.pmask = 0u;
    n.base = 0ull;
    *S = n;
    return;
  }
  if (a.phase == SHARD_RACE) {
    struct KT {
      double key;
      int32_t t;
      float z;
    };
    KT b{-HUGE_VAL, INT_MAX, CDS_NEG_INF};
    for (int p = tid; p < np; p += 64) {
      const ShardPartial& q = part[(int64_t)p * B + r];
      if (better(q.key, q.t, b.key, b.t)) b = KT{q.key, q.t, q.z};
    }
    b = wave_allreduce(b, [](const KT& x, const KT& y) { return better(y.key, y.t, x.key, x.t) ? y : x; });
    if (tid != 0) return;
    const double Td = (double)rp.temperature;
    if (b.t == INT_MAX)
      out(-1, CDS_NEG_INF, 2);
    else
      out(b.t, (float)((double)b.z / Td - s.m - s.log_z), 0);
  }
}

template <bool BF16, bool VEC>
static hipError_t launch_pass(const ShardArgs& a, hipStream_t s) {
  const unsigned subs = (unsigned)((a.width + kShardSub - 1) / kShardSub);
  hipLaunchKernelGGL((shard_pass_kernel<kShardNT, BF16, VEC>), dim3((unsigned)a.B * subs),
                     dim3(kShardNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_shard_pass(const ShardArgs& a, bool bf16, bool vec, hipStream_t stream) {
  if (bf16) return vec ? launch_pass<true, true>(a, stream) : launch_pass<true, false>(a, stream);
  return vec ? launch_pass<false, true>(a, stream) : launch_pass<false, false>(a, stream);
}

hipError_t launch_shard_merge(const ShardArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((shard_merge_kernel<kMergeNT>), dim3((unsigned)a.B), dim3(kMergeNT), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace cds
