// outputs.hip -- further per-row outputs of the sampling step, for gfx950.
//
// What the sampler returns beside the drawn token ("SGLang 源码完全拆解(十)",
// section LogitsProcessorOutput 的五段结构): the chosen token's logprob, the
// top-N logprobs (the most likely tokens and their logprobs), the logprobs of
// tokens a request names, and the sampling support set (the tokens the row's
// draw was made from, with their renormalised logprobs and a status ordered
// by severity, OK < OVERFLOW < INVALID).  Same page, section logprobs
// 的数值一致性: an option returns logprobs of the distribution before the
// temperature; section LogitsProcessor 与 LogitsProcessorOutput: scoring
// requests take logprobs of the same preprocessed logits with no draw.
//
// Row blocks (one workgroup per row) give the chosen and named tokens'
// logprobs and the top-N.  With a workspace, a slice pass first summarises
// every 16384-token slice (maximum, normaliser in the requested basis, the
// slice's top-N keys) and the row blocks fold those records; without one, a
// row block streams its row: maximum and normaliser in one pass, then the
// top-N from an LDS candidate list of every token at or above the N-th
// largest of the threads' maxima, sorted by a bitonic network (an exact radix
// select on the fp32 order key, ties broken by id, if the list would
// overflow).  Support sets: with the sampling call's thresholds and a
// workspace, one pass over 4096-token slices records counts and kept mass
// and a second writes each slice's kept tokens in id order at its offset;
// otherwise one workgroup per support row finds the threshold with the exact
// path's selection (row_cut) when none was given, sums the kept mass, and
// writes the kept tokens by a block-wide prefix sum per chunk.
#include <hip/hip_runtime.h>

#include <cfloat>

#include "device_common.h"
#include "exact_path.h"
#include "kernels.h"

namespace cds {

constexpr int kOutNT = 512;
constexpr int kOutK = 16;      // chunks of 4 tokens in flight per thread and pass
constexpr int kMaxTopN = 256;  // SAMPLER_MAX_TOP_N
constexpr int kCandCap = 2048; // top-N candidates held in LDS

constexpr int kSliceNT = 256;                                // slice pass workgroup
constexpr int kSliceChunks = kOutSlice / (4 * kSliceNT);      // 16 chunks of 4 per thread
constexpr int kMergeCap = 8192;  // slice top-N keys the merge holds in LDS

template <int NT>
struct OutShared {
  ExactShared<NT> ex;
  unsigned long long cand[kCandCap];  // okey(z) << 32 | ~id: larger = earlier in the order
  float tmax[NT];
  uint32_t cnt;
  uint32_t wt[NT / 64];
  unsigned long long mlist[kMergeCap];  // the slices' top-N keys, N slots per slice
};

// z of token t as the sampling kernel sees it: bf16 upcast, mask applied
// (-inf if disallowed), -0 read as +0.
template <bool BF16>
__device__ __forceinline__ float token_z(const RowView& rv, int64_t t) {
  if (rv.mrow && !(((uint32_t)rv.mrow[t >> 5] >> (uint32_t)(t & 31)) & 1u)) return CDS_NEG_INF;
  const float v = BF16 ? __uint_as_float((uint32_t)rv.b16[t] << 16) : rv.f32[t];
  return v + 0.0f;
}

__device__ __forceinline__ bool finite_f(float x) { return x > CDS_NEG_INF && x < CDS_POS_INF; }

// Radix select over 8-bit digits of a 32-bit key (most significant first):
// the `need`-th largest key among the tokens `sel` admits, counting with
// `key`.  Returns the key; *tie_rem = how many tokens with exactly that key
// the `need` largest hold, *tie_cnt = how many tokens have it.
template <int NT, bool BF16, bool VEC, int K, typename Sel, typename Key>
__device__ __forceinline__ uint32_t radix_select(const RowView& rv, int64_t V, uint32_t need, Sel sel,
                                                 Key key, ExactShared<NT>& sh, uint32_t* tie_rem,
                                                 uint32_t* tie_cnt) {
  uint32_t prefix = 0, pmask = 0;
  unsigned long long krem = need;
  unsigned long long cnt_d = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0ull;
    __syncthreads();
    uint32_t nonfin = 0;
    for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t t0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!sel(x[q], t0 + q)) continue;
        const uint32_t u = key(x[q], t0 + q);
        if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], 1ull);
      }
    });
    __syncthreads();
    unsigned long long above;
    const int d = pick_digit<NT>(sh, (double)krem, 0ull, &above);
    if (shift == 0) cnt_d = sh.hist[d];  // no later round clears it
    krem -= above;
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
  }
  __syncthreads();  // every thread has read the last round's count
  *tie_rem = (uint32_t)krem;
  *tie_cnt = (uint32_t)cnt_d;
  return prefix;
}

// One pass: max z (lowest index on ties), finite count, non-finite flag and
// sum over finite tokens of exp((z - zm) * invT), the last kept per thread
// against the thread's running maximum (rescaled when it grows) and brought
// to the row maximum in fp64 at the end.  Also returns the thread's maximum.
struct RowLse {
  float zm;
  int32_t am;
  int32_t nf;
  uint32_t nonfin;
  double se;
  float tmax;
};

template <int NT, bool BF16, bool VEC, int K>
__device__ __forceinline__ RowLse row_stats_lse(const RowView& rv, int64_t V, float invT32,
                                                ExactShared<NT>& sh) {
  uint32_t nonfin = 0;
  float mt = CDS_NEG_INF;
  int32_t am = INT_MAX;
  int32_t nf = 0;
  double st = 0.0;
  const float c = invT32 * kLog2e;
  for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t t0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v = x[q];
      if (!finite_f(v)) continue;
      ++nf;
      if (v > mt) {  // exp2(-inf) = 0 on the first one
        st = st * (double)exp2f((mt - v) * c) + 1.0;
        mt = v;
        am = (int32_t)(t0 + q);
      } else {
        st += (double)exp2f((v - mt) * c);
      }
    }
  });
  RowLse r;
  r.tmax = mt;
  float zm = mt;
  int32_t a = am;
  block_argmax<NT>(zm, a, sh.red);
  r.zm = zm;
  r.am = a;
  r.nf = block_sum_i32<NT>(nf, sh.red);
  r.nonfin = block_or_u32<NT>(nonfin, sh.red);
  const double part = mt > CDS_NEG_INF ? st * exp(((double)mt - (double)zm) * (double)invT32) : 0.0;
  r.se = block_sum_f64<NT>(part, sh.red);
  return r;
}

// With the kept-set threshold given: one pass for the row's max, finite
// count, non-finite flag, and the size and mass (sum of exp((z - zm) * invT))
// of {allowed z >= cut}, the mass kept per thread against the thread's
// running maximum and brought to the row maximum in fp64 at the end.
struct CutStats {
  float zm;
  int32_t nf;
  uint32_t nonfin;
  int32_t cnt;
  double mass;
};

template <int NT, bool BF16, bool VEC, int K>
__device__ __forceinline__ CutStats row_stats_cut(const RowView& rv, int64_t V, float cut,
                                                  float invT32, ExactShared<NT>& sh) {
  uint32_t nonfin = 0;
  float mt = CDS_NEG_INF;
  int32_t nf = 0, cnt = 0;
  double st = 0.0;
  const float c = invT32 * kLog2e;
  for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v = x[q];
      if (!finite_f(v)) continue;
      ++nf;
      const bool kept = v >= cut;
      cnt += kept ? 1 : 0;
      if (v > mt) {  // exp2(-inf) = 0 on the first one
        st = st * (double)exp2f((mt - v) * c) + (kept ? 1.0 : 0.0);
        mt = v;
      } else if (kept) {
        st += (double)exp2f((v - mt) * c);
      }
    }
  });
  CutStats r;
  r.zm = block_max_f32<NT>(mt, sh.red);
  r.nf = block_sum_i32<NT>(nf, sh.red);
  r.nonfin = block_or_u32<NT>(nonfin, sh.red);
  r.cnt = block_sum_i32<NT>(cnt, sh.red);
  const double part = mt > CDS_NEG_INF ? st * exp(((double)mt - (double)r.zm) * (double)invT32) : 0.0;
  r.mass = block_sum_f64<NT>(part, sh.red);
  return r;
}

// Sort the first n entries of sh.cand in descending order (bitonic network
// over the next power of two, padded with zeros, which sort last).
template <int NT>
__device__ __forceinline__ void sort_desc(unsigned long long* cand, int n) {
  int P = 1;
  while (P < n) P <<= 1;
  for (int i = n + (int)threadIdx.x; i < P; i += NT) cand[i] = 0ull;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += NT) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long x = cand[i], y = cand[l];
          // descending runs where (i & k) == 0, ascending elsewhere
          if (((i & k) == 0) ? (x < y) : (x > y)) {
            cand[i] = y;
            cand[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// ---- slice pass: per row and 16384-token slice, its statistics and top-N ----
// One workgroup per slice with the slice in registers: max (lowest id),
// finite count, exp-sum against the slice max in the requested basis, and
// the slice's N largest keys: every token at or above the smallest of the
// waves' ceil(N/W)-th largest thread maxima is a candidate (at least N thread
// maxima, distinct tokens, reach it), sorted in LDS.  A candidate list over the LDS capacity flags the slice and its row
// falls back to the row-serial passes.
// A slice's running statistics: largest value, the lowest index holding it,
// the exp-sum relative to that value, the non-finite flag, the finite count.
struct OutStat {
  float m;
  int32_t a;
  double s;
  uint32_t nonfin;
  int32_t nf;
};

__device__ __forceinline__ OutStat out_stat_merge(const OutStat& x, const OutStat& y, float c) {
  OutStat r;
  r.m = fmaxf(x.m, y.m);
  r.a = x.m > y.m ? x.a : (y.m > x.m ? y.a : min(x.a, y.a));
  const double sx = x.m == CDS_NEG_INF ? 0.0 : x.s * (double)__builtin_amdgcn_exp2f((x.m - r.m) * c);
  const double sy = y.m == CDS_NEG_INF ? 0.0 : y.s * (double)__builtin_amdgcn_exp2f((y.m - r.m) * c);
  r.s = sx + sy;
  r.nonfin = x.nonfin | y.nonfin;
  r.nf = x.nf + y.nf;
  return r;
}

template <int NT>
struct SliceShared {
  float m[NT / 64];
  int32_t a[NT / 64];
  double s[NT / 64];
  uint32_t nonfin[NT / 64];
  int32_t nf[NT / 64];
  unsigned long long cand[kCandCap];
  uint32_t cnt;
  float wk[NT / 64];
};

__device__ __forceinline__ int row_top_n(const OutputArgs& o, int r) {
  const int ncol = o.top_ids ? o.top_n_max : 0;
  return (ncol > 0 && o.top_n) ? min(max(o.top_n[r], 0), ncol) : ncol;
}

// The records of row r, slice q (tokens s0 ..), from the slice's values:
// thread chunk i holds tokens s0 + 4*(i*NT + tid) .. +3 (disallowed and
// out-of-range tokens -inf; nonfin: a NaN or +inf among the allowed ones).
// Statistics and the slice's n_top largest keys.
template <int NT, int KS>
__device__ __forceinline__ void slice_summary(const OutputArgs& o, int r, int q, int64_t s0,
                                              const float (&x)[KS][4], uint32_t nonfin,
                                              int n_top, bool greedy, float temperature,
                                              SliceShared<NT>& sh) {
  const int Q = o.n_slices;
  const int tid = threadIdx.x;
  // (a NaN or +inf sets nonfin, and such a row's outputs ignore every sum
  // and list, so the sums and lists below only test against -inf)
  OutStat t{CDS_NEG_INF, INT_MAX, 0.0, nonfin, 0};
#pragma unroll
  for (int i = 0; i < KS; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = x[i][k];
      t.nf += finite_f(v) ? 1 : 0;
      if (v > t.m) {  // tokens in increasing order per thread: the lowest id wins ties
        t.m = v;
        t.a = 4 * (i * NT + tid) + k;
      }
    }
  const float zt = t.m;  // the thread's own maximum
  const double Tb = (o.basis == 1 || greedy) ? 1.0 : (double)temperature;
  const float c = (float)(1.0 / Tb) * kLog2e;
  // exp-sum against the thread's maximum, four terms in fp32 then fp64
  if (zt > CDS_NEG_INF) {
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      float p = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        p += x[i][k] > CDS_NEG_INF ? __builtin_amdgcn_exp2f((x[i][k] - zt) * c) : 0.0f;
      t.s += (double)p;
    }
  }
  // one workgroup merge (a fixed tree: deterministic), one barrier
  t = wave_allreduce(t, [c](const OutStat& u, const OutStat& v) { return out_stat_merge(u, v, c); });
  if ((tid & 63) == 0) {
    const int w = tid >> 6;
    sh.m[w] = t.m;
    sh.a[w] = t.a;
    sh.s[w] = t.s;
    sh.nonfin[w] = t.nonfin;
    sh.nf[w] = t.nf;
  }
  __syncthreads();
  OutStat bs{sh.m[0], sh.a[0], sh.s[0], sh.nonfin[0], sh.nf[0]};
#pragma unroll
  for (int w = 1; w < NT / 64; ++w)
    bs = out_stat_merge(bs, OutStat{sh.m[w], sh.a[w], sh.s[w], sh.nonfin[w], sh.nf[w]}, c);
  const float zm = bs.m;
  const int32_t am = bs.a, nf = bs.nf;
  const double se = zm < CDS_POS_INF ? bs.s : 0.0;
  uint32_t flags = bs.nonfin ? 1u : 0u;
  int nc = 0;
  const int n = min(n_top, nf);
  if (n > 0 && !bs.nonfin) {
    auto key = [&](float v, int i, int k) -> unsigned long long {
      return ((unsigned long long)okey(v + 0.0f) << 32) |
             (uint32_t)~(uint32_t)(s0 + 4 * (i * NT + tid) + k);
    };
    // a value bound: each wave's ceil(n/W)-th largest thread maximum (W
    // waves), the smallest of them -- at least n thread maxima, distinct
    // tokens, reach it
    constexpr int NW = NT / 64;
    const float wk = wave_kth_largest(zt, (n + NW - 1) / NW);
    if ((tid & 63) == 0) sh.wk[tid >> 6] = wk;
    if (tid == 0) sh.cnt = 0u;
    __syncthreads();
    float tz = sh.wk[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) tz = fminf(tz, sh.wk[w]);
#pragma unroll
    for (int i = 0; i < KS; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float v = x[i][k];
        if (!(v > CDS_NEG_INF && v >= tz)) continue;
        const uint32_t slot = atomicAdd(&sh.cnt, 1u);
        if (slot < (uint32_t)kCandCap) sh.cand[slot] = key(v, i, k);
      }
    __syncthreads();
    const int cnt = (int)sh.cnt;
    unsigned long long* out = o.sl_keys + ((int64_t)r * Q + q) * o.top_n_max;
    if (cnt > kCandCap) {
      flags |= 2u;
    } else if (cnt <= NT) {
      // each candidate's rank is the number of larger keys (keys are
      // distinct): no sort, no further barrier
      nc = min(n, cnt);
      const unsigned long long mine = tid < cnt ? sh.cand[tid] : 0ull;
      uint32_t rank = 0u;
      for (int j = 0; j < cnt; ++j) rank += sh.cand[j] > mine ? 1u : 0u;
      if (tid < cnt && rank < (uint32_t)nc) out[rank] = mine;
    } else {
      sort_desc<NT>(sh.cand, cnt);
      nc = min(n, cnt);
      for (int j = tid; j < nc; j += NT) out[j] = sh.cand[j];
    }
  }
  if (tid == 0) {
    OutSliceStat rec;
    rec.zm = zm;
    rec.am = nf > 0 ? (int32_t)(s0 + am) : INT_MAX;
    rec.nf = nf;
    rec.flags = flags;
    rec.se = se;
    rec.nc = nc;
    rec.pad = 0;
    o.sl_stat[(int64_t)r * Q + q] = rec;
  }
}

// One workgroup per (row, slice).
template <int NT, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void outputs_slice_kernel(const SampleArgs a, const OutputArgs o) {
  constexpr int KS = kSliceChunks;
  __shared__ SliceShared<NT> sh;
  const int Q = o.n_slices;
  const int r = (int)blockIdx.x / Q, q = (int)blockIdx.x % Q;
  const int n_top = row_top_n(o, r);
  const bool named = o.tok_off && o.tok_off[r + 1] > o.tok_off[r];
  if (n_top == 0 && !named && !o.next_lp) return;  // nothing asked of this row
  const RowParams rp = a.rows[r];
  RowView rv = row_view<BF16>(a, r);
  const int64_t s0 = (int64_t)q * kOutSlice;
  if (BF16)
    rv.b16 += s0;
  else
    rv.f32 += s0;
  if (rv.mrow) rv.mrow += s0 / 32;
  const int64_t W = min((int64_t)kOutSlice, (int64_t)a.V - s0);
  float x[KS][4];
  uint32_t nonfin = 0;
  load_chunks<NT, KS, BF16, VEC>(rv, 0, W, 0, x, nonfin);
  slice_summary<NT, KS>(o, r, q, s0, x, nonfin, n_top, (rp.flags & ROW_GREEDY) != 0,
                        rp.temperature, sh);
}

// ---- row blocks: chosen-token, named-token and top-N logprobs ----------------
template <int NT, bool BF16, bool VEC>
__device__ __forceinline__ void row_outputs(const SampleArgs& a, const OutputArgs& o, int r,
                                            OutShared<NT>& sh) {
  constexpr int K = kOutK;
  const int64_t V = a.V;
  const int ncol = o.top_ids ? o.top_n_max : 0;
  int n_top = ncol;
  if (ncol > 0 && o.top_n) n_top = min(max(o.top_n[r], 0), ncol);
  const int64_t tlo = o.tok_off ? o.tok_off[r] : 0;
  const int64_t thi = o.tok_off ? o.tok_off[r + 1] : 0;
  int32_t* top_ids = ncol > 0 ? o.top_ids + (int64_t)r * ncol : nullptr;
  float* top_vals = ncol > 0 ? o.top_vals + (int64_t)r * ncol : nullptr;
  // columns past the row's N
  for (int j = n_top + (int)threadIdx.x; j < ncol; j += NT) {
    top_ids[j] = -1;
    top_vals[j] = CDS_NEG_INF;
  }
  if (n_top == 0 && thi <= tlo && !o.next_lp) return;

  const RowParams rp = a.rows[r];
  const RowView rv = row_view<BF16>(a, r);
  const bool greedy = (rp.flags & ROW_GREEDY) != 0;
  // the basis: the row's sampling distribution (greedy rows: the logits
  // before the temperature, as for the drawn token's logprob), or the logits
  // before the temperature for every row
  const double Tb = (o.basis == 1 || greedy) ? 1.0 : (double)rp.temperature;
  RowLse st;
  bool slices = o.sl_stat != nullptr;  // the slice pass summarised the row
  bool ovf = false;
  if (slices) {
    // fold the slices' records: max (lowest id), finite count, flags, and the
    // exp-sums brought to the row max in fp64
    // (every wave on its own, lane k taking records k, k + 64, ...: one
    // round of loads, a fixed reduction tree, the same result in each wave)
    const int Q = o.n_slices;
    const OutSliceStat* S = o.sl_stat + (int64_t)r * Q;
    const int lane = threadIdx.x & 63;
    float zm = CDS_NEG_INF;
    int32_t nf = 0;
    uint32_t fl = 0;
    for (int q = lane; q < Q; q += 64) {
      const OutSliceStat sq = S[q];
      zm = sq.nf > 0 ? fmaxf(zm, sq.zm) : zm;
      nf += sq.nf;
      fl |= sq.flags;
    }
    zm = wave_allreduce(zm, [](float u, float v) { return fmaxf(u, v); });
    nf = wave_allreduce(nf, [](int32_t u, int32_t v) { return u + v; });
    fl = wave_allreduce(fl, [](uint32_t u, uint32_t v) { return u | v; });
    double se = 0.0;
    for (int q = lane; q < Q; q += 64) {
      const OutSliceStat sq = S[q];
      if (sq.nf > 0) se += sq.se * exp(((double)sq.zm - (double)zm) / Tb);
    }
    se = wave_allreduce(se, [](double u, double v) { return u + v; });
    st.zm = zm;
    st.nf = nf;
    st.nonfin = fl & 1u;
    st.se = se;
    st.tmax = CDS_NEG_INF;
    st.am = INT_MAX;
    ovf = (fl & 2u) != 0 || (int64_t)Q * o.top_n_max > kMergeCap;
  } else {
    st = row_stats_lse<NT, BF16, VEC, K>(rv, V, (float)(1.0 / Tb), sh.ex);
  }
  const int status = st.nf == 0 ? 2 : (st.nonfin ? 1 : 0);
  double mb = 0.0, lz = 0.0;
  if (status == 0) {
    mb = (double)st.zm / Tb;
    lz = log(st.se);
  }
  const float qnan = __builtin_nanf("");
  auto lp_of = [&](float z) -> float {
    return z == CDS_NEG_INF ? CDS_NEG_INF : (float)((double)z / Tb - mb - lz);
  };
  auto named = [&](int64_t t) -> float {
    if (status == 1 || t < 0 || t >= V) return qnan;
    return lp_of(token_z<BF16>(rv, t));  // an INVALID row's allowed tokens are all -inf
  };
  if (o.next_lp && threadIdx.x == 0) {
    float v;
    if (status == 1)
      v = qnan;
    else if (status == 2)
      v = CDS_NEG_INF;
    else
      v = named(o.sel_ids[r]);
    o.next_lp[r] = v;
  }
  for (int64_t j = tlo + threadIdx.x; j < thi; j += NT) o.tok_vals[j] = named(o.tok_ids[j]);
  if (n_top == 0) return;

  int n = 0;  // real entries
  if (status == 0 && slices && !ovf) {
    // the slices' sorted top-N lists, N slots each (zero keys pad them and
    // sort last); a key's rank in the row is its index in its own list plus
    // the keys above it in the other lists (binary search), and every key of
    // the row's top n is in its slice's top n
    n = min(n_top, st.nf);
    const int Q = o.n_slices, N = o.top_n_max;
    const OutSliceStat* S = o.sl_stat + (int64_t)r * Q;
    const unsigned long long* K0 = o.sl_keys + (int64_t)r * Q * N;
    for (int j = threadIdx.x; j < Q * N; j += NT) {
      const int q = j / N, i = j % N;
      sh.mlist[j] = i < S[q].nc ? K0[j] : 0ull;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < Q * N; j += NT) {
      const unsigned long long e = sh.mlist[j];
      if (e == 0ull) continue;
      const int q = j / N;
      int rank = j % N;
      for (int p = 0; p < Q && rank < n; ++p) {
        if (p == q) continue;
        const unsigned long long* L = sh.mlist + p * N;
        int lo = 0, hi = N;  // count of entries > e: the first index with L[i] < e
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (L[mid] > e)
            lo = mid + 1;
          else
            hi = mid;
        }
        rank += lo;
      }
      if (rank < n) {
        top_ids[rank] = (int32_t)~(uint32_t)e;
        top_vals[rank] = lp_of(from_okey((uint32_t)(e >> 32)));
      }
    }
  } else if (status == 0) {
    if (slices) st = row_stats_lse<NT, BF16, VEC, K>(rv, V, (float)(1.0 / Tb), sh.ex);
    n = min(n_top, st.nf);
    // Candidates: every finite z >= tau, where tau is the n-th largest of the
    // threads' maxima (those n maxima are distinct tokens, so at least n
    // tokens reach tau, and every one of the n largest does).
    float tau = CDS_NEG_INF;
    if (n < st.nf) {
      sh.tmax[threadIdx.x] = st.tmax;
      __syncthreads();
      int c = 0;
      for (int j = 0; j < NT; ++j) c += sh.tmax[j] >= st.tmax ? 1 : 0;
      tau = block_max_f32<NT>(st.tmax > CDS_NEG_INF && c >= n ? st.tmax : CDS_NEG_INF, sh.ex.red);
    }
    if (threadIdx.x == 0) sh.cnt = 0u;
    __syncthreads();
    uint32_t nonfin = 0;
    const float tf = tau;
    for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t t0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!finite_f(x[q]) || x[q] < tf) continue;
        const uint32_t slot = atomicAdd(&sh.cnt, 1u);
        if (slot < (uint32_t)kCandCap)
          sh.cand[slot] = ((unsigned long long)okey(x[q] + 0.0f) << 32) | (uint32_t)~(uint32_t)(t0 + q);
      }
    });
    __syncthreads();
    int nc = (int)sh.cnt;
    if (nc > kCandCap) {
      // too many candidates (values concentrated in few threads): exact radix
      // select of the n-th largest key, then of the id among its ties; the
      // token set {key > kthr} + {key == kthr, ~id >= ithr} has n members
      uint32_t rem, cnt;
      const uint32_t kthr = radix_select<NT, BF16, VEC, K>(
          rv, V, (uint32_t)n, [](float x, int64_t) { return finite_f(x); },
          [](float x, int64_t) { return okey(x + 0.0f); }, sh.ex, &rem, &cnt);
      uint32_t ithr = 0u;
      if (cnt > rem) {
        uint32_t rem2, cnt2;
        ithr = radix_select<NT, BF16, VEC, K>(
            rv, V, rem, [&](float x, int64_t) { return finite_f(x) && okey(x + 0.0f) == kthr; },
            [](float, int64_t t) { return ~(uint32_t)t; }, sh.ex, &rem2, &cnt2);
      }
      if (threadIdx.x == 0) sh.cnt = 0u;
      __syncthreads();
      for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t t0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (!finite_f(x[q])) continue;
          const uint32_t u = okey(x[q] + 0.0f);
          const uint32_t iu = ~(uint32_t)(t0 + q);
          if (u > kthr || (u == kthr && iu >= ithr)) {
            const uint32_t slot = atomicAdd(&sh.cnt, 1u);
            if (slot < (uint32_t)kCandCap) sh.cand[slot] = ((unsigned long long)u << 32) | iu;
          }
        }
      });
      __syncthreads();
      nc = min((int)sh.cnt, kCandCap);
    }
    sort_desc<NT>(sh.cand, nc);
    n = min(n, nc);
    for (int i = threadIdx.x; i < n; i += NT) {
      const unsigned long long e = sh.cand[i];
      top_ids[i] = (int32_t)~(uint32_t)e;
      top_vals[i] = lp_of(from_okey((uint32_t)(e >> 32)));
    }
  }
  const float pad = status == 1 ? qnan : CDS_NEG_INF;
  for (int j = n + (int)threadIdx.x; j < n_top; j += NT) {
    top_ids[j] = -1;
    top_vals[j] = pad;
  }
}

// ---- support blocks: the set the row's draw was made from ------------------
template <int NT, bool BF16, bool VEC>
__device__ __forceinline__ void support_outputs(const SampleArgs& a, const OutputArgs& o, int j,
                                                OutShared<NT>& sh) {
  const int64_t V = a.V;
  const int cap = o.sup_cap;
  int32_t* ids_out = o.sup_ids ? o.sup_ids + (int64_t)j * cap : nullptr;
  float* lp_out = o.sup_lp ? o.sup_lp + (int64_t)j * cap : nullptr;
  const float qnan = __builtin_nanf("");
  auto finish = [&](int len, int status, float sel) {
    if (threadIdx.x == 0) {
      o.sup_len[j] = len;
      o.sup_st[j] = status;
      if (o.sup_sel) o.sup_sel[j] = sel;
    }
  };
  const int r = o.sup_rows[j];
  if (r < 0 || r >= a.B) {
    finish(0, 2, qnan);
    return;
  }
  const RowParams rp = a.rows[r];
  const RowView rv = row_view<BF16>(a, r);
  constexpr int K = kOutK;
  const bool greedy = (rp.flags & ROW_GREEDY) != 0;
  const double Td = (double)rp.temperature;
  const float invT32 = (float)(1.0 / Td);
  const int64_t tsel = o.sel_ids ? (int64_t)o.sel_ids[r] : -1;
  const bool has_sel = o.sel_ids && tsel >= 0 && tsel < V;
  float zm, zcut;
  int32_t cnt;
  double mass;
  if (o.cuts && !greedy) {
    // the sampling call's threshold: one pass for the row's status and the
    // size and mass of {allowed z >= cut}
    zcut = o.cuts[r];
    const CutStats cs = row_stats_cut<NT, BF16, VEC, K>(rv, V, zcut, invT32, sh.ex);
    if (cs.nf == 0 || cs.nonfin) {  // no distribution
      finish(0, 2, qnan);
      return;
    }
    zm = cs.zm;
    cnt = cs.cnt;
    mass = cs.mass;
  } else {
    const RowStats st = row_stats<NT, BF16, VEC, K>(rv, V, sh.ex);
    if (st.nf == 0 || st.nonfin) {  // no distribution
      finish(0, 2, qnan);
      return;
    }
    if (greedy) {  // the argmax alone
      if (threadIdx.x == 0 && cap > 0) {
        if (ids_out) ids_out[0] = st.am;
        if (lp_out) lp_out[0] = 0.0f;
      }
      finish(min(1, cap), cap >= 1 ? 0 : 1, !has_sel ? qnan : (tsel == st.am ? 0.0f : CDS_NEG_INF));
      return;
    }
    zm = st.zm;
    zcut = row_cut<NT, BF16, VEC, K>(rv, V, rp, zm, st.nf, sh.ex);
    // size and mass of {allowed z >= zcut}
    cnt = 0;
    mass = 0.0;
    uint32_t nonfin = 0;
    const float zc = zcut, zmax = zm;
    for_row4<NT, BF16, VEC, K>(rv, V, nonfin, [&](const float* x, int64_t) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (x[q] != CDS_NEG_INF && x[q] >= zc) {
          ++cnt;
          mass += (double)exp2f((x[q] - zmax) * invT32 * kLog2e);
        }
    });
    cnt = block_sum_i32<NT>(cnt, sh.ex.red);
    mass = block_sum_f64<NT>(mass, sh.ex.red);
  }
  const double m = (double)zm / Td;
  const double lmass = log(mass);
  auto lp_s = [&](float z) -> float { return (float)((double)z / Td - m - lmass); };
  // the kept tokens in id order, at most cap: chunk by chunk (thread order
  // within a chunk is id order), an exclusive prefix sum places each thread's
  // members after those of lower ids
  if (cap > 0 && ids_out) {
    uint32_t written = 0u;
    constexpr int KW = 8;
    for (int g = 0; (int64_t)g * 4 * NT < V && written < (uint32_t)cap; g += KW) {
      float x[KW][4];
      uint32_t nf2 = 0;
      load_chunks<NT, KW, BF16, VEC>(rv, 0, V, g, x, nf2);
#pragma unroll
      for (int i = 0; i < KW; ++i) {
        const int64_t t0 = 4 * ((int64_t)(g + i) * NT + threadIdx.x);
        uint32_t c = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) c += (x[i][q] != CDS_NEG_INF && x[i][q] >= zcut) ? 1u : 0u;
        uint32_t total;
        uint32_t pos = written + block_excl<NT>(c, sh.wt, total);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (x[i][q] != CDS_NEG_INF && x[i][q] >= zcut) {
            if (pos < (uint32_t)cap) {
              ids_out[pos] = (int32_t)(t0 + q);
              if (lp_out) lp_out[pos] = lp_s(x[i][q]);
            }
            ++pos;
          }
        written += total;
        __syncthreads();  // sh.wt is read again by the next chunk's sum
      }
    }
  }
  float sel = qnan;
  if (has_sel) {
    const float z = token_z<BF16>(rv, tsel);
    sel = (z != CDS_NEG_INF && z >= zcut) ? lp_s(z) : CDS_NEG_INF;
  }
  finish(min(cnt, cap), cnt > cap ? 1 : 0, sel);
}

// ---- support sets by slices ----------------------------------------------------
// With the sampling call's thresholds and a workspace, a support request is
// two launches over (support row, 4096-token slice) workgroups instead of one
// workgroup per row: the first records each slice's statistics
// (SupSliceStat); the second folds its row's records -- every wave of every
// workgroup of the row in the same fixed order, so all agree bit for bit on
// the row's maximum, counts and kept mass -- and writes the slice's kept
// tokens in id order after the kept tokens of the slices before it.
constexpr int kSupNT = 256;
constexpr int kSupChunks = kSupSlice / (4 * kSupNT);  // chunks of 4 tokens per thread

template <int NT, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void support_stats_kernel(const SampleArgs a, const OutputArgs o) {
  __shared__ RedScratch<NT> red;
  const int Qs = o.n_sup_slices;
  const int j = (int)(blockIdx.x / (unsigned)Qs), q = (int)(blockIdx.x % (unsigned)Qs);
  const int r = o.sup_rows[j];
  if (r < 0 || r >= a.B) return;  // the write pass reports it
  const RowParams rp = a.rows[r];
  const RowView rv = row_view<BF16>(a, r);
  const int64_t s0 = (int64_t)q * kSupSlice, s1 = min(s0 + (int64_t)kSupSlice, (int64_t)a.V);
  float x[kSupChunks][4];
  uint32_t nonfin = 0u;
  load_chunks<NT, kSupChunks, BF16, VEC>(rv, s0, s1, 0, x, nonfin);
  const bool greedy = (rp.flags & ROW_GREEDY) != 0;
  const float cut = greedy ? CDS_POS_INF : o.cuts[r];
  // thread: largest finite z and its lowest id, finite and kept counts
  float mt = CDS_NEG_INF;
  int32_t at = INT_MAX, nf = 0, cnt = 0;
#pragma unroll
  for (int i = 0; i < kSupChunks; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = x[i][k];
      const bool fin = finite_f(v);
      nf += fin ? 1 : 0;
      cnt += (fin && v >= cut) ? 1 : 0;
      if (fin && v > mt) {  // ids increase along (i, k): the first one stays
        mt = v;
        at = (int32_t)(s0 + 4 * ((int64_t)i * NT + threadIdx.x) + k);
      }
    }
  float zm = mt;
  int32_t am = at;
  block_argmax<NT>(zm, am, red);
  const uint64_t counts = block_sum_u64<NT>((uint64_t)(uint32_t)nf | ((uint64_t)(uint32_t)cnt << 32), red);
  const uint32_t nonf = block_or_u32<NT>(nonfin, red);
  // kept mass relative to the slice's largest z (which is kept if anything is)
  double st = 0.0;
  if (!greedy && zm > CDS_NEG_INF) {
    const float c = (float)(1.0 / (double)rp.temperature) * kLog2e;
#pragma unroll
    for (int i = 0; i < kSupChunks; ++i) {
      float part = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        part += (finite_f(x[i][k]) && x[i][k] >= cut) ? exp2f((x[i][k] - zm) * c) : 0.0f;
      st += (double)part;
    }
  }
  st = block_sum_f64<NT>(st, red);
  if (threadIdx.x == 0) {
    SupSliceStat rec;
    rec.zm = zm;
    rec.am = am;
    rec.nf = (int32_t)(uint32_t)counts;
    rec.cnt = (int32_t)(uint32_t)(counts >> 32);
    rec.st = st;
    rec.nonfin = nonf;
    rec.pad = 0u;
    o.sup_stat[(size_t)j * (size_t)Qs + (size_t)q] = rec;
  }
}

template <int NT, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void support_write_kernel(const SampleArgs a, const OutputArgs o) {
  __shared__ uint32_t wt[kSupChunks][NT / 64];
  const int Qs = o.n_sup_slices;
  const int j = (int)(blockIdx.x / (unsigned)Qs), q = (int)(blockIdx.x % (unsigned)Qs);
  const int cap = o.sup_cap;
  const float qnan = __builtin_nanf("");
  const bool lead = q == 0 && threadIdx.x == 0;  // reports the row
  auto finish = [&](int len, int status, float sel) {
    if (lead) {
      o.sup_len[j] = len;
      o.sup_st[j] = status;
      if (o.sup_sel) o.sup_sel[j] = sel;
    }
  };
  const int r = o.sup_rows[j];
  if (r < 0 || r >= a.B) {
    finish(0, 2, qnan);
    return;
  }
  const RowParams rp = a.rows[r];
  const RowView rv = row_view<BF16>(a, r);
  // fold the row's records, each wave on its own (no barrier)
  const SupSliceStat* rec = o.sup_stat + (size_t)j * (size_t)Qs;
  const int lane = threadIdx.x & 63;
  struct ZA {
    float z;
    int32_t a;
  };
  ZA za{CDS_NEG_INF, INT_MAX};
  int32_t nf = 0, cnt = 0, before = 0;
  uint32_t nonfin = 0u;
  for (int k = lane; k < Qs; k += 64) {
    const SupSliceStat sr = rec[k];
    if (sr.zm > za.z || (sr.zm == za.z && sr.am < za.a)) za = ZA{sr.zm, sr.am};
    nf += sr.nf;
    cnt += sr.cnt;
    before += k < q ? sr.cnt : 0;
    nonfin |= sr.nonfin;
  }
  za = wave_allreduce(za, [](const ZA& p, const ZA& u) {
    return (u.z > p.z || (u.z == p.z && u.a < p.a)) ? u : p;
  });
  nf = wave_allreduce(nf, [](int32_t u, int32_t v) { return u + v; });
  cnt = wave_allreduce(cnt, [](int32_t u, int32_t v) { return u + v; });
  before = wave_allreduce(before, [](int32_t u, int32_t v) { return u + v; });
  nonfin = wave_allreduce(nonfin, [](uint32_t u, uint32_t v) { return u | v; });
  if (nf == 0 || nonfin) {  // no distribution
    finish(0, 2, qnan);
    return;
  }
  const int64_t tsel = o.sel_ids ? (int64_t)o.sel_ids[r] : -1;
  const bool has_sel = o.sel_ids && tsel >= 0 && tsel < a.V;
  if ((rp.flags & ROW_GREEDY) != 0) {  // the argmax alone
    if (lead && cap > 0) {
      if (o.sup_ids) o.sup_ids[(int64_t)j * cap] = za.a;
      if (o.sup_lp) o.sup_lp[(int64_t)j * cap] = 0.0f;
    }
    finish(min(1, cap), cap >= 1 ? 0 : 1,
           !has_sel ? qnan : (tsel == (int64_t)za.a ? 0.0f : CDS_NEG_INF));
    return;
  }
  const double Td = (double)rp.temperature;
  const double invT = 1.0 / Td;
  double mass = 0.0;
  for (int k = lane; k < Qs; k += 64) {
    const SupSliceStat sr = rec[k];
    if (sr.zm > CDS_NEG_INF) mass += sr.st * exp(((double)sr.zm - (double)za.z) * invT);
  }
  mass = wave_allreduce(mass, [](double u, double v) { return u + v; });
  const double m = (double)za.z / Td;
  const double lmass = log(mass);
  const float zcut = o.cuts[r];
  auto lp_s = [&](float z) -> float { return (float)((double)z / Td - m - lmass); };
  if (lead) {
    float sel = qnan;
    if (has_sel) {
      const float z = token_z<BF16>(rv, tsel);
      sel = (z != CDS_NEG_INF && z >= zcut) ? lp_s(z) : CDS_NEG_INF;
    }
    o.sup_len[j] = min(cnt, cap);
    o.sup_st[j] = cnt > cap ? 1 : 0;
    if (o.sup_sel) o.sup_sel[j] = sel;
  }
  if (cap == 0 || !o.sup_ids || before >= cap) return;  // uniform over the workgroup
  // this slice's kept tokens, in id order: chunk, then thread, then token
  const int64_t s0 = (int64_t)q * kSupSlice, s1 = min(s0 + (int64_t)kSupSlice, (int64_t)a.V);
  float x[kSupChunks][4];
  uint32_t nf2 = 0u;
  load_chunks<NT, kSupChunks, BF16, VEC>(rv, s0, s1, 0, x, nf2);
  const int w = threadIdx.x >> 6;
  uint32_t excl[kSupChunks];
#pragma unroll
  for (int i = 0; i < kSupChunks; ++i) {
    uint32_t e = 0u, tot = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned long long bal = __ballot(x[i][k] != CDS_NEG_INF && x[i][k] >= zcut);
      e += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      tot += (uint32_t)__popcll(bal);
    }
    excl[i] = e;
    if (lane == 0) wt[i][w] = tot;
  }
  __syncthreads();
  uint32_t base = (uint32_t)before;
  int32_t* ids_out = o.sup_ids + (int64_t)j * cap;
  float* lp_out = o.sup_lp ? o.sup_lp + (int64_t)j * cap : nullptr;
#pragma unroll
  for (int i = 0; i < kSupChunks; ++i) {
    uint32_t pos = base + excl[i];
#pragma unroll
    for (int w2 = 0; w2 < NT / 64; ++w2) {
      const uint32_t tw = wt[i][w2];
      pos += w2 < w ? tw : 0u;
      base += tw;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (x[i][k] != CDS_NEG_INF && x[i][k] >= zcut) {
        if (pos < (uint32_t)cap) {
          ids_out[pos] = (int32_t)(s0 + 4 * ((int64_t)i * NT + threadIdx.x) + k);
          if (lp_out) lp_out[pos] = lp_s(x[i][k]);
        }
        ++pos;
      }
  }
}

template <int NT, bool BF16, bool VEC>
__global__ __launch_bounds__(NT) void outputs_kernel(const SampleArgs a, const OutputArgs o) {
  __shared__ OutShared<NT> sh;
  if ((int)blockIdx.x < o.n_row_blocks)
    row_outputs<NT, BF16, VEC>(a, o, blockIdx.x, sh);
  else
    support_outputs<NT, BF16, VEC>(a, o, (int)blockIdx.x - o.n_row_blocks, sh);
}

template <bool BF16, bool VEC>
static hipError_t launch_out(const SampleArgs& a, const OutputArgs& o, const KernelEvents* ev,
                             hipStream_t s) {
  // support rows by slices (their own launches) or one block each here
  const bool sup_sliced = o.sup_stat && o.n_sup > 0;
  const unsigned grid = (unsigned)o.n_row_blocks + (sup_sliced ? 0u : (unsigned)o.n_sup);
  if (grid == 0u && !sup_sliced) return hipSuccess;
  if (ev && ev->start) (void)hipEventRecord(ev->start, s);
  if (o.sl_stat && o.n_row_blocks > 0)
    hipLaunchKernelGGL((outputs_slice_kernel<kSliceNT, BF16, VEC>),
                       dim3((unsigned)a.B * (unsigned)o.n_slices), dim3(kSliceNT), 0, s, a, o);
  if (grid > 0u)
    hipLaunchKernelGGL((outputs_kernel<kOutNT, BF16, VEC>), dim3(grid), dim3(kOutNT), 0, s, a, o);
  if (sup_sliced) {
    const unsigned sgrid = (unsigned)o.n_sup * (unsigned)o.n_sup_slices;
    hipLaunchKernelGGL((support_stats_kernel<kSupNT, BF16, VEC>), dim3(sgrid), dim3(kSupNT), 0, s,
                       a, o);
    hipLaunchKernelGGL((support_write_kernel<kSupNT, BF16, VEC>), dim3(sgrid), dim3(kSupNT), 0, s,
                       a, o);
  }
  if (ev && ev->stop) (void)hipEventRecord(ev->stop, s);
  return hipGetLastError();
}

hipError_t launch_outputs(const SampleArgs& a, const OutputArgs& o, bool bf16, bool vec,
                          const KernelEvents* ev, hipStream_t stream) {
  if (o.top_n_max > kMaxTopN) return hipErrorInvalidValue;
  if (bf16)
    return vec ? launch_out<true, true>(a, o, ev, stream) : launch_out<true, false>(a, o, ev, stream);
  return vec ? launch_out<false, true>(a, o, ev, stream) : launch_out<false, false>(a, o, ev, stream);
}

}  // namespace cds
