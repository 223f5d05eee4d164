// device_common.h -- device helpers of libcd_sampler.so: order keys, Philox,
// the race key, row loads with the fused bitmask, and workgroup reductions.
// Wave size is 64 (CDNA); every workgroup size used here is a multiple of 64.
#pragma once
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "layout.h"

namespace cds {

#define CDS_NEG_INF (-__builtin_inff())
#define CDS_POS_INF (__builtin_inff())

// ---- order-preserving uint32 key of a float (larger key = larger value) ----
__device__ __forceinline__ uint32_t okey(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_okey(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---- Philox-4x32-10 --------------------------------------------------------
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11), section 3.2: each round multiplies counter words 0 and 2 by the two
// round multipliers; the high halves, xored with words 1 / 3 and the round key,
// and the low halves form the next counter; the key advances by the Weyl
// constants (golden ratio and sqrt(3) fraction bits) between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // full 64-bit products: one v_mad_u64_u32 each instead of a lo / hi pair
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1,
                   (uint32_t)p0);
  }
  return c;
}

// ---- the race ----------------------------------------------------------------
// Token t of a row draws x = word (t & 3) of Philox(counter = (t>>2, lo(off),
// hi(off), 0), key = (lo(seed), hi(seed))), U = (2*(x>>9)+1) * 2^-24 (exact in
// fp32), and its key is (s_t - m) - ln(-ln U) with s = z/T, m = max s.  The
// largest key wins (lowest index on an exact tie); maximising s_t + Gumbel
// noise draws t with probability proportional to exp(s_t) over the candidate
// set, i.e. from the renormalised distribution.
//
// Bounds used for pruning: U lies in [2^-24, 1-2^-24], so -ln(-ln U) lies in
// [-2.8094, 16.6355].  The row maximum is always a candidate, so the winning
// key is >= -2.8094 and a token with s_t - m < -19.45 can never win.
struct RaceCtx {
  double Td;        // T as double
  double m;         // zmax / T
  float zmax;
  float invT32;     // (float)(1 / T)
  uint32_t k0, k1;  // Philox key
  uint32_t off_lo, off_hi;
};

__device__ __forceinline__ RaceCtx make_race_ctx(const RowParams& rp, float zmax) {
  RaceCtx c;
  c.Td = (double)rp.temperature;
  c.m = (double)zmax / c.Td;
  c.zmax = zmax;
  c.invT32 = (float)(1.0 / c.Td);
  c.k0 = (uint32_t)rp.seed;
  c.k1 = (uint32_t)(rp.seed >> 32);
  c.off_lo = (uint32_t)rp.offset;
  c.off_hi = (uint32_t)(rp.offset >> 32);
  return c;
}

__device__ __forceinline__ uint4 race_block(const RaceCtx& c, int64_t t0) {
  return philox4x32_10(make_uint4((uint32_t)(t0 >> 2), c.off_lo, c.off_hi, 0u), c.k0, c.k1);
}

// -ln(-ln U) in fp32, branch-free: E2 = -log2 U by a degree-5 series in
// d = 1-U when d < 1/16 (relative error < 2e-7; U near 1 would lose -log2 U to
// cancellation in a log), by the hardware log2 otherwise; then
// -ln(-ln U) = -ln(E2 ln 2) = -ln 2 log2(E2) - ln ln 2.  Both logs take normal
// arguments (U >= 2^-24, E2 > 8e-8), where the hardware log2 is within 1 ulp.
__device__ __forceinline__ float gumbel_fast(uint32_t x) {
  const float u = fmaf((float)(x >> 9), 0x1p-23f, 0x1p-24f);  // (2 (x>>9) + 1) 2^-24, exact
  const float d = 1.0f - u;                                   // exact
  constexpr float L = 1.4426950408889634f;                    // 1 / ln 2
  const float ser = d * fmaf(d, fmaf(d, fmaf(d, fmaf(d, L / 5, L / 4), L / 3), L / 2), L);
  const float e2 = d < 0.0625f ? ser : -__builtin_amdgcn_logf(u);
  return fmaf(-0.6931471805599453f, __builtin_amdgcn_logf(e2), 0.36651292058166435f);
}

// The exact key, in fp64 with the same operation order as the definition.
__device__ __forceinline__ double race_key64(float z, const RaceCtx& c, uint32_t x) {
  const double u = (double)(2u * (x >> 9) + 1u) * 0x1p-24;
  const double s = (double)z / c.Td;
  return (s - c.m) - log(-log(u));
}

struct Best {
  double key;
  int32_t t;
  float key32;  // fp32 copy of key for pruning
  float z;      // logit of the best token
};

__device__ __forceinline__ Best best_init() {
  Best b;
  b.key = CDS_NEG_INF;
  b.t = INT_MAX;
  b.key32 = CDS_NEG_INF;
  b.z = CDS_NEG_INF;
  return b;
}

__device__ __forceinline__ bool better(double k1, int t1, double k2, int t2) {
  return k1 > k2 || (k1 == k2 && t1 < t2);
}

// Cheap test before drawing bits: can token value z still beat b?
__device__ __forceinline__ bool race_hopeful(const Best& b, float z, const RaceCtx& c) {
  const float sd = (z - c.zmax) * c.invT32;
  return sd >= -19.5f && sd + 16.7f >= b.key32;
}

__device__ __forceinline__ void race_consider(Best& b, float z, int32_t t, uint32_t x,
                                              const RaceCtx& c) {
  const float sd = (z - c.zmax) * c.invT32;
  if (sd < -19.5f || sd + 16.7f < b.key32) return;
  // (for a token that can win, k32 is within 1e-5 of the exact key, as in
  // the fp32 race below: far inside the 1e-3 margin)
  const float k32 = sd + gumbel_fast(x);
  if (k32 + 1e-3f < b.key32) return;
  const double k64 = race_key64(z, c, x);
  if (better(k64, t, b.key, b.t)) {
    b.key = k64;
    b.t = t;
    b.key32 = (float)k64;
    b.z = z;
  }
}

// ---- fp32 race with a top-two margin ------------------------------------------
// The fast path ranks candidates by an fp32 key; |key32 - exact key| < 1e-5 for
// every token that can win (sd error <= 20 * 1.8e-7, Gumbel term < 3e-6, final
// rounding 1.2e-6), so when the best fp32 key beats the second by more than
// 2 * kRaceEps the fp32 winner is the exact winner.  Otherwise the row is
// re-raced in fp64 by the row's finisher.
constexpr float kRaceEps = 2e-5f;

struct Top2 {
  float k1;    // best key
  int32_t t1;  // its token (lowest index on an exact fp32 tie)
  float z1;    // its logit
  float k2;    // second-best key
};

__device__ __forceinline__ Top2 top2_init() {
  Top2 b;
  b.k1 = CDS_NEG_INF;
  b.t1 = INT_MAX;
  b.z1 = CDS_NEG_INF;
  b.k2 = CDS_NEG_INF;
  return b;
}

// (branch-free: selects instead of divergent paths)
__device__ __forceinline__ void top2_add(Top2& b, float k, int32_t t, float z) {
  const bool gt = (k > b.k1) | ((k == b.k1) & (t < b.t1));  // no short circuit: no branches
  b.k2 = fmaxf(b.k2, gt ? b.k1 : k);
  b.k1 = gt ? k : b.k1;
  b.t1 = gt ? t : b.t1;
  b.z1 = gt ? z : b.z1;
}

__device__ __forceinline__ void top2_merge(Top2& a, const Top2& o) {
  if (o.k1 > a.k1 || (o.k1 == a.k1 && o.t1 < a.t1)) {
    a.k2 = fmaxf(fmaxf(a.k1, a.k2), o.k2);
    a.k1 = o.k1;
    a.t1 = o.t1;
    a.z1 = o.z1;
  } else {
    a.k2 = fmaxf(a.k2, fmaxf(o.k1, o.k2));
  }
}

// Can a token with value z still enter the top two?
__device__ __forceinline__ bool race32_hopeful(const Top2& b, float z, float zmax, float invT32) {
  const float sd = (z - zmax) * invT32;
  return sd >= -19.5f && sd + 16.7f >= b.k2;
}

// Token t (value z, Gumbel term g = gumbel_fast of its draw) enters the race
// if ok; branch-free.  A token with s_t - m < -19.5 (including z = -inf) never
// wins and is left out.
__device__ __forceinline__ void race32_g_if(Top2& b, bool ok, float z, int32_t t, float g,
                                            float zmax, float invT32) {
  const float sd = (z - zmax) * invT32;
  const float k = sd + g;
  const bool in2 = ok & (sd >= -19.5f);  // bitwise: no short circuit, no branches
  const bool gt = in2 & ((k > b.k1) | ((k == b.k1) & (t < b.t1)));
  b.k2 = fmaxf(b.k2, gt ? b.k1 : (in2 ? k : CDS_NEG_INF));
  b.k1 = gt ? k : b.k1;
  b.t1 = gt ? t : b.t1;
  b.z1 = gt ? z : b.z1;
}

// As race32_g_if, from the token's 32-bit draw x.
__device__ __forceinline__ void race32_if(Top2& b, bool ok, float z, int32_t t, uint32_t x,
                                          float zmax, float invT32) {
  race32_g_if(b, ok, z, t, gumbel_fast(x), zmax, invT32);
}

__device__ __forceinline__ void race32(Top2& b, float z, int32_t t, uint32_t x, float zmax,
                                       float invT32) {
  race32_if(b, true, z, t, x, zmax, invT32);
}

// ---- histogram bins ------------------------------------------------------------
struct BinGeom {
  float delta;      // 2^floor(log2(T/16))
  float inv_delta;  // 1 / delta (exact)
  float c_bin;      // delta * log2(e) / T: exp2((off - 1) * c_bin) = mass vs bin top
};

__device__ __forceinline__ BinGeom bin_geom(float T) {
  int e;
  (void)frexpf(T * 0.0625f, &e);  // T/16 = f * 2^e, f in [0.5, 1)
  BinGeom g;
  g.delta = ldexpf(1.0f, e - 1);
  g.inv_delta = ldexpf(1.0f, 1 - e);
  g.c_bin = (float)((double)g.delta * 1.4426950408889634 / (double)T);
  return g;
}

// ---- wave-parallel search ------------------------------------------------------
// Smallest order key k in (lo, hi] with pred(k) true, for a predicate that is
// monotone in k, given pred(lo) false and pred(hi) true.  64 probes per step:
// six steps for a 32-bit range.  Called by all 64 lanes of one wave.
template <typename Pred>
__device__ __forceinline__ uint32_t wave_first_true(uint32_t lo, uint32_t hi, Pred pred) {
  const int lane = threadIdx.x & 63;
  while (hi - lo > 1u) {
    const uint64_t span = (uint64_t)(hi - lo);
    const uint32_t probe = lo + (uint32_t)((span * (uint64_t)(lane + 1)) >> 6);
    const bool ok = (lane == 63) || (probe > lo && pred(probe));
    const unsigned long long msk = __ballot(ok);
    const int first = __ffsll((long long)msk) - 1;
    const uint32_t nhi = (uint32_t)__builtin_amdgcn_readlane((int)probe, first);
    const uint32_t nlo = first > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)probe, first - 1) : lo;
    hi = nhi;
    lo = (nlo < nhi) ? nlo : lo;
  }
  return hi;
}

// ---- loads -------------------------------------------------------------------
struct RowView {
  const float* f32;
  const uint16_t* b16;
  const int32_t* mrow;  // bitmask words of the row, or nullptr
};

// Four consecutive tokens t0..t0+3 (t0 % 4 == 0, t0 < hi).  Disallowed and
// out-of-range tokens read as -inf; a NaN or +inf among allowed tokens sets
// `nonfin` and reads as -inf; -0 is canonicalised to +0 so that value
// comparisons and value order agree.
template <bool BF16, bool VEC>
__device__ __forceinline__ void load4(const RowView& rv, int64_t t0, int64_t hi, float x[4],
                                      uint32_t& nonfin) {
  if (VEC && t0 + 3 < hi) {
    if (BF16) {
      const uint2 u = *reinterpret_cast<const uint2*>(rv.b16 + t0);
      x[0] = __uint_as_float(u.x << 16);
      x[1] = __uint_as_float(u.x & 0xFFFF0000u);
      x[2] = __uint_as_float(u.y << 16);
      x[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      const float4 f = *reinterpret_cast<const float4*>(rv.f32 + t0);
      x[0] = f.x;
      x[1] = f.y;
      x[2] = f.z;
      x[3] = f.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = t0 + q;
      if (t < hi)
        x[q] = BF16 ? __uint_as_float((uint32_t)rv.b16[t] << 16) : rv.f32[t];
      else
        x[q] = CDS_NEG_INF;
    }
  }
  uint32_t bits = 0xFu;
  if (rv.mrow) bits = ((uint32_t)rv.mrow[t0 >> 5] >> (uint32_t)(t0 & 31)) & 0xFu;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!((bits >> q) & 1u) || t0 + q >= hi) {
      x[q] = CDS_NEG_INF;
    } else {
      if (x[q] != x[q] || x[q] == CDS_POS_INF) {
        nonfin = 1u;
        x[q] = CDS_NEG_INF;
      }
      x[q] = x[q] + 0.0f;
    }
  }
}

// N chunks of four tokens, chunk i at t0 = lo + 4*((first+i)*NT + tid).
// Vector path (VEC: row starts aligned and V % 4 == 0, so every chunk below
// hi is whole): every load -- logits, then mask words -- is issued before any
// value is used, with no branch between them; chunks at or beyond hi load
// chunk `lo` (in bounds) and are discarded.  Otherwise guarded scalar loads.
// CHECK_NF = false (vector path only): no per-token non-finite test; the
// caller detects NaN / +inf from its own reductions instead.
template <int NT, int N, bool BF16, bool VEC, bool STREAM = false, bool CHECK_NF = true>
__device__ __forceinline__ void load_chunks(const RowView& rv, int64_t lo, int64_t hi, int first,
                                            float x[N][4], uint32_t& nonfin) {
  if (!VEC) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int64_t t0 = lo + 4 * ((int64_t)(first + i) * NT + threadIdx.x);
      if (t0 < hi) {
        load4<BF16, false>(rv, t0, hi, x[i], nonfin);
      } else {
        x[i][0] = x[i][1] = x[i][2] = x[i][3] = CDS_NEG_INF;
      }
    }
    return;
  }
  // 32-bit unsigned byte offsets (V < 2^24) from the row base, which is the
  // same for the whole workgroup: loads take the scalar-base + 32-bit vector
  // offset form, and no 64-bit address per chunk stays live
  const uint32_t tb = (uint32_t)lo + 4u * (uint32_t)threadIdx.x + 4u * (uint32_t)(NT * first);
  const uint32_t hi32 = (uint32_t)hi, lo32 = (uint32_t)lo;
  auto tok = [&](int i) {
    const uint32_t t = tb + 4u * (uint32_t)(NT * i);
    return t < hi32 ? t : lo32;
  };
  const unsigned char* base = BF16 ? reinterpret_cast<const unsigned char*>(rv.b16)
                                   : reinterpret_cast<const unsigned char*>(rv.f32);
  // STREAM: non-temporal loads, for data no later pass reads again
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  uint32_t raw[N][4];
  // every chunk in range and no mask (all slices of an unmasked row but the
  // last): no clamp, no masking, offsets from one base (uniform branch)
  if (!rv.mrow && hi32 - lo32 >= 4u * (uint32_t)(NT * (first + N))) {
    // chunk i: a uniform base (scalar registers) plus the thread's own 32-bit
    // byte offset, so no address arithmetic per chunk in vector registers
    // (readfirstlane pins the base to scalar registers: the compiler would
    // otherwise fold the thread offset into a 64-bit vector address per chunk)
    const uint32_t toff = tb * (BF16 ? 2u : 4u);
    typedef const __attribute__((address_space(1))) unsigned char gbyte;
    auto sbase = [](const unsigned char* q) {
      const uint64_t v = reinterpret_cast<uint64_t>(q);
      const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
      const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
      return (gbyte*)((hi << 32) | lo);  // global memory: global, not flat, loads
    };
    typedef const __attribute__((address_space(1))) u32x2 gu32x2;
    typedef const __attribute__((address_space(1))) u32x4 gu32x4;
    if (BF16) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        gbyte* bi = sbase(base + (size_t)i * NT * 8);
        gu32x2* src = (gu32x2*)(bi + toff);
        const u32x2 u = STREAM ? __builtin_nontemporal_load(src) : *src;
        x[i][0] = __uint_as_float(u.x << 16);
        x[i][1] = __uint_as_float(u.x & 0xFFFF0000u);
        x[i][2] = __uint_as_float(u.y << 16);
        x[i][3] = __uint_as_float(u.y & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        gbyte* bi = sbase(base + (size_t)i * NT * 16);
        gu32x4* src = (gu32x4*)(bi + toff);
        const u32x4 u = STREAM ? __builtin_nontemporal_load(src) : *src;
        x[i][0] = __uint_as_float(u.x);
        x[i][1] = __uint_as_float(u.y);
        x[i][2] = __uint_as_float(u.z);
        x[i][3] = __uint_as_float(u.w);
      }
    }
    if (CHECK_NF) {
      uint32_t nf = 0u;
#pragma unroll
      for (int i = 0; i < N; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) nf |= __builtin_amdgcn_class(x[i][q], 0x203) ? 1u : 0u;
      nonfin |= nf;
    }
    return;
  }
  if (BF16) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const u32x2* src = reinterpret_cast<const u32x2*>(base + tok(i) * 2u);
      const u32x2 u = STREAM ? __builtin_nontemporal_load(src) : *src;
      raw[i][0] = u.x << 16;
      raw[i][1] = u.x & 0xFFFF0000u;
      raw[i][2] = u.y << 16;
      raw[i][3] = u.y & 0xFFFF0000u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const u32x4* src = reinterpret_cast<const u32x4*>(base + tok(i) * 4u);
      const u32x4 u = STREAM ? __builtin_nontemporal_load(src) : *src;
      raw[i][0] = u.x;
      raw[i][1] = u.y;
      raw[i][2] = u.z;
      raw[i][3] = u.w;
    }
  }
  // Masking is applied per chunk, only where some token of the chunk is
  // disallowed or out of range; the non-finite test (NaN or +inf among allowed
  // tokens) is one class test per token.  Non-finite values are left in place:
  // such a row ends with status OVERFLOW whatever the kernels compute for it,
  // so consumers only have to keep their indexing in bounds for them.
  uint32_t nf = 0u;
  // token offsets again, from an opaque copy of the base: the compiler would
  // otherwise keep every chunk's offset live from the loads to here
  uint32_t tb2 = tb;
  asm volatile("" : "+v"(tb2));
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t t = tb2 + 4u * (uint32_t)(NT * i);
    uint32_t bits = 0xFu;
    if (rv.mrow) {
      const uint32_t tc = t < hi32 ? t : lo32;
      bits = (*reinterpret_cast<const uint32_t*>(reinterpret_cast<const unsigned char*>(rv.mrow) +
                                                  ((tc >> 5) << 2)) >> (t & 31u)) & 0xFu;
    }
    if (t >= hi32) bits = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) x[i][q] = __uint_as_float(raw[i][q]);
    if (bits != 0xFu) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (!((bits >> q) & 1u)) x[i][q] = CDS_NEG_INF;
    }
    if (CHECK_NF) {
#pragma unroll
      for (int q = 0; q < 4; ++q) nf |= __builtin_amdgcn_class(x[i][q], 0x203) ? 1u : 0u;
    }
  }
  nonfin |= nf;
}

// Number of set bits of m below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---- wave-level inclusive prefix sums by DPP (no LDS, no barrier) --------------
// Hillis-Steele within each row of 16 lanes (row_shr 1, 2, 4, 8), then the
// last lane of a row is added into the rows above it (row_bcast 15 and 31).
// Fixed combination order: bit-reproducible.  All 64 lanes must call it.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return (uint64_t)dpp_u32<CTRL, ROWS>((uint32_t)v) |
         ((uint64_t)dpp_u32<CTRL, ROWS>((uint32_t)(v >> 32)) << 32);
}
template <typename T, typename Mov>
__device__ __forceinline__ T wave_incl_sum_impl(T v, Mov mov) {
  const int lane = threadIdx.x & 63;
  T t;
  t = mov(v, 0);
  if ((lane & 15) >= 1) v = v + t;
  t = mov(v, 1);
  if ((lane & 15) >= 2) v = v + t;
  t = mov(v, 2);
  if ((lane & 15) >= 4) v = v + t;
  t = mov(v, 3);
  if ((lane & 15) >= 8) v = v + t;
  t = mov(v, 4);
  if ((lane & 31) >= 16) v = v + t;
  t = mov(v, 5);
  if (lane >= 32) v = v + t;
  return v;
}

__device__ __forceinline__ unsigned long long wave_incl_sum(unsigned long long v) {
  return wave_incl_sum_impl(v, [](unsigned long long x, int k) -> unsigned long long {
    switch (k) {
      case 0: return dpp_u64<0x111, 0xf>(x);
      case 1: return dpp_u64<0x112, 0xf>(x);
      case 2: return dpp_u64<0x114, 0xf>(x);
      case 3: return dpp_u64<0x118, 0xf>(x);
      case 4: return dpp_u64<0x142, 0xa>(x);
      default: return dpp_u64<0x143, 0xc>(x);
    }
  });
}
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  return wave_incl_sum_impl(v, [](uint32_t x, int k) -> uint32_t {
    switch (k) {
      case 0: return dpp_u32<0x111, 0xf>(x);
      case 1: return dpp_u32<0x112, 0xf>(x);
      case 2: return dpp_u32<0x114, 0xf>(x);
      case 3: return dpp_u32<0x118, 0xf>(x);
      case 4: return dpp_u32<0x142, 0xa>(x);
      default: return dpp_u32<0x143, 0xc>(x);
    }
  });
}
__device__ __forceinline__ double wave_incl_sum(double v) {
  return wave_incl_sum_impl(v, [](double x, int k) -> double {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    switch (k) {
      case 0: u = dpp_u64<0x111, 0xf>(u); break;
      case 1: u = dpp_u64<0x112, 0xf>(u); break;
      case 2: u = dpp_u64<0x114, 0xf>(u); break;
      case 3: u = dpp_u64<0x118, 0xf>(u); break;
      case 4: u = dpp_u64<0x142, 0xa>(u); break;
      default: u = dpp_u64<0x143, 0xc>(u); break;
    }
    return __longlong_as_double((long long)u);
  });
}

// Value of lane l-1 (0 for lane 0): the exclusive prefix from an inclusive one.
__device__ __forceinline__ uint32_t wave_shift_up(uint32_t v) { return dpp_u32<0x138, 0xf>(v); }
__device__ __forceinline__ unsigned long long wave_shift_up(unsigned long long v) {
  return dpp_u64<0x138, 0xf>(v);
}
__device__ __forceinline__ double wave_shift_up(double v) {
  return __longlong_as_double((long long)dpp_u64<0x138, 0xf>((uint64_t)__double_as_longlong(v)));
}

// Inclusive prefix sum, in place, over n <= 64*K values of an LDS array, by
// one wave (`wave`, default 0) alone: lane l owns elements [K*l, K*l + K).
// The caller synchronises the workgroup before (values written) and after
// (results read).
template <int K, typename T>
__device__ __forceinline__ void wave_scan_inplace(T* v, int n, int wave = 0) {
  if ((int)(threadIdx.x >> 6) != wave) return;
  const int l = threadIdx.x & 63;
  T loc[K];
  T run = T(0);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int i = K * l + j;
    run = run + (i < n ? v[i] : T(0));
    loc[j] = run;
  }
  const T incl = wave_incl_sum(run);
  const T ex = wave_shift_up(incl);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int i = K * l + j;
    if (i < n) v[i] = ex + loc[j];
  }
}


// First index i < n with v[i] >= x in an LDS array that is non-decreasing
// (n if none), by wave 0 alone with one ballot: lane l owns [K*l, K*l + K).
// Every lane of wave 0 gets the result.
template <int K, typename T>
__device__ __forceinline__ int wave0_first_ge(const T* v, int n, T x) {
  const int l = threadIdx.x & 63;
  const int last = min(K * l + K, n) - 1;
  const bool any = K * l < n && v[last] >= x;
  const unsigned long long m = __ballot(any);
  if (!m) return n;
  const int f = __ffsll((long long)m) - 1;
  // inside lane f's range (whose last value is >= x): one element per lane,
  // one LDS round instead of a walk
  static_assert(K <= 64, "one ballot covers a lane's range");
  const int i = K * f + l;
  const unsigned long long m2 = __ballot(l < K && i < n && v[i] >= x);
  return K * f + (__ffsll((long long)m2) - 1);
}

// ---- wave all-reduce by DPP row rotations ----------------------------------------
// Each 16-lane row is reduced by rotations (row_ror 8, 4, 2, 1), then the four
// row results are read from lanes 0, 16, 32, 48 into scalar registers and
// combined.  No lane-address registers, no LDS; a fixed combination order, so
// the result is deterministic, and it is the same (uniform) value in every
// lane.  All 64 lanes must be active; op must be commutative and associative
// up to rounding.
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_obj(const T& v) {
  static_assert(sizeof(T) % 4 == 0, "32-bit words");
  uint32_t w[sizeof(T) / 4];
  __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 4); ++k)
    w[k] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w[k], CTRL, 0xf, 0xf, false);
  T r;
  __builtin_memcpy(&r, w, sizeof(T));
  return r;
}
template <typename T>
__device__ __forceinline__ T readlane_obj(const T& v, int lane) {
  uint32_t w[sizeof(T) / 4];
  __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 4); ++k)
    w[k] = (uint32_t)__builtin_amdgcn_readlane((int)w[k], lane);
  T r;
  __builtin_memcpy(&r, w, sizeof(T));
  return r;
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op) {
  v = op(v, dpp_obj<0x128>(v));  // row_ror:8
  v = op(v, dpp_obj<0x124>(v));  // row_ror:4
  v = op(v, dpp_obj<0x122>(v));  // row_ror:2
  v = op(v, dpp_obj<0x121>(v));  // row_ror:1
  const T r0 = readlane_obj(v, 0), r1 = readlane_obj(v, 16);
  const T r2 = readlane_obj(v, 32), r3 = readlane_obj(v, 48);
  return op(op(r0, r1), op(r2, r3));
}

// q-th largest (1 <= q <= 64) of one value per lane, by a walk over the order
// key bits with ballots (scalar work, no LDS); every lane gets the result.  All
// 64 lanes must be active.
__device__ __forceinline__ float wave_kth_largest(float v, int q) {
  const uint32_t key = okey(v + 0.0f);
  unsigned long long cand = ~0ull;
  uint32_t prefix = 0u;
  int need = q;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned long long ones = __ballot((key >> bit) & 1u) & cand;
    const int n1 = __popcll(ones);
    if (n1 >= need) {
      cand = ones;
      prefix |= 1u << bit;
    } else {
      need -= n1;
      cand &= ~ones;
    }
  }
  return from_okey(prefix);
}

// q-th largest (1 <= q <= 64 N) of N values per lane, the same walk with one
// candidate mask per value.
template <int N>
__device__ __forceinline__ float wave_kth_largest_n(const float (&v)[N], int q) {
  uint32_t k[N];
  unsigned long long c[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    k[j] = okey(v[j] + 0.0f);
    c[j] = ~0ull;
  }
  uint32_t prefix = 0u;
  int need = q;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    unsigned long long o[N];
    int n1 = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      o[j] = __ballot((k[j] >> bit) & 1u) & c[j];
      n1 += __popcll(o[j]);
    }
    if (n1 >= need) {
#pragma unroll
      for (int j = 0; j < N; ++j) c[j] = o[j];
      prefix |= 1u << bit;
    } else {
      need -= n1;
#pragma unroll
      for (int j = 0; j < N; ++j) c[j] &= ~o[j];
    }
  }
  return from_okey(prefix);
}

// ---- one-pass slice summary ----------------------------------------------------
// The per-thread summary of a thread's values, and its merge: max, the lowest
// index holding it, sum exp2((x - max) * c) relative to that max, the
// non-finite flag, and the minimum of a per-thread lower bound (top-k filter).
struct SliceStat {
  float m;      // max (-inf if none)
  int32_t a;    // lowest index holding it (INT_MAX if none)
  double s;     // sum exp2((x - m) * c)
  uint32_t nf;  // a non-finite value seen
  float lb;     // min of the per-thread bounds
};

__device__ __forceinline__ SliceStat stat_merge(const SliceStat& x, const SliceStat& y, float c) {
  SliceStat r;
  r.m = fmaxf(x.m, y.m);
  r.a = x.m > y.m ? x.a : (y.m > x.m ? y.a : min(x.a, y.a));
  const double sx = x.m == CDS_NEG_INF ? 0.0 : x.s * (double)__builtin_amdgcn_exp2f((x.m - r.m) * c);
  const double sy = y.m == CDS_NEG_INF ? 0.0 : y.s * (double)__builtin_amdgcn_exp2f((y.m - r.m) * c);
  r.s = sx + sy;
  r.nf = x.nf | y.nf;
  r.lb = fminf(x.lb, y.lb);
  return r;
}

template <int NT>
struct StatScratch {
  float m[NT / 64];
  int32_t a[NT / 64];
  double s[NT / 64];
  uint32_t nf[NT / 64];
  float lb[NT / 64];
};

// Workgroup merge of the threads' summaries (a fixed tree: deterministic);
// every thread gets the result.  One barrier.
template <int NT>
__device__ __forceinline__ SliceStat block_stat(SliceStat v, float c, StatScratch<NT>& sc) {
  v = wave_allreduce(v, [c](const SliceStat& x, const SliceStat& y) { return stat_merge(x, y, c); });
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sc.m[w] = v.m;
    sc.a[w] = v.a;
    sc.s[w] = v.s;
    sc.nf[w] = v.nf;
    sc.lb[w] = v.lb;
  }
  __syncthreads();
  SliceStat r;
  r.m = sc.m[0];
  r.a = sc.a[0];
  r.s = sc.s[0];
  r.nf = sc.nf[0];
  r.lb = sc.lb[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k) {
    SliceStat y;
    y.m = sc.m[k];
    y.a = sc.a[k];
    y.s = sc.s[k];
    y.nf = sc.nf[k];
    y.lb = sc.lb[k];
    r = stat_merge(r, y, c);
  }
  return r;
}

// ---- workgroup reductions (fixed trees: deterministic) -------------------------
template <int NT>
struct RedScratch {
  double d[NT / 64];
  float f[NT / 64];
  int32_t i[NT / 64];
  uint64_t u[NT / 64];
};

template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, RedScratch<NT>& s) {
  v = wave_allreduce(v, [](double x, double y) { return x + y; });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.d[w] = v;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) tot += s.d[k];
  return tot;
}

template <int NT>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, RedScratch<NT>& s) {
  v = wave_allreduce(v, [](uint64_t x, uint64_t y) { return x + y; });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.u[w] = v;
  __syncthreads();
  uint64_t tot = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) tot += s.u[k];
  return tot;
}

template <int NT>
__device__ __forceinline__ int32_t block_sum_i32(int32_t v, RedScratch<NT>& s) {
  v = wave_allreduce(v, [](int32_t x, int32_t y) { return x + y; });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.i[w] = v;
  __syncthreads();
  int32_t tot = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) tot += s.i[k];
  return tot;
}

template <int NT>
__device__ __forceinline__ uint32_t block_or_u32(uint32_t v, RedScratch<NT>& s) {
  v = wave_allreduce(v, [](uint32_t x, uint32_t y) { return x | y; });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.i[w] = (int32_t)v;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) tot |= (uint32_t)s.i[k];
  return tot;
}

template <int NT>
__device__ __forceinline__ float block_max_f32(float v, RedScratch<NT>& s) {
  v = wave_allreduce(v, [](float x, float y) { return fmaxf(x, y); });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.f[w] = v;
  __syncthreads();
  float tot = s.f[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k) tot = fmaxf(tot, s.f[k]);
  return tot;
}

template <int NT>
__device__ __forceinline__ int32_t block_min_i32(int32_t v, RedScratch<NT>& s) {
  v = wave_allreduce(v, [](int32_t x, int32_t y) { return min(x, y); });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.i[w] = v;
  __syncthreads();
  int32_t tot = s.i[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k) tot = min(tot, s.i[k]);
  return tot;
}

template <int NT>
__device__ __forceinline__ void block_top2(Top2& b, RedScratch<NT>& s) {
  b = wave_allreduce(b, [](Top2 x, const Top2& y) {
    top2_merge(x, y);
    return x;
  });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    s.f[w] = b.k1;
    s.i[w] = b.t1;
    s.d[w] = (double)b.z1;
    s.u[w] = (uint64_t)__float_as_uint(b.k2);
  }
  __syncthreads();
  Top2 r = top2_init();
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    Top2 p;
    p.k1 = s.f[k];
    p.t1 = s.i[k];
    p.z1 = (float)s.d[k];
    p.k2 = __uint_as_float((uint32_t)s.u[k]);
    top2_merge(r, p);
  }
  b = r;
}

// max value, lowest index among equal maxima
// Exclusive prefix sum of c over the block (thread order) and its total, with
// one barrier; wt is LDS scratch of NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_excl(uint32_t c, uint32_t* wt, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_sum(c);
  if (lane == 63) wt[w] = incl;
  __syncthreads();
  uint32_t base = 0u;
  total = 0u;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const uint32_t tk = wt[k];
    base += k < w ? tk : 0u;
    total += tk;
  }
  return base + incl - c;
}

template <int NT>
__device__ __forceinline__ void block_argmax(float& z, int32_t& t, RedScratch<NT>& s) {
  struct ZT {
    float z;
    int32_t t;
  };
  const ZT zt = wave_allreduce(ZT{z, t}, [](const ZT& p, const ZT& q) {
    return (q.z > p.z || (q.z == p.z && q.t < p.t)) ? q : p;
  });
  z = zt.z;
  t = zt.t;
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    s.f[w] = z;
    s.i[w] = t;
  }
  __syncthreads();
  z = s.f[0];
  t = s.i[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k)
    if (s.f[k] > z || (s.f[k] == z && s.i[k] < t)) {
      z = s.f[k];
      t = s.i[k];
    }
}

template <int NT>
__device__ __forceinline__ void block_best(Best& b, RedScratch<NT>& s) {
  b = wave_allreduce(b, [](const Best& p, const Best& q) { return better(q.key, q.t, p.key, p.t) ? q : p; });
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    s.d[w] = b.key;
    s.i[w] = b.t;
    s.f[w] = b.z;
  }
  __syncthreads();
  b.key = s.d[0];
  b.t = s.i[0];
  b.z = s.f[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k)
    if (better(s.d[k], s.i[k], b.key, b.t)) {
      b.key = s.d[k];
      b.t = s.i[k];
      b.z = s.f[k];
    }
  b.key32 = (float)b.key;
}

}  // namespace cds
