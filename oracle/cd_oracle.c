/*
 * cd_oracle.c -- CPU oracle for the batched per-request sampling step.
 *
 * TEST INFRASTRUCTURE ONLY (see cd_oracle.h).  Plain single-threaded C,
 * built with -O2 -ffp-contract=off and no fast-math, so every fp32 and fp64
 * operation below is the IEEE operation written in the source.
 *
 * Precision: the logit transforms run in fp32, the precision the pages'
 * engines apply them in (in-place adds/multiplies on the fp32 logits tensor).
 * Everything the method defines as a real number -- s = z/T, softmax
 * weights, masses, race keys, logprobs -- is computed in fp64.
 *
 * Citation handles ([SGL], [VLP], [SO], [GLM], [PHX]) are listed in
 * cd_oracle.h.
 */
#include "cd_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Philox [PHX, section 3.2 "Philox"; constants from its Table 2].            */
/*                                                                          */
/* One round on a 4-word counter (c0,c1,c2,c3) with a 2-word key (k0,k1):   */
/* form the double-width products M0*c0 and M1*c2; the new counter is        */
/* (hi(M1*c2)^c1^k0, lo(M1*c2), hi(M0*c0)^c3^k1, lo(M0*c0)).  The key is      */
/* advanced by the Weyl constants (W0,W1) between rounds; 10 rounds.        */
/* Both widths come from this one macro, so the 4x64 instance (which the    */
/* tests compare with numpy.random.Philox) pins the round structure that    */
/* the 4x32 instance uses.                                                  */
/* ------------------------------------------------------------------------ */
#define CDO_DEFINE_PHILOX4(NAME, UW, UD, SHIFT, M0, M1, W0, W1)               \
  void NAME(const UW ctr[4], const UW key[2], UW out[4]) {                    \
    UW c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];                    \
    UW k0 = key[0], k1 = key[1];                                              \
    for (int round = 0; round < 10; ++round) {                                \
      if (round > 0) {                                                        \
        k0 = (UW)(k0 + (UW)(W0));                                             \
        k1 = (UW)(k1 + (UW)(W1));                                             \
      }                                                                       \
      UD p0 = (UD)(UW)(M0) * (UD)c0;                                          \
      UD p1 = (UD)(UW)(M1) * (UD)c2;                                          \
      UW n0 = (UW)(p1 >> (SHIFT)) ^ c1 ^ k0;                                  \
      UW n1 = (UW)p1;                                                         \
      UW n2 = (UW)(p0 >> (SHIFT)) ^ c3 ^ k1;                                  \
      UW n3 = (UW)p0;                                                         \
      c0 = n0;                                                                \
      c1 = n1;                                                                \
      c2 = n2;                                                                \
      c3 = n3;                                                                \
    }                                                                         \
    out[0] = c0;                                                              \
    out[1] = c1;                                                              \
    out[2] = c2;                                                              \
    out[3] = c3;                                                              \
  }

/* Multipliers from the paper's table; Weyl increments are the leading
 * fraction bits of the golden ratio and of sqrt(3) (tests recompute both
 * from their closed forms through cdo_philox_constants). */
#define CDO_P32_M0 0xD2511F53u
#define CDO_P32_M1 0xCD9E8D57u
#define CDO_P32_W0 0x9E3779B9u
#define CDO_P32_W1 0xBB67AE85u
#define CDO_P64_M0 0xD2E7470EE14C6C93ull
#define CDO_P64_M1 0xCA5A826395121157ull
#define CDO_P64_W0 0x9E3779B97F4A7C15ull
#define CDO_P64_W1 0xBB67AE8584CAA73Bull

CDO_DEFINE_PHILOX4(cdo_philox4x32_10, uint32_t, uint64_t, 32, CDO_P32_M0,
                   CDO_P32_M1, CDO_P32_W0, CDO_P32_W1)
CDO_DEFINE_PHILOX4(cdo_philox4x64_10, uint64_t, unsigned __int128, 64,
                   CDO_P64_M0, CDO_P64_M1, CDO_P64_W0, CDO_P64_W1)

void cdo_philox_constants(uint64_t out[8]) {
  out[0] = CDO_P32_M0;
  out[1] = CDO_P32_M1;
  out[2] = CDO_P32_W0;
  out[3] = CDO_P32_W1;
  out[4] = CDO_P64_M0;
  out[5] = CDO_P64_M1;
  out[6] = CDO_P64_W0;
  out[7] = CDO_P64_W1;
}

uint32_t cdo_race_bits(uint64_t seed, uint64_t offset, int64_t t) {
  uint32_t ctr[4] = {(uint32_t)(t >> 2), (uint32_t)offset,
                     (uint32_t)(offset >> 32), 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t o[4];
  cdo_philox4x32_10(ctr, key, o);
  return o[t & 3];
}

/* Midpoints of a 2^23-point grid on (0,1): exact in fp32 and fp64. */
double cdo_uniform24(uint32_t x) {
  return (double)(2u * (x >> 9) + 1u) * 0x1p-24;
}

/* ------------------------------------------------------------------------ */
/* Transforms [SGL, "惩罚项的顺序语义" (order of penalty terms): additive       */
/* penalties first, the repetition penalty (divide or multiply) on the       */
/* updated logits second, then the grammar mask, then the logit_bias add;    */
/* SGL, "位掩码" (bitmask): int32 words, bit 0 -> -inf, -1 = all allowed;      */
/* SGL, "logit_bias 为什么用三元组构造": ids deduplicated, last value wins].     */
/* ------------------------------------------------------------------------ */
static float bf16_bits_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int cdo_transform_row(const void *logits, int dtype, int32_t V,
                      const int32_t *hist_ids, int64_t n_hist, float rep,
                      float freq, float pres, const int32_t *bias_ids,
                      const float *bias_vals, int64_t n_bias,
                      const int32_t *mask, float *out) {
  for (int32_t t = 0; t < V; ++t)
    out[t] = (dtype == CDO_DTYPE_BF16)
                 ? bf16_bits_to_f32(((const uint16_t *)logits)[t])
                 : ((const float *)logits)[t];

  if (n_hist > 0) {
    int32_t *cnt = (int32_t *)calloc((size_t)V, sizeof(int32_t));
    for (int64_t i = 0; i < n_hist; ++i) {
      int32_t id = hist_ids[i];
      if (id < 0 || id >= V) {
        free(cnt);
        return -1;
      }
      cnt[id] += 1;
    }
    for (int32_t t = 0; t < V; ++t) {
      if (cnt[t] == 0) continue;
      float scaled_count = freq * (float)cnt[t];
      float pen = scaled_count + pres;          /* f*c + p*[c>0]      */
      float v = out[t] - pen;                   /* additive first     */
      if (rep != 1.0f) v = (v > 0.0f) ? v / rep : v * rep; /* scaling */
      out[t] = v;
    }
    free(cnt);
  }

  if (mask) {
    for (int32_t t = 0; t < V; ++t) {
      uint32_t word = (uint32_t)mask[t >> 5];
      if (((word >> (t & 31)) & 1u) == 0u) out[t] = -INFINITY;
    }
  }

  if (n_bias > 0) {
    float *bv = (float *)malloc((size_t)V * sizeof(float));
    uint8_t *has = (uint8_t *)calloc((size_t)V, 1);
    for (int64_t i = 0; i < n_bias; ++i) {
      int32_t id = bias_ids[i];
      if (id < 0 || id >= V) {
        free(bv);
        free(has);
        return -1;
      }
      bv[id] = bias_vals[i]; /* a later duplicate overwrites: last wins */
      has[id] = 1;
    }
    for (int32_t t = 0; t < V; ++t)
      if (has[t]) out[t] = out[t] + bv[t];
    free(bv);
    free(has);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Sampling of one row.                                                      */
/*                                                                           */
/* Order (vLLM's, [GLM, "采样: temperature、top-k/top-p 与一次分布式随机"] and */
/* [VLP, "将 Logits Processors 应用于模型输出的 Logits"]): greedy rows take the */
/* argmax of the temperature-free logits; other rows divide by T, apply      */
/* min-p (argmax invariant), then top-k, then top-p, then draw from the     */
/* renormalised distribution.                                               */
/* Set definitions [SGL, "概率裁剪的数学: 三把刀的不同"]:                        */
/*   softmax   p_t = exp(z_t/T) / sum_j exp(z_j/T)                           */
/*   top-k     tokens of rank < k (ties at rank k all kept)   */
/*   top-p     tokens whose strictly-greater mass is < p (ties all in/out)  */
/*   min-p     tokens with p_t >= p_max * min_p                              */
/* and the renormalised draw p'_t = w_t 1[t in S] / sum_{S} w               */
/* [GLM, same section].  The draw is an exponential race: token t gets the   */
/* key (s_t - m) - ln(-ln U_t) with U_t its Philox uniform, and the largest */
/* key wins (a Gumbel-max draw, exact for the renormalised distribution).   */
/* The logprob is the log-softmax of z/T before truncation [SGL, "logprobs  */
/* 的数值一致性"], computed in log form; greedy rows use T = 1 [SGL, "贪心路径"]. */
/* ------------------------------------------------------------------------ */
typedef struct {
  double s;
  int32_t t;
} cdo_entry;

static int cdo_entry_cmp(const void *a, const void *b) {
  const cdo_entry *x = (const cdo_entry *)a;
  const cdo_entry *y = (const cdo_entry *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->t < y->t) ? -1 : (x->t > y->t ? 1 : 0);
}

/* Mass of the top-k set over every finite token (ties at the k-th value all
 * in), by its definition: a full sort of the finite values, the k-th largest
 * value, and the sum of w over the tokens at or above it.  Used by the
 * top-k -> top-p -> min-p order, whose top-p cut is normalised by the mass
 * the top-k cut leaves [SGL, "后端分支": top_k_renorm_prob, then
 * top_p_renorm_prob, then min_p_sampling_from_probs]. */
static int cdo_cmp_desc(const void *a, const void *b) {
  const double x = *(const double *)a, y = *(const double *)b;
  return x > y ? -1 : (x < y ? 1 : 0);
}

static double cdo_topk_mass_all(const double *s, const double *w, int32_t V,
                                int32_t top_k) {
  double *v = (double *)malloc((size_t)V * sizeof(double));
  int64_t n = 0;
  for (int32_t t = 0; t < V; ++t)
    if (s[t] != -INFINITY) v[n++] = s[t];
  qsort(v, (size_t)n, sizeof(double), cdo_cmp_desc); /* full sort */
  const double tau = v[top_k - 1];
  double mass = 0.0;
  for (int32_t t = 0; t < V; ++t)
    if (s[t] != -INFINITY && s[t] >= tau) mass += w[t];
  free(v);
  return mass;
}

static int cdo_sample_row_impl(const float *z, int32_t V, float T,
                               int32_t top_k, float top_p, float min_p,
                               uint64_t seed, uint64_t offset, int32_t order,
                               cdo_result *out, uint8_t *set_out);

int cdo_sample_row(const float *z, int32_t V, float T, int32_t top_k,
                   float top_p, float min_p, uint64_t seed, uint64_t offset,
                   cdo_result *out, uint8_t *set_out) {
  return cdo_sample_row_impl(z, V, T, top_k, top_p, min_p, seed, offset,
                             CDO_ORDER_MINP_FIRST, out, set_out);
}

int cdo_sample_row_order(const float *z, int32_t V, float T, int32_t top_k,
                         float top_p, float min_p, uint64_t seed,
                         uint64_t offset, int32_t order, cdo_result *out,
                         uint8_t *set_out) {
  if (order < CDO_ORDER_MINP_FIRST || order > CDO_ORDER_MINP_LAST) return -1;
  return cdo_sample_row_impl(z, V, T, top_k, top_p, min_p, seed, offset,
                             order, out, set_out);
}

static int cdo_sample_row_impl(const float *z, int32_t V, float T,
                               int32_t top_k, float top_p, float min_p,
                               uint64_t seed, uint64_t offset, int32_t order,
                               cdo_result *out, uint8_t *set_out) {
  memset(out, 0, sizeof *out);
  out->id = -1;
  out->zcut = NAN;
  out->best_key = -INFINITY;
  out->second_key = -INFINITY;
  if (set_out) memset(set_out, 0, (size_t)V);

  /* status [SGL, "LogitsProcessorOutput": severity-ordered statuses] */
  int nonfinite = 0;
  int64_t nfin = 0;
  float zmax = -INFINITY;
  int32_t arg = -1;
  for (int32_t t = 0; t < V; ++t) {
    float v = z[t];
    if (isnan(v) || v == INFINITY) {
      nonfinite = 1;
    } else if (v != -INFINITY) {
      ++nfin;
      if (v > zmax) { /* strict: the lowest index wins ties */
        zmax = v;
        arg = t;
      }
    }
  }
  if (nfin == 0) {
    out->status = CDO_STATUS_INVALID;
    out->logprob = -INFINITY;
    return 0;
  }
  if (nonfinite) {
    out->status = CDO_STATUS_OVERFLOW;
    out->logprob = NAN;
    return 0;
  }

  if (T < 1e-5f || top_k == 1) { /* greedy [GLM; SGL "贪心路径"] */
    double sum = 0.0;
    for (int32_t t = 0; t < V; ++t)
      if (z[t] != -INFINITY) sum += exp((double)z[t] - (double)zmax);
    out->greedy = 1;
    out->id = arg;
    out->m = (double)zmax;
    out->log_z = log(sum);
    out->logprob = (double)z[arg] - (double)zmax - log(sum);
    out->n1 = out->n2 = out->n3 = 1;
    out->zcut = zmax;
    return 0;
  }

  const double Td = (double)T;
  double *s = (double *)malloc((size_t)V * sizeof(double));
  double *w = (double *)malloc((size_t)V * sizeof(double));
  uint8_t *in = (uint8_t *)calloc((size_t)V, 1); /* bits: S1, S2, S3 */
  const double m = (double)zmax / Td;
  double Z = 0.0;
  for (int32_t t = 0; t < V; ++t) {
    if (z[t] == -INFINITY) {
      s[t] = -INFINITY;
      w[t] = 0.0;
      continue;
    }
    s[t] = (double)z[t] / Td;
    w[t] = exp(s[t] - m);
    Z += w[t];
  }

  /* S1: min-p */
  int64_t n1 = 0;
  for (int32_t t = 0; t < V; ++t) {
    if (z[t] == -INFINITY) continue;
    int keep = 1;
    if (min_p > 0.0f) {
      keep = (w[t] >= (double)min_p);
      if (fabs(w[t] - (double)min_p) <= 1e-6 * (double)min_p)
        out->flags |= CDO_F_MINP;
    }
    if (keep) {
      in[t] |= 1;
      ++n1;
    }
  }

  const int topk_on = (top_k > 1 && (int64_t)top_k < n1);
  const int topp_on = (top_p < 1.0f);
  int64_t n2 = n1;
  cdo_entry *ent = NULL;
  if (topk_on || topp_on) {
    ent = (cdo_entry *)malloc((size_t)n1 * sizeof(cdo_entry));
    int64_t j = 0;
    for (int32_t t = 0; t < V; ++t)
      if (in[t] & 1) {
        ent[j].s = s[t];
        ent[j].t = t;
        ++j;
      }
    qsort(ent, (size_t)n1, sizeof(cdo_entry), cdo_entry_cmp); /* full sort */
  }

  /* S2: top-k within S1; every token tying the k-th value is kept */
  if (topk_on) {
    double tau = ent[top_k - 1].s;
    if (w[ent[top_k].t] >= (1.0 - 1e-6) * w[ent[top_k - 1].t])
      out->flags |= CDO_F_TOPK;
    n2 = 0;
    while (n2 < n1 && ent[n2].s >= tau) ++n2;
  }
  for (int64_t i = 0; i < n2 && ent; ++i) in[ent[i].t] |= 2;
  if (!ent)
    for (int32_t t = 0; t < V; ++t)
      if (in[t] & 1) in[t] |= 2;

  /* S3: top-p within S2, walked in sorted order one value-group at a time.
   * The mass the cut is normalised by depends on the filter order: the mass
   * of S2 when min-p and top-k come first (vLLM's order [GLM, "采样"]); the
   * mass of the top-k set over every token when min-p comes last (top-k,
   * renormalise, top-p, renormalise, min-p [SGL, "后端分支"]); the mass of
   * every token when top-k and top-p are applied jointly to one distribution
   * and the kept set is their intersection [SGL, "后端分支",
   * filter_apply_order="joint"].  Every set here is a prefix of the sorted
   * order, so the mass strictly above t is the same whichever set t is
   * measured in. */
  int64_t n3 = 0;
  if (topp_on) {
    double M2 = 0.0;
    for (int64_t i = 0; i < n2; ++i) M2 += w[ent[i].t];
    if (order == CDO_ORDER_JOINT) {
      M2 = Z;
    } else if (order == CDO_ORDER_MINP_LAST) {
      int64_t nfin_all = 0;
      for (int32_t t = 0; t < V; ++t) nfin_all += (z[t] != -INFINITY);
      M2 = (top_k > 1 && (int64_t)top_k < nfin_all)
               ? cdo_topk_mass_all(s, w, V, top_k)
               : Z;
    }
    const double target = (double)top_p * M2;
    double cum = 0.0;
    int64_t i = 0;
    while (i < n2) {
      int64_t j = i;
      double gmass = 0.0;
      while (j < n2 && ent[j].s == ent[i].s) {
        gmass += w[ent[j].t];
        ++j;
      }
      const double above = cum; /* mass strictly above this value */
      if (fabs(above / M2 - (double)top_p) <= 1e-6) out->flags |= CDO_F_TOPP;
      if (above < target)
        for (int64_t q = i; q < j; ++q) {
          in[ent[q].t] |= 4;
          ++n3;
        }
      cum += gmass;
      i = j;
    }
  } else {
    for (int32_t t = 0; t < V; ++t)
      if (in[t] & 2) {
        in[t] |= 4;
        ++n3;
      }
  }

  /* exponential race over S3 */
  double best = -INFINITY, second = -INFINITY;
  int32_t best_t = -1;
  float zcut = INFINITY;
  for (int32_t t = 0; t < V; ++t) {
    if (!(in[t] & 4)) continue;
    if (z[t] < zcut) zcut = z[t];
    double u = cdo_uniform24(cdo_race_bits(seed, offset, t));
    double key = (s[t] - m) - log(-log(u));
    if (key > best) {
      second = best;
      best = key;
      best_t = t;
    } else if (key > second) {
      second = key;
    }
  }
  if (n3 >= 2 && fabs(best - second) <= 1e-6) out->flags |= CDO_F_RACE;

  out->id = best_t;
  out->m = m;
  out->log_z = log(Z);
  out->logprob = s[best_t] - m - log(Z);
  out->n1 = n1;
  out->n2 = n2;
  out->n3 = n3;
  out->zcut = zcut;
  out->best_key = best;
  out->second_key = second;
  if (set_out) memcpy(set_out, in, (size_t)V);
  free(ent);
  free(in);
  free(w);
  free(s);
  return 0;
}

int cdo_sample_batch(const float *z, int64_t ld, int32_t B, int32_t V,
                     const float *T, const int32_t *top_k, const float *top_p,
                     const float *min_p, const uint64_t *seed,
                     const uint64_t *offset, cdo_result *out) {
  return cdo_sample_batch_order(z, ld, B, V, T, top_k, top_p, min_p, seed,
                                offset, CDO_ORDER_MINP_FIRST, out);
}

int cdo_sample_batch_order(const float *z, int64_t ld, int32_t B, int32_t V,
                           const float *T, const int32_t *top_k,
                           const float *top_p, const float *min_p,
                           const uint64_t *seed, const uint64_t *offset,
                           int32_t order, cdo_result *out) {
  for (int32_t r = 0; r < B; ++r)
    if (cdo_sample_row_order(z + (int64_t)r * ld, V, T[r], top_k[r], top_p[r],
                             min_p[r], seed[r], offset[r], order, &out[r],
                             NULL) != 0)
      return -1;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Further outputs [SGL, "LogitsProcessorOutput 的五段结构": the chosen        */
/* token's logprob, the top logprobs (the most likely tokens and their      */
/* logprobs), the logprobs of tokens the request names, and the sampling    */
/* support set with its logprobs and a severity-ordered status; "logprobs   */
/* 的数值一致性": an option returns logprobs of the distribution before the   */
/* temperature; "LogitsProcessor 与 LogitsProcessorOutput": scoring requests */
/* take logprobs of the same preprocessed logits without a draw].           */
/* ------------------------------------------------------------------------ */

int64_t cdo_set_log_softmax(const float *z, int32_t V, double T,
                            const uint8_t *set, uint8_t bit, double *out) {
  /* the tokens in play: finite z, and in the set when one is given */
  int64_t n = 0;
  int bad = 0;
  double m = -INFINITY;
  for (int32_t t = 0; t < V; ++t) {
    out[t] = -INFINITY;
    if (set && !(set[t] & bit)) continue;
    if (isnan(z[t]) || z[t] == INFINITY) {
      bad = 1;
      continue;
    }
    if (z[t] == -INFINITY) continue;
    ++n;
    const double s = (double)z[t] / T;
    if (s > m) m = s;
  }
  if (bad) {
    for (int32_t t = 0; t < V; ++t) out[t] = NAN;
    return -1;
  }
  if (n == 0) return 0;
  /* log form: s - m - log(sum exp(s - m)) */
  double sum = 0.0;
  for (int32_t t = 0; t < V; ++t) {
    if (set && !(set[t] & bit)) continue;
    if (z[t] == -INFINITY) continue;
    sum += exp((double)z[t] / T - m);
  }
  const double log_sum = log(sum);
  for (int32_t t = 0; t < V; ++t) {
    if (set && !(set[t] & bit)) continue;
    if (z[t] == -INFINITY) continue;
    out[t] = (double)z[t] / T - m - log_sum;
  }
  return n;
}

int32_t cdo_top_n(const float *z, const double *lp, int32_t V, int32_t N,
                  int32_t *ids, double *vals) {
  cdo_entry *ent = (cdo_entry *)malloc((size_t)(V > 0 ? V : 1) * sizeof(cdo_entry));
  int64_t n = 0;
  for (int32_t t = 0; t < V; ++t)
    if (z[t] != -INFINITY && !isnan(z[t])) {
      ent[n].s = (double)z[t];
      ent[n].t = t;
      ++n;
    }
  /* full sort: larger value first, the lower id first among equal values */
  qsort(ent, (size_t)n, sizeof(cdo_entry), cdo_entry_cmp);
  int32_t k = 0;
  for (; k < N && k < n; ++k) {
    ids[k] = ent[k].t;
    vals[k] = lp[ent[k].t];
  }
  for (int32_t j = k; j < N; ++j) {
    ids[j] = -1;
    vals[j] = -INFINITY;
  }
  free(ent);
  return k;
}

/* ------------------------------------------------------------------------ */
/* Vocabulary shards [GLM, "输出侧的通信与开销账本": sampling after a gather of */
/* per-shard results instead of the full logits; "从最后一层 hidden 到 token  */
/* id": the LM head's output is split along the vocabulary under TP].  The  */
/* race key of token t depends only on (seed, offset, t) and s_t - m, so the */
/* row's winner is the best of the shards' winners when every shard uses   */
/* global token ids.                                                         */
/* ------------------------------------------------------------------------ */
int32_t cdo_race_best(const float *z, int32_t V, float T, double m,
                      uint64_t seed, uint64_t offset, int32_t v0,
                      int32_t width, const uint8_t *set, uint8_t bit,
                      double *best_key) {
  const double Td = (double)T;
  double best = -INFINITY;
  int32_t best_t = -1;
  for (int32_t t = v0; t < v0 + width && t < V; ++t) {
    if (!(set[t] & bit)) continue;
    const double u = cdo_uniform24(cdo_race_bits(seed, offset, t));
    const double key = ((double)z[t] / Td - m) - log(-log(u));
    if (key > best) { /* strict: the lowest id wins an exact tie */
      best = key;
      best_t = t;
    }
  }
  *best_key = best;
  return best_t;
}

/* ------------------------------------------------------------------------ */
/* Speculative verification [GLM, "投机解码的输出行: 一次前向里的 k+1 个      */
/* token": one verification forward gives k+1 rows per request (the token    */
/* after the committed prefix, then after each of the k draft tokens); each  */
/* row is sampled; the accepted tokens are kept and the rejected suffix's KV */
/* rolled back; SGL, "逐 token 推进: accept_token、rollback 与跳步": the draft */
/* is rolled back from the first position that does not match; SO, 4.4     */
/* "推进与终止": the tail past a terminator is dropped].  Row j's sample y_j is compared with draft */
/* token j+1: the first n drafts are accepted while y_j equals them, and the */
/* request emits y_0 .. y_n (the accepted drafts and the row's own token at  */
/* the first mismatch).  A row without a token (status not OK) ends the     */
/* emission before it; a terminator ends it after itself.                    */
/* ------------------------------------------------------------------------ */
int32_t cdo_spec_accept(const int32_t *sampled, const int32_t *status,
                        int32_t k, const int32_t *draft, int32_t eos,
                        int32_t *tokens, int32_t *rollback) {
  int32_t count = 0;
  for (int32_t j = 0; j <= k; ++j) {
    if (status && status[j] != CDO_STATUS_OK) break; /* no token here   */
    tokens[count++] = sampled[j];
    if (eos >= 0 && sampled[j] == eos) break;        /* terminator       */
    if (j == k || sampled[j] != draft[j]) break;     /* first mismatch   */
  }
  for (int32_t j = count; j <= k; ++j) tokens[j] = -1;
  *rollback = k + 1 - count; /* positions written by the verification but not kept */
  return count;
}
