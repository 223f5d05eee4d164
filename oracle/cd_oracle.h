/*
 * cd_oracle.h -- CPU oracle for the batched per-request sampling step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py load this library.  It shares no code, header,
 * table or helper with the HIP path under constrained_decoding_amd/.
 *
 * Sources, cited by page title and section:
 *   [SGL] "SGLang 源码完全拆解(十): Sampling、Grammar 与结构化输出"
 *   [VLP] vLLM design document "Logits Processors" (Chinese translation)
 *   [SO]  "04 · 结构化输出: 在采样器上强制合法"
 *   [GLM] "GLM-5.3 推理全链路(七): 输出侧的最后一公里"
 *   [PHX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *         1, 2, 3" (SC'11): the Philox-4xW-R counter-based generator.
 *
 * Parity pins: every function below is pinned by tests/test_oracle_*.py
 * against closed forms, numpy/scipy routines, brute force or chi-square,
 * except the two Philox-4x32 multiplier constants, which are taken from the
 * paper's table and are "parity unpinned" (the round structure they feed is
 * pinned through the 4x64 instance of the same code against numpy).
 */
#ifndef CD_ORACLE_H
#define CD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CDO_DTYPE_F32 0
#define CDO_DTYPE_BF16 1

#define CDO_STATUS_OK 0
#define CDO_STATUS_OVERFLOW 1 /* a NaN or +inf among the allowed logits */
#define CDO_STATUS_INVALID 2  /* no finite allowed logit at all         */

/* near-tie flags: a GPU/oracle id mismatch on a row carrying one of these is
 * accounted for, any other mismatch is a failure. */
#define CDO_F_TOPP 1u /* a normalised prefix mass lies within 1e-6 of top_p  */
#define CDO_F_RACE 2u /* best two race keys within 1e-6                      */
#define CDO_F_MINP 4u /* some w_t within 1e-6 * min_p of min_p               */
#define CDO_F_TOPK 8u /* rank-k and rank-(k+1) weights within 1e-6 (info)    */

typedef struct cdo_result {
  int32_t id;         /* sampled / argmax token, -1 on OVERFLOW / INVALID     */
  int32_t status;     /* CDO_STATUS_*                                         */
  int32_t greedy;     /* 1 if the row took the argmax path                    */
  uint32_t flags;     /* CDO_F_*                                              */
  double logprob;     /* log-softmax of the chosen token (see cdo_sample_row) */
  double m;           /* max of s = z/T (greedy rows: max z)                  */
  double log_z;       /* log sum exp(s - m) over the allowed finite tokens   */
  int64_t n1, n2, n3; /* |S1|, |S2|, |S3| (sampled rows)                      */
  float zcut;         /* smallest z in S3 (sampled rows)                      */
  float pad_;
  double best_key;    /* winning race key                                     */
  double second_key;  /* runner-up race key (-inf if |S3| == 1)               */
} cdo_result;

/* Philox-4x32-10 and Philox-4x64-10 block functions [PHX, section 3.2]. */
void cdo_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                       uint32_t out[4]);
void cdo_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2],
                       uint64_t out[4]);

/* The constants the two instances use: M0, M1, W0, W1 of 4x32, then of 4x64. */
void cdo_philox_constants(uint64_t out[8]);

/* The race uniform of token t for a row: 32 random bits from the Philox
 * block at counter (t>>2, lo(offset), hi(offset), 0) under key (lo(seed),
 * hi(seed)), word t&3; mapped to U = (2*(x>>9)+1) * 2^-24 in (0,1). */
uint32_t cdo_race_bits(uint64_t seed, uint64_t offset, int64_t t);
double cdo_uniform24(uint32_t x);

/* Logit transforms for one row, in the pages' order [SGL, penalty-order
 * section; bitmask section; logit_bias section]:
 *   penalties (frequency/presence additive, then repetition scaling) on the
 *   tokens of the row's history, then the grammar bitmask (bit 0 -> -inf),
 *   then the sparse logit bias (duplicate ids: last entry wins).
 * logits: V values, fp32 or bf16 (upcast by bits<<16, exact).
 * mask: ceil(V/32) int32 words or NULL.  Returns 0, or -1 on an id outside
 * [0, V). */
int cdo_transform_row(const void *logits, int dtype, int32_t V,
                      const int32_t *hist_ids, int64_t n_hist, float rep,
                      float freq, float pres, const int32_t *bias_ids,
                      const float *bias_vals, int64_t n_bias,
                      const int32_t *mask, float *out);

/* Filter orders.  MINP_FIRST: temperature -> min-p -> top-k -> top-p, each
 * cut on what the previous ones left (vLLM's order, [GLM] "采样"; the
 * default).  JOINT: top-k and top-p applied to one distribution, the kept set
 * their intersection (with min-p's set) [SGL, "后端分支",
 * filter_apply_order="joint"].  MINP_LAST: top-k, renormalise, top-p,
 * renormalise, min-p [SGL, "后端分支" and "概率裁剪的数学"]. */
#define CDO_ORDER_MINP_FIRST 0
#define CDO_ORDER_JOINT 1
#define CDO_ORDER_MINP_LAST 2

/* Sampling for one row of transformed logits z (post penalties, mask and
 * bias), in the MINP_FIRST order.  set_out (optional, V bytes): bit0 = in
 * S1 (min-p), bit1 = in S2 (and top-k), bit2 = in S3 (the drawn-from set).
 * Returns 0. */
int cdo_sample_row(const float *z, int32_t V, float T, int32_t top_k,
                   float top_p, float min_p, uint64_t seed, uint64_t offset,
                   cdo_result *out, uint8_t *set_out);

/* cdo_sample_row in a given filter order (CDO_ORDER_*); -1 on an unknown
 * order.  In every order the drawn-from set is S1 & Tk & {t : mass strictly
 * above t < top_p * M}, where M is the mass of S1 & Tk (MINP_FIRST), of Tk
 * (MINP_LAST) or of every finite token (JOINT); set_out's bit2 marks it. */
int cdo_sample_row_order(const float *z, int32_t V, float T, int32_t top_k,
                         float top_p, float min_p, uint64_t seed,
                         uint64_t offset, int32_t order, cdo_result *out,
                         uint8_t *set_out);

/* Row loop over cdo_sample_row; ld is the row stride in elements (0 repeats
 * row 0 for every row, used for many draws of one distribution). */
int cdo_sample_batch(const float *z, int64_t ld, int32_t B, int32_t V,
                     const float *T, const int32_t *top_k, const float *top_p,
                     const float *min_p, const uint64_t *seed,
                     const uint64_t *offset, cdo_result *out);
int cdo_sample_batch_order(const float *z, int64_t ld, int32_t B, int32_t V,
                           const float *T, const int32_t *top_k,
                           const float *top_p, const float *min_p,
                           const uint64_t *seed, const uint64_t *offset,
                           int32_t order, cdo_result *out);


/* ---- further outputs [SGL, "LogitsProcessorOutput 的五段结构"] ----------- */

/* Log-softmax of s = z/T over a set of tokens, in log form (s - m - log sum
 * exp(s - m), m the largest s of the set) [SGL, "logprobs 的数值一致性"]:
 * out[t] for every t in the set with finite z, -inf elsewhere.  The set is
 * {t : set[t] & bit} (set == NULL: every token).  T = 1 gives the logprobs
 * of the logits before the temperature.  Returns the number of finite
 * tokens in the set (0: every out is -inf), or -1 if a NaN or +inf lies in
 * the set (then every out is NaN). */
int64_t cdo_set_log_softmax(const float *z, int32_t V, double T,
                            const uint8_t *set, uint8_t bit, double *out);

/* The N tokens with the largest z (NaN and -inf excluded), larger value
 * first and the lower id first among equal values, with their lp values;
 * entries past the number of such tokens get id -1 and -inf.  Returns the
 * number of real entries. */
int32_t cdo_top_n(const float *z, const double *lp, int32_t V, int32_t N,
                  int32_t *ids, double *vals);

/* ---- vocabulary shards [GLM, "输出侧的通信与开销账本"] --------------------- */

/* The race over the tokens of [v0, v0 + width) that are in a set
 * ({t : set[t] & bit}), with global token ids: the largest key
 * (z_t/T - m) - ln(-ln U_t) (U_t as in cdo_race_bits / cdo_uniform24), the
 * lowest id on an exact tie.  Returns its token (-1 if none) and sets
 * *best_key (-inf if none).  z and set are the whole row (V entries). */
int32_t cdo_race_best(const float *z, int32_t V, float T, double m,
                      uint64_t seed, uint64_t offset, int32_t v0,
                      int32_t width, const uint8_t *set, uint8_t bit,
                      double *best_key);

/* ---- speculative verification [GLM, "投机解码的输出行"] ------------------- */

/* One request's k+1 sampled rows (sampled[j], status[j] or NULL) against its
 * k draft tokens: the emitted tokens y_0 .. y_n (n = the number of leading
 * drafts equal to the rows' samples, draft[j] compared with sampled[j]),
 * cut before a row whose status is not OK and after the terminator `eos`
 * (-1: none).  tokens [k+1] gets the emitted tokens then -1; *rollback =
 * k + 1 - count.  Returns count. */
int32_t cdo_spec_accept(const int32_t *sampled, const int32_t *status,
                        int32_t k, const int32_t *draft, int32_t eos,
                        int32_t *tokens, int32_t *rollback);

#ifdef __cplusplus
}
#endif
#endif
