/*
 * cd_sampler.h -- C ABI of libcd_sampler.so, the MI355X (gfx950) batched
 * per-request sampling step: [B, V] logits + per-row parameters -> one token
 * id and one logprob per row.
 *
 * Sources, cited by page title and section:
 *   [SGL] "SGLang 源码完全拆解(十): Sampling、Grammar 与结构化输出"
 *         (pinghaoyang.com.cn)
 *   [VLP] vLLM design document "Logits Processors" (Chinese translation)
 *   [SO]  "04 · 结构化输出: 在采样器上强制合法"
 *   [GLM] "GLM-5.3 推理全链路(七): 输出侧的最后一公里" (pinghaoyang.com.cn)
 *   [PHX] Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11
 *
 * Pipeline (order fixed by [SGL] "惩罚项的顺序语义" and [GLM] "采样"):
 *   1. sampler_pack_params      host: validate, batch flags, dedup, CSR, H2D
 *   2. sampler_apply_transforms penalties then logit bias, in place (fp32)
 *   3. sampler_apply_bitmask    grammar bitmask -> -inf, in place (optional:
 *                               sampler_sample can take the mask fused)
 *   4. sampler_sample           greedy rows: argmax; other rows: temperature,
 *                               min-p, top-k, top-p, seeded exponential race
 *
 * Conventions
 *   - Every call returns int: SAMPLER_OK (0) or a negative SAMPLER_E* code;
 *     sampler_strerror() describes it.  Nothing throws across the ABI.
 *   - "dev" pointers are device memory, "host" pointers host memory.  All
 *     device memory is allocated and owned by the caller; the library keeps
 *     no device allocation.  Its only process-wide state is an atomic call
 *     counter and a per-device cache of the device wall-clock rate, so calls
 *     on different streams and workspaces may run concurrently from any
 *     threads.  Calls that share a workspace must not overlap.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     No call synchronises the stream, except sampler_pack_params without a
 *     staging buffer (documented there).  Device inputs must stay alive and
 *     unmodified until the stream reaches the call.
 *   - A call that returns an error has launched nothing and written no
 *     device memory (a caller's host staging buffer may hold partial data).
 *   - Data-dependent failures never return an error: they come back per row
 *     in out_status (OK=0 < OVERFLOW=1 < INVALID=2, ordered by severity as
 *     [SGL] "LogitsProcessorOutput" orders its mask statuses).
 */
#ifndef CD_SAMPLER_H
#define CD_SAMPLER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define SAMPLER_OK 0
#define SAMPLER_EINVAL (-1)       /* invalid argument or parameter value     */
#define SAMPLER_ERANGE (-2)       /* size outside the supported range        */
#define SAMPLER_ENOSPC (-3)       /* caller buffer or workspace too small    */
#define SAMPLER_EUNSUPPORTED (-4) /* valid request the library does not do  */
#define SAMPLER_EHIP (-5)         /* a HIP runtime call failed               */

/* ---- dtypes of the logits ----------------------------------------------- */
#define SAMPLER_DTYPE_F32 0
#define SAMPLER_DTYPE_BF16 1 /* upcast exactly (bits << 16) on load; [GLM]
                                "从最后一层 hidden 到 token id": sampling runs
                                on fp32 values                              */

/* ---- per-row output status ---------------------------------------------- */
#define SAMPLER_STATUS_OK 0
#define SAMPLER_STATUS_OVERFLOW 1 /* a NaN or +inf among the allowed logits:
                                     id = -1, logprob = NaN                  */
#define SAMPLER_STATUS_INVALID 2  /* no finite allowed logit (e.g. the mask
                                     allows nothing): id = -1, logprob = -inf
                                     (takes precedence over OVERFLOW)        */

/* ---- batch flags (sampler_batch.flags), computed by sampler_pack_params --
 * Host-side booleans that let whole kernels be skipped ([SGL] "字段分组":
 * is_all_greedy / need_top_k_sampling / ...; [VLP] "将 Logits Processors
 * 应用于模型输出的 Logits": argmax-invariant work skipped for all-greedy
 * batches).  NEED_* are evaluated over the non-greedy rows only.          */
#define SAMPLER_FLAG_ALL_GREEDY (1u << 0)
#define SAMPLER_FLAG_ANY_GREEDY (1u << 1)
#define SAMPLER_FLAG_NEED_TOP_K (1u << 2)
#define SAMPLER_FLAG_NEED_TOP_P (1u << 3)
#define SAMPLER_FLAG_NEED_MIN_P (1u << 4)
#define SAMPLER_FLAG_NEED_PENALTY (1u << 5)
#define SAMPLER_FLAG_HAS_BIAS (1u << 6)
/* Layout, not semantics: the n_hold rows' second-pass tasks each take half a
 * slice (set when n_hold is small against B, so that those rows' latency is
 * spread over twice the workgroups).                                      */
#define SAMPLER_FLAG_SPLIT_PASS2 (1u << 7)

/* ---- host-side per-request parameters ------------------------------------
 * All arrays are host memory, [B] unless noted; NULL selects the default.
 *   temperature  required. Row is greedy if temperature < 1e-5 ([GLM] "采样":
 *                the sampling epsilon) or top_k == 1 ([SGL] "字段分组":
 *                top_k <= 1 rows are argmax; top_k <= 0 here means "off").
 *                Must be finite and >= 0.
 *   top_k        int32; <= 0 or >= V: off (the pages' "-1 / whole vocab").
 *   top_p        (0, 1]; 1: off.                     default 1
 *   min_p        [0, 1]; 0: off.                     default 0
 *   repetition_penalty  > 0, finite; 1: off.         default 1
 *   frequency_penalty   finite; 0: off.              default 0
 *   presence_penalty    finite; 0: off.              default 0
 *   hist_indptr  int64 [B+1], hist_ids int32: each row's generated-token
 *                history (CSR); counts are taken from it for the
 *                frequency / presence / repetition penalties.  NULL: none.
 *   bias_indptr  int64 [B+1], bias_ids int32, bias_vals float: sparse
 *                logit bias (CSR).  Duplicate ids in a row: the later entry
 *                wins ([SGL] "logit_bias 为什么用三元组构造").  Values may be
 *                -inf (ban a token) but not NaN or +inf.  NULL: none.
 *   seed         uint64: Philox key of the row's draw.      default 0
 *   offset       uint64: Philox counter words 1-2 of the row's draw, e.g.
 *                the decode position ([SGL] "调用点": positions seed the
 *                draw, so a request's stream does not depend on the batch).
 *                default: the row index.
 *   filter_order (a scalar for the whole batch) SAMPLER_ORDER_*: how min-p,
 *                top-k and top-p stack.  Each cut keeps a prefix of the
 *                tokens by value; the kept set is always S1 & Tk &
 *                {t : mass strictly above t < top_p * M} (S1 the min-p set,
 *                Tk the top-k set over every token) and the orders differ in
 *                the mass M the top-p cut is normalised by:
 *                  MINP_FIRST (0, default): M = mass of S1 & Tk -- min-p,
 *                    then top-k, then top-p on what is left ([GLM] "采样",
 *                    vLLM's order);
 *                  JOINT (1): M = mass of every allowed token -- top-k and
 *                    top-p cut one distribution and the intersection is kept
 *                    ([SGL] "后端分支", filter_apply_order="joint"; min-p, if
 *                    set, is intersected too);
 *                  MINP_LAST (2): M = mass of Tk -- top-k, renormalise,
 *                    top-p, renormalise, min-p ([SGL] "后端分支" and
 *                    "概率裁剪的数学").
 *                Any other value -> SAMPLER_EINVAL.
 * -------------------------------------------------------------------------- */
#define SAMPLER_ORDER_MINP_FIRST 0
#define SAMPLER_ORDER_JOINT 1
#define SAMPLER_ORDER_MINP_LAST 2
typedef struct sampler_host_params {
  int32_t B;
  int32_t V;
  const float *temperature;
  const int32_t *top_k;
  const float *top_p;
  const float *min_p;
  const float *repetition_penalty;
  const float *frequency_penalty;
  const float *presence_penalty;
  const int64_t *hist_indptr;
  const int32_t *hist_ids;
  const int64_t *bias_indptr;
  const int32_t *bias_ids;
  const float *bias_vals;
  const uint64_t *seed;
  const uint64_t *offset;
  int32_t filter_order;
} sampler_host_params;

/* ---- packed batch descriptor (plain data, returned by value) ------------- */
typedef struct sampler_batch {
  int32_t B;
  int32_t V;
  uint32_t flags;       /* SAMPLER_FLAG_*                                      */
  int32_t max_top_k;    /* max top_k over non-greedy rows if every one of them
                           has 1 < top_k < V, else 0 ([SGL] "max_top_k")      */
  int64_t n_pen;        /* packed (token, count) penalty entries (histories
                           longer than 4096 tokens, counted on the host)    */
  int64_t n_bias;       /* packed (token, value) bias entries after dedup    */
  const void *d_rows;   /* dev: per-row records inside the caller's d_buf    */
  const void *d_pen;    /* dev: penalty entries inside d_buf                 */
  const void *d_bias;   /* dev: bias entries inside d_buf                    */
  size_t bytes;         /* bytes of d_buf in use                             */
  int32_t n_sampled;    /* rows that are not greedy                          */
  int32_t n_hold;       /* of these, rows whose cut needs the whole row's
                           histogram (the first n_hold of d_sampled): their
                           slices race in a second pass, after the plan     */
  const void *d_sampled; /* dev: int32 row order [B] inside d_buf, the order
                            in which sampler_sample dispatches the rows: the
                            n_sampled rows that are not greedy (first those
                            whose cut needs the whole row's histogram: top-p
                            as the only cut, or a top_k above a bound that
                            depends on V; then top-k rows without min-p whose
                            candidate lists are long), then the greedy rows;
                            ascending within each group.  The sampling
                            kernel's task table follows it (after the order
                            padded to 16 bytes)                             */
  int64_t n_hist_raw;   /* raw history ids (histories of up to 4096 tokens,
                           counted on the device by the transforms kernel)  */
  const void *d_hist_raw; /* dev: int32 raw history ids inside d_buf        */
  const void *d_slots;  /* dev: per-row workspace places inside d_buf       */
  uint64_t ws_list_entries; /* workspace the batch's rows need: candidate-  */
  uint64_t ws_records;      /* list entries, list records and slice         */
  uint64_t ws_hist_slices;  /* histograms (see sampler_workspace_bytes_batch) */
} sampler_batch;

/* Message for a SAMPLER_* return code (static storage). */
const char *sampler_strerror(int code);

/* Library version string (static storage). */
const char *sampler_version(void);

/* Upper bound of the device bytes sampler_pack_params needs for B rows,
 * n_hist history ids and n_bias bias entries in total. */
size_t sampler_params_bytes(int32_t B, int64_t n_hist, int64_t n_bias);

/* Validate `h`, compute the batch flags and max_top_k, pack each row's
 * history (rows of up to 4096 history tokens as raw int32 ids, counted on
 * the device by sampler_apply_transforms; longer rows as (token, count)
 * entries counted here), deduplicate the bias, and copy the packed block to
 * d_buf (dev, >= sampler_params_bytes(...) bytes) on
 * `stream`.  h_staging: pinned host memory of >= the same size used as the
 * copy source (it must stay untouched until the copy has run), or NULL:
 * then the call copies from a temporary host buffer and synchronises
 * `stream` before returning.  Validation follows the fail-fast rule of
 * [SGL] "后端分支" and vLLM's validate_params ([VLP] "Logits Processor 编程
 * 模型"): any invalid value -> SAMPLER_EINVAL and nothing is copied.
 * d_bytes too small -> SAMPLER_ENOSPC.  On success *out describes the batch;
 * its device pointers point into d_buf, which the kernels of every call given
 * *out read: d_buf must not be packed into again (nor h_staging rewritten)
 * before those calls and the copy have run on the stream. */
int sampler_pack_params(const sampler_host_params *h, void *d_buf,
                        size_t d_bytes, void *h_staging, void *stream,
                        sampler_batch *out);

/* Host-only variant for inspection and CPU tests: packs into `host_buf`
 * (host memory, >= sampler_params_bytes(...)) with the same validation;
 * out->d_* then point into host_buf.  Makes no HIP call. */
int sampler_pack_host(const sampler_host_params *h, void *host_buf,
                      size_t bytes, sampler_batch *out);

/* Pre-grammar penalties and post-grammar bias, in place on fp32 logits
 * (dev, row stride `ld` >= V elements, 4-byte aligned).  Per penalised
 * token with history count c > 0, in fp32 without contraction:
 *   z -= frequency*c + presence;  then if repetition != 1:
 *   z = z > 0 ? z / repetition : z * repetition
 * ([SGL] "惩罚项的顺序语义": additive before scaling), then z += bias for
 * each deduplicated bias entry ([SGL] same section: bias after the mask;
 * applying it before a later mask is identical because -inf + b = -inf).
 * Repeated history tokens are merged into one count per token on the device
 * (an LDS hash table per row), so each token is updated once.
 * Tokens outside history and bias are not touched.  Skipped (no launch) when
 * the batch has neither NEED_PENALTY nor HAS_BIAS.  bf16 logits would round
 * the transformed values, so only fp32 is accepted here. */
int sampler_apply_transforms(const sampler_batch *b, float *logits, int64_t ld,
                             void *stream);

/* Grammar bitmask in place ([SGL] "位掩码"; [SO] 4.2): token t of row r is
 * allowed iff bit (t & 31) of word bitmask[r*mask_ld + (t >> 5)] is 1;
 * disallowed tokens become exactly -inf.  bitmask: dev int32 [B, mask_ld],
 * mask_ld >= ceil(V/32); a word of -1 allows all its tokens; bits at
 * positions >= V are ignored.  row_has_mask: dev uint8 [B] or NULL (every
 * row has a mask row); rows with 0 are untouched.  dtype: SAMPLER_DTYPE_*. */
int sampler_apply_bitmask(void *logits, int dtype, int64_t ld, int32_t B,
                          int32_t V, const int32_t *bitmask, int64_t mask_ld,
                          const uint8_t *row_has_mask, void *stream);

/* Device workspace bytes sampler_sample needs for any batch of B rows of V
 * tokens (every row with room for its largest class). */
size_t sampler_workspace_bytes(int32_t B, int32_t V);

/* Device workspace bytes sampler_sample needs for this packed batch: only
 * the rows that list candidates get lists (sized by their class), only rows
 * whose cut needs the row's histogram get histograms.  At most
 * sampler_workspace_bytes(b->B, b->V); 0 on an invalid descriptor. */
size_t sampler_workspace_bytes_batch(const sampler_batch *b);

/* Zero a workspace on `stream` (a fill kernel, safe under graph capture).
 * A workspace must be zero before its first sampler_sample; every
 * sampler_sample leaves its synchronisation counters zero again, so one init
 * per allocation is enough, also for later calls with other B or V that fit
 * in it.  Two calls that share a workspace must not overlap. */
int sampler_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/* The sampling step.
 *   logits      dev [B, ld] (ld >= V), dtype SAMPLER_DTYPE_*; read only.
 *   bitmask     dev int32 [B, mask_ld] or NULL: applied on the fly with the
 *               semantics of sampler_apply_bitmask (nothing is written).
 *   row_has_mask dev uint8 [B] or NULL.
 *   out_ids     dev int32 [B] (required); out_logprobs dev float [B] or NULL;
 *               out_status dev int32 [B] or NULL.
 *   workspace   dev, >= sampler_workspace_bytes_batch(b) (at most
 *               sampler_workspace_bytes(B, V)), zeroed once.
 * Per row, on the transformed (and masked) logits z:
 *   greedy rows: id = lowest index of max z; logprob = log_softmax(z)[id]
 *     ([SGL] "贪心路径"; [GLM] "采样": greedy rows use the logits before
 *     the temperature).
 *   other rows: s = z/T ([SGL] "采样主路径的骨架"); S1 = min-p set
 *     {p_t >= min_p * p_max}; S2 = top-k of S1 (ties at the k-th value all
 *     kept); S3 = top-p of S2 {t : mass of S2 strictly above t < top_p *
 *     mass(S2)} (ties all in or all out) ([SGL] "概率裁剪的数学"; order
 *     min-p -> top-k -> top-p as vLLM applies its argmax-invariant processors
 *     after the temperature, [GLM] "采样"); the drawn token maximises
 *     (s_t - max s) - ln(-ln U_t) over S3, an exponential race equivalent to a
 *     draw from the renormalised distribution ([GLM] "采样" formula for p'),
 *     with U_t = (2*(x>>9)+1) * 2^-24 and x word (t&3) of Philox-4x32-10
 *     [PHX] at counter (t>>2, lo(offset), hi(offset), 0), key (lo(seed),
 *     hi(seed)); logprob = log_softmax(s)[id] over all allowed tokens, before
 *     truncation ([SGL] "logprobs 的数值一致性").
 * Errors: B or V mismatch with `b`, bad dtype or strides -> EINVAL;
 * workspace too small -> ENOSPC; launch failure -> EHIP. */
int sampler_sample(const sampler_batch *b, const void *logits, int dtype,
                   int64_t ld, const int32_t *bitmask, int64_t mask_ld,
                   const uint8_t *row_has_mask, int32_t *out_ids,
                   float *out_logprobs, int32_t *out_status, void *workspace,
                   size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, allocation-free serving loops, harnesses that forbid hipMalloc:
 * sampler_sample with no workspace argument.  The workspace is the library's
 * own device array of SAMPLER_STATIC_WORKSPACE_BYTES (64 MiB), one per
 * device, held until the process ends; the call allocates nothing.  The first
 * call on a device clears the array's row counters on its stream (a fill
 * kernel).  Every call on a device shares that array: calls that overlap on
 * one device race (keep them on one stream).  A batch that needs more than
 * the array (sampler_workspace_bytes_batch) -> SAMPLER_ENOSPC, nothing
 * launched.  Other arguments and errors as sampler_sample. */
#define SAMPLER_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int sampler_sample_static(const sampler_batch *b, const void *logits, int dtype,
                          int64_t ld, const int32_t *bitmask, int64_t mask_ld,
                          const uint8_t *row_has_mask, int32_t *out_ids,
                          float *out_logprobs, int32_t *out_status, void *stream);

/* ---- per-call options -----------------------------------------------------
 * sampler_sample_ex is sampler_sample with a per-call options record; every
 * option belongs to that one call (nothing is kept between calls).
 * opt == NULL, or all fields zero: the same call as sampler_sample.
 *   size        sizeof(sampler_options) as the caller compiled it (a record of
 *               another size -> SAMPLER_EINVAL).
 *   algo        SAMPLER_ALGO_FAST (0): the fused kernel; SAMPLER_ALGO_EXACT
 *               (1): the row-serial exact path for every row (one workgroup
 *               per row, several passes; the fallback the fast path takes for
 *               rows whose boundary sets do not fit on chip).  Same results.
 *   wait_ns     how long a workgroup that needs its row's plan waits for it
 *               before the row falls back to the exact path, in nanoseconds:
 *               0 = the default (5 ms); SAMPLER_WAIT_NONE (-1) = no wait at
 *               all (every such row takes the exact path; used to exercise
 *               that path); other negative values -> SAMPLER_EINVAL.
 *   trace       dev uint64 buffer or NULL: diagnostic phase timestamps, 8
 *               words per workgroup of the sampling kernel (8 * (ceil(B/8) +
 *               2 * ceil(n_hold/8)) * P workgroups, P = slices per row, at
 *               most 64; never more than 24 * ceil(B/8) * P): word 0 = row |
 *               slice << 20 | class << 28 | planner << 31 (class 4: a pass-2
 *               task), words 1..7 = the 100 MHz device wall clock at the
 *               start, after the slice maximum, after the summary pass, after
 *               the class work, after the arrival ticket, after the plan (or
 *               the wait for it), and at the end.
 *   start_event, stop_event  hipEvent_t (as void*) or NULL: recorded on the
 *               call's stream right before and after the sampling kernel.
 *   cut         dev float [B] or NULL: for each sampled row with status OK the
 *               value threshold of the set its token was drawn from (that
 *               set is {allowed z >= cut}); other rows are not written.
 *               sampler_logprobs takes it to return support sets without
 *               selecting the cut again.
 * -------------------------------------------------------------------------- */
#define SAMPLER_ALGO_FAST 0
#define SAMPLER_ALGO_EXACT 1
#define SAMPLER_WAIT_NONE (-1)
typedef struct sampler_options {
  uint32_t size;
  int32_t algo;
  int64_t wait_ns;
  void *trace;
  void *start_event;
  void *stop_event;
  void *cut;
} sampler_options;

int sampler_sample_ex(const sampler_batch *b, const void *logits, int dtype,
                      int64_t ld, const int32_t *bitmask, int64_t mask_ld,
                      const uint8_t *row_has_mask, int32_t *out_ids,
                      float *out_logprobs, int32_t *out_status,
                      void *workspace, size_t ws_bytes, void *stream,
                      const sampler_options *opt);

/* ---- further outputs ------------------------------------------------------
 * What the sampler returns beside the drawn token ([SGL]
 * "LogitsProcessorOutput 的五段结构"): the chosen token's logprob, the top-N
 * logprobs (next_token_top_logprobs_val / _idx), the logprobs of tokens a
 * request names (next_token_token_ids_logprobs_val), and the sampling support
 * set (SamplingMaskOutput: token_ids, lengths, selected_logprobs,
 * support_logprobs, statuses).  sampler_logprobs computes them for a packed
 * batch from the same logits sampler_sample read (after the transforms, the
 * bitmask fused or applied), on `stream`, after the draw when `selected` is
 * given; with `selected` NULL it is the scoring path: logprobs of the same
 * preprocessed logits with no draw ([SGL] "LogitsProcessor 与
 * LogitsProcessorOutput": compute_logprobs_only).
 *
 * Basis of every logprob but the support set's ([SGL] "logprobs 的数值一致
 * 性"): SAMPLER_LOGPROB_SAMPLED (0): log_softmax(z/T) over the allowed
 * tokens, greedy rows log_softmax(z) -- the basis of sampler_sample's
 * out_logprobs; SAMPLER_LOGPROB_ORIGINAL (1): log_softmax(z) for every row,
 * the logits before the temperature.
 *
 * Request (all device arrays; NULL = not asked for):
 *   selected        int32 [B]: the drawn tokens (sampler_sample's out_ids).
 *   top_n_max       columns of the top-N outputs, 0..SAMPLER_MAX_TOP_N.
 *   top_n           int32 [B]: the row's N (top_logprobs_nums), clamped to
 *                   [0, top_n_max]; NULL: top_n_max for every row.
 *   token_indptr    int64 [B+1], token_ids int32: the named tokens per row
 *                   (token_ids_logprobs, CSR).
 *   cuts            float [B]: the thresholds sampler_sample_ex returned
 *                   (option `cut`) for the same batch and logits: support
 *                   sets then take two passes over their row (with a
 *                   workspace, by 4096-token slices, one workgroup each);
 *                   NULL: the threshold is selected again (several more
 *                   passes, one workgroup per support row).
 *   mask_rows       int32 [n_mask_rows]: the rows that return their support
 *                   set (sampling_mask_batch_indices); a row may appear more
 *                   than once; an index outside [0, B) gives status INVALID.
 *   mask_cap        ids kept per support set.
 *   workspace       dev, >= sampler_logprobs_workspace_bytes(B, V,
 *                   top_n_max, n_mask_rows) bytes, 16-byte aligned, or NULL.
 *                   With it the rows are first summarised by 16384-token
 *                   slices (each slice's statistics and top-N) and the
 *                   per-row outputs fold the slices' records,
 *                   and support sets with `cuts` are made by slices; without
 *                   it one workgroup per row streams the row (slower).  Same
 *                   results either way (logprobs within rounding).  Not kept
 *                   between calls; calls that share it must not overlap.
 * Outputs (device; NULL = not written):
 *   next_token_logprobs   float [B]: logprob of selected[r] in the basis
 *                   (needs selected); NaN on an OVERFLOW row or for an id
 *                   outside [0, V), -inf on an INVALID row or a masked id.
 *   top_logprobs_idx int32 [B, top_n_max], top_logprobs_val float: the row's
 *                   N largest z, larger first, the lower id first among equal
 *                   values, with their logprobs; entries past the allowed
 *                   tokens and columns past the row's N are -1 / -inf; an
 *                   OVERFLOW row's N entries are -1 / NaN.  Both or neither;
 *                   required when top_n_max > 0.
 *   token_ids_logprobs float [token_indptr[B]]: logprob of each named token
 *                   (NaN for an id outside [0, V) or on an OVERFLOW row,
 *                   -inf if masked).  Required with token_indptr.
 *   mask_token_ids  int32 [n_mask_rows, mask_cap]: the support set in
 *                   ascending id order, at most mask_cap of it: the tokens the
 *                   row's draw is made from (the set sampler_sample defines;
 *                   a greedy row's is its argmax alone).
 *   mask_support_logprobs float [n_mask_rows, mask_cap]: their logprobs
 *                   renormalised over the whole support (the distribution the
 *                   draw used, at the row's temperature, whatever the basis).
 *   mask_lengths    int32 [n_mask_rows]: ids written, min(|support|, cap).
 *   mask_selected_logprobs float [n_mask_rows]: the renormalised logprob of
 *                   selected[row] (-inf outside the support, NaN without
 *                   selected or for an id outside [0, V)).
 *   mask_statuses   int32 [n_mask_rows]: SAMPLER_STATUS_OK; OVERFLOW: the
 *                   support has more than mask_cap tokens; INVALID: the row has
 *                   no distribution (no finite allowed logit, or a NaN / +inf
 *                   among them).  Severity-ordered so that a MAX reduction
 *                   reaches one decision ([SGL] "LogitsProcessorOutput").
 *   mask_lengths and mask_statuses are required when n_mask_rows > 0, and
 *   mask_token_ids when mask_cap > 0 as well.
 * Other arguments as sampler_sample.  Errors: an inconsistent request (an
 * output without its input, a missing required output, a record of another
 * size, basis or top_n_max out of range, a misaligned workspace) ->
 * SAMPLER_EINVAL; a workspace below the size query -> SAMPLER_ENOSPC;
 * n_mask_rows times the 4096-token slices of a row beyond 2^31 - 1 with a
 * workspace -> SAMPLER_ERANGE; launch failure -> SAMPLER_EHIP.  Nothing asked
 * for: SAMPLER_OK, no launch.
 * -------------------------------------------------------------------------- */
#define SAMPLER_LOGPROB_SAMPLED 0
#define SAMPLER_LOGPROB_ORIGINAL 1
#define SAMPLER_MAX_TOP_N 256
typedef struct sampler_logprob_request {
  uint32_t size; /* sizeof(sampler_logprob_request) as the caller compiled it */
  int32_t basis;
  const int32_t *selected;
  int32_t top_n_max;
  int32_t n_mask_rows;
  const int32_t *top_n;
  const int64_t *token_indptr;
  const int32_t *token_ids;
  const int32_t *mask_rows;
  int32_t mask_cap;
  int32_t pad_;
  const float *cuts;
  void *workspace;
  size_t workspace_bytes;
} sampler_logprob_request;

/* Workspace bytes of sampler_logprobs's slice passes for B rows of V
 * tokens, top_n_max columns and n_mask_rows support rows (0 on an invalid
 * size). */
size_t sampler_logprobs_workspace_bytes(int32_t B, int32_t V, int32_t top_n_max,
                                        int32_t n_mask_rows);

typedef struct sampler_logprob_outputs {
  uint32_t size; /* sizeof(sampler_logprob_outputs) as the caller compiled it */
  int32_t pad_;
  float *next_token_logprobs;
  int32_t *top_logprobs_idx;
  float *top_logprobs_val;
  float *token_ids_logprobs;
  int32_t *mask_token_ids;
  float *mask_support_logprobs;
  int32_t *mask_lengths;
  float *mask_selected_logprobs;
  int32_t *mask_statuses;
} sampler_logprob_outputs;

int sampler_logprobs(const sampler_batch *b, const void *logits, int dtype,
                     int64_t ld, const int32_t *bitmask, int64_t mask_ld,
                     const uint8_t *row_has_mask,
                     const sampler_logprob_request *req,
                     const sampler_logprob_outputs *out, void *stream);

/* ---- vocabulary-parallel sampling: one rank's share ------------------------
 * Under tensor parallelism each rank holds the logits of a slice of the
 * vocabulary ([GLM] "从最后一层 hidden 到 token id": the LM head's output is
 * split along the vocabulary and normally all-gathered before sampling).
 * These calls sample from the shards without gathering the logits ([GLM]
 * "输出侧的通信与开销账本": sample on per-shard results, exchange only what
 * the draw needs): the row's draw is the exact path's (SAMPLER_ALGO_EXACT)
 * decomposed into phases; in each phase every shard makes a small partial
 * record per row (sampler_shard_pass), the ranks all-gather the records, and
 * every rank folds them into the same per-row state (sampler_shard_merge).
 * The race uses global token ids in the Philox counter, so the winner is the
 * best of the shards' winners, and every threshold is summed from exact
 * per-shard integer counts and fixed-point masses: the results are those of
 * sampler_sample_ex with SAMPLER_ALGO_EXACT on the gathered logits (ids and
 * statuses bit for bit; logprobs within rounding).
 *
 * A step: sampler_shard_phases(b) gives the phases the batch needs (bit p
 * set: run phase p); for each p in 0 .. SAMPLER_SHARD_PHASES-1 with its bit
 * set, in order on one stream: sampler_shard_pass on every shard, writing
 * its record block (sampler_shard_partial_bytes(B, width) bytes: the pass
 * splits each row of its shard into slices of 4096 tokens and makes one
 * record per slice, sampler_shard_records(width) per row), then the blocks
 * of all shards side by side (records of n_records = the shards'
 * sampler_shard_records summed, [n_records][B], in any order: ties are
 * broken by global id; what an all-gather of the blocks delivers), then
 * sampler_shard_merge.  The merges
 * write out_ids / out_logprobs / out_status (greedy, INVALID and OVERFLOW
 * rows after phase 0, sampled rows after the last phase).
 *
 *   b         the packed batch of the whole vocabulary (b->V = every shard's
 *             width summed); every rank packs the same parameters.
 *   logits    dev [B, ld]: the shard, tokens v0 .. v0 + width - 1 (after the
 *             transforms, which touch only the shard's own tokens).
 *   v0        global id of the shard's first token: a multiple of 4 (four
 *             tokens share a Philox block), 0 <= v0, v0 + width <= b->V.
 *   bitmask   dev int32 [B, mask_ld] or NULL: the shard's own bitmask, bit j
 *             of the shard's row (bit j&31 of word j>>5) for token v0 + j --
 *             the mask split by vocabulary shard ([GLM] "结构化输出"); mask_ld
 *             >= ceil(width/32).  row_has_mask as sampler_sample.
 *   state     dev, sampler_shard_state_bytes(B), 16-byte aligned: written by
 *             the merges, read by the passes; one per rank.
 * Errors: bad phase, v0, width, strides or sizes -> SAMPLER_EINVAL; launch
 * failure -> SAMPLER_EHIP.  Phases run out of order, or records from other
 * steps, give unspecified results (never out-of-bounds accesses).
 * -------------------------------------------------------------------------- */
#define SAMPLER_SHARD_PHASES 11
size_t sampler_shard_state_bytes(int32_t B);
int32_t sampler_shard_records(int32_t width);
size_t sampler_shard_partial_bytes(int32_t B, int32_t width);
uint32_t sampler_shard_phases(const sampler_batch *b);
int sampler_shard_pass(const sampler_batch *b, int32_t phase, const void *logits,
                       int dtype, int64_t ld, int32_t v0, int32_t width,
                       const int32_t *bitmask, int64_t mask_ld,
                       const uint8_t *row_has_mask, const void *state,
                       void *partial, void *stream);
int sampler_shard_merge(const sampler_batch *b, int32_t phase, void *state,
                        const void *partials, int32_t n_records,
                        int32_t *out_ids, float *out_logprobs,
                        int32_t *out_status, void *stream);

/* ---- speculative verification -----------------------------------------------
 * One verification forward of a linear draft gives k+1 rows per request
 * ([GLM] "投机解码的输出行"): row j of request i (row i*(k+1) + j of the
 * batch) is the distribution after the committed prefix and the first j
 * draft tokens.  After sampler_sample has drawn y_j from every row, draft
 * token j+1 (draft[i*k + j]) is accepted while y_j equals it; the request
 * emits y_0 .. y_n -- the n accepted drafts, then the row's own token at the
 * first mismatch (the bonus token when all k are accepted) -- and the KV the
 * verification wrote past what is kept is rolled back ([SGL] "逐 token 推进":
 * rollback from the first mismatching position).  Emission also stops after
 * the request's terminator token (the tail past it is dropped: [SO] 4.4
 * "推进与终止") and before a row whose status is not OK.
 * Every emitted token is a draw from the target's own distribution given the
 * tokens before it: the rule changes how many tokens a step yields, not
 * their distribution.  Greedy rows verify greedily.
 *   sampled   dev int32 [n_req, k+1] (sampler_sample's out_ids)
 *   status    dev int32 [n_req, k+1] or NULL (sampler_sample's out_status)
 *   draft     dev int32 [n_req, k]
 *   eos       dev int32 [n_req] or NULL: terminator per request, -1 = none
 *   tokens    dev int32 [n_req, k+1]: emitted tokens, then -1
 *   count     dev int32 [n_req]: tokens emitted, 0 .. k+1 (0: row 0 of the
 *             request had no token)
 *   rollback  dev int32 [n_req] or NULL: k + 1 - count, the verified
 *             positions whose KV is not kept
 * Errors: n_req < 0, k < 0, or a required pointer NULL -> SAMPLER_EINVAL;
 * launch failure -> SAMPLER_EHIP.  n_req = 0: SAMPLER_OK, no launch. */
int sampler_spec_accept(int32_t n_req, int32_t k, const int32_t *sampled,
                        const int32_t *status, const int32_t *draft,
                        const int32_t *eos, int32_t *tokens, int32_t *count,
                        int32_t *rollback, void *stream);

#ifdef __cplusplus
}
#endif
#endif
