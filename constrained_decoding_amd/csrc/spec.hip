// spec.hip -- speculative verification of linear drafts, for gfx950.
//
// One verification forward gives k+1 rows per request: the distribution of
// the token after the committed prefix, then after each of the k draft
// tokens ("GLM-5.3 推理全链路(七)", section 投机解码的输出行).  The sampling
// step draws a token y_j from every row; draft token j+1 is accepted while
// y_j equals it, and the request emits y_0 .. y_n: the n accepted drafts and
// the row's own token at the first mismatch (the bonus token when every
// draft is accepted).  The KV the verification wrote past what is kept is
// rolled back ("SGLang 源码完全拆解(十)", section 逐 token 推进: rollback from
// the first mismatching position; "04 · 结构化输出", 4.4 推进与终止: the tail
// past a terminator is dropped).
// Each emitted token is a sample of the target's own distribution given the
// tokens before it, so the rule changes how many tokens a step yields, never
// their distribution.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace cds {

constexpr int kSpecNT = 256;

// One thread per request; the request's k+1 rows are consecutive.
__global__ __launch_bounds__(kSpecNT) void spec_accept_kernel(const SpecArgs a) {
  const int i = blockIdx.x * kSpecNT + threadIdx.x;
  if (i >= a.n_req) return;
  const int k = a.k;
  const int32_t* y = a.sampled + (int64_t)i * (k + 1);
  const int32_t* st = a.status ? a.status + (int64_t)i * (k + 1) : nullptr;
  const int32_t* d = a.draft + (int64_t)i * k;
  int32_t* out = a.tokens + (int64_t)i * (k + 1);
  const int32_t eos = a.eos ? a.eos[i] : -1;
  int count = 0;
  for (int j = 0; j <= k; ++j) {
    if (st && st[j] != 0) break;             // no token at this row
    const int32_t t = y[j];
    out[count++] = t;
    if (eos >= 0 && t == eos) break;         // terminator: nothing after it
    if (j == k || t != d[j]) break;          // first mismatch (or the bonus token)
  }
  for (int j = count; j <= k; ++j) out[j] = -1;
  a.count[i] = count;
  if (a.rollback) a.rollback[i] = k + 1 - count;
}

hipError_t launch_spec_accept(const SpecArgs& a, hipStream_t stream) {
  if (a.n_req <= 0) return hipSuccess;
  hipLaunchKernelGGL(spec_accept_kernel, dim3((unsigned)((a.n_req + kSpecNT - 1) / kSpecNT)),
                     dim3(kSpecNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cds
