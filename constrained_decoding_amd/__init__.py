"""MI355X (gfx950) batched per-request sampling step.

[B, V] logits + per-row temperature / top-k / top-p / min-p / penalties /
sparse logit bias / grammar bitmask -> one token id and one logprob per row
(and on request the top-N / named-token logprobs and the sampling support
set), in hand-written HIP kernels behind the C ABI of libcd_sampler.so
(include/cd_sampler.h).  This package is the thin Python binding.
"""
from ._binding import (  # noqa: F401
    ALGO_EXACT, ALGO_FAST, DTYPE_BF16, DTYPE_F32, EXPORTS, FLAG_ALL_GREEDY, FLAG_ANY_GREEDY,
    FLAG_HAS_BIAS, FLAG_NEED_MIN_P, FLAG_NEED_PENALTY, FLAG_NEED_TOP_K, FLAG_NEED_TOP_P,
    FLAG_SPLIT_PASS2, LIB_PATH, LOGPROB_ORIGINAL, LOGPROB_SAMPLED, MAX_TOP_N, STATUS_INVALID,
    STATUS_OK, STATUS_OVERFLOW, WAIT_NONE, Batch, HostParams, LogprobOutputs, LogprobRequest,
    Options, PackedBatch, SamplerError, Workspace, apply_bitmask, apply_transforms,
    bias_from_dict, csr, logprobs, SHARD_PHASES, ShardBuffers, shard_sample, spec_accept,
    ORDER_JOINT, ORDER_MINP_FIRST, ORDER_MINP_LAST, lib, pack_host, sample, strerror, version,
)
