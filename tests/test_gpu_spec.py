"""GPU parity of speculative verification (sampler_spec_accept) against the
oracle ("GLM-5.3 推理全链路(七)", section 投机解码的输出行; "SGLang 源码完全
拆解(十)", section 逐 token 推进): the emitted tokens, their count and the
rolled-back positions, bit for bit."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_harness import run_gpu, run_oracle_parallel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import constrained_decoding_amd  # noqa: F401  (must load: no fallback)


def _oracle_accept(sampled, draft, status, eos):
    n_req, k1 = sampled.shape
    tok = np.full((n_req, k1), -1, np.int32)
    cnt = np.zeros(n_req, np.int32)
    rb = np.zeros(n_req, np.int32)
    for i in range(n_req):
        t, n, r = oracle.spec_accept(sampled[i], draft[i],
                                     None if status is None else status[i],
                                     -1 if eos is None else int(eos[i]))
        tok[i, :n] = t
        cnt[i] = n
        rb[i] = r
    return tok, cnt, rb


def _gpu_accept(sampled, draft, status, eos):
    import torch
    import constrained_decoding_amd as cds
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    tok, cnt, rb = cds.spec_accept(d(sampled), d(draft), status=d(status), eos=d(eos))
    torch.cuda.synchronize()
    return tok.cpu().numpy(), cnt.cpu().numpy(), rb.cpu().numpy()


@pytest.mark.parametrize("k", [0, 1, 7, 15])
def test_accept_rule_random_inputs(k):
    """Seeded random rows, drafts that match for a random prefix, statuses
    with INVALID / OVERFLOW rows and terminators; 1000 requests (several
    workgroups and a ragged tail)."""
    rng = np.random.default_rng(800 + k)
    n_req, V = 1000, 50
    sampled = rng.integers(0, V, (n_req, k + 1)).astype(np.int32)
    draft = rng.integers(0, V, (n_req, k)).astype(np.int32)
    for i in range(n_req):                    # a matching prefix of random length
        m = int(rng.integers(0, k + 1))
        draft[i, :m] = sampled[i, :m]
    status = np.zeros((n_req, k + 1), np.int32)
    bad = rng.random((n_req, k + 1)) < 0.03
    status[bad] = rng.choice([1, 2], int(bad.sum()))
    sampled[status != 0] = -1
    eos = np.where(rng.random(n_req) < 0.3, rng.integers(0, V, n_req), -1).astype(np.int32)
    for st, eo in ((None, None), (status, None), (status, eos)):
        got = _gpu_accept(sampled, draft, st, eo)
        ref = _oracle_accept(sampled, draft, st, eo)
        for g, r in zip(got, ref):
            np.testing.assert_array_equal(g, r)


@pytest.mark.parametrize("variant", ["a", "b"])
def test_verify_step_spec_shape(variant):
    """The spec-verify step: 64 requests x 8 rows (k = 7), V = 151936, greedy
    (c5a) or T = 1, top_k = 50 (c5b), sampled on the GPU; drafts made from the
    oracle's draws of the same rows, each request's matching prefix cut at a
    random position.  The GPU's emitted tokens, counts and rollbacks equal
    the oracle's."""
    batch = workloads.c5_spec(variant)
    n_req, k1 = 64, 8
    print(f"[case] spec verify c5{variant}", flush=True)
    ids, _, st = run_gpu(batch)
    ref = run_oracle_parallel(batch)
    o_ids = ref["id"].astype(np.int32).reshape(n_req, k1)
    rng = np.random.default_rng(810)
    draft = o_ids[:, :k1 - 1].copy()
    cut = rng.integers(0, k1, n_req)
    for i in range(n_req):
        if cut[i] < k1 - 1:
            draft[i, cut[i]] = (draft[i, cut[i]] + 1 + int(rng.integers(0, 1000))) % batch.V
    got = _gpu_accept(ids.reshape(n_req, k1), draft, st.reshape(n_req, k1), None)
    want = _oracle_accept(o_ids, draft, ref["status"].astype(np.int32).reshape(n_req, k1), None)
    for g, r in zip(got, want):
        np.testing.assert_array_equal(g, r)
    assert got[1].min() >= 1 and got[1].max() == k1
