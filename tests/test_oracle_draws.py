"""Distributional pin of the oracle's draw.

For V <= 16, 10^6 seeded draws (offsets 0..10^6-1) are compared by a
chi-square test with the closed-form renormalised distribution
p'_t = w_t 1[t in S] / sum_S w  (GLM-5.3 推理全链路(七), section 采样,
renormalised-draw formula), where S is computed here directly from the set
definitions of SGLang 源码完全拆解(十), section 概率裁剪的数学 -- not from
the oracle's sort-based code.
"""
import numpy as np
import pytest
from scipy.stats import chisquare

import oracle
import workloads

N_DRAWS = 1_000_000


def _support(z, T, k, p, mp):
    fin = np.isfinite(z)
    s = np.where(fin, z.astype(np.float64) / np.float64(np.float32(T)), -np.inf)
    w = np.where(fin, np.exp(s - s.max()), 0.0)
    S = fin.copy()
    if mp > 0:
        S &= w >= np.float64(np.float32(mp))
    if 1 < k < S.sum():
        rank = np.array([np.sum(S & (s > s[t])) for t in range(len(z))])
        S &= rank < k
    if p < 1:
        M = w[S].sum()
        above = np.array([w[S & (s > s[t])].sum() for t in range(len(z))])
        S &= above < np.float64(np.float32(p)) * M
    q = np.where(S, w, 0.0)
    return q / q.sum()


MODES = {
    "none":     dict(T=0.9, k=0, p=1.0, mp=0.0, mask=None),
    "min_p":    dict(T=1.1, k=0, p=1.0, mp=0.12, mask=None),
    "top_k":    dict(T=0.8, k=5, p=1.0, mp=0.0, mask=None),
    "top_p":    dict(T=1.0, k=0, p=0.7, mp=0.0, mask=None),
    "mask":     dict(T=1.3, k=0, p=1.0, mp=0.0, mask=[0, 2, 3, 5, 8, 9, 11, 12, 15]),
    "combined": dict(T=0.7, k=7, p=0.9, mp=0.02, mask=[1, 2, 3, 4, 6, 7, 9, 10, 12, 13, 14]),
}


@pytest.mark.slow
@pytest.mark.parametrize("mode", list(MODES))
def test_draws_match_renormalised_distribution(mode):
    cfg = MODES[mode]
    rng = workloads.rng_for(200, salt=list(MODES).index(mode))
    V = 16
    z = (rng.standard_normal(V) * 1.5).astype(np.float32)
    if cfg["mask"] is not None:
        z = oracle.transform_row(z, mask=workloads.pack_bitmask([np.array(cfg["mask"])], V)[0])
    q = _support(z, cfg["T"], cfg["k"], cfg["p"], cfg["mp"])
    n = N_DRAWS
    res = oracle.sample_batch(
        z, T=np.full(n, cfg["T"], np.float32), top_k=np.full(n, cfg["k"], np.int32),
        top_p=np.full(n, cfg["p"], np.float32), min_p=np.full(n, cfg["mp"], np.float32),
        seed=np.full(n, 0x5EED0000 + V, np.uint64), offset=np.arange(n, dtype=np.uint64),
        broadcast=True)
    ids = res["id"]
    counts = np.bincount(ids, minlength=V)
    assert np.all(counts[q == 0] == 0), "drew a token outside the support"
    sup = q > 0
    assert sup.sum() >= 2
    pv = chisquare(counts[sup], n * q[sup]).pvalue
    assert pv > 1e-3, (mode, pv, counts, q)


def test_masked_tokens_never_drawn_100k():
    rng = workloads.rng_for(201)
    V = 64
    z = (rng.standard_normal(V) * 3).astype(np.float32)
    allowed = rng.choice(V, size=9, replace=False)
    zt = oracle.transform_row(z, mask=workloads.pack_bitmask([allowed], V)[0])
    n = 100_000
    for T, k, p in [(1.0, 0, 1.0), (0.5, 3, 0.9), (2.0, 0, 0.99)]:
        ids = oracle.sample_batch(zt, T=np.full(n, T, np.float32),
                                  top_k=np.full(n, k, np.int32),
                                  top_p=np.full(n, p, np.float32),
                                  min_p=np.zeros(n, np.float32),
                                  seed=np.full(n, 11, np.uint64),
                                  offset=np.arange(n, dtype=np.uint64), broadcast=True)["id"]
        assert set(np.unique(ids).tolist()) <= set(allowed.tolist())
