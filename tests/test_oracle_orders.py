"""Pins of the oracle's filter orders (CPU only).

The pages give three ways to stack min-p, top-k and top-p ("SGLang 源码完全
拆解(十)", section 概率裁剪的数学 and section 后端分支; "GLM-5.3 推理全链路(七)",
section 采样):
  - min-p first, then top-k, then top-p on what is left (vLLM's order; the
    default);
  - top-k, renormalise, top-p, renormalise, min-p (SGLang's FlashInfer path
    when a row has min-p);
  - top-k and top-p applied jointly to one distribution, keeping their
    intersection (SGLang's fused sampler, filter_apply_order="joint").
Every cut keeps a prefix of the tokens by value, so each order keeps
S1 & Tk & {t : mass strictly above t < top_p * M} and they differ only in
the mass M the top-p cut is normalised by.  The tests below compute the
kept set straight from the definitions (pairwise comparisons over the
tokens, no sorting, nothing from the oracle) and compare, check a row on
which the three orders keep three different sets, and compare 10^6 draws
per order with the renormalised distribution by chi-square.
"""
import numpy as np
import pytest
from scipy.stats import chisquare

import oracle
import workloads

ORDERS = [oracle.ORDER_MINP_FIRST, oracle.ORDER_JOINT, oracle.ORDER_MINP_LAST]


def _kept_by_definition(z, T, k, p, mp, order):
    """The drawn-from set, from the definitions, in float64."""
    fin = np.isfinite(z)
    s = np.where(fin, z.astype(np.float64) / np.float64(np.float32(T)), -np.inf)
    w = np.where(fin, np.exp(s - s[fin].max()), 0.0)
    V = len(z)
    # min-p: weight relative to the maximum (renormalising never moves it)
    S1 = fin & (w >= np.float64(np.float32(mp))) if mp > 0 else fin.copy()
    # top-k over every finite token: fewer than k tokens strictly above
    nfin = int(fin.sum())
    if 1 < k < nfin:
        rank = np.array([np.sum(fin & (s > s[t])) for t in range(V)])
        Tk = fin & (rank < k)
    else:
        Tk = fin.copy()
    # top-k within the min-p set (first order): fewer than k of S1 above
    if 1 < k < int(S1.sum()):
        rank1 = np.array([np.sum(S1 & (s > s[t])) for t in range(V)])
        S2 = S1 & (rank1 < k)
    else:
        S2 = S1.copy()
    if order == oracle.ORDER_MINP_FIRST:
        kept = S2
        norm = S2
    elif order == oracle.ORDER_MINP_LAST:
        kept = Tk & S1
        norm = Tk
    else:
        kept = Tk & S1
        norm = fin
    if p < 1:
        M = w[norm].sum()
        above = np.array([w[fin & (s > s[t])].sum() for t in range(V)])
        kept = kept & (above < np.float64(np.float32(p)) * M)
    return kept, w


def test_first_order_reads_as_top_k_within_min_p():
    """Reading of the first order: top-k within the min-p set equals the
    min-p set intersected with the top-k set over every token (both cut a
    prefix of the tokens by value), on random rows with ties."""
    rng = workloads.rng_for(300)
    for trial in range(300):
        V = int(rng.integers(2, 14))
        z = np.round(rng.standard_normal(V) * 2).astype(np.float32)
        z[rng.random(V) < 0.2] = -np.inf
        if not np.isfinite(z).any():
            continue
        k, mp = int(rng.integers(0, V + 2)), float(rng.choice([0.0, 0.1, 0.4]))
        a, _ = _kept_by_definition(z, 1.0, k, 1.0, mp, oracle.ORDER_MINP_FIRST)
        b, _ = _kept_by_definition(z, 1.0, k, 1.0, mp, oracle.ORDER_MINP_LAST)
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("order", ORDERS)
def test_kept_set_matches_definition_random_small(order):
    rng = workloads.rng_for(301, salt=order)
    for trial in range(400):
        V = int(rng.integers(1, 13))
        z = (rng.standard_normal(V) * 2).astype(np.float32)
        if trial % 3 == 0:
            z = np.round(z).astype(np.float32)           # ties
        z[rng.random(V) < 0.15] = -np.inf
        if not np.isfinite(z).any():
            continue
        T = float(rng.choice([0.5, 1.0, 1.7]))
        k = int(rng.integers(0, V + 2))
        p = float(rng.choice([1.0, 0.3, 0.6, 0.9]))
        mp = float(rng.choice([0.0, 0.05, 0.3]))
        r, sets = oracle.sample_row(z, T=T, top_k=k, top_p=p, min_p=mp, seed=trial,
                                    offset=trial, want_sets=True, order=order)
        if T < 1e-5 or k == 1:
            continue
        kept, _ = _kept_by_definition(z, T, k, p, mp, order)
        np.testing.assert_array_equal((sets & 4) != 0, kept,
                                      err_msg=f"order {order} z={z} T={T} k={k} p={p} mp={mp}")
        assert kept[r["id"]]


def test_three_orders_keep_three_different_sets():
    """Weights (T = 1, relative to the maximum) 1, 0.45, 0.40 above min_p =
    0.35; 0.34 and 0.33 complete the top-5; twenty tokens of 0.05 below.
    top_p = 0.5 normalises by 1.85 (min-p first), 2.52 (min-p last) or 3.52
    (joint): the kept sets are {0}, {0, 1} and {0, 1, 2}."""
    w = np.array([1.0, 0.45, 0.40, 0.34, 0.33] + [0.05] * 20)
    z = np.log(w).astype(np.float32)
    got = {}
    for order in ORDERS:
        _, sets = oracle.sample_row(z, T=1.0, top_k=5, top_p=0.5, min_p=0.35, want_sets=True,
                                    order=order)
        got[order] = np.nonzero(sets & 4)[0].tolist()
        kept, _ = _kept_by_definition(z, 1.0, 5, 0.5, 0.35, order)
        assert got[order] == np.nonzero(kept)[0].tolist()
    assert got[oracle.ORDER_MINP_FIRST] == [0]
    assert got[oracle.ORDER_MINP_LAST] == [0, 1]
    assert got[oracle.ORDER_JOINT] == [0, 1, 2]


def test_orders_agree_without_a_second_cut():
    """With top-p as the only cut, or without top-p, the three orders keep
    the same set and draw the same token (same Philox stream)."""
    rng = workloads.rng_for(302)
    z = (rng.standard_normal(3000) * 2).astype(np.float32)
    for k, p, mp in [(0, 0.8, 0.0), (40, 1.0, 0.0), (0, 1.0, 0.05), (40, 1.0, 0.05)]:
        ids = {oracle.sample_row(z, T=0.9, top_k=k, top_p=p, min_p=mp, seed=5, offset=9,
                                 order=o)["id"] for o in ORDERS}
        assert len(ids) == 1, (k, p, mp, ids)


def test_unknown_order_rejected():
    with pytest.raises(ValueError):
        oracle.sample_row(np.zeros(4, np.float32), T=1.0, order=7)


N_DRAWS = 1_000_000


@pytest.mark.slow
@pytest.mark.parametrize("order", ORDERS)
def test_draws_match_renormalised_distribution_per_order(order):
    """10^6 draws with all three cuts active (V = 16): chi-square against
    w_t 1[t kept] / sum_kept w, the kept set from the definitions."""
    rng = workloads.rng_for(303)
    V = 16
    z = (rng.standard_normal(V) * 1.5).astype(np.float32)
    T, k, p, mp = 0.9, 9, 0.75, 0.03
    kept, w = _kept_by_definition(z, T, k, p, mp, order)
    q = np.where(kept, w, 0.0)
    q /= q.sum()
    n = N_DRAWS
    res = oracle.sample_batch(
        z, T=np.full(n, T, np.float32), top_k=np.full(n, k, np.int32),
        top_p=np.full(n, p, np.float32), min_p=np.full(n, mp, np.float32),
        seed=np.full(n, 0x0DE5 + order, np.uint64), offset=np.arange(n, dtype=np.uint64),
        broadcast=True, order=order)
    counts = np.bincount(res["id"], minlength=V)
    assert np.all(counts[q == 0] == 0)
    sup = q > 0
    assert sup.sum() >= 2
    pv = chisquare(counts[sup], n * q[sup]).pvalue
    assert pv > 1e-3, (order, pv, counts, q)
