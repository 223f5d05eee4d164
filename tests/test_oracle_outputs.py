"""Pins of the oracle's further outputs: top logprobs, logprobs of named
tokens, the pre-temperature basis and the sampling support set
("SGLang 源码完全拆解(十)", sections LogitsProcessorOutput 的五段结构,
logprobs 的数值一致性, LogitsProcessor 与 LogitsProcessorOutput).

Each check compares the oracle with a library routine (scipy's log_softmax,
numpy's lexsort), a closed form, an invariant or an independent brute-force
formulation of the set the row is drawn from.  CPU only.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
import workloads


def _z(rng, V, scale=2.0, ninf=0.0, quant=None):
    z = (rng.standard_normal(V) * scale).astype(np.float32)
    if quant:
        z = (np.round(z * quant) / quant).astype(np.float32)
    if ninf:
        z[rng.random(V) < ninf] = -np.inf
    return z


# ------------------------------------------------------------ log-softmax --

@pytest.mark.parametrize("T", [0.3, 1.0, 1.7])
def test_set_log_softmax_matches_scipy(T):
    rng = workloads.rng_for(301)
    for trial in range(30):
        V = int(rng.integers(1, 4000))
        z = _z(rng, V, ninf=0.2 if trial % 2 else 0.0)
        sel = None if trial % 3 == 0 else (rng.random(V) < 0.5).astype(np.uint8) * 4
        n, lp = oracle.set_log_softmax(z, T, sel, 4)
        keep = np.isfinite(z) & (True if sel is None else sel > 0)
        assert n == int(keep.sum())
        if n == 0:
            assert np.all(lp == -np.inf)
            continue
        ref = scipy.special.log_softmax(z[keep].astype(np.float64) / np.float64(T))
        np.testing.assert_allclose(lp[keep], ref, rtol=0, atol=1e-12)
        assert np.all(lp[~keep] == -np.inf)
        # invariant: the set's probabilities sum to one
        assert abs(math.fsum(np.exp(lp[keep])) - 1.0) < 1e-12


def test_set_log_softmax_two_token_closed_form():
    for a, b, T in [(0.0, 1.0, 1.0), (3.5, -2.0, 0.4), (10.0, 10.0, 2.0), (-7.0, 5.0, 0.9)]:
        z = np.array([a, b], np.float32)
        _, lp = oracle.set_log_softmax(z, T)
        d = (float(np.float32(b)) - float(np.float32(a))) / T
        assert abs(lp[0] - (-math.log1p(math.exp(d)))) < 1e-13
        assert abs(lp[1] - (-math.log1p(math.exp(-d)))) < 1e-13


def test_set_log_softmax_nonfinite():
    z = np.array([0.0, np.nan, 1.0, np.inf], np.float32)
    n, lp = oracle.set_log_softmax(z, 1.0)
    assert n == -1 and np.all(np.isnan(lp))
    # outside the set they do not count
    sel = np.array([1, 0, 1, 0], np.uint8)
    n, lp = oracle.set_log_softmax(z, 1.0, sel, 1)
    assert n == 2 and lp[1] == -np.inf and lp[3] == -np.inf
    assert abs(lp[2] - (-math.log1p(math.exp(-1.0)))) < 1e-13


# ------------------------------------------------------------------ top-N --

def test_top_n_matches_lexsort_with_ties_and_padding():
    rng = workloads.rng_for(302)
    for trial in range(60):
        V = int(rng.integers(1, 300))
        z = _z(rng, V, quant=2 if trial % 2 else None, ninf=0.3 if trial % 3 == 0 else 0.0)
        _, lp = oracle.set_log_softmax(z, 0.8)
        for N in (0, 1, 5, 40, V + 3):
            ids, vals = oracle.top_n(z, lp, N)
            fin = np.flatnonzero(np.isfinite(z))
            order = fin[np.lexsort((fin, -z[fin].astype(np.float64)))]
            want = np.full(N, -1)
            k = min(N, order.shape[0])
            want[:k] = order[:k]
            np.testing.assert_array_equal(ids, want)
            np.testing.assert_array_equal(vals[:k], lp[want[:k]])
            assert np.all(vals[k:] == -np.inf)


# ------------------------------------------------------------ row outputs --

def _support_def(z, T, k, p, mp):
    """The drawn-from set by its definition written directly (min-p, rank
    below k counting strictly larger members, strictly-greater mass below
    p times the mass of what min-p and top-k left)."""
    fin = np.isfinite(z)
    s = np.where(fin, z.astype(np.float64) / np.float64(np.float32(T)), -np.inf)
    w = np.where(fin, np.exp(s - s.max()), 0.0)
    S = fin & ((w >= np.float64(np.float32(mp))) if mp > 0 else True)
    if 1 < k < int(S.sum()):
        S = S & np.array([np.sum(S & (s > s[t])) < k for t in range(len(z))])
    if p < 1:
        M = w[S].sum()
        S = S & np.array([w[S & (s > s[t])].sum() < np.float64(np.float32(p)) * M
                          for t in range(len(z))])
    return S


def test_support_set_is_the_drawn_set_renormalised():
    rng = workloads.rng_for(303)
    for trial in range(200):
        V = int(rng.integers(2, 60))
        z = _z(rng, V, scale=float(rng.choice([0.5, 2.0])), quant=2 if trial % 4 == 0 else None,
               ninf=0.25 if trial % 5 == 0 else 0.0)
        if not np.isfinite(z).any():
            continue
        T = float(rng.choice([0.3, 1.0, 2.5]))
        k = int(rng.choice([0, 2, 3, 100]))
        p = float(rng.choice([1.0, 0.9, 0.5]))
        mp = float(rng.choice([0.0, 0.1]))
        cap = int(rng.choice([1, 4, 1000]))
        o = oracle.row_outputs(z, T=T, top_k=k, top_p=p, min_p=mp, seed=trial,
                               selected=None, support_cap=cap)
        S = _support_def(z, T, k, p, mp)
        allids = np.flatnonzero(S)
        assert o["sup_n"] == allids.shape[0]
        np.testing.assert_array_equal(o["sup_ids"], allids[:cap])
        assert o["sup_status"] == (oracle.STATUS_OVERFLOW if allids.shape[0] > cap
                                   else oracle.STATUS_OK)
        ref = scipy.special.log_softmax(z[S].astype(np.float64) / np.float64(np.float32(T)))
        np.testing.assert_allclose(o["sup_vals"], ref[:cap], rtol=0, atol=1e-12)
        # the drawn token lies in the support; its renormalised logprob is
        # its logprob minus the log of the support's probability mass
        o2 = oracle.row_outputs(z, T=T, top_k=k, top_p=p, min_p=mp, seed=trial,
                                selected=int(o["res"]["id"]), support_cap=cap)
        t = int(o["res"]["id"])
        assert S[t]
        full = scipy.special.log_softmax(z[np.isfinite(z)].astype(np.float64) / np.float64(np.float32(T)))
        mass = scipy.special.logsumexp(full[S[np.isfinite(z)]])
        assert abs(o2["sup_sel"] - (o2["next"] - mass)) < 1e-12
        # a token outside the support has probability zero
        out = np.flatnonzero(np.isfinite(z) & ~S)
        if out.shape[0]:
            o3 = oracle.row_outputs(z, T=T, top_k=k, top_p=p, min_p=mp, seed=trial,
                                    selected=int(out[0]), support_cap=cap)
            assert o3["sup_sel"] == -np.inf


def test_greedy_support_is_the_argmax_and_basis_is_unscaled():
    rng = workloads.rng_for(304)
    z = _z(rng, 500)
    for T, k in [(0.0, 0), (0.7, 1)]:
        o = oracle.row_outputs(z, T=T, top_k=k, n_top=3, token_ids=[5, 6], selected=int(np.argmax(z)),
                               support_cap=8)
        assert o["res"]["greedy"] == 1
        np.testing.assert_array_equal(o["sup_ids"], [int(np.argmax(z))])
        assert o["sup_vals"][0] == 0.0 and o["sup_sel"] == 0.0 and o["sup_status"] == 0
        ref = scipy.special.log_softmax(z.astype(np.float64))
        np.testing.assert_allclose(o["tok_vals"], ref[[5, 6]], rtol=0, atol=1e-12)
        assert abs(o["next"] - ref.max()) < 1e-12
        np.testing.assert_array_equal(o["top_ids"], np.argsort(-z.astype(np.float64), kind="stable")[:3])


def test_original_basis_is_the_pre_temperature_log_softmax():
    rng = workloads.rng_for(305)
    z = _z(rng, 3000, ninf=0.1)
    fin = np.isfinite(z)
    ids = [0, 17, 2999, -1, 3000]
    for T in (0.3, 1.0, 1.9):
        samp = oracle.row_outputs(z, T=T, top_p=0.9, n_top=10, token_ids=ids, seed=3)
        orig = oracle.row_outputs(z, T=T, top_p=0.9, n_top=10, token_ids=ids, seed=3,
                                  basis=oracle.BASIS_ORIGINAL)
        ref_o = np.full(3000, -np.inf)
        ref_o[fin] = scipy.special.log_softmax(z[fin].astype(np.float64))
        ref_s = np.full(3000, -np.inf)
        ref_s[fin] = scipy.special.log_softmax(z[fin].astype(np.float64) / np.float64(np.float32(T)))
        for o, ref in ((samp, ref_s), (orig, ref_o)):
            np.testing.assert_allclose(o["tok_vals"][:3], ref[ids[:3]], rtol=0, atol=1e-12)
            assert np.all(np.isnan(o["tok_vals"][3:]))
            np.testing.assert_allclose(o["top_vals"], ref[o["top_ids"]], rtol=0, atol=1e-12)
        # the ranking does not depend on the basis; the values do unless T = 1
        np.testing.assert_array_equal(samp["top_ids"], orig["top_ids"])
        if T == 1.0:
            np.testing.assert_array_equal(samp["top_vals"], orig["top_vals"])
        else:
            assert np.max(np.abs(samp["top_vals"] - orig["top_vals"])) > 1e-3


def test_status_rows():
    z = np.array([0.0, 1.0, np.nan, 2.0], np.float32)
    o = oracle.row_outputs(z, T=0.8, n_top=2, token_ids=[0, 1], selected=1, support_cap=4)
    assert o["res"]["status"] == oracle.STATUS_OVERFLOW
    assert np.all(o["top_ids"] == -1) and np.all(np.isnan(o["top_vals"]))
    assert np.all(np.isnan(o["tok_vals"])) and math.isnan(o["next"])
    assert o["sup_status"] == oracle.STATUS_INVALID and o["sup_len"] == 0
    z = np.full(4, -np.inf, np.float32)
    o = oracle.row_outputs(z, T=0.8, n_top=2, token_ids=[0, 9], selected=-1, support_cap=4)
    assert o["res"]["status"] == oracle.STATUS_INVALID
    assert np.all(o["top_ids"] == -1) and np.all(o["top_vals"] == -np.inf)
    assert o["tok_vals"][0] == -np.inf and math.isnan(o["tok_vals"][1])
    assert o["next"] == -np.inf
    assert o["sup_status"] == oracle.STATUS_INVALID and o["sup_len"] == 0
