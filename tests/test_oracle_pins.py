"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a figure the pages print
(tests/golden/), a textbook or library routine (numpy, scipy, torch, Python
dict semantics), an independent brute-force formulation of a set definition,
or a distributional test.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ Philox --

def test_philox_round_structure_matches_numpy_4x64():
    """numpy.random.Philox is Philox-4x64-10; it advances the 256-bit counter
    before producing each block, so block n of counter c is philox(c + n + 1).
    The oracle's 4x32 instance is generated from the same macro body."""
    rng = np.random.Generator(np.random.PCG64(1))
    for _ in range(25):
        key = rng.integers(0, 2**64, size=2, dtype=np.uint64)
        ctr = rng.integers(0, 2**63, size=4, dtype=np.uint64)
        bg = np.random.Philox(key=key, counter=ctr)
        ref = bg.random_raw(8).astype(np.uint64)
        c1 = ctr.copy(); c1[0] += np.uint64(1)
        c2 = ctr.copy(); c2[0] += np.uint64(2)
        got = np.concatenate([oracle.philox4x64_10(c1, key), oracle.philox4x64_10(c2, key)])
        np.testing.assert_array_equal(got, ref)


def test_philox_weyl_constants_closed_form():
    """W0/W1 are the leading fraction bits of the golden ratio and sqrt(3)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    phi = (Decimal(1) + Decimal(5).sqrt()) / 2
    s3 = Decimal(3).sqrt()
    def frac_bits(x, bits):
        f = x - int(x)
        return int(f * (Decimal(2) ** bits))
    c = oracle.philox_constants()
    assert c[2] == frac_bits(phi, 32) and c[3] == frac_bits(s3, 32)
    assert c[6] == frac_bits(phi, 64) and c[7] == frac_bits(s3, 64)
    # multipliers: odd (bijective mod 2^w), as the round function requires
    assert all(v & 1 for v in (c[0], c[1], c[4], c[5]))


def test_philox_counter_and_key_sensitivity():
    """Flipping any single input bit changes about half the output bits
    (avalanche) -- a dropped xor or a dead counter word fails this."""
    rng = np.random.Generator(np.random.PCG64(2))
    flips = []
    for _ in range(200):
        ctr = rng.integers(0, 2**32, size=4, dtype=np.uint64).astype(np.uint32)
        key = rng.integers(0, 2**32, size=2, dtype=np.uint64).astype(np.uint32)
        base = oracle.philox4x32_10(ctr, key)
        word = rng.integers(0, 6)
        bit = np.uint32(1 << int(rng.integers(0, 32)))
        c2, k2 = ctr.copy(), key.copy()
        if word < 4:
            c2[word] ^= bit
        else:
            k2[word - 4] ^= bit
        out = oracle.philox4x32_10(c2, k2)
        flips.append(sum(bin(int(a) ^ int(b)).count("1") for a, b in zip(base, out)))
    mean = np.mean(flips)
    assert 60 < mean < 68, mean  # 64 expected out of 128 bits


def test_race_bits_layout():
    """Token t reads word t&3 of the block at counter (t>>2, off_lo, off_hi, 0)
    under key (seed_lo, seed_hi)."""
    seed, off = 0x0123456789ABCDEF, 0xFEDCBA9876543210
    for t in [0, 1, 2, 3, 4, 7, 1023, 151935]:
        blk = oracle.philox4x32_10([t >> 2, off & 0xFFFFFFFF, off >> 32, 0],
                                   [seed & 0xFFFFFFFF, seed >> 32])
        assert oracle.race_bits(seed, off, t) == int(blk[t & 3])


def test_uniform24_closed_forms():
    assert oracle.uniform24(0) == 2.0 ** -24
    assert oracle.uniform24(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert oracle.uniform24(0x80000000) == 0.5 + 2.0 ** -24
    assert oracle.uniform24(0x1FF) == 2.0 ** -24          # low 9 bits dropped
    # symmetric grid: U(x) + U(~x) == 1 exactly
    for x in [0, 12345, 0xDEADBEEF, 0x7FFFFFFF]:
        assert oracle.uniform24(x) + oracle.uniform24(~x & 0xFFFFFFFF) == 1.0


def test_race_uniforms_are_uniform():
    """Chi-square of 2^16 uniforms over 64 bins, and lag-1 correlation."""
    seed = 0xC0FFEE
    u = np.array([oracle.uniform24(oracle.race_bits(seed, 3, t)) for t in range(1 << 16)])
    counts = np.bincount((u * 64).astype(int), minlength=64)
    from scipy.stats import chisquare
    assert chisquare(counts).pvalue > 1e-4
    r = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(r) < 0.02


# -------------------------------------------------------------- transforms --

def test_transforms_hand_closed_forms():
    for case in _golden("transforms_hand.json")["cases"]:
        z = np.array(case["z"], np.float32)
        got = oracle.transform_row(z, hist_ids=np.array(case["hist"]), rep=case["rep"],
                                   freq=case["freq"], pres=case["pres"])
        np.testing.assert_allclose(got, np.array(case["expected"]), rtol=1e-6, atol=1e-7,
                                   err_msg=case["name"])
        if "reverse_order_would_give" in case:
            assert not np.allclose(got, case["reverse_order_would_give"])


def test_transform_untouched_tokens_bit_identical():
    rng = workloads.rng_for(90)
    z = rng.standard_normal(4096).astype(np.float32)
    hist = rng.integers(0, 4096, size=300)
    got = oracle.transform_row(z, hist_ids=hist, rep=1.3, freq=0.2, pres=0.1)
    untouched = np.setdiff1d(np.arange(4096), hist)
    np.testing.assert_array_equal(got[untouched].view(np.uint32), z[untouched].view(np.uint32))
    assert np.all(got[np.unique(hist)] != z[np.unique(hist)])


def test_bias_key_collision_last_wins():
    """The page's '1' vs '01' example: an int-keyed dict comprehension keeps one
    entry per token, the later value (Python dict semantics)."""
    g = _golden("page_figures.json")["bias_key_collision"]
    dedup = {int(k): v for k, v in g["keys"].items()}   # the library behaviour
    assert list(dedup) == [1]
    z = np.zeros(4, np.float32)
    got = oracle.transform_row(z, bias_ids=np.array([1, 1]), bias_vals=np.array([5.0, -3.0]))
    np.testing.assert_array_equal(got, np.array([0.0, dedup[1], 0.0, 0.0], np.float32))


def test_mask_semantics_and_row_width():
    """-1 words allow everything; bit t&31 of word t>>5 is token t; bit 0 ->
    exactly -inf; bias cannot lift a masked token.  Row width at the page's
    vocab (152064) is 19008 bytes."""
    g = _golden("page_figures.json")
    V = g["bitmask_row"]["V"]
    W = (V + 31) // 32
    assert W * 4 == g["bitmask_row"]["bytes"]
    assert V // 1000 == g["bitmask_row"]["bool_mask_kb"]
    assert V * 4 // 1000 == g["bitmask_row"]["fp32_mask_kb"]
    rng = workloads.rng_for(91)
    z = rng.standard_normal(V).astype(np.float32)
    full = np.full(W, g["bitmask_fill"]["unconstrained_word"], np.int32)
    np.testing.assert_array_equal(oracle.transform_row(z, mask=full), z)
    allowed = rng.choice(V, size=777, replace=False)
    mask = workloads.pack_bitmask([allowed], V)[0]
    assert mask.shape[0] == W
    bias_ids = np.concatenate([allowed[:3], np.setdiff1d(np.arange(V), allowed)[:3]])
    got = oracle.transform_row(z, mask=mask, bias_ids=bias_ids,
                               bias_vals=np.full(6, 50.0, np.float32))
    ref = np.full(V, -np.inf, np.float32)
    ref[allowed] = z[allowed]
    ref[allowed[:3]] += np.float32(50.0)
    np.testing.assert_array_equal(got, ref)
    with pytest.raises(ValueError):
        oracle.transform_row(z, mask=mask[:-1])


def test_bf16_upcast_matches_torch():
    import torch
    rng = workloads.rng_for(92)
    x = (rng.standard_normal(5000) * 7).astype(np.float32)
    bits = workloads.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.transform_row(bits, bf16=True)
    np.testing.assert_array_equal(got, ref)   # exact upcast, RNE downcast


def test_page_size_figures():
    g = _golden("page_figures.json")
    b = g["fp32_logits_buffer"]
    assert b["B"] * b["V"] * 4 == 116_686_848
    assert round(b["B"] * b["V"] * 4 / 1e6) == b["approx_MB"]
    a = g["vocab_allgather"]
    ag = a["B"] * a["V"] * 4 * (a["TP"] - 1) // a["TP"]
    assert ag == 102_100_992 and round(ag / 1e6) == a["approx_MB"]
    d = g["dense_bias"]
    assert round(d["B"] * d["V"] * 4 / 1e6) == d["approx_MB"]
    assert (151936 + 31) // 32 == 4748


# ---------------------------------------------------------- greedy / status --

def _random_z(rng, V, scale=2.0):
    return (rng.standard_normal(V) * scale).astype(np.float32)


def test_greedy_equals_numpy_argmax_and_scipy_logprob():
    rng = workloads.rng_for(93)
    for trial in range(20):
        V = int(rng.integers(2, 3000))
        z = _random_z(rng, V)
        if trial % 3 == 0:                       # plant ties at the max
            z[rng.choice(V, size=min(3, V), replace=False)] = z.max() + 1
        for T, k in [(0.0, 0), (1e-6, 50), (0.7, 1), (2.0, 1)]:
            r = oracle.sample_row(z, T=T, top_k=k, top_p=0.5, min_p=0.3, seed=trial)
            assert r["greedy"] == 1
            assert r["id"] == int(np.argmax(z))  # first occurrence
            ref = scipy.special.log_softmax(z.astype(np.float64))[r["id"]]
            assert abs(r["logprob"] - ref) < 1e-12


def test_greedy_threshold_is_the_pages_epsilon():
    eps = _golden("page_figures.json")["greedy_eps"]["temperature_below"]
    z = np.array([0.0, 1.0, 2.0], np.float32)
    below = np.nextafter(np.float32(eps), np.float32(0))
    assert oracle.sample_row(z, T=below)["greedy"] == 1
    assert oracle.sample_row(z, T=np.float32(eps))["greedy"] == 0


def test_status_cases():
    z = np.array([0.0, 1.0, 2.0, 3.0], np.float32)
    for bad in [np.nan, np.inf]:
        zz = z.copy(); zz[1] = bad
        for T in (0.0, 1.0):
            r = oracle.sample_row(zz, T=T)
            assert r["status"] == oracle.STATUS_OVERFLOW and r["id"] == -1
            assert math.isnan(r["logprob"])
    zz = np.full(4, -np.inf, np.float32)
    r = oracle.sample_row(zz, T=1.0)
    assert r["status"] == oracle.STATUS_INVALID and r["id"] == -1 and r["logprob"] == -np.inf
    # a NaN that the mask removes does not count
    zz = z.copy(); zz[0] = np.nan
    masked = oracle.transform_row(zz, mask=np.array([~1], np.int32))
    r = oracle.sample_row(masked, T=1.0, seed=4)
    assert r["status"] == oracle.STATUS_OK and r["id"] != 0
    # nothing allowed at all
    masked = oracle.transform_row(z, mask=np.array([0], np.int32))
    assert oracle.sample_row(masked, T=0.0)["status"] == oracle.STATUS_INVALID


def test_single_allowed_token_logprob_zero():
    rng = workloads.rng_for(94)
    z = _random_z(rng, 1000)
    mask = workloads.pack_bitmask([np.array([617])], 1000)[0]
    zt = oracle.transform_row(z, mask=mask)
    for T in (0.0, 0.5, 1.7):
        for s in range(5):
            r = oracle.sample_row(zt, T=T, top_p=0.3, top_k=7, min_p=0.2, seed=s)
            assert r["id"] == 617 and r["logprob"] == 0.0


# --------------------------------------------------------- sets, by brute force

def _defs(z, T, top_k, top_p, min_p):
    """The pages' set definitions written directly (no sorting):
    min-p: p_t >= p_max*min_p; top-k: rank(t) < k with rank = number of
    strictly larger members; top-p: mass strictly above t < p * mass(S2)."""
    fin = np.isfinite(z)
    s = np.where(fin, z.astype(np.float64) / np.float64(T), -np.inf)
    m = s.max()
    w = np.where(fin, np.exp(s - m), 0.0)
    S1 = fin & ((w >= np.float64(np.float32(min_p))) if min_p > 0 else True)
    n1 = int(S1.sum())
    if 1 < top_k < n1:
        rank = np.array([np.sum(S1 & (s > s[t])) for t in range(len(z))])
        S2 = S1 & (rank < top_k)
    else:
        S2 = S1.copy()
    if top_p < 1:
        M2 = w[S2].sum()
        above = np.array([w[S2 & (s > s[t])].sum() for t in range(len(z))])
        S3 = S2 & (above < np.float64(np.float32(top_p)) * M2)
    else:
        S3 = S2.copy()
    return S1, S2, S3, w


def _oracle_sets(z, **kw):
    r, sets = oracle.sample_row(z, want_sets=True, **kw)
    return (sets & 1) > 0, (sets & 2) > 0, (sets & 4) > 0, r


def test_sets_match_definitions_random_small():
    rng = workloads.rng_for(95)
    for trial in range(300):
        V = int(rng.integers(2, 40))
        z = _random_z(rng, V, scale=float(rng.choice([0.5, 2.0, 5.0])))
        if trial % 4 == 0:  # ties: quantise
            z = np.round(z * 2) / 2
        if trial % 7 == 0:
            z[rng.choice(V, size=V // 3, replace=False)] = -np.inf
        if not np.isfinite(z).any():
            continue
        T = float(rng.choice([0.3, 1.0, 2.5]))
        k = int(rng.choice([0, 2, 3, 5, 100]))
        p = float(rng.choice([1.0, 0.95, 0.6, 0.2]))
        mp = float(rng.choice([0.0, 0.05, 0.3]))
        S1, S2, S3, r = _oracle_sets(z, T=T, top_k=k, top_p=p, min_p=mp, seed=trial)
        D1, D2, D3, _ = _defs(z, np.float32(T), k, p, mp)
        np.testing.assert_array_equal(S1, D1)
        np.testing.assert_array_equal(S2, D2)
        np.testing.assert_array_equal(S3, D3)
        assert S3[r["id"]]
        assert r["n3"] == D3.sum()


def test_top_p_smallest_prefix_brute_force():
    """Second formulation: S3 is the smallest prefix of the tokens ordered by
    probability, cut only between distinct values (ties all in or all out),
    whose mass reaches p * M.  Every prefix is enumerated (V <= 10)."""
    rng = workloads.rng_for(96)
    checked = 0
    for trial in range(200):
        V = int(rng.integers(1, 11))
        z = (np.round(_random_z(rng, V) * (3 if trial % 2 else 100)) / 3).astype(np.float32)
        p = float(rng.choice([0.1, 0.5, 0.75, 0.9, 0.99]))
        _, _, S3, _ = _oracle_sets(z, T=1.0, top_p=p, seed=trial)
        s = z.astype(np.float64)
        w = np.exp(s - s.max())
        target = np.float64(np.float32(p)) * w.sum()
        prefixes = [s >= lo for lo in np.unique(s)]
        masses = [w[sel].sum() for sel in prefixes]
        if min(abs(m - target) for m in masses) < 1e-12 * w.sum():
            continue                                # exact-boundary case: see flag test
        best = min((sel for sel, m in zip(prefixes, masses) if m >= target),
                   key=lambda sel: sel.sum())
        np.testing.assert_array_equal(S3, best, err_msg=f"trial {trial} z={z} p={p}")
        checked += 1
    assert checked > 150


def test_top_p_tie_group_all_in_or_all_out():
    # two tokens tied in the middle, p chosen so the cut falls inside the tie
    z = np.log(np.array([0.4, 0.2, 0.2, 0.2], np.float64)).astype(np.float32)
    z[2] = z[1]; z[3] = z[1]
    for p in (0.45, 0.5, 0.55, 0.7):
        _, _, S3, _ = _oracle_sets(z, T=1.0, top_p=p)
        assert S3[1] == S3[2] == S3[3]
        assert S3[0]


def test_top_k_matches_argpartition_and_max_top_k_invariant():
    rng = workloads.rng_for(97)
    for trial in range(30):
        V = int(rng.integers(50, 5000))
        z = _random_z(rng, V)
        k = int(rng.integers(2, min(V, 300)))
        K = int(rng.integers(k, min(V, 400) + 1))          # a batch-wide bound
        _, S2, _, _ = _oracle_sets(z, T=0.8, top_k=k, seed=trial)
        ref = np.zeros(V, bool)
        ref[np.argpartition(-z, k - 1)[:k]] = True          # no ties in N(0,1)
        np.testing.assert_array_equal(S2, ref)
        # partial sort of the leading K columns, then the top-k mask, gives the
        # same support as the full sort (the max_top_k argument of the pages)
        lead = np.argpartition(-z, K - 1)[:K]
        lead = lead[np.argsort(-z[lead], kind="stable")]
        part = np.zeros(V, bool)
        part[lead[:k]] = True
        np.testing.assert_array_equal(S2, part)


def test_top_k_ties_at_rank_k_all_kept():
    z = np.array([5, 4, 3, 3, 3, 1, 0], np.float32)
    _, S2, _, r = _oracle_sets(z, T=1.0, top_k=3)
    np.testing.assert_array_equal(S2, [1, 1, 1, 1, 1, 0, 0])
    assert r["n2"] == 5


def test_min_p_closed_form_and_argmax_invariance():
    w = np.array([1.0, 0.5, 0.2, 0.05])
    z = np.log(w).astype(np.float32)
    for mp, expect in [(0.3, [1, 1, 0, 0]), (0.1, [1, 1, 1, 0]), (0.6, [1, 0, 0, 0]),
                       (0.01, [1, 1, 1, 1])]:
        S1, _, _, _ = _oracle_sets(z, T=1.0, min_p=mp)
        np.testing.assert_array_equal(S1, np.array(expect, bool))
    rng = workloads.rng_for(98)
    for trial in range(50):
        z = _random_z(rng, 300, scale=3.0)
        mp = float(rng.uniform(0.0, 1.0))
        S1, _, _, _ = _oracle_sets(z, T=float(rng.uniform(0.2, 2)), min_p=mp)
        assert S1[np.argmax(z)]                      # argmax always survives
        g0 = oracle.sample_row(z, T=0.0)["id"]
        g1 = oracle.sample_row(z, T=0.0, min_p=mp)["id"]
        assert g0 == g1 == np.argmax(z)


def test_min_p_flag_near_boundary():
    z = np.log(np.array([1.0, 0.25], np.float64)).astype(np.float32)
    w1 = math.exp(float(z[1]) - float(z[0]))
    r = oracle.sample_row(z, T=1.0, min_p=np.float32(w1))
    assert r["flags"] & oracle.F_MINP
    r = oracle.sample_row(z, T=1.0, min_p=0.1)
    assert not r["flags"] & oracle.F_MINP


def test_top_p_flag_at_exact_boundary():
    z = np.array([1.0, 1.0, 0.0], np.float32)   # above(t2) = 2e/(2e+1) exactly
    s = z.astype(np.float64)
    w = np.exp(s - 1.0)
    frac = (w[0] + w[1]) / w.sum()
    r = oracle.sample_row(z, T=1.0, top_p=np.float32(frac))
    assert r["flags"] & oracle.F_TOPP
    assert not oracle.sample_row(z, T=1.0, top_p=0.5)["flags"] & oracle.F_TOPP


# --------------------------------------------------------------- logprobs --

def test_logprob_is_log_softmax_of_scaled_logits():
    rng = workloads.rng_for(99)
    for trial in range(20):
        V = int(rng.integers(10, 20000))
        z = _random_z(rng, V, 3.0)
        T = float(rng.uniform(0.2, 2.0))
        r = oracle.sample_row(z, T=T, top_k=int(rng.choice([0, 10])),
                              top_p=float(rng.choice([1.0, 0.9])), seed=trial)
        ref = scipy.special.log_softmax(z.astype(np.float64) / np.float64(np.float32(T)))
        assert abs(r["logprob"] - ref[r["id"]]) < 1e-12
        assert abs(r["log_z"] - scipy.special.logsumexp(
            z.astype(np.float64) / np.float64(np.float32(T)) - r["m"])) < 1e-12


def test_log_of_softmax_fp32_gap_is_order_1e6():
    """The pages' point: in fp32, log(softmax(x)) and log_softmax(x) differ at
    about 1e-6, which is why the oracle works in log form and in fp64."""
    import torch
    g = _golden("page_figures.json")["logprob_gap"]["order_of_magnitude"]
    rng = workloads.rng_for(100)
    x = torch.from_numpy((rng.standard_normal((8, 151936)) * 2).astype(np.float32))
    gap = (torch.log(torch.softmax(x, -1)) - torch.log_softmax(x, -1)).abs().max().item()
    assert g / 100 < gap < g * 100
    r = oracle.sample_row(x[0].numpy(), T=1.0, seed=1)
    ref = scipy.special.log_softmax(x[0].numpy().astype(np.float64))[r["id"]]
    assert abs(r["logprob"] - ref) < 1e-12


# ------------------------------------------------------------------ order --

def test_mask_before_truncation_differs_from_reverse_order():
    """The grammar's allowed set is applied before truncation; truncating first
    and masking afterwards gives a different answer on these cases."""
    # (i) greedy (top_k = 1): mask first -> token 1; truncate first keeps only
    # token 0, which the mask then removes: nothing left.
    z = np.array([5, 4, 0, 0], np.float32)
    mask = workloads.pack_bitmask([np.array([1, 2, 3])], 4)[0]
    zt = oracle.transform_row(z, mask=mask)
    assert oracle.sample_row(zt, T=1.0, top_k=1)["id"] == 1
    trunc_first = np.zeros(4, bool); trunc_first[np.argmax(z)] = True
    assert not (trunc_first & np.isfinite(zt)).any()
    # (ii) top-p: mask first renormalises over the allowed set and widens the
    # nucleus to {1, 2}; truncating first keeps {0, 1} and then only {1}.
    w = np.array([0.6, 0.2, 0.15, 0.05])
    z = np.log(w).astype(np.float32)
    mask = workloads.pack_bitmask([np.array([1, 2, 3])], 4)[0]
    zt = oracle.transform_row(z, mask=mask)
    _, _, S3, _ = _oracle_sets(zt, T=1.0, top_p=0.75)
    np.testing.assert_array_equal(S3, [False, True, True, False])
    _, _, S3_raw, _ = _oracle_sets(z, T=1.0, top_p=0.75)
    np.testing.assert_array_equal(S3_raw & np.isfinite(zt), [False, True, False, False])
    ids = oracle.sample_batch(zt, T=np.ones(400, np.float32), top_k=np.zeros(400, np.int32),
                              top_p=np.full(400, 0.75, np.float32),
                              min_p=np.zeros(400, np.float32),
                              seed=np.full(400, 7, np.uint64),
                              offset=np.arange(400, dtype=np.uint64), broadcast=True)["id"]
    assert set(ids.tolist()) == {1, 2}


# ---------------------------------------------------- batch / reproducibility

def test_batch_invariance_and_reproducibility():
    b = workloads.c2_decode(B=24, V=3000)
    res = oracle.sample_batch(b.logits, T=b.temperature, top_k=b.top_k, top_p=b.top_p,
                              min_p=b.min_p, seed=b.seed, offset=b.offset)
    perm = workloads.rng_for(101).permutation(24)
    sub = b.subset(perm[:11])
    res2 = oracle.sample_batch(sub.logits, T=sub.temperature, top_k=sub.top_k,
                               top_p=sub.top_p, min_p=sub.min_p, seed=sub.seed,
                               offset=sub.offset)
    np.testing.assert_array_equal(res2["id"], res["id"][perm[:11]])
    np.testing.assert_array_equal(res2["logprob"], res["logprob"][perm[:11]])
    res3 = oracle.sample_batch(b.logits, T=b.temperature, top_k=b.top_k, top_p=b.top_p,
                               min_p=b.min_p, seed=b.seed, offset=b.offset)
    np.testing.assert_array_equal(res3["id"], res["id"])


def test_temperature_limits():
    rng = workloads.rng_for(102)
    z = rng.standard_normal(8).astype(np.float32)
    n = 40000
    common = dict(top_k=np.zeros(n, np.int32), top_p=np.ones(n, np.float32),
                  min_p=np.zeros(n, np.float32), seed=np.full(n, 3, np.uint64),
                  offset=np.arange(n, dtype=np.uint64), broadcast=True)
    hot = oracle.sample_batch(z, T=np.full(n, 1e4, np.float32), **common)["id"]
    from scipy.stats import chisquare
    assert chisquare(np.bincount(hot, minlength=8)).pvalue > 1e-3     # ~uniform
    zc = np.array([0.0, 0.02, 0.5, 0.49], np.float32)
    cold = oracle.sample_batch(zc, T=np.full(n, 1e-4, np.float32), **common)["id"]
    assert np.all(cold == 2)                                          # one-hot


# ------------------------------------------------- near-tie flag thresholds --
# Each flag is pinned from both sides of its 1e-6 threshold: a row built so
# that the flagged quantity sits about 5e-7 from its boundary must carry the
# flag, one built 5e-6 away must not.  The distances are computed here in
# float64 straight from the definitions (Philox words through race_bits only),
# not from the oracle's own key or mass code, so a wrong threshold, a dropped
# term or a wrong comparison in the flag code fails one of the two cases.

def _uniform_from_bits(x):
    return (2.0 * float(x >> 9) + 1.0) * 2.0 ** -24


def _gumbel(seed, offset, t):
    return -math.log(-math.log(_uniform_from_bits(oracle.race_bits(seed, offset, t))))


@pytest.mark.parametrize("gap,flagged", [(5e-7, True), (5e-6, False), (2e-6, False),
                                         (0.0, True)])
def test_race_flag_threshold_two_sided(gap, flagged):
    """F_RACE: the best two race keys over S3 within 1e-6.  Tokens 3 and 5
    are the only finite ones besides a far-down token 0; z[5] is set so that
    key_3 - key_5 = gap (up to fp32 rounding of z[5], measured below)."""
    seed, offset, T = 0x1234_5678_9ABC_DEF0, 77, 1.0
    V = 8
    g = [_gumbel(seed, offset, t) for t in range(V)]
    z = np.full(V, -np.inf, np.float32)
    z[0] = np.float32(-40.0)
    z[3] = np.float32(0.0)
    z[5] = np.float32(g[3] - g[5] - gap)
    s = z.astype(np.float64) / T
    m = float(np.max(s))
    keys = sorted(((s[t] - m) + g[t] for t in (0, 3, 5)), reverse=True)
    d = keys[0] - keys[1]
    assert abs(d - gap) < 2e-7                 # the construction worked
    r = oracle.sample_row(z, T=T, seed=seed, offset=offset)
    assert r["n3"] == 3
    assert bool(r["flags"] & oracle.F_RACE) == (abs(d) <= 1e-6), d
    assert bool(r["flags"] & oracle.F_RACE) == flagged
    # the winner is the larger key (lowest index on an exact tie)
    k3, k5 = (s[3] - m) + g[3], (s[5] - m) + g[5]
    assert r["id"] == (3 if k3 >= k5 else 5)


@pytest.mark.parametrize("rel,flagged", [(5e-7, True), (-5e-7, True), (5e-6, False),
                                         (-5e-6, False)])
def test_min_p_flag_threshold_two_sided(rel, flagged):
    """F_MINP: some weight w_t = exp(s_t - m) within 1e-6 * min_p of min_p."""
    min_p = np.float32(0.25)
    z = np.array([0.0, np.log(float(min_p) * (1.0 + rel)), -5.0], np.float32)
    w = np.exp(z.astype(np.float64) - 0.0)
    d = abs(w[1] - float(min_p)) / float(min_p)
    assert abs(d - abs(rel)) < 1e-7
    r = oracle.sample_row(z, T=1.0, min_p=min_p)
    assert bool(r["flags"] & oracle.F_MINP) == flagged
    assert r["n1"] == (2 if w[1] >= float(min_p) else 1)


@pytest.mark.parametrize("rel,flagged", [(5e-7, True), (5e-6, False)])
def test_top_k_flag_threshold_two_sided(rel, flagged):
    """F_TOPK: the weight at rank k+1 is at least (1 - 1e-6) times the weight
    at rank k (k = 2 here)."""
    z = np.array([0.0, -1.0, -1.0 + np.log1p(-rel), -6.0], np.float32)
    w = np.exp(z.astype(np.float64))
    ratio = w[2] / w[1]
    assert abs((1.0 - ratio) - rel) < 1e-7
    r = oracle.sample_row(z, T=1.0, top_k=2)
    assert bool(r["flags"] & oracle.F_TOPK) == flagged
    assert r["n2"] == 2


@pytest.mark.parametrize("dist,flagged", [(5e-7, True), (-5e-7, True), (5e-6, False),
                                          (-5e-6, False)])
def test_top_p_flag_threshold_two_sided(dist, flagged):
    """F_TOPP: a normalised prefix mass above(t) / M2 within 1e-6 of top_p.
    The prefix masses of z are 0, w0/M, (w0 + w1)/M, ...; top_p is placed
    `dist` from the second one (fp32 rounding of top_p measured)."""
    z = np.array([1.0, 0.3, -0.2, -2.0], np.float32)
    w = np.exp(z.astype(np.float64) - 1.0)
    M = w.sum()
    f = w[0] / M
    top_p = np.float32(f + dist)
    d = float(top_p) - f
    assert abs(d - dist) < 1e-7
    r = oracle.sample_row(z, T=1.0, top_p=top_p)
    assert bool(r["flags"] & oracle.F_TOPP) == flagged
    # S3 is the smallest prefix whose mass reaches top_p: one token if
    # top_p <= w0/M, else two
    assert r["n3"] == (1 if float(top_p) <= f else 2)
