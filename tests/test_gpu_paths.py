"""GPU tests of the paths the full-size workloads do not reach, through the
C ABI, against the CPU oracle (same bar as test_gpu_parity.py):

  - the bounded wait for a row's plan giving up (forced from the host with a
    zero wait limit): every row whose slices need the plan takes the
    row-serial exact path;
  - histogram bins that would lose exactness (|max z / bin width| >= 2^22 at
    temperatures just above the greedy threshold): the plan sends the row to
    the exact path;
  - parameter extremes: min_p = 1, top_p near 0, top_k = V - 1, T just above
    the greedy threshold;
  - bf16 rows with V % 4 != 0 and an odd row stride (scalar loads) through
    the sampling kernel;
  - logprobs at low temperature with large logits (the exp-sum must not
    carry the rounding of max / T);
  - a NaN among the few tokens a mask allows, on the vector-load path (the
    NaN's thread sees no other allowed token);
  - the kept-set threshold of top-k rows whose k-th token lies below the
    histogram window (large k at low temperature): the threshold a caller
    asks for is the k-th value itself, not the window's bottom.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_harness import compare, record_parity, run_gpu, run_oracle, run_oracle_parallel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import constrained_decoding_amd  # noqa: F401  (must load: no fallback)


def _batch(z, T, k=None, p=None, mp=None, seed=None, masks=None, rhm=None, bf16=False):
    B = z.shape[0]
    f = lambda v, dt=np.float32: np.full(B, v, dt)
    return workloads.Batch("paths", z, bf16, np.asarray(T, np.float32),
                           f(0, np.int32) if k is None else np.asarray(k, np.int32),
                           f(1.0) if p is None else np.asarray(p, np.float32),
                           f(0.0) if mp is None else np.asarray(mp, np.float32),
                           np.arange(1, B + 1, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
                           if seed is None else seed,
                           np.arange(B, dtype=np.uint64), masks=masks, row_has_mask=rhm)


def test_plan_wait_give_up_takes_exact_path():
    """A decode-shaped batch (B=192, V=151936) of top-p-only rows, whose slices
    need the row's plan before they race: with no wait allowed every such
    row gives up at once and is resolved by the exact path; results match
    the oracle, and the default path's ids and statuses bit for bit (the two
    paths sum the logprob's normaliser differently: within 1e-5)."""
    import constrained_decoding_amd as cds
    b = workloads.c2_decode(salt=41)
    b.top_k[:] = 0
    b.min_p[:] = 0.0
    print("[case] give-up B=192 V=151936 top-p only", flush=True)
    gave_up = run_gpu(b, wait_ns=cds.WAIT_NONE)
    ref = run_oracle_parallel(b)
    record_parity("wait-give-up", compare(b, gave_up, ref, label="give-up"))
    normal = run_gpu(b)
    np.testing.assert_array_equal(gave_up[0], normal[0])
    np.testing.assert_array_equal(gave_up[2], normal[2])
    assert np.max(np.abs(gave_up[1] - normal[1])) <= 1e-5


def test_bins_lost_rows_take_exact_path():
    """Top-p-only rows at T in {1.2e-5, 3e-5, 1e-4} whose logits reach |z| =
    50: the histogram's bin width 2^floor(log2(T/16)) puts |max z / width|
    past 2^22, so the row's bins would not be exact and the plan sends it to
    the exact path.  Rows at T = 1e-4 and max z = 8 keep the fast path."""
    rng = np.random.default_rng(51)
    B, V = 12, 40000
    z = (rng.standard_normal((B, V)) * 2.0).astype(np.float32)
    T = np.array([1.2e-5, 3e-5, 1e-4] * 4, np.float32)
    for r in range(B):
        hot = rng.choice(V, 6, replace=False)
        top = 50.0 if r < 9 else 8.0
        z[r, hot] = top - rng.uniform(0, 2e-4, 6).astype(np.float32)
        z[r, hot[:2]] = np.float32(top)       # an exact tie at the top
    b = _batch(z, T, p=np.full(B, 0.9, np.float32))
    print("[case] bins-lost", flush=True)
    gpu = run_gpu(b)
    ref, _ = run_oracle(b)
    record_parity("bins-lost", compare(b, gpu, ref, label="bins-lost"))


@pytest.mark.parametrize("V", [151936, 40003])
def test_parameter_extremes(V):
    """min_p = 1 (only the maximum and its ties), top_p = 1e-6 (only the top
    token), top_k = V - 1 (one token cut), top_k = 2, T = 1.01e-5 (just above
    greedy), all mixed in one batch; V = 40003 adds a ragged tail."""
    rng = np.random.default_rng(52 + V)
    B = 24
    z = (rng.standard_normal((B, V)) * 2.0).astype(np.float32)
    z[::5, 7] = z[::5].max(axis=1) + 0.0      # an exact tie at the max on some rows
    z[::5, 11] = z[::5, 7]
    T = np.tile(np.array([1.0, 0.7, 1.3, 1.01e-5], np.float32), B // 4)
    k = np.tile(np.array([0, V - 1, 2, 0, V - 1, 0], np.int32), B // 6)
    p = np.tile(np.array([1.0, 1e-6, 0.9, 1.0, 1.0, 1e-6, 0.5, 1.0], np.float32), B // 8)
    mp = np.tile(np.array([1.0, 0.0, 0.0, 1.0, 0.5, 0.0], np.float32), B // 6)
    b = _batch(z, T, k=k, p=p, mp=mp)
    print(f"[case] extremes V={V}", flush=True)
    for algo in (0, 1):
        gpu = run_gpu(b, algo=algo)
        ref, _ = run_oracle(b)
        record_parity(f"extremes-V{V}-algo{algo}", compare(b, gpu, ref, label="extremes"))


@pytest.mark.parametrize("ld_extra", [0, 1, 3])
def test_bf16_ragged_vocab_and_odd_stride(ld_extra):
    """bf16 logits with V % 4 != 0 (and odd row strides): the sampling kernel's
    guarded scalar loads, with and without a fused mask."""
    import torch
    import constrained_decoding_amd as cds
    b = workloads.c4_grammar(B=24, V=30001, sizes=(1, 50, 900, 12000), salt=53)
    B, V = b.B, b.V
    pad = np.zeros((B, V + ld_extra), np.uint16)
    pad[:, :V] = b.logits
    x = torch.from_numpy(pad.view(np.int16)).view(torch.bfloat16).cuda()[:, :V]
    assert x.stride(0) == V + ld_extra
    print(f"[case] bf16 V={V} ld=V+{ld_extra}", flush=True)
    pk = cds.PackedBatch(B, V, b.temperature, top_k=b.top_k, top_p=b.top_p, min_p=b.min_p,
                         seed=b.seed, offset=b.offset)
    mask = torch.from_numpy(b.masks).cuda()
    rhm = torch.from_numpy(b.row_has_mask).cuda()
    ids, lp, st = cds.sample(pk, x, bitmask=mask, row_has_mask=rhm)
    torch.cuda.synchronize()
    ref, _ = run_oracle(b)
    record_parity(f"bf16-ragged-ld+{ld_extra}",
                  compare(b, (ids.cpu().numpy(), lp.cpu().numpy(), st.cpu().numpy()), ref,
                          label="bf16-ragged"))


def test_low_temperature_logprobs_large_logits():
    """T in {0.05, 0.1} with logits shifted by +30: greedy, top-k and min-p rows
    (the slice exp-sum path) keep their logprobs within 1e-5 of the oracle."""
    rng = np.random.default_rng(54)
    B, V = 24, 151936
    z = (rng.standard_normal((B, V)) * 2.0 + 30.0).astype(np.float32)
    for r in range(B):
        z[r, rng.choice(V, 5, replace=False)] += np.float32(4.0)
    T = np.tile(np.array([0.05, 0.1, 0.0], np.float32), B // 3)
    k = np.tile(np.array([20, 0, 50, 1000], np.int32), B // 4)
    mp = np.tile(np.array([0.0, 0.05], np.float32), B // 2)
    mp[k == 0] = 0.05                              # every sampled row has a LIST cut
    b = _batch(z, T, k=k, mp=mp)
    print("[case] low-T large logits", flush=True)
    gpu = run_gpu(b)
    ref = run_oracle_parallel(b)
    record_parity("low-T-logprobs", compare(b, gpu, ref, label="low-T"))


def test_nan_among_masked_tokens_vector_path():
    """V % 4 == 0 and aligned rows (vector loads).  Each row's mask allows a
    NaN token and three finite ones, far apart, so the NaN's thread holds no
    other allowed token: greedy, top-k and min-p rows must all report
    OVERFLOW.  Control rows without the NaN are sampled normally."""
    rng = np.random.default_rng(55)
    B, V = 12, 151936
    z = (rng.standard_normal((B, V)) * 2.0).astype(np.float32)
    allowed = []
    for r in range(B):
        toks = rng.choice(V, 4, replace=False)
        if r < 9:
            z[r, toks[0]] = np.nan
        allowed.append(toks)
    masks = workloads.pack_bitmask(allowed, V)
    T = np.tile(np.array([0.0, 0.8, 1.1], np.float32), B // 3)
    k = np.tile(np.array([0, 3, 0], np.int32), B // 3)
    mp = np.tile(np.array([0.0, 0.0, 0.1], np.float32), B // 3)
    b = _batch(z, T, k=k, mp=mp, masks=masks, rhm=np.ones(B, np.uint8))
    print("[case] NaN among masked tokens", flush=True)
    gpu = run_gpu(b)
    ref, _ = run_oracle(b)
    compare(b, gpu, ref, label="nan-masked")
    assert (gpu[2][:9] == oracle.STATUS_OVERFLOW).all()
    assert (gpu[2][9:] == oracle.STATUS_OK).all()


def _kept_sets(b, zs, rows):
    """The oracle's kept set of each row (bool [V]), "SGLang 源码完全拆解(十)",
    section LogitsProcessor 与 LogitsProcessorOutput: the support the draw is
    made from."""
    out = {}
    for r in rows:
        _, sets = oracle.sample_row(zs[r], T=float(b.temperature[r]), top_k=int(b.top_k[r]),
                                    top_p=float(b.top_p[r]), min_p=float(b.min_p[r]),
                                    seed=int(b.seed[r]), offset=int(b.offset[r]),
                                    want_sets=True, order=b.order)
        out[r] = (sets & 4) > 0
    return out


@pytest.mark.parametrize("V", [151936, 5003])
def test_cut_of_topk_below_histogram_window(V):
    """Top-k rows too large for the slices' lists, at T = 0.05, where the
    k-th largest value lies more than the histogram window (1120 bins of
    width 2^-9, about 2.2 in z) below the maximum, with min-p below or
    inside the window, with top-p, and with a mask allowing fewer tokens
    than k; control rows at T = 0.3 and 1.  On the fast and the exact path
    the returned threshold keeps exactly the oracle's kept set; asking for
    it changes no id, logprob or status."""
    import torch
    import constrained_decoding_amd as cds
    from gpu_harness import pack, to_device
    rng = np.random.default_rng(57)
    B = 16
    z = workloads.decode_logits(rng, B, V)
    k = np.full(B, 3000 if V > 100000 else 1000, np.int32)
    T = np.full(B, 0.05, np.float32)
    T[8:10] = 1.0
    T[12:14] = 0.3
    mp = np.zeros(B, np.float32)
    mp[4:6] = 1e-20                    # min-p cut below the window
    mp[6:8] = 1e-6                     # ... inside it (about 14 units of z/T)
    p = np.ones(B, np.float32)
    p[10:12] = 0.9
    allowed = [np.arange(V)] * B
    allowed = list(allowed)
    allowed[14] = rng.choice(V, int(k[14]) // 2, replace=False)   # fewer tokens than k
    allowed[15] = rng.choice(V, V // 2, replace=False)
    rhm = np.zeros(B, np.uint8)
    rhm[14:] = 1
    b = _batch(z, T, k=k, p=p, mp=mp, masks=workloads.pack_bitmask(allowed, V), rhm=rhm)
    print(f"[case] cut below window V={V}", flush=True)
    ref, zs = run_oracle(b)
    kept = _kept_sets(b, zs, range(B))
    plain = run_gpu(b)
    record_parity(f"cut-below-window-{V}", compare(b, plain, ref, label="cut-below-window"))
    for algo in (cds.ALGO_FAST, cds.ALGO_EXACT):
        x = to_device(b)
        mask = torch.from_numpy(b.masks).cuda()
        rh = torch.from_numpy(b.row_has_mask).cuda()
        cut = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
        ids, lp, st = cds.sample(pack(b), x, bitmask=mask, row_has_mask=rh, cut=cut, algo=algo)
        torch.cuda.synchronize()
        ids, lp, st, c = (t.cpu().numpy() for t in (ids, lp, st, cut))
        np.testing.assert_array_equal(ids, plain[0])
        np.testing.assert_array_equal(st, plain[2])
        assert np.max(np.abs(lp - plain[1])) <= 1e-5
        for r in range(B):
            fin = np.isfinite(zs[r])
            got = fin & (zs[r] >= c[r])
            assert np.array_equal(got, kept[r]), \
                f"algo {algo} row {r}: cut {c[r]} keeps {got.sum()} tokens, the oracle {kept[r].sum()}"
