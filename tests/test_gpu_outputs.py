"""GPU parity of the further outputs (sampler_logprobs) against the oracle:
the chosen token's logprob in either basis, top-N logprobs, logprobs of
named tokens, and the sampling support set ("SGLang 源码完全拆解(十)",
sections LogitsProcessorOutput 的五段结构, logprobs 的数值一致性,
LogitsProcessor 与 LogitsProcessorOutput).

Bar: ids (top-N, support) bit-exact; logprobs within 1e-5; statuses and
lengths exact.  A support set may differ from the oracle's only on rows the
oracle flags as a near-tie of the top-p or min-p cut; there the GPU set must
still be a value-threshold set that differs from the oracle's by one value
group at the boundary.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import workloads
from gpu_harness import pack, run_oracle, to_device

pytestmark = pytest.mark.gpu

LP_TOL = 1e-5
SET_EXCUSE = oracle.F_TOPP | oracle.F_MINP


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import constrained_decoding_amd  # noqa: F401  (must load: no fallback)


def _close(a, b, tol=LP_TOL):
    """a: the GPU's fp32 logprobs, b: the oracle's fp64 values; within tol,
    or within one fp32 spacing of b where that spacing is coarser than tol
    (|b| >= 128: the outputs' own precision)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_nan = np.isnan(a) & np.isnan(b)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    fin = np.isfinite(a) & np.isfinite(b)
    with np.errstate(invalid="ignore"):
        ulp = np.spacing(np.abs(np.where(fin, b, 0.0)).astype(np.float32)).astype(np.float64)
    ok = same_nan | same_inf | (fin & (np.abs(a - b) <= np.maximum(tol, ulp)))
    return bool(ok.all()), np.flatnonzero(~ok)


def _run(batch, *, basis, top_n, tok_rows, mask_rows, cap, with_selected=True, use_cuts=True,
         use_ws=True):
    """Pack, transform, sample (fused mask), then sampler_logprobs; returns
    (ids, status, logprobs, dict of host arrays).  use_cuts: the support sets
    take the sampling call's kept-set thresholds (else they select them
    again)."""
    import torch
    import constrained_decoding_amd as cds
    x = to_device(batch)
    pk = pack(batch)
    if batch.rep is not None or batch.bias_indptr is not None:
        cds.apply_transforms(pk, x)
    mask = rhm = None
    if batch.masks is not None:
        mask = torch.from_numpy(batch.masks).cuda()
        rhm = None if batch.row_has_mask is None else \
            torch.from_numpy(batch.row_has_mask.astype(np.uint8)).cuda()
    cut = torch.full((batch.B,), float("nan"), dtype=torch.float32, device="cuda")
    ids, lp, st = cds.sample(pk, x, bitmask=mask, row_has_mask=rhm, cut=cut)
    indptr, flat = cds.csr(tok_rows)
    top_n_max = int(max(top_n)) if len(top_n) else 0
    res = cds.logprobs(
        pk, x, selected=ids if with_selected else None, basis=basis, top_n_max=top_n_max,
        top_n=torch.from_numpy(np.asarray(top_n, np.int32)).cuda() if top_n_max else None,
        token_indptr=torch.from_numpy(indptr).cuda(),
        token_ids=torch.from_numpy(flat.astype(np.int32)).cuda(),
        mask_rows=torch.from_numpy(np.asarray(mask_rows, np.int32)).cuda() if len(mask_rows) else None,
        mask_cap=cap, cuts=cut if use_cuts else None, bitmask=mask, row_has_mask=rhm,
        workspace=use_ws)
    torch.cuda.synchronize()
    host = {k: v.cpu().numpy() for k, v in res.items()}
    return ids.cpu().numpy(), st.cpu().numpy(), lp.cpu().numpy(), host


def _oracle_rows(batch, zs, rows, *, basis, top_n, tok_rows, selected, cap, want_support):
    """oracle.row_outputs for each of `rows`, in threads (the C calls release
    the GIL)."""
    def one(k):
        r = rows[k]
        return oracle.row_outputs(
            zs[r], T=float(batch.temperature[r]), top_k=int(batch.top_k[r]),
            top_p=float(batch.top_p[r]), min_p=float(batch.min_p[r]), seed=int(batch.seed[r]),
            offset=int(batch.offset[r]), order=batch.order, basis=basis, n_top=int(top_n[r]),
            token_ids=tok_rows[r], selected=None if selected is None else int(selected[r]),
            support_cap=cap if want_support[k] else None)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(one, range(len(rows))))


def _threshold_set_ok(z, gpu_ids, ref_ids, ref_full):
    """A flagged row's GPU support must be {allowed z >= g} for its own
    smallest value g, and differ from the oracle's by tokens of one value."""
    if len(gpu_ids) == 0:
        return False
    g = z[gpu_ids].min()
    want = np.flatnonzero(np.isfinite(z) & (z >= g))
    if not np.array_equal(np.sort(gpu_ids), want[:len(gpu_ids)]):
        return False
    diff = np.setxor1d(want, ref_full)
    return len(np.unique(z[diff])) <= 1


def _check(batch, zs, gpu, refs, rows, *, top_n, tok_rows, mask_rows, cap, with_selected, label):
    ids, st, lp_sample, h = gpu
    bad = []
    flagged_sets = 0
    B = batch.B
    tok_off = np.concatenate([[0], np.cumsum([len(t) for t in tok_rows])])
    for r in range(B):
        o = refs[r]
        if st[r] != o["res"]["status"]:
            bad.append(f"row {r}: sample status {st[r]} vs {o['res']['status']}")
            continue
        n = int(top_n[r])
        if "top_idx" in h:
            if not np.array_equal(h["top_idx"][r, :n], o["top_ids"]):
                bad.append(f"row {r}: top ids {h['top_idx'][r, :n][:8]} vs {o['top_ids'][:8]}")
            ok, where = _close(h["top_val"][r, :n], o["top_vals"])
            if not ok:
                bad.append(f"row {r}: top vals at {where[:4]}: {h['top_val'][r, where[:4]]} vs "
                           f"{o['top_vals'][where[:4]]}")
            if not (np.all(h["top_idx"][r, n:] == -1) and np.all(h["top_val"][r, n:] == -np.inf)):
                bad.append(f"row {r}: columns past N not padded")
        ok, where = _close(h["token"][tok_off[r]:tok_off[r + 1]], o["tok_vals"])
        if not ok:
            bad.append(f"row {r}: named-token logprobs at {where[:4]}")
        if with_selected:
            ok, _ = _close([h["next"][r]], [o["next"]])
            if not ok:
                bad.append(f"row {r}: next {h['next'][r]} vs {o['next']}")
    for k, r in enumerate(mask_rows):
        if not 0 <= r < B:
            if h["mask_status"][k] != oracle.STATUS_INVALID or h["mask_len"][k] != 0:
                bad.append(f"mask entry {k} (row {r} out of range): not INVALID")
            continue
        o = refs[r]
        L = int(h["mask_len"][k])
        gids = h["mask_ids"][k, :L] if cap > 0 else np.zeros(0, np.int32)
        flagged = bool(o["res"]["flags"] & SET_EXCUSE)
        if flagged and not (L == o["sup_len"] and np.array_equal(gids, o["sup_ids"])):
            flagged_sets += 1
            ref_full = np.flatnonzero(_oracle_member(batch, zs, r))
            if L < cap and not _threshold_set_ok(zs[r], gids, None, ref_full):
                bad.append(f"mask entry {k} row {r}: flagged row, GPU set is not a threshold set")
            continue
        if h["mask_status"][k] != o["sup_status"] or L != o["sup_len"]:
            bad.append(f"mask entry {k} row {r}: status/len {h['mask_status'][k]}/{L} vs "
                       f"{o['sup_status']}/{o['sup_len']}")
            continue
        if not np.array_equal(gids, o["sup_ids"]):
            bad.append(f"mask entry {k} row {r}: ids differ")
            continue
        if "mask_lp" in h and L:
            ok, where = _close(h["mask_lp"][k, :L], o["sup_vals"])
            if not ok:
                bad.append(f"mask entry {k} row {r}: support logprobs at {where[:4]}")
        ok, _ = _close([h["mask_sel"][k]], [o["sup_sel"]])
        if not ok:
            bad.append(f"mask entry {k} row {r}: selected {h['mask_sel'][k]} vs {o['sup_sel']}")
    assert not bad, f"{label}: {len(bad)} mismatches:\n" + "\n".join(bad[:20])
    print(f"[outputs] {label}: rows={B} mask rows={len(mask_rows)} "
          f"flagged support sets differing={flagged_sets}", flush=True)


def _oracle_member(batch, zs, r):
    res, sets = oracle.sample_row(zs[r], T=float(batch.temperature[r]), top_k=int(batch.top_k[r]),
                                  top_p=float(batch.top_p[r]), min_p=float(batch.min_p[r]),
                                  seed=int(batch.seed[r]), offset=int(batch.offset[r]),
                                  want_sets=True, order=batch.order)
    if res["greedy"]:
        m = np.zeros(len(zs[r]), bool)
        m[int(res["id"])] = True
        return m
    return (sets & 4) > 0


def _case(batch, *, basis, top_n, tok_rows, mask_rows, cap, with_selected=True, use_cuts=True,
          use_ws=True, label=""):
    print(f"[case] {label} B={batch.B} V={batch.V} bf16={batch.bf16} basis={basis} "
          f"cap={cap} selected={with_selected} cuts={use_cuts} slices={use_ws}", flush=True)
    gpu = _run(batch, basis=basis, top_n=top_n, tok_rows=tok_rows, mask_rows=mask_rows, cap=cap,
               with_selected=with_selected, use_cuts=use_cuts, use_ws=use_ws)
    ids = gpu[0]
    _, zs = run_oracle(batch)
    want = np.zeros(batch.B, bool)
    for r in mask_rows:
        if 0 <= r < batch.B:
            want[r] = True
    refs = _oracle_rows(batch, zs, np.arange(batch.B), basis=basis, top_n=top_n,
                        tok_rows=tok_rows, selected=ids if with_selected else None, cap=cap,
                        want_support=want)
    _check(batch, zs, gpu, refs, np.arange(batch.B), top_n=top_n, tok_rows=tok_rows,
           mask_rows=mask_rows, cap=cap, with_selected=with_selected, label=label)
    return gpu, refs


def _mixed_batch(rng, B, V, bf16=False, masked=True):
    z = workloads.decode_logits(rng, B, V)
    if bf16:
        z = workloads.to_bf16_bits(z)
    T = rng.choice(np.array([0.0, 0.05, 0.3, 0.7, 1.0, 1.3], np.float32), B)
    k = rng.choice(np.array([0, 1, 5, 50, 1000], np.int32), B)
    p = rng.choice(np.array([1.0, 0.9, 0.5, 0.99], np.float32), B)
    mp = rng.choice(np.array([0.0, 0.05, 0.3], np.float32), B)
    masks = rhm = None
    if masked:
        allowed = []
        rhm = np.zeros(B, np.uint8)
        for r in range(B):
            if r % 3 == 0:
                allowed.append(rng.choice(V, int(rng.choice([1, 7, 300, V // 2])), replace=False))
                rhm[r] = 1
            else:
                allowed.append(np.arange(V))
        masks = workloads.pack_bitmask(allowed, V)
    return workloads.Batch("outputs", z, bf16, T.astype(np.float32), k, p, mp,
                           workloads.seeds(rng, B), np.arange(B, dtype=np.uint64),
                           masks=masks, row_has_mask=rhm)


def _requests(rng, B, V, n_max=40):
    top_n = rng.integers(0, n_max + 1, B).astype(np.int32)
    top_n[0] = n_max
    tok_rows = []
    for r in range(B):
        t = list(rng.integers(0, V, int(rng.integers(0, 6))))
        if r % 4 == 0:
            t += [-1, V, V + 5]            # outside [0, V)
        tok_rows.append(np.asarray(t, np.int64))
    return top_n, tok_rows


@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("V,bf16", [(5003, False), (20000, False), (20000, True), (7001, True)])
def test_outputs_small_parity(V, bf16, use_ws):
    """Mixed rows (greedy, low T, top-k, top-p, min-p, masks allowing 1 to
    V/2 tokens), ragged V (scalar loads) and V % 4 == 0 (vector loads), fp32
    and bf16 (many ties); both bases; a support set per row plus an index out
    of range and a repeated row; the per-row outputs from the slice pass's
    records and from the row-serial passes."""
    rng = np.random.default_rng(700 + V + bf16)
    B = 24
    batch = _mixed_batch(rng, B, V, bf16=bf16)
    top_n, tok_rows = _requests(rng, B, V)
    mask_rows = list(range(B)) + [B, -3, 5]
    # support sets from the sampling call's thresholds (by slices with the
    # workspace: whole, and cut at 64 ids across slice boundaries), and with
    # the thresholds selected again
    for basis, cuts, cap in ((oracle.BASIS_SAMPLED, True, V), (oracle.BASIS_SAMPLED, True, 64),
                             (oracle.BASIS_ORIGINAL, False, 64)):
        _case(batch, basis=basis, top_n=top_n, tok_rows=tok_rows, mask_rows=mask_rows,
              cap=cap, use_cuts=cuts, use_ws=use_ws, label=f"small V={V} bf16={bf16}")


def test_outputs_scoring_without_draw():
    """selected = NULL: the scoring path; the same logprobs, no chosen-token
    output, and the support's selected logprob is NaN."""
    rng = np.random.default_rng(711)
    B, V = 16, 12000
    batch = _mixed_batch(rng, B, V)
    top_n, tok_rows = _requests(rng, B, V, n_max=256)
    gpu, refs = _case(batch, basis=oracle.BASIS_SAMPLED, top_n=top_n, tok_rows=tok_rows,
                      mask_rows=list(range(B)), cap=300, with_selected=False, use_cuts=False,
                      label="scoring")
    assert "next" not in gpu[3]
    ok = gpu[3]["mask_status"] == oracle.STATUS_INVALID
    assert np.all(np.isnan(gpu[3]["mask_sel"][~ok]))


def test_outputs_next_matches_sample_logprob():
    """In the sampled basis the chosen token's logprob is sampler_sample's own
    out_logprobs (two kernels, one definition)."""
    rng = np.random.default_rng(712)
    batch = _mixed_batch(rng, 32, 30000, masked=False)
    ids, st, lp, h = _run(batch, basis=oracle.BASIS_SAMPLED, top_n=np.zeros(32, np.int32),
                          tok_rows=[np.zeros(0, np.int64)] * 32, mask_rows=[], cap=0)
    ok, where = _close(h["next"], lp, tol=LP_TOL)
    assert ok, where


@pytest.mark.parametrize("cfg", ["c2", "c4"])
def test_outputs_full_size(cfg):
    """Full decode shape (B=192, V=151936): top-20 logprobs and 4 named tokens
    for every row, the support set of every 12th row with room for 40000
    tokens, the sampled basis; c2 fp32 (mixed top-k / top-p / min-p / greedy)
    and c4 bf16 with grammar masks."""
    batch = workloads.c2_decode(salt=3) if cfg == "c2" else workloads.c4_grammar(salt=3)
    rng = np.random.default_rng(713)
    B, V = batch.B, batch.V
    top_n = np.full(B, 20, np.int32)
    tok_rows = [rng.integers(0, V, 4) for _ in range(B)]
    mask_rows = list(range(0, B, 12))
    _case(batch, basis=oracle.BASIS_SAMPLED, top_n=top_n, tok_rows=tok_rows, mask_rows=mask_rows,
          cap=40000, label=f"full {cfg}")
    # the same support sets with the thresholds selected again
    _case(batch, basis=oracle.BASIS_SAMPLED, top_n=np.zeros(B, np.int32),
          tok_rows=[np.zeros(0, np.int64)] * B, mask_rows=mask_rows, cap=40000, use_cuts=False,
          label=f"full {cfg} reselected")


def test_outputs_original_basis_full_size():
    """Pre-temperature logprobs on the decode shape, T spread over
    [0.3, 1.3]: top-5 and the chosen token."""
    batch = workloads.c2_decode(salt=4)
    B = batch.B
    _case(batch, basis=oracle.BASIS_ORIGINAL, top_n=np.full(B, 5, np.int32),
          tok_rows=[np.zeros(0, np.int64)] * B, mask_rows=[], cap=0, label="original basis")


@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("V", [20000, 20003])
def test_outputs_edge_rows(V, use_ws):
    """Rows without a distribution and other edges, through the per-row
    outputs and the support sets from the sampling call's thresholds (by
    slices with the workspace, row by row without): a NaN and a +inf among
    the allowed tokens (statuses OVERFLOW / INVALID), a row with nothing
    allowed, one allowed token, a masked greedy row, a NaN on a masked token
    (ignored), ties under top-k, and a support cut at 3 ids; V % 4 == 0 (vector
    loads) and ragged."""
    rng = np.random.default_rng(716 + V)
    B = 8
    z = (rng.standard_normal((B, V)) * 2.0).astype(np.float32)
    z[0, 1234] = np.nan
    z[1, V - 7] = np.inf
    z[6, 17] = np.nan                       # masked below
    z[7, :] = np.round(z[7] * 2) / 2        # ties
    allowed = [np.arange(V)] * B
    allowed = list(allowed)
    allowed[2] = np.zeros(0, np.int64)      # nothing allowed
    allowed[3] = np.array([V - 1])          # one token
    allowed[4] = rng.choice(V, 500, replace=False)
    allowed[6] = np.setdiff1d(np.arange(V), [17])
    masks = workloads.pack_bitmask(allowed, V)
    rhm = np.array([0, 0, 1, 1, 1, 0, 1, 0], np.uint8)
    T = np.array([0.8, 1.0, 0.9, 0.7, 0.0, 1.1, 0.6, 1.0], np.float32)
    k = np.array([0, 0, 0, 0, 0, 40, 0, 5], np.int32)
    p = np.array([0.9, 0.9, 1.0, 0.5, 1.0, 0.95, 0.8, 1.0], np.float32)
    mp = np.array([0.0, 0.0, 0.0, 0.0, 0.0, 0.05, 0.0, 0.0], np.float32)
    batch = workloads.Batch("outputs-edge", z, False, T, k, p, mp, workloads.seeds(rng, B),
                            np.arange(B, dtype=np.uint64), masks=masks, row_has_mask=rhm)
    top_n = np.array([20, 20, 20, 20, 20, 20, 20, 20], np.int32)
    tok_rows = [np.array([0, 17, 1234, V - 1, V - 7], np.int64)] * B
    for cap in (V, 3):
        gpu, refs = _case(batch, basis=oracle.BASIS_SAMPLED, top_n=top_n, tok_rows=tok_rows,
                          mask_rows=list(range(B)) + [3], cap=cap, use_ws=use_ws,
                          label=f"edge rows V={V} cap={cap}")
        st = gpu[3]["mask_status"]
        assert st[0] == oracle.STATUS_INVALID and st[1] == oracle.STATUS_INVALID
        assert st[2] == oracle.STATUS_INVALID and gpu[3]["mask_len"][2] == 0
        assert gpu[3]["mask_len"][3] == 1 and gpu[3]["mask_ids"][3, 0] == V - 1


def test_outputs_top_n_candidate_overflow_and_ties():
    """Rows whose candidate list (tokens at or above the N-th largest
    thread maximum) overflows LDS: all-equal values, two values, and the
    large values packed into a few threads; top-N then takes the exact radix
    select with the id tie-break.  V = 151936, N up to 256."""
    rng = np.random.default_rng(714)
    B, V = 8, 151936
    z = (rng.standard_normal((B, V)) * 2.0).astype(np.float32)
    z[0, :] = 0.25                                   # all equal
    z[1, :] = np.where(rng.random(V) < 0.5, 1.0, 2.0).astype(np.float32)
    idx = np.arange(V)
    z[2, (idx % 2048) < 4] += 30.0                   # every large value in thread 0's groups
    z[3, :] = np.round(z[3] * 4) / 4                 # many ties
    z[4, :] = np.float32(-3.0)
    z[4, rng.choice(V, 300, replace=False)] = 5.0     # 300 tied maxima
    T = np.array([0.7, 1.0, 0.5, 0.9, 1.2, 0.0, 0.8, 1.0], np.float32)
    batch = workloads.Batch("ties", z, False, T, np.zeros(B, np.int32),
                            np.full(B, 0.9, np.float32), np.zeros(B, np.float32),
                            workloads.seeds(rng, B), np.arange(B, dtype=np.uint64))
    top_n = np.array([256, 256, 40, 256, 256, 20, 1, 256], np.int32)
    for ws in (True, False):
        _case(batch, basis=oracle.BASIS_SAMPLED, top_n=top_n, tok_rows=[np.array([0, 5])] * B,
              mask_rows=[0, 1, 4], cap=V, use_ws=ws, label="candidate overflow")
