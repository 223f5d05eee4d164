"""Host-side checks of the C ABI: the library loads and exports every function
include/cd_sampler.h declares; sampler_pack_host validates and packs as
documented.  No GPU call is made."""
import ctypes as ct
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def cds():
    import constrained_decoding_amd as m
    return m


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "cd_sampler.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sampler_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(cds):
    declared = _declared_functions()
    assert len(declared) >= 10
    lib = ct.CDLL(cds.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(cds.EXPORTS) == declared


def test_strerror_and_version(cds):
    assert cds.strerror(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert cds.strerror(code) != "unknown error"
    assert "gfx950" in cds.version()


def _rowparams(buf, B):
    dt = np.dtype([("T", "<f4"), ("top_p", "<f4"), ("min_p", "<f4"), ("top_k", "<i4"),
                   ("rep", "<f4"), ("freq", "<f4"), ("pres", "<f4"), ("flags", "<u4"),
                   ("pen_lo", "<i4"), ("pen_hi", "<i4"), ("bias_lo", "<i4"), ("bias_hi", "<i4"),
                   ("seed", "<u8"), ("offset", "<u8")])
    assert dt.itemsize == 64
    return np.frombuffer(buf[:64 * B].tobytes(), dt)


def test_flags_greedy_and_max_top_k(cds):
    T = np.array([0.0, 0.7, 1.0, 1e-6, 0.9], np.float32)
    k = np.array([0, 50, 1, 0, 20], np.int32)
    p = np.array([1.0, 0.9, 1.0, 0.5, 1.0], np.float32)
    mp = np.array([0.3, 0.0, 0.0, 0.0, 0.05], np.float32)
    buf, b = cds.pack_host(5, 1000, T, top_k=k, top_p=p, min_p=mp)
    rows = _rowparams(buf, 5)
    greedy = rows["flags"] & 1
    np.testing.assert_array_equal(greedy, [1, 0, 1, 1, 0])   # T<1e-5 or top_k==1
    assert b.flags & cds.FLAG_ANY_GREEDY and not b.flags & cds.FLAG_ALL_GREEDY
    assert b.flags & cds.FLAG_NEED_TOP_K and b.flags & cds.FLAG_NEED_TOP_P
    assert b.flags & cds.FLAG_NEED_MIN_P                       # row 4 (row 0 is greedy)
    assert b.max_top_k == 50                                  # every sampled row has k
    np.testing.assert_array_equal(rows["offset"], np.arange(5))  # default offset = row
    # greedy rows do not raise NEED_* flags
    _, b2 = cds.pack_host(2, 1000, np.array([0.0, 0.0], np.float32),
                          top_p=np.array([0.5, 0.5], np.float32),
                          min_p=np.array([0.2, 0.2], np.float32))
    assert b2.flags & cds.FLAG_ALL_GREEDY
    assert not b2.flags & (cds.FLAG_NEED_TOP_P | cds.FLAG_NEED_MIN_P | cds.FLAG_NEED_TOP_K)
    # top_k off (0 or >= V) on a sampled row -> no max_top_k
    _, b3 = cds.pack_host(2, 1000, np.array([1.0, 1.0], np.float32),
                          top_k=np.array([20, 1000], np.int32))
    assert b3.max_top_k == 0


def test_penalty_counts_and_bias_dedup(cds):
    hist = [[3, 3, 7, 3], [], [5]]
    hp, hi = cds.csr(hist)
    ids, vals = cds.bias_from_dict({"1": 5.0, "01": -3.0, "7": 2.0})
    bp = np.array([0, 3, 3, 3], np.int64)
    buf, b = cds.pack_host(3, 100, np.ones(3, np.float32),
                           repetition_penalty=np.array([1.1, 1.1, 1.0], np.float32),
                           frequency_penalty=np.array([0.5, 0.5, 0.0], np.float32),
                           presence_penalty=np.zeros(3, np.float32),
                           hist_indptr=hp, hist_ids=hi, bias_indptr=bp, bias_ids=ids,
                           bias_vals=vals)
    rows = _rowparams(buf, 3)
    assert b.n_sampled == 3
    assert np.frombuffer(buf[64 * 3:64 * 3 + 12].tobytes(), "<i4").tolist() == [0, 1, 2]
    # the row order (room for B int32, 16-byte padded), then the task table (one
    # group of 8 task rows, int32: no row needs a second pass), then the rows'
    # workspace places (8 bytes each)
    pen_off = 64 * 3 + 16 + 32 + 8 * 3
    assert b.n_pen == 0 and b.n_hist_raw == 4
    raw_off = pen_off + 8 * b.n_bias
    pen = np.frombuffer(buf[raw_off:raw_off + 4 * b.n_hist_raw].tobytes(), "<i4")
    # rows of up to 4096 history tokens are packed as they come, as raw int32
    # ids after the bias entries (the transforms kernel merges repeats); row 2
    # has no active penalty
    np.testing.assert_array_equal(pen, [3, 3, 7, 3])
    assert (rows["pen_lo"][0], rows["pen_hi"][0]) == (0, 4)
    assert rows["flags"][0] & (1 << 6)                      # ROW_PEN_RAW
    assert b.flags & cds.FLAG_NEED_PENALTY and b.flags & cds.FLAG_HAS_BIAS
    off = pen_off
    bias = np.frombuffer(buf[off:off + 8 * b.n_bias].tobytes(),
                         [("id", "<i4"), ("val", "<f4")])
    assert bias["id"].tolist() == [1, 7]
    assert bias["val"].tolist() == [-3.0, 2.0]                # "01" came later: it wins


@pytest.mark.parametrize("field,value", [
    ("temperature", -0.1), ("temperature", np.nan), ("temperature", np.inf),
    ("top_p", 0.0), ("top_p", 1.5), ("top_p", np.nan),
    ("min_p", -0.1), ("min_p", 1.1), ("min_p", np.nan),
    ("repetition_penalty", 0.0), ("repetition_penalty", np.nan),
    ("frequency_penalty", np.nan), ("presence_penalty", np.inf),
])
def test_invalid_parameters_rejected(cds, field, value):
    kw = dict(temperature=np.ones(2, np.float32))
    arr = np.ones(2, np.float32) if field != "frequency_penalty" and field != "presence_penalty" \
        and field != "min_p" else np.zeros(2, np.float32)
    if field == "top_p":
        arr = np.ones(2, np.float32)
    arr[1] = value
    kw[field] = arr
    with pytest.raises(cds.SamplerError) as e:
        cds.pack_host(2, 100, **kw)
    assert e.value.code == -1


def test_invalid_ids_and_sizes_rejected(cds):
    T = np.ones(2, np.float32)
    with pytest.raises(cds.SamplerError) as e:
        cds.pack_host(2, 100, T, hist_indptr=np.array([0, 1, 2]), hist_ids=np.array([3, 100]))
    assert e.value.code == -1
    with pytest.raises(cds.SamplerError):
        cds.pack_host(2, 100, T, bias_indptr=np.array([0, 1, 1]), bias_ids=np.array([-1]),
                      bias_vals=np.array([1.0]))
    with pytest.raises(cds.SamplerError):   # +inf bias is not a valid value
        cds.pack_host(2, 100, T, bias_indptr=np.array([0, 1, 1]), bias_ids=np.array([1]),
                      bias_vals=np.array([np.inf]))
    cds.pack_host(2, 100, T, bias_indptr=np.array([0, 1, 1]), bias_ids=np.array([1]),
                  bias_vals=np.array([-np.inf]))           # -inf bans a token: allowed
    with pytest.raises(cds.SamplerError):   # non-monotone indptr
        cds.pack_host(2, 100, T, hist_indptr=np.array([0, 2, 1]), hist_ids=np.array([1, 2]))
    with pytest.raises(cds.SamplerError) as e:
        cds.pack_host(1, 1 << 25, np.ones(1, np.float32))
    assert e.value.code == -2
    buf = np.zeros(8, np.uint8)
    out = cds.Batch()
    h = cds._binding._HostArrays(2, 100, T)
    rc = cds.lib.sampler_pack_host(ct.byref(h.hp), buf.ctypes.data, 8, ct.byref(out))
    assert rc == -3                           # ENOSPC


def test_workspace_size_closed_form(cds):
    n = cds.lib.sampler_workspace_bytes(192, 151936)
    assert n > 192 * 151936 // 64                    # holds histograms and lists
    assert cds.lib.sampler_workspace_bytes(0, 10) == 0
    assert cds.lib.sampler_workspace_bytes(4, 1024) > 0


def test_sampled_row_list(cds):
    """The packed block holds the dispatch order of the rows: the rows that are
    not greedy (T >= 1e-5 and top_k != 1) -- those whose only cut is top-p
    first, hotter rows first within a group -- then the greedy rows,
    ascending."""
    T = np.array([0.0, 0.7, 1e-6, 1.0, 0.9, 0.8], np.float32)
    k = np.array([0, 0, 0, 1, 50, 0], np.int32)
    p = np.array([1, 1, 1, 1, 1, 0.9], np.float32)
    buf, b = cds.pack_host(6, 1000, T, top_k=k, top_p=p)
    assert b.n_sampled == 3
    order = [5, 4, 1, 0, 2, 3]
    assert np.frombuffer(buf[64 * 6:64 * 6 + 24].tobytes(), "<i4").tolist() == order
    # the kernel's task table: 24 task slots (three groups of 8 for B = 6); pass
    # 1 takes the ordered rows, the one top-p-only row (5) gets two pass-2
    # tasks (bit 30), one per slice half (bit 28: split; bit 29: second half),
    # as one such row in six is few
    assert b.n_hold == 1 and b.flags & cds.FLAG_SPLIT_PASS2
    t0 = 64 * 6 + 32
    tasks = np.frombuffer(buf[t0:t0 + 96].tobytes(), "<i4")
    assert tasks[:8].tolist() == order + [-1, -1]
    assert tasks[8] == 5 | (1 << 30) | (1 << 28) and (tasks[9:16] == -1).all()
    assert tasks[16] == 5 | (1 << 30) | (1 << 29) | (1 << 28) and (tasks[17:] == -1).all()
    # when most rows need the second pass, its tasks take whole slices (the
    # table holds the groups in use: one pass-1 and one pass-2 group)
    buf, b = cds.pack_host(4, 1000, np.ones(4, np.float32), top_p=np.full(4, 0.9, np.float32))
    assert b.n_hold == 4 and not b.flags & cds.FLAG_SPLIT_PASS2
    tasks = np.frombuffer(buf[64 * 4 + 16:64 * 4 + 16 + 64].tobytes(), "<i4")
    assert tasks[8:12].tolist() == [(1 << 30) | r for r in range(4)] and (tasks[12:] == -1).all()

    buf, b = cds.pack_host(2, 1000, np.zeros(2, np.float32))
    assert b.n_sampled == 0 and b.flags & cds.FLAG_ALL_GREEDY


def test_row_classes_follow_list_capacity(cds):
    """Top-k rows list candidates only while the lists fit the finisher:
    q = min(k, ceil(2k/P) + 64) <= 384 and 1.5 q P <= 4096 (P = ceil(V/15360)
    slices); other top-k rows need the row's histogram first (n_hold, listed
    first in the order).  Top-p as the only cut always needs it."""
    def holds(V, k, p=1.0):
        buf, b = cds.pack_host(2, V, np.ones(2, np.float32), top_k=np.full(2, k, np.int32),
                               top_p=np.full(2, p, np.float32))
        return b.n_hold
    assert holds(151936, 1000) == 0     # P=10: q=264, 1.5*264*10 = 3960
    assert holds(151936, 50) == 0
    assert holds(32000, 1000) == 2      # P=3: q=731 > 384
    assert holds(200000, 1000) == 2     # P=14: 1.5*207*14 = 4347 > 4096
    assert holds(200000, 100) == 0
    assert holds(151936, 0, 0.9) == 2   # top-p only


def test_dispatch_order_by_list_length(cds):
    """Sampled rows go out in the order: rows that need the row's histogram
    first; top-k rows with long lists (q P > 1024, no min-p); other top-k rows
    whose lists pass the finisher's one-wave limit (q P > 256); the rest; then
    the greedy rows; within a group by falling temperature, then by row
    index.  V = 151936 gives P = 10 slices, so k = 20, 50, 1000 list
    q P = 200, 500, 2640."""
    T = np.array([0.8, 0.8, 0.8, 0.8, 0.8, 0.8, 0.0], np.float32)
    k = np.array([20, 50, 1000, 1000, 0, 0, 0], np.int32)
    p = np.array([1, 1, 1, 1, 1, 0.9, 1], np.float32)
    mp = np.array([0, 0, 0, 0.05, 0.05, 0, 0], np.float32)
    buf, b = cds.pack_host(7, 151936, T, top_k=k, top_p=p, min_p=mp)
    assert b.n_sampled == 6 and b.n_hold == 1
    order = np.frombuffer(buf[64 * 7:64 * 7 + 28].tobytes(), "<i4").tolist()
    assert order == [5, 2, 1, 3, 0, 4, 6]
    # within a group, hotter rows first (ties keep the row order)
    T2 = np.array([0.5, 1.2, 0.5, 0.9], np.float32)
    buf, b = cds.pack_host(4, 151936, T2, top_k=np.full(4, 50, np.int32))
    assert np.frombuffer(buf[64 * 4:64 * 4 + 16].tobytes(), "<i4").tolist() == [1, 3, 0, 2]


def test_filter_order_validated_and_flagged_where_it_matters(cds):
    T = np.ones(4, np.float32)
    k = np.array([20, 0, 20, 0], np.int32)
    p = np.array([0.9, 0.9, 1.0, 0.9], np.float32)
    mp = np.array([0.0, 0.1, 0.1, 0.0], np.float32)
    for order, bit in ((0, 0), (1, 1 << 8), (2, 1 << 9)):
        buf, b = cds.pack_host(4, 1000, T, top_k=k, top_p=p, min_p=mp, filter_order=order)
        flags = _rowparams(buf, 4)["flags"]
        # top-p with top-k, top-p with min-p: flagged; top-k + min-p without
        # top-p, and top-p alone: the orders agree, no flag
        assert [(f & (3 << 8)) for f in flags] == [bit, bit, 0, 0]
    for bad in (-1, 3):
        with pytest.raises(cds.SamplerError) as e:
            cds.pack_host(4, 1000, T, top_k=k, top_p=p, min_p=mp, filter_order=bad)
        assert e.value.code == -1


def test_workspace_per_batch_smaller_than_bound(cds):
    """Workspace a packed batch needs: lists only for rows that list
    candidates (top-k rows at their class's capacity), histograms only for
    rows whose cut needs the row's histogram; the per-shape bound covers
    every batch."""
    V, P = 151936, 10
    B = 8
    T = np.ones(B, np.float32)
    T[0] = 0.0                                              # greedy: nothing
    k = np.array([0, 20, 0, 0, 50, 0, 1000, 0], np.int32)
    p = np.array([1, 0.9, 0.9, 1, 1, 1, 0.9, 1], np.float32)
    mp = np.array([0, 0, 0, 0.05, 0, 0, 0, 0], np.float32)
    _, b = cds.pack_host(B, V, T, top_k=k, top_p=p, min_p=mp)
    need = cds.lib.sampler_workspace_bytes_batch(ct.byref(b))
    bound = cds.lib.sampler_workspace_bytes(B, V)
    assert 0 < need < bound
    # row 2 (top-p only) and row 6 (k = 1000 lists) ... row 2 is the only
    # HOLD row: P histograms
    assert b.ws_hist_slices == P
    # lists: rows 1, 3, 4, 6 (LIST) P each, row 2 (HOLD) 2P (half slices),
    # rows 5, 7 (no cut: RACE) records only
    assert b.ws_records == P * (4 + 2 + 2)
    caps = {20: 128, 50: 192, 1000: 640}     # 2q + 64 rounded up to 64 entries
    assert b.ws_list_entries == P * (caps[20] + 2048 + caps[50] + caps[1000]) + 2 * P * 2048


def test_logprobs_request_validation(cds):
    """sampler_logprobs rejects inconsistent requests before any launch, and
    returns OK without a launch when nothing is asked for (host pointers stand
    in for device ones: nothing reaches the GPU)."""
    _, b = cds.pack_host(4, 1000, np.ones(4, np.float32))
    logits = np.zeros((4, 1000), np.float32)
    dummy = np.zeros(4096, np.int64)
    P = dummy.ctypes.data

    def call(req=None, out=None, **kw):
        r = cds.LogprobRequest(size=ct.sizeof(cds.LogprobRequest))
        o = cds.LogprobOutputs(size=ct.sizeof(cds.LogprobOutputs))
        for k, v in (req or {}).items():
            setattr(r, k, v)
        for k, v in (out or {}).items():
            setattr(o, k, v)
        return cds.lib.sampler_logprobs(ct.byref(b), logits.ctypes.data, 0, 1000, None, 0, None,
                                        ct.byref(r), ct.byref(o), None)

    assert call() == 0                                        # nothing asked: no launch
    bad = [
        ({"size": 8}, {}),
        ({"basis": 2}, {}),
        ({"top_n_max": cds.MAX_TOP_N + 1}, {"top_logprobs_idx": P, "top_logprobs_val": P}),
        ({"top_n_max": 5}, {}),                               # no top-N outputs
        ({}, {"top_logprobs_idx": P, "top_logprobs_val": P}),  # outputs, top_n_max 0
        ({"top_n": P}, {}),
        ({}, {"next_token_logprobs": P}),                     # needs selected
        ({"token_indptr": P, "token_ids": P}, {}),            # no output
        ({"token_indptr": P}, {"token_ids_logprobs": P}),     # no ids
        ({"n_mask_rows": 3, "mask_rows": P, "mask_cap": 4},
         {"mask_lengths": P, "mask_statuses": P}),            # no ids output
        ({"n_mask_rows": 3, "mask_rows": P}, {"mask_statuses": P}),
        ({"n_mask_rows": 3}, {"mask_lengths": P, "mask_statuses": P}),
        ({}, {"mask_lengths": P}),                            # outputs without rows
        ({"n_mask_rows": -1}, {}),
        ({"n_mask_rows": 2, "mask_rows": P, "mask_cap": -1},
         {"mask_lengths": P, "mask_statuses": P}),
    ]
    for req, out in bad:
        assert call(req, out) == -1, (req, out)
    # the workspace: row slice records and keys (16384-token slices), then
    # the support slice records (4096-token slices), 16-byte aligned
    rows = -(-4 * 1 * (32 + 8 * 5) // 16) * 16
    ws = cds.lib.sampler_logprobs_workspace_bytes
    assert ws(4, 1000, 5, 0) == rows
    assert ws(4, 1000, 5, 3) == rows + 3 * 1 * 32
    assert ws(4, 151936, 0, 16) == -(-4 * 10 * 32 // 16) * 16 + 16 * 38 * 32
    assert ws(4, 1000, 5, -1) == 0 and ws(4, 1000, cds.MAX_TOP_N + 1, 0) == 0
    assert ws(0, 1000, 5, 0) == 0
    sup_req = {"n_mask_rows": 3, "mask_rows": P, "mask_cap": 4, "cuts": P, "workspace": P}
    sup_out = {"mask_token_ids": P, "mask_lengths": P, "mask_statuses": P}
    need = ws(4, 1000, 0, 3)
    assert call(dict(sup_req, workspace_bytes=need - 16), sup_out) == -3   # too small
    assert call(dict(sup_req, workspace=P + 8, workspace_bytes=need), sup_out) == -1  # misaligned
    # a record of another size
    r = cds.LogprobRequest(size=ct.sizeof(cds.LogprobRequest))
    o = cds.LogprobOutputs(size=ct.sizeof(cds.LogprobOutputs) - 8)
    assert cds.lib.sampler_logprobs(ct.byref(b), logits.ctypes.data, 0, 1000, None, 0, None,
                                    ct.byref(r), ct.byref(o), None) == -1


def test_shard_calls_validated_without_launch(cds):
    """The vocabulary-parallel calls: sizes, the phase set of a batch, and
    rejected arguments (host pointers stand in: nothing is launched)."""
    assert cds.lib.sampler_shard_state_bytes(192) == 80 * 192
    assert cds.lib.sampler_shard_records(18992) == 5 and cds.lib.sampler_shard_records(4096) == 1
    assert cds.lib.sampler_shard_partial_bytes(192, 18992) == 2112 * 192 * 5
    assert cds.lib.sampler_shard_state_bytes(0) == 0
    T = np.array([0.0, 0.0], np.float32)
    _, b = cds.pack_host(2, 1000, T)
    assert cds.lib.sampler_shard_phases(ct.byref(b)) == 1            # all greedy: stats only
    T = np.array([0.7, 0.0], np.float32)
    _, b = cds.pack_host(2, 1000, T, top_k=np.array([5, 0], np.int32),
                         top_p=np.array([0.9, 1.0], np.float32))
    assert cds.lib.sampler_shard_phases(ct.byref(b)) == (1 << 11) - 1  # every phase
    _, b = cds.pack_host(2, 1000, T)
    assert cds.lib.sampler_shard_phases(ct.byref(b)) == 1 | (1 << 10)  # stats and race
    x = np.zeros((2, 1000), np.float32)
    buf = np.zeros(8192, np.uint8)
    p = buf.ctypes.data + (-buf.ctypes.data) % 256
    pas = lambda **kw: cds.lib.sampler_shard_pass(
        ct.byref(b), kw.get("phase", 0), x.ctypes.data, 0, kw.get("ld", 1000), kw.get("v0", 0),
        kw.get("width", 500), None, 0, None, p, p, None)
    for bad in ({"phase": -1}, {"phase": 11}, {"v0": 2}, {"v0": -4}, {"width": 0},
                {"v0": 600, "width": 500}, {"ld": 400}):
        assert pas(**bad) == -1, bad
    mer = lambda ph, n: cds.lib.sampler_shard_merge(ct.byref(b), ph, p, p, n, p, None, None, None)
    assert mer(0, 0) == -1 and mer(11, 2) == -1


def test_spec_accept_validated_without_launch(cds):
    P = np.zeros(64, np.int32).ctypes.data
    f = cds.lib.sampler_spec_accept
    assert f(0, 7, None, None, None, None, None, None, None, None) == 0   # nothing to do
    assert f(-1, 7, P, None, P, None, P, P, None, None) == -1
    assert f(4, -1, P, None, P, None, P, P, None, None) == -1
    assert f(4, 7, None, None, P, None, P, P, None, None) == -1
    assert f(4, 7, P, None, None, None, P, P, None, None) == -1         # drafts required
    assert f(4, 7, P, None, P, None, P, None, None, None) == -1         # counts required
