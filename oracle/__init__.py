"""CPU oracle for the batched per-request sampling step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this package.  It shares no
code with the HIP path in ``constrained_decoding_amd``; neither imports the
other.  The arithmetic lives in ``cd_oracle.c`` (plain C, fp64); this module
only marshals numpy arrays.

Parity status: all functions are pinned by ``tests/test_oracle_*.py``; the
two Philox-4x32 multiplier constants are "parity unpinned" (taken from the
Philox paper's table; the round structure is pinned via the 4x64 instance).
"""
import ctypes as _ct
import os as _os

import numpy as _np

from . import build as _build

DTYPE_F32 = 0
DTYPE_BF16 = 1
# filter orders (see cd_oracle.h): min-p first (default), joint top-k/top-p,
# min-p last
ORDER_MINP_FIRST, ORDER_JOINT, ORDER_MINP_LAST = 0, 1, 2
STATUS_OK, STATUS_OVERFLOW, STATUS_INVALID = 0, 1, 2
# logprob basis of the further outputs: the distribution the row is sampled
# from (z/T; greedy rows z), or the logits before the temperature (z)
BASIS_SAMPLED, BASIS_ORIGINAL = 0, 1
F_TOPP, F_RACE, F_MINP, F_TOPK = 1, 2, 4, 8
# flags that excuse an id mismatch (F_TOPK is informational: top-k is decided
# on exact fp32 values on both sides)
F_EXCUSE = F_TOPP | F_RACE | F_MINP

RESULT_DTYPE = _np.dtype([
    ("id", _np.int32), ("status", _np.int32), ("greedy", _np.int32),
    ("flags", _np.uint32), ("logprob", _np.float64), ("m", _np.float64),
    ("log_z", _np.float64), ("n1", _np.int64), ("n2", _np.int64),
    ("n3", _np.int64), ("zcut", _np.float32), ("pad_", _np.float32),
    ("best_key", _np.float64), ("second_key", _np.float64),
])
assert RESULT_DTYPE.itemsize == 88

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # CDS_ORACLE_SANITIZE=1: the AddressSanitizer / UBSan build (the process
    # must preload the ASan runtime; tests/test_sanitizers.py does)
    if _os.environ.get("CDS_ORACLE_SANITIZE") == "1":
        path = _build.build(force=False, sanitize=True)
    else:
        path = _build.LIB
        if not _os.path.exists(path) or \
                _os.path.getmtime(path) < _os.path.getmtime(_build.SRC):
            _build.build(force=True)
    lib = _ct.CDLL(path)
    P = _ct.c_void_p
    lib.cdo_philox4x32_10.argtypes = [P, P, P]
    lib.cdo_philox4x64_10.argtypes = [P, P, P]
    lib.cdo_philox_constants.argtypes = [P]
    lib.cdo_race_bits.argtypes = [_ct.c_uint64, _ct.c_uint64, _ct.c_int64]
    lib.cdo_race_bits.restype = _ct.c_uint32
    lib.cdo_uniform24.argtypes = [_ct.c_uint32]
    lib.cdo_uniform24.restype = _ct.c_double
    lib.cdo_transform_row.argtypes = [P, _ct.c_int, _ct.c_int32, P, _ct.c_int64,
                                      _ct.c_float, _ct.c_float, _ct.c_float,
                                      P, P, _ct.c_int64, P, P]
    lib.cdo_sample_row.argtypes = [P, _ct.c_int32, _ct.c_float, _ct.c_int32,
                                   _ct.c_float, _ct.c_float, _ct.c_uint64,
                                   _ct.c_uint64, P, P]
    lib.cdo_sample_batch.argtypes = [P, _ct.c_int64, _ct.c_int32, _ct.c_int32,
                                     P, P, P, P, P, P, P]
    lib.cdo_sample_row_order.argtypes = [P, _ct.c_int32, _ct.c_float, _ct.c_int32,
                                         _ct.c_float, _ct.c_float, _ct.c_uint64,
                                         _ct.c_uint64, _ct.c_int32, P, P]
    lib.cdo_sample_batch_order.argtypes = [P, _ct.c_int64, _ct.c_int32, _ct.c_int32,
                                           P, P, P, P, P, P, _ct.c_int32, P]
    lib.cdo_set_log_softmax.argtypes = [P, _ct.c_int32, _ct.c_double, P, _ct.c_uint8, P]
    lib.cdo_set_log_softmax.restype = _ct.c_int64
    lib.cdo_top_n.argtypes = [P, P, _ct.c_int32, _ct.c_int32, P, P]
    lib.cdo_top_n.restype = _ct.c_int32
    lib.cdo_race_best.argtypes = [P, _ct.c_int32, _ct.c_float, _ct.c_double, _ct.c_uint64,
                                  _ct.c_uint64, _ct.c_int32, _ct.c_int32, P, _ct.c_uint8, P]
    lib.cdo_race_best.restype = _ct.c_int32
    lib.cdo_spec_accept.argtypes = [P, P, _ct.c_int32, P, _ct.c_int32, P, P]
    lib.cdo_spec_accept.restype = _ct.c_int32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_ct.c_void_p)


def philox4x32_10(ctr, key):
    c = _np.ascontiguousarray(ctr, dtype=_np.uint32)
    k = _np.ascontiguousarray(key, dtype=_np.uint32)
    o = _np.zeros(4, _np.uint32)
    _load().cdo_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def philox4x64_10(ctr, key):
    c = _np.ascontiguousarray(ctr, dtype=_np.uint64)
    k = _np.ascontiguousarray(key, dtype=_np.uint64)
    o = _np.zeros(4, _np.uint64)
    _load().cdo_philox4x64_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def philox_constants():
    """(M0, M1, W0, W1) of the 4x32 instance, then of the 4x64 instance."""
    o = _np.zeros(8, _np.uint64)
    _load().cdo_philox_constants(_ptr(o))
    return [int(v) for v in o]


def race_bits(seed, offset, t):
    return int(_load().cdo_race_bits(int(seed), int(offset), int(t)))


def uniform24(x):
    return float(_load().cdo_uniform24(int(x)))


def transform_row(logits, *, hist_ids=None, rep=1.0, freq=0.0, pres=0.0,
                  bias_ids=None, bias_vals=None, mask=None, bf16=False):
    """Penalties -> bitmask -> bias on one row.

    ``logits``: float32 array, or uint16 bf16 bit patterns with ``bf16=True``.
    ``mask``: int32 words (ceil(V/32)) or None.  Returns float32 [V].
    """
    if bf16:
        x = _np.ascontiguousarray(logits, dtype=_np.uint16)
    else:
        x = _np.ascontiguousarray(logits, dtype=_np.float32)
    V = x.shape[0]
    h = None if hist_ids is None else _np.ascontiguousarray(hist_ids, _np.int32)
    bi = None if bias_ids is None else _np.ascontiguousarray(bias_ids, _np.int32)
    bv = None if bias_vals is None else _np.ascontiguousarray(bias_vals, _np.float32)
    mk = None if mask is None else _np.ascontiguousarray(mask, _np.int32)
    if mk is not None and mk.shape[0] < (V + 31) // 32:
        raise ValueError("mask row too short")
    out = _np.empty(V, _np.float32)
    rc = _load().cdo_transform_row(
        _ptr(x), DTYPE_BF16 if bf16 else DTYPE_F32, V, _ptr(h),
        0 if h is None else h.shape[0], rep, freq, pres, _ptr(bi), _ptr(bv),
        0 if bi is None else bi.shape[0], _ptr(mk), _ptr(out))
    if rc != 0:
        raise ValueError("token id out of range")
    return out


def sample_row(z, *, T, top_k=0, top_p=1.0, min_p=0.0, seed=0, offset=0,
               want_sets=False, order=ORDER_MINP_FIRST):
    """Sample one row of transformed logits; returns a RESULT_DTYPE record
    (and the V-byte set-membership array if ``want_sets``).  ``order``: the
    filter order (ORDER_*)."""
    zz = _np.ascontiguousarray(z, dtype=_np.float32)
    V = zz.shape[0]
    res = _np.zeros(1, RESULT_DTYPE)
    sets = _np.zeros(V, _np.uint8) if want_sets else None
    rc = _load().cdo_sample_row_order(_ptr(zz), V, float(T), int(top_k), float(top_p),
                                      float(min_p), int(seed), int(offset), int(order),
                                      _ptr(res), _ptr(sets))
    if rc != 0:
        raise ValueError(f"unknown filter order {order}")
    return (res[0], sets) if want_sets else res[0]


def sample_batch(z, *, T, top_k, top_p, min_p, seed, offset, broadcast=False,
                 order=ORDER_MINP_FIRST):
    """Row loop; ``z`` is [B, V] (or [V] with ``broadcast=True`` and B given
    by the parameter arrays).  Returns RESULT_DTYPE [B]."""
    zz = _np.ascontiguousarray(z, dtype=_np.float32)
    T = _np.ascontiguousarray(T, _np.float32)
    B = T.shape[0]
    if broadcast:
        V, ld = zz.shape[-1], 0
    else:
        assert zz.ndim == 2 and zz.shape[0] == B
        V, ld = zz.shape[1], zz.shape[1]
    k = _np.ascontiguousarray(top_k, _np.int32)
    p = _np.ascontiguousarray(top_p, _np.float32)
    mp = _np.ascontiguousarray(min_p, _np.float32)
    sd = _np.ascontiguousarray(seed, _np.uint64)
    of = _np.ascontiguousarray(offset, _np.uint64)
    for a in (k, p, mp, sd, of):
        assert a.shape[0] == B
    out = _np.zeros(B, RESULT_DTYPE)
    rc = _load().cdo_sample_batch_order(_ptr(zz), ld, B, V, _ptr(T), _ptr(k), _ptr(p),
                                        _ptr(mp), _ptr(sd), _ptr(of), int(order), _ptr(out))
    if rc != 0:
        raise ValueError(f"unknown filter order {order}")
    return out


def pipeline(logits, params, *, bf16=False, masks=None, row_has_mask=None,
             rows=None):
    """Oracle for the whole step on a batch described by plain arrays.

    ``logits``: [B, V] float32 (or uint16 bf16 bits).  ``params``: dict with
    per-row arrays ``temperature, top_k, top_p, min_p, seed, offset`` and
    optional ``rep, freq, pres`` plus per-row lists ``hist`` (int arrays) and
    ``bias`` (lists of (id, value) pairs, applied in order).  ``masks``:
    [B, W] int32 or None; ``row_has_mask``: [B] bool or None (all rows).
    ``rows``: subset of row indices to evaluate (default all).  An optional
    ``params["order"]`` (scalar) selects the filter order (ORDER_*).
    Returns (RESULT_DTYPE records, transformed logits) for the chosen rows.
    """
    B = logits.shape[0]
    rows = range(B) if rows is None else rows
    res, zs = [], []
    for r in rows:
        hist = params.get("hist")
        h = None if hist is None or hist[r] is None or len(hist[r]) == 0 \
            else _np.asarray(hist[r], _np.int32)
        bias = params.get("bias")
        bi = bv = None
        if bias is not None and bias[r]:
            bi = _np.asarray([b[0] for b in bias[r]], _np.int32)
            bv = _np.asarray([b[1] for b in bias[r]], _np.float32)
        mk = None
        if masks is not None and (row_has_mask is None or row_has_mask[r]):
            mk = masks[r]
        z = transform_row(
            logits[r], hist_ids=h,
            rep=float(params["rep"][r]) if "rep" in params else 1.0,
            freq=float(params["freq"][r]) if "freq" in params else 0.0,
            pres=float(params["pres"][r]) if "pres" in params else 0.0,
            bias_ids=bi, bias_vals=bv, mask=mk, bf16=bf16)
        res.append(sample_row(
            z, T=params["temperature"][r], top_k=params["top_k"][r],
            top_p=params["top_p"][r], min_p=params["min_p"][r],
            seed=params["seed"][r], offset=params["offset"][r],
            order=params.get("order", ORDER_MINP_FIRST)))
        zs.append(z)
    return _np.array(res, dtype=RESULT_DTYPE), _np.array(zs)


# ------------------------------------------------------------ further outputs

def set_log_softmax(z, T=1.0, in_set=None, bit=1):
    """log_softmax(z/T) over the finite tokens of a set (all tokens when
    ``in_set`` is None; else those with ``in_set & bit``), -inf elsewhere.
    Returns (count, float64 [V]); count -1 means a NaN/+inf lay in the set
    (every value NaN)."""
    zz = _np.ascontiguousarray(z, dtype=_np.float32)
    V = zz.shape[0]
    st = None if in_set is None else _np.ascontiguousarray(in_set, _np.uint8)
    out = _np.empty(V, _np.float64)
    n = _load().cdo_set_log_softmax(_ptr(zz), V, float(T), _ptr(st), int(bit), _ptr(out))
    return int(n), out


def top_n(z, lp, N):
    """The N largest z (lower id first among equal values) with their lp."""
    zz = _np.ascontiguousarray(z, dtype=_np.float32)
    ll = _np.ascontiguousarray(lp, dtype=_np.float64)
    ids = _np.empty(max(N, 1), _np.int32)
    vals = _np.empty(max(N, 1), _np.float64)
    _load().cdo_top_n(_ptr(zz), _ptr(ll), zz.shape[0], int(N), _ptr(ids), _ptr(vals))
    return ids[:N], vals[:N]


def row_outputs(z, *, T, top_k=0, top_p=1.0, min_p=0.0, seed=0, offset=0,
                order=ORDER_MINP_FIRST, basis=BASIS_SAMPLED, n_top=0,
                token_ids=(), selected=None, support_cap=None):
    """The further outputs of one row of transformed logits ``z``.

    Basis: the row's sampling distribution (s = z/T; greedy rows z, as for
    the chosen token's logprob), or with ``basis=BASIS_ORIGINAL`` the logits
    before the temperature.  Returns a dict with
      ``top_ids, top_vals``  the ``n_top`` most likely tokens (larger z first,
                             lower id first among equal values; -1 / -inf past
                             the allowed tokens; -1 / NaN on an OVERFLOW row);
      ``tok_vals``           logprobs of ``token_ids`` (NaN for an id outside
                             [0, V) or on an OVERFLOW row, -inf if masked);
      ``next``               logprob of token ``selected`` (if given): NaN on
                             OVERFLOW, -inf on INVALID;
      and, if ``support_cap`` is given, the support set (the set the row's
      draw is made from; a greedy row's is its argmax): ``sup_ids`` (ascending,
      at most ``support_cap``), ``sup_vals`` (logprobs renormalised over the
      whole support, under the sampling distribution), ``sup_n`` (its true
      size), ``sup_len``, ``sup_status`` (OK; OVERFLOW: larger than the
      capacity; INVALID: no distribution -- no finite allowed logit, or a NaN
      or +inf among them), ``sup_sel`` (renormalised logprob of ``selected``,
      -inf outside the support, NaN if ``selected`` is not a token id or the
      row is INVALID).
    Also ``res``: the row's sampling record (RESULT_DTYPE)."""
    zz = _np.ascontiguousarray(z, dtype=_np.float32)
    V = zz.shape[0]
    T32 = float(_np.float32(T))
    res, sets = sample_row(zz, T=T32, top_k=top_k, top_p=top_p, min_p=min_p,
                           seed=seed, offset=offset, want_sets=True, order=order)
    status = int(res["status"])
    greedy = bool(res["greedy"])
    Tb = 1.0 if (basis == BASIS_ORIGINAL or greedy) else T32
    if status == STATUS_OVERFLOW:
        lp = _np.full(V, _np.nan)
    else:
        _, lp = set_log_softmax(zz, Tb)
    out = {"res": res}
    if status == STATUS_OVERFLOW:
        out["top_ids"] = _np.full(n_top, -1, _np.int32)
        out["top_vals"] = _np.full(n_top, _np.nan)
    else:
        out["top_ids"], out["top_vals"] = top_n(zz, lp, n_top)

    def at(i):
        return float(lp[i]) if 0 <= i < V else float("nan")
    out["tok_vals"] = _np.array([at(int(i)) for i in token_ids], _np.float64)
    if selected is not None:
        if status == STATUS_OVERFLOW:
            out["next"] = float("nan")
        elif status == STATUS_INVALID:
            out["next"] = float("-inf")
        else:
            out["next"] = at(int(selected))
    if support_cap is not None:
        sel = None if selected is None else int(selected)
        if status != STATUS_OK:
            ids = _np.zeros(0, _np.int64)
            vals = _np.zeros(0)
            n_sup, sst, ssel = 0, STATUS_INVALID, float("nan")
        else:
            if greedy:
                member = _np.zeros(V, _np.uint8)
                member[int(res["id"])] = 1
                _, slp = set_log_softmax(zz, 1.0, member, 1)
            else:
                member = (sets & 4).astype(_np.uint8)
                _, slp = set_log_softmax(zz, T32, member, 4)
            allids = _np.flatnonzero(member)
            n_sup = int(allids.shape[0])
            ids = allids[:support_cap]
            vals = slp[ids]
            sst = STATUS_OVERFLOW if n_sup > support_cap else STATUS_OK
            ssel = float("nan") if sel is None or not 0 <= sel < V else float(slp[sel])
        out.update(sup_ids=ids.astype(_np.int32), sup_vals=vals, sup_n=n_sup,
                   sup_len=int(ids.shape[0]), sup_status=sst, sup_sel=ssel)
    return out


# ------------------------------------------------------------ vocabulary shards

def race_best(z, in_set, *, T, m, seed, offset, v0, width, bit=4):
    """The race over the set's tokens in [v0, v0 + width), global ids: returns
    (token or -1, key)."""
    zz = _np.ascontiguousarray(z, dtype=_np.float32)
    st = _np.ascontiguousarray(in_set, _np.uint8)
    key = _np.zeros(1, _np.float64)
    t = _load().cdo_race_best(_ptr(zz), zz.shape[0], float(T), float(m), int(seed), int(offset),
                              int(v0), int(width), _ptr(st), int(bit), _ptr(key))
    return int(t), float(key[0])


# --------------------------------------------------------- speculative verify

def spec_accept(sampled, draft, status=None, eos=-1):
    """One request's k+1 sampled rows against its k drafts: returns
    (emitted tokens [count], count, rollback)."""
    sm = _np.ascontiguousarray(sampled, _np.int32)
    k = sm.shape[0] - 1
    dr = _np.ascontiguousarray(draft, _np.int32)
    assert dr.shape[0] == k
    st = None if status is None else _np.ascontiguousarray(status, _np.int32)
    tok = _np.empty(k + 1, _np.int32)
    rb = _np.zeros(1, _np.int32)
    n = _load().cdo_spec_accept(_ptr(sm), _ptr(st), k, _ptr(dr), int(eos), _ptr(tok), _ptr(rb))
    return tok[:n], int(n), int(rb[0])
