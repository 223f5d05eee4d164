"""Seeded synthetic workloads for the batched sampling step.

These generators are the only code shared by the oracle side (tests, bench
cpu_baseline) and the HIP side.  They hold none of the sampling method's
arithmetic: they draw logits, per-row parameters, token histories, bias
entries and grammar bitmasks, and pack them into the input layouts the
method consumes (row-major logits, CSR lists, int32 bitmask words with token
t at bit t&31 of word t>>5).

Workload recipes (stand-ins for GLM-5.3 decode logits at B=192,
V=151936 -- no model weights or datasets are used):

  C1 tiny        B=4, V=1024, fp32 N(0,3^2); rows {greedy; T=.7 p=.9;
                 T=1 k=20; T=1.2 min_p=.05}
  C2 decode      B=192, V=151936, fp32 N(0,2^2) plus +8 added to 5 distinct
                 random tokens per row; T=0 on exactly B/4 random rows, else
                 U[0.3,1.3]; top_p U[0.8,1]; top_k from {0,20,50,1000};
                 min_p from {0,0.05}
  C3 penalties   C2 logits; 512-token history per row, bounded Zipf(1.1) over
                 ranks 1..V mapped through a fixed seeded permutation;
                 rep 1.1, freq 0.5, pres 0.3; 16 distinct bias ids per row at
                 +-5; T=0.8, top_p=0.95
  C4 grammar     C2 fp32 draw rounded to bf16 (round-to-nearest-even); B/2
                 random rows carry a bitmask allowing a uniform random subset
                 of size from {1, 50, 5000, 60000}; T=0.7, top_p=0.9
  C5 spec-verify 64 requests x 8 draft positions = 512 rows of C2 logits;
                 parameters repeated per request, offset = position;
                 variant "a": all greedy; variant "b": T=1, top_k=50

Every function takes explicit sizes so tests can use the same recipe at
sizes the oracle finishes in seconds.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_BASE = 20261202 * 10


def rng_for(config_no: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(SEED_BASE + config_no + 7919 * salt))


@dataclass
class Batch:
    name: str
    logits: np.ndarray            # [B, V] float32, or uint16 bf16 bits
    bf16: bool
    temperature: np.ndarray       # [B] float32
    top_k: np.ndarray             # [B] int32 (<=0 or >=V: off)
    top_p: np.ndarray             # [B] float32 (1: off)
    min_p: np.ndarray             # [B] float32 (0: off)
    seed: np.ndarray              # [B] uint64
    offset: np.ndarray            # [B] uint64
    rep: Optional[np.ndarray] = None
    freq: Optional[np.ndarray] = None
    pres: Optional[np.ndarray] = None
    hist_indptr: Optional[np.ndarray] = None   # [B+1] int64
    hist_ids: Optional[np.ndarray] = None      # int32
    bias_indptr: Optional[np.ndarray] = None   # [B+1] int64
    bias_ids: Optional[np.ndarray] = None      # int32
    bias_vals: Optional[np.ndarray] = None     # float32
    masks: Optional[np.ndarray] = None         # [B, ceil(V/32)] int32
    row_has_mask: Optional[np.ndarray] = None  # [B] uint8
    meta: dict = field(default_factory=dict)
    order: int = 0                             # filter order (0: min-p first)

    @property
    def B(self) -> int:
        return self.logits.shape[0]

    @property
    def V(self) -> int:
        return self.logits.shape[1]

    def hist(self, r):
        if self.hist_indptr is None:
            return None
        return self.hist_ids[self.hist_indptr[r]:self.hist_indptr[r + 1]]

    def bias_pairs(self, r):
        if self.bias_indptr is None:
            return []
        lo, hi = self.bias_indptr[r], self.bias_indptr[r + 1]
        return list(zip(self.bias_ids[lo:hi].tolist(), self.bias_vals[lo:hi].tolist()))

    def oracle_params(self) -> dict:
        """Per-row parameters in the dict form ``oracle.pipeline`` takes."""
        p = dict(temperature=self.temperature, top_k=self.top_k, top_p=self.top_p,
                 min_p=self.min_p, seed=self.seed, offset=self.offset, order=self.order)
        if self.rep is not None:
            p.update(rep=self.rep, freq=self.freq, pres=self.pres)
        if self.hist_indptr is not None:
            p["hist"] = [self.hist(r) for r in range(self.B)]
        if self.bias_indptr is not None:
            p["bias"] = [self.bias_pairs(r) for r in range(self.B)]
        return p

    def subset(self, rows) -> "Batch":
        """The same requests, restricted to ``rows`` (in the given order)."""
        rows = np.asarray(rows)
        def take(a):
            return None if a is None else a[rows]
        def csr(indptr, *arrs):
            if indptr is None:
                return (None,) * (1 + len(arrs))
            lens = indptr[1:] - indptr[:-1]
            new_ptr = np.zeros(len(rows) + 1, np.int64)
            new_ptr[1:] = np.cumsum(lens[rows])
            outs = [np.concatenate([a[indptr[r]:indptr[r + 1]] for r in rows])
                    if len(rows) else a[:0] for a in arrs]
            return (new_ptr, *outs)
        hp, hi = csr(self.hist_indptr, self.hist_ids) if self.hist_indptr is not None \
            else (None, None)
        bp, bi, bv = csr(self.bias_indptr, self.bias_ids, self.bias_vals) \
            if self.bias_indptr is not None else (None, None, None)
        return Batch(self.name + "[subset]", self.logits[rows], self.bf16,
                     take(self.temperature), take(self.top_k), take(self.top_p),
                     take(self.min_p), take(self.seed), take(self.offset),
                     take(self.rep), take(self.freq), take(self.pres), hp, hi,
                     bp, bi, bv, take(self.masks), take(self.row_has_mask),
                     dict(self.meta), self.order)


# ---------------------------------------------------------------- pieces ---

def decode_logits(rng, B, V, sigma=2.0, n_spikes=5, spike=8.0):
    """N(0, sigma^2) fp32 logits with +spike added to n_spikes distinct tokens
    per row (adding, not setting, avoids artificial exact ties)."""
    z = rng.standard_normal((B, V), dtype=np.float32)
    z *= np.float32(sigma)
    for r in range(B):
        idx = rng.choice(V, size=min(n_spikes, V), replace=False)
        z[r, idx] += np.float32(spike)
    return z


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def seeds(rng, B):
    return rng.integers(0, 2**64, size=B, dtype=np.uint64)


def zipf_history(rng, B, V, n=512, a=1.1):
    """n ids per row: bounded Zipf(a) ranks 1..V via an inverse-CDF table,
    mapped to token ids by one fixed seeded permutation of [0, V)."""
    ranks = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-a))
    cdf /= cdf[-1]
    perm = rng.permutation(V).astype(np.int32)
    u = rng.random((B, n))
    r = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1)
    ids = perm[r].astype(np.int32)
    indptr = np.arange(0, (B + 1) * n, n, dtype=np.int64)
    return indptr, ids.reshape(-1)


def sparse_bias(rng, B, V, n=16, mag=5.0):
    ids = np.stack([rng.choice(V, size=min(n, V), replace=False) for _ in range(B)])
    signs = rng.choice(np.array([-1.0, 1.0], np.float32), size=ids.shape)
    vals = (signs * np.float32(mag)).astype(np.float32)
    n_eff = ids.shape[1]
    indptr = np.arange(0, (B + 1) * n_eff, n_eff, dtype=np.int64)
    return indptr, ids.reshape(-1).astype(np.int32), vals.reshape(-1)


def pack_bitmask(allowed_rows, V):
    """allowed_rows: list of int arrays (or None = unconstrained).  Returns
    [B, ceil(V/32)] int32 words, -1 for unconstrained rows."""
    W = (V + 31) // 32
    out = np.full((len(allowed_rows), W), -1, dtype=np.int32)
    for r, allowed in enumerate(allowed_rows):
        if allowed is None:
            continue
        bits = np.zeros(W * 32, dtype=np.uint8)
        bits[np.asarray(allowed, np.int64)] = 1
        words = np.packbits(bits.reshape(W, 32), axis=1, bitorder="little")
        out[r] = words.view("<u4").reshape(W).view(np.int32)
    return out


# --------------------------------------------------------------- configs ---

def c1_tiny(B=4, V=1024):
    rng = rng_for(1)
    z = (rng.standard_normal((B, V), dtype=np.float32) * np.float32(3.0))
    T = np.array([0.0, 0.7, 1.0, 1.2] * ((B + 3) // 4), np.float32)[:B]
    k = np.array([0, 0, 20, 0] * ((B + 3) // 4), np.int32)[:B]
    p = np.array([1.0, 0.9, 1.0, 1.0] * ((B + 3) // 4), np.float32)[:B]
    mp = np.array([0.0, 0.0, 0.0, 0.05] * ((B + 3) // 4), np.float32)[:B]
    return Batch("C1 tiny mixed", z, False, T, k, p, mp, seeds(rng, B),
                 np.zeros(B, np.uint64))


def c2_decode(B=192, V=151936, step=0, salt=0):
    rng = rng_for(2, salt)
    z = decode_logits(rng, B, V)
    T = rng.uniform(0.3, 1.3, size=B).astype(np.float32)
    T[rng.choice(B, size=B // 4, replace=False)] = 0.0
    p = rng.uniform(0.8, 1.0, size=B).astype(np.float32)
    k = rng.choice(np.array([0, 20, 50, 1000], np.int32), size=B)
    mp = rng.choice(np.array([0.0, 0.05], np.float32), size=B)
    return Batch("C2 decode", z, False, T, k, p, mp, seeds(rng, B),
                 np.full(B, step, np.uint64))


def c3_penalties(B=192, V=151936, n_hist=512, n_bias=16, salt=0):
    rng = rng_for(3, salt)
    z = decode_logits(rng, B, V)
    hp, hi = zipf_history(rng, B, V, n=n_hist)
    bp, bi, bv = sparse_bias(rng, B, V, n=n_bias)
    f = lambda v: np.full(B, v, np.float32)
    return Batch("C3 penalties+bias", z, False, f(0.8), np.zeros(B, np.int32),
                 f(0.95), f(0.0), seeds(rng, B), np.zeros(B, np.uint64),
                 rep=f(1.1), freq=f(0.5), pres=f(0.3), hist_indptr=hp,
                 hist_ids=hi, bias_indptr=bp, bias_ids=bi, bias_vals=bv)


def c4_grammar(B=192, V=151936, sizes=(1, 50, 5000, 60000), salt=0):
    rng = rng_for(4, salt)
    z = to_bf16_bits(decode_logits(rng, B, V))
    masked = np.zeros(B, np.uint8)
    masked[rng.choice(B, size=B // 2, replace=False)] = 1
    allowed = []
    sizes = [min(s, V) for s in sizes]
    for r in range(B):
        if masked[r]:
            n = int(rng.choice(sizes))
            allowed.append(rng.choice(V, size=n, replace=False))
        else:
            allowed.append(None)
    masks = pack_bitmask(allowed, V)
    f = lambda v: np.full(B, v, np.float32)
    return Batch("C4 grammar bf16", z, True, f(0.7), np.zeros(B, np.int32),
                 f(0.9), f(0.0), seeds(rng, B), np.zeros(B, np.uint64),
                 masks=masks, row_has_mask=masked,
                 meta={"allowed": allowed})


def c5_spec(variant="b", n_req=64, n_pos=8, V=151936):
    rng = rng_for(5)
    B = n_req * n_pos
    z = decode_logits(rng, B, V)
    req_seed = seeds(rng, n_req)
    seed = np.repeat(req_seed, n_pos)
    offset = np.tile(np.arange(n_pos, dtype=np.uint64), n_req)
    f = lambda v: np.full(B, v, np.float32)
    if variant == "a":
        T, k = f(0.0), np.zeros(B, np.int32)
    else:
        T, k = f(1.0), np.full(B, 50, np.int32)
    return Batch(f"C5{variant} spec-verify", z, False, T, k, f(1.0), f(0.0),
                 seed, offset)


def spec_drafts(batch, n_pos=8):
    """Draft tokens for a spec-verify batch (rows request-major, n_pos rows per
    request): draft token j+1 of a request is the most likely token of its row
    j (a draft model that agrees with the target's greedy choice), so greedy
    rows accept every draft and sampled rows accept while their draws hit the
    mode.  [n_req, n_pos - 1] int32."""
    z = batch.logits
    if batch.bf16:
        z = (z.astype(np.uint32) << 16).view(np.float32)
    am = np.argmax(z, axis=1).astype(np.int32).reshape(-1, n_pos)
    return np.ascontiguousarray(am[:, :n_pos - 1])


CONFIGS = {
    "c1": c1_tiny, "c2": c2_decode, "c3": c3_penalties, "c4": c4_grammar,
    "c5a": lambda **kw: c5_spec("a", **kw), "c5b": lambda **kw: c5_spec("b", **kw),
}


def input_set(name: str, s: int) -> Batch:
    """Input set s of a full-size workload, as the benchmark rotates them:
    another salt of the same recipe (C5: the same logits with every request
    seed shifted by s, as its recipe fixes the logits)."""
    if name in ("c5a", "c5b"):
        b = CONFIGS[name]()
        if s:
            b.seed = b.seed + np.uint64(s)
        return b
    return CONFIGS[name](salt=s)
