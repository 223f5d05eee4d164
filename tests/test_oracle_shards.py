"""Pin of the property vocabulary-parallel sampling rests on ("GLM-5.3 推理全
链路(七)", section 输出侧的通信与开销账本: sampling on per-shard results
instead of a gather of the full logits): with global token ids in the
counter, the race's winner over the whole row is the best of the shards'
winners, for any split of the vocabulary.  Checked against the oracle's
full-row draw, and the shard race against a numpy restatement of the key.
CPU only."""
import numpy as np

import oracle
import workloads


def _splits(rng, V, n):
    cuts = np.sort(rng.choice(np.arange(4, V, 4), n - 1, replace=False))
    return [0, *cuts.tolist(), V]


def test_race_decomposes_over_shards():
    rng = workloads.rng_for(401)
    checked = 0
    for trial in range(120):
        V = int(rng.integers(40, 3000))
        z = (rng.standard_normal(V) * 2.0).astype(np.float32)
        if trial % 3 == 0:
            z[rng.random(V) < 0.3] = -np.inf
        if not np.isfinite(z).any():
            continue
        T = float(rng.choice([0.3, 0.8, 1.4]))
        k = int(rng.choice([0, 5, 50]))
        p = float(rng.choice([1.0, 0.9, 0.6]))
        mp = float(rng.choice([0.0, 0.05]))
        seed = int(rng.integers(0, 2**63))
        res, sets = oracle.sample_row(z, T=T, top_k=k, top_p=p, min_p=mp, seed=seed,
                                      offset=trial, want_sets=True)
        if res["greedy"]:
            continue
        bounds = _splits(rng, V, int(rng.integers(2, 9)))
        best = (-np.inf, -1)
        for a, b in zip(bounds[:-1], bounds[1:]):
            t, key = oracle.race_best(z, sets, T=T, m=res["m"], seed=seed, offset=trial,
                                      v0=a, width=b - a)
            if t >= 0 and (key > best[0] or (key == best[0] and t < best[1])):
                best = (key, t)
        assert best[1] == res["id"], (trial, best, res["id"])
        assert best[0] == res["best_key"]
        checked += 1
    assert checked > 60


def test_shard_race_key_restated_in_numpy():
    """The shard race's key is (z/T - m) - ln(-ln U) with U from the Philox
    bits of the global id; a numpy restatement over one shard agrees."""
    rng = workloads.rng_for(402)
    V = 2000
    z = (rng.standard_normal(V) * 2.0).astype(np.float32)
    allset = np.full(V, 4, np.uint8)
    for v0, w in ((0, 500), (500, 1000), (1500, 500)):
        t, key = oracle.race_best(z, allset, T=0.7, m=1.5, seed=77, offset=9, v0=v0, width=w)
        ts = np.arange(v0, v0 + w)
        x = np.array([oracle.race_bits(77, 9, int(tt)) for tt in ts], np.float64)
        u = (2.0 * np.floor(x / 512.0) + 1.0) * 2.0 ** -24
        keys = (z[ts].astype(np.float64) / np.float64(np.float32(0.7)) - 1.5) - np.log(-np.log(u))
        j = int(np.argmax(keys))
        assert t == v0 + j and abs(key - keys[j]) < 1e-12
