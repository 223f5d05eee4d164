"""GPU parity of vocabulary-parallel sampling (sampler_shard_pass / merge)
with every shard on one device ("GLM-5.3 推理全链路(七)", sections 从最后一层
hidden 到 token id and 输出侧的通信与开销账本): the rows' results must equal
the oracle's on the whole row (ids bit-exact except oracle-flagged near-ties,
logprobs within 1e-5, statuses exact) and the exact path's on the gathered
logits (ids and statuses bit for bit).  Shards hold global token ids in the
race counter and their own slice of the bitmask."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_harness import compare, pack, record_parity, run_gpu, run_oracle_parallel, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import constrained_decoding_amd  # noqa: F401  (must load: no fallback)


def _mask_bits(masks, V):
    """[B, W] int32 words -> [B, V] bool."""
    w = masks.view(np.uint32)
    bits = (w[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(masks.shape[0], -1)[:, :V].astype(bool)


def _split(batch, bounds, x_full):
    """Shards of the (transformed) device logits and their own bitmasks."""
    import torch
    shards = []
    bits = None if batch.masks is None else _mask_bits(batch.masks, batch.V)
    for a, b in zip(bounds[:-1], bounds[1:]):
        xs = x_full[:, a:b].contiguous()
        m = None
        if bits is not None:
            sub = [np.flatnonzero(bits[r, a:b]) for r in range(batch.B)]
            m = torch.from_numpy(workloads.pack_bitmask(sub, b - a)).cuda()
        shards.append((xs, a, m))
    return shards


def _run_shards(batch, bounds, order=None):
    import torch
    import constrained_decoding_amd as cds
    x = to_device(batch)
    pk = pack(batch)
    if batch.rep is not None or batch.bias_indptr is not None:
        cds.apply_transforms(pk, x)
    shards = _split(batch, bounds, x)
    if order is not None:
        shards = [shards[i] for i in order]     # the merge breaks ties by global id
    rhm = None if batch.row_has_mask is None else \
        torch.from_numpy(batch.row_has_mask.astype(np.uint8)).cuda()
    ids, lp, st = cds.shard_sample(pk, shards, row_has_mask=rhm)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), lp.cpu().numpy(), st.cpu().numpy()


def _even(V, n):
    step = (V // n + 3) // 4 * 4
    return [min(i * step, V) for i in range(n)] + [V]


def _check(batch, bounds, label, order=None):
    print(f"[case] {label} B={batch.B} V={batch.V} shards={len(bounds) - 1}", flush=True)
    got = _run_shards(batch, bounds, order)
    ref = run_oracle_parallel(batch)
    record_parity(label, compare(batch, got, ref, label=label))
    ex = run_gpu(batch, algo=1)
    np.testing.assert_array_equal(got[0], ex[0])
    np.testing.assert_array_equal(got[2], ex[2])
    ok = np.isfinite(ex[1])
    assert np.max(np.abs(got[1][ok] - ex[1][ok]), initial=0.0) <= 1e-5


def test_shards_decode_tp8():
    """The decode batch (B=192, V=151936) as TP=8 ranks' [192, 18992] shards."""
    _check(workloads.c2_decode(salt=21), _even(151936, 8), "shards c2 TP8")


def test_shards_grammar_bf16_tp8():
    """bf16 with grammar masks split by shard (rows whose allowed tokens lie
    in one shard only, or in none)."""
    _check(workloads.c4_grammar(salt=22), _even(151936, 8), "shards c4 TP8")


def test_shards_penalties_tp4():
    """Penalties and bias applied to the full row before the split; TP=4."""
    _check(workloads.c3_penalties(salt=23), _even(151936, 4), "shards c3 TP4")


@pytest.mark.parametrize("order", [oracle.ORDER_JOINT, oracle.ORDER_MINP_LAST])
def test_shards_filter_orders_uneven(order):
    """Uneven shards (a ragged last one), every cut combination, both other
    filter orders; the shards handed over out of vocabulary order."""
    rng = np.random.default_rng(731 + order)
    B, V = 32, 20003
    z = workloads.decode_logits(rng, B, V)
    T = rng.choice(np.array([0.0, 0.4, 0.8, 1.2], np.float32), B)
    k = rng.choice(np.array([0, 1, 7, 40, 700], np.int32), B)
    p = rng.choice(np.array([1.0, 0.9, 0.6], np.float32), B)
    mp = rng.choice(np.array([0.0, 0.02, 0.2], np.float32), B)
    b = workloads.Batch("shards-orders", z, False, T, k, p, mp, workloads.seeds(rng, B),
                        np.arange(B, dtype=np.uint64), order=order)
    bounds = [0, 2400, 9600, 9604, 16000, V]
    _check(b, bounds, f"shards order {order}", order=[3, 0, 4, 2, 1])


def test_shards_edge_rows():
    """A row with one shard fully masked, a row whose only allowed tokens lie
    in one shard, a NaN in one shard (OVERFLOW), a row with nothing allowed
    (INVALID), tied maxima across shards (lowest global id), and one shard
    holding the whole row."""
    rng = np.random.default_rng(741)
    B, V = 8, 12000
    z = (rng.standard_normal((B, V)) * 2.0).astype(np.float32)
    z[3, 5003] = np.nan
    z[4, [100, 6000, 11999]] = 40.0                 # tied maxima in three shards
    allowed = [np.arange(V)] * B
    allowed = list(allowed)
    allowed[0] = np.arange(4000, V)                  # shard 0 fully masked
    allowed[1] = np.array([8001, 8007, 8100])        # one shard only
    allowed[2] = np.zeros(0, np.int64)               # nothing allowed
    masks = workloads.pack_bitmask(allowed, V)
    T = np.array([0.8, 1.0, 0.7, 0.9, 0.0, 1.1, 0.6, 1.3], np.float32)
    k = np.array([0, 2, 0, 0, 0, 30, 0, 500], np.int32)
    p = np.array([0.9, 1.0, 0.9, 0.8, 1.0, 0.95, 0.7, 1.0], np.float32)
    mp = np.array([0.0, 0.0, 0.0, 0.0, 0.0, 0.1, 0.0, 0.05], np.float32)
    b = workloads.Batch("shards-edge", z, False, T, k, p, mp, workloads.seeds(rng, B),
                        np.arange(B, dtype=np.uint64), masks=masks,
                        row_has_mask=np.ones(B, np.uint8))
    _check(b, [0, 4000, 8000, V], "shards edge")
    got = _run_shards(b, [0, V])
    ex = run_gpu(b, algo=1)
    np.testing.assert_array_equal(got[0], ex[0])
    assert got[2][2] == oracle.STATUS_INVALID and got[2][3] == oracle.STATUS_OVERFLOW
    assert got[0][4] == 100
