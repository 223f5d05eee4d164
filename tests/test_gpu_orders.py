"""GPU parity of the filter orders (min-p first, joint top-k/top-p, min-p
last; include/cd_sampler.h, sampler_host_params.filter_order) against the
oracle's cdo_sample_row_order, through the C ABI, fast and exact paths.
Sources: "SGLang 源码完全拆解(十)", sections 后端分支 and 概率裁剪的数学;
"GLM-5.3 推理全链路(七)", section 采样."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_harness import compare, record_parity, run_gpu, run_oracle, run_oracle_parallel

pytestmark = pytest.mark.gpu

ORDERS = [oracle.ORDER_MINP_FIRST, oracle.ORDER_JOINT, oracle.ORDER_MINP_LAST]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import constrained_decoding_amd  # noqa: F401  (must load: no fallback)


def _mixed(B, V, salt, order):
    """Decode-like rows where the order matters: top-p with top-k and/or
    min-p, at several temperatures (short and long candidate lists)."""
    b = workloads.c2_decode(B=B, V=V, salt=salt)
    rng = np.random.default_rng(600 + salt)
    b.temperature[:] = rng.uniform(0.4, 1.4, B).astype(np.float32)
    b.top_k[:] = rng.choice(np.array([0, 8, 20, 50, 300, 1000], np.int32), B)
    b.min_p[:] = rng.choice(np.array([0.0, 0.02, 0.1], np.float32), B)
    b.top_p[:] = rng.uniform(0.3, 0.95, B).astype(np.float32)
    b.order = order
    return b


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("order", ORDERS)
def test_orders_small(order, algo):
    b = _mixed(48, 20000, 61, order)
    print(f"[case] orders small order={order} algo={algo}", flush=True)
    gpu = run_gpu(b, algo=algo)
    ref, _ = run_oracle(b)
    record_parity(f"order{order}-small-algo{algo}", compare(b, gpu, ref, label=f"order{order}"))


@pytest.mark.parametrize("order", [oracle.ORDER_JOINT, oracle.ORDER_MINP_LAST])
def test_orders_full_size(order):
    b = _mixed(192, 151936, 62, order)
    print(f"[case] orders full order={order}", flush=True)
    gpu = run_gpu(b)
    ref = run_oracle_parallel(b)
    record_parity(f"order{order}-full", compare(b, gpu, ref, label=f"order{order}-full"))


def test_three_orders_three_sets():
    """The row the oracle pins cut three ways (kept sets {0}, {0, 1},
    {0, 1, 2}), padded to V = 4096 with masked tokens: every draw lies in its
    order's set and matches the oracle."""
    w = np.array([1.0, 0.45, 0.40, 0.34, 0.33] + [0.05] * 20)
    V, B = 4096, 64
    z = np.full((B, V), -np.inf, np.float32)
    z[:, :len(w)] = np.log(w).astype(np.float32)
    expect = {oracle.ORDER_MINP_FIRST: {0}, oracle.ORDER_MINP_LAST: {0, 1},
              oracle.ORDER_JOINT: {0, 1, 2}}
    for order in ORDERS:
        f = lambda v, dt=np.float32: np.full(B, v, dt)
        b = workloads.Batch("3sets", z.copy(), False, f(1.0), f(5, np.int32), f(0.5), f(0.35),
                            np.arange(B, dtype=np.uint64) + np.uint64(99),
                            np.arange(B, dtype=np.uint64), order=order)
        ids, lp, st = run_gpu(b)
        assert set(ids.tolist()) <= expect[order], (order, sorted(set(ids.tolist())))
        assert len(set(ids.tolist())) == len(expect[order])
        ref, _ = run_oracle(b)
        compare(b, (ids, lp, st), ref, label=f"3sets-order{order}")


@pytest.mark.parametrize("order", [oracle.ORDER_JOINT, oracle.ORDER_MINP_LAST])
def test_large_top_k_rows_in_other_orders(order):
    """Rows whose top-k is too large for candidate lists (their cut needs the
    row's histogram) with top-p on top, in the other orders: routed to the
    exact path, results match."""
    b = workloads.c2_decode(B=16, V=60000, salt=63)
    b.temperature[:] = np.linspace(0.6, 1.3, 16).astype(np.float32)
    b.top_k[:] = 20000
    b.top_p[:] = np.linspace(0.5, 0.95, 16).astype(np.float32)
    b.min_p[:] = np.array([0.0, 0.01] * 8, np.float32)
    b.order = order
    gpu = run_gpu(b)
    ref, _ = run_oracle(b)
    record_parity(f"order{order}-large-k", compare(b, gpu, ref, label="large-k"))
