"""GPU test of sampler_sample_static, the entry point for callers that cannot
allocate: called through the C ABI, its output is checked bit for bit against
sampler_sample's (own workspace) on two calls in a row, the second with a
smaller batch, and a batch whose workspace need exceeds the library's array
is refused without a launch."""
import ctypes as ct

import numpy as np
import pytest

import workloads
from gpu_harness import pack, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import constrained_decoding_amd  # noqa: F401  (must load: no fallback)


def _static(pk, x, bitmask=None, rhm=None):
    import torch
    import constrained_decoding_amd as cds
    B = x.shape[0]
    ids = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    lp = torch.full((B,), 7.0, dtype=torch.float32, device="cuda")
    st = torch.full((B,), 7, dtype=torch.int32, device="cuda")
    rc = cds.lib.sampler_sample_static(
        ct.byref(pk.batch), x.data_ptr(), cds._binding._dtype_code(x), x.stride(0),
        None if bitmask is None else bitmask.data_ptr(),
        0 if bitmask is None else bitmask.stride(0),
        None if rhm is None else rhm.data_ptr(), ids.data_ptr(), lp.data_ptr(), st.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    return rc, (ids, lp, st)


def _own(pk, x, bitmask=None, rhm=None):
    import constrained_decoding_amd as cds
    return cds.sample(pk, x, bitmask=bitmask, row_has_mask=rhm)


def test_static_workspace_matches_own_workspace_two_calls():
    import torch
    cases = [workloads.c2_decode(salt=71),                       # B=192, V=151936
             workloads.c4_grammar(B=40, V=40001, salt=72)]       # smaller, bf16, masked
    for b in cases:
        print(f"[case] static workspace B={b.B} V={b.V}", flush=True)
        x = to_device(b)
        pk = pack(b)
        mask = None if b.masks is None else torch.from_numpy(b.masks).cuda()
        rhm = None if b.row_has_mask is None else torch.from_numpy(b.row_has_mask).cuda()
        rc, got = _static(pk, x, mask, rhm)
        assert rc == 0, rc
        ref = _own(pk, x, mask, rhm)
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            np.testing.assert_array_equal(g.cpu().numpy(), r.cpu().numpy())


def test_static_workspace_refuses_batches_beyond_its_size():
    import torch
    import constrained_decoding_amd as cds
    B, V = 2048, 151936
    T = np.full(B, 0.9, np.float32)
    pk = cds.PackedBatch(B, V, T, top_p=np.full(B, 0.9, np.float32))
    need = cds.lib.sampler_workspace_bytes_batch(ct.byref(pk.batch))
    assert need > (64 << 20)
    x = torch.zeros((B, V), dtype=torch.float32, device="cuda")   # full size: never read
    ids = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    rc = cds.lib.sampler_sample_static(ct.byref(pk.batch), x.data_ptr(), 0, V, None, 0, None,
                                       ids.data_ptr(), None, None,
                                       torch.cuda.current_stream().cuda_stream)
    assert rc == cds._binding.ENOSPC
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == -7).all()                         # nothing launched
