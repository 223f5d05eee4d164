"""Helpers shared by the GPU tests: run a workloads.Batch through the HIP path
(via the C ABI binding) and through the oracle, and compare them."""
import numpy as np

import oracle
import workloads


def to_device(batch: workloads.Batch):
    import torch
    if batch.bf16:
        t = torch.from_numpy(np.ascontiguousarray(batch.logits).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(batch.logits))
    return t.cuda()


def pack(batch: workloads.Batch, stream=None):
    import constrained_decoding_amd as cds
    kw = dict(top_k=batch.top_k, top_p=batch.top_p, min_p=batch.min_p, seed=batch.seed,
              offset=batch.offset, filter_order=batch.order)
    if batch.rep is not None:
        kw.update(repetition_penalty=batch.rep, frequency_penalty=batch.freq,
                  presence_penalty=batch.pres)
    if batch.hist_indptr is not None:
        kw.update(hist_indptr=batch.hist_indptr, hist_ids=batch.hist_ids)
    if batch.bias_indptr is not None:
        kw.update(bias_indptr=batch.bias_indptr, bias_ids=batch.bias_ids,
                  bias_vals=batch.bias_vals)
    return cds.PackedBatch(batch.B, batch.V, batch.temperature, stream=stream, **kw)


def run_gpu(batch: workloads.Batch, *, algo=0, fused_mask=True, logits=None, packed=None,
            workspace=None, return_logits=False, wait_ns=0):
    """Full step on the GPU: pack -> transforms -> (mask) -> sample."""
    import torch
    import constrained_decoding_amd as cds
    x = to_device(batch) if logits is None else logits
    pk = pack(batch) if packed is None else packed
    if batch.rep is not None or batch.bias_indptr is not None:
        cds.apply_transforms(pk, x)
    mask = rhm = None
    if batch.masks is not None:
        mask = torch.from_numpy(batch.masks).cuda()
        rhm = None if batch.row_has_mask is None else \
            torch.from_numpy(batch.row_has_mask.astype(np.uint8)).cuda()
        if not fused_mask:
            cds.apply_bitmask(x, mask, rhm)
            mask = rhm = None
    ids, lp, st = cds.sample(pk, x, bitmask=mask, row_has_mask=rhm, workspace=workspace,
                             algo=algo, wait_ns=wait_ns)
    torch.cuda.synchronize()
    out = (ids.cpu().numpy(), lp.cpu().numpy(), st.cpu().numpy())
    if return_logits:
        return out, x
    return out


def run_oracle(batch: workloads.Batch, rows=None):
    masks = batch.masks
    return oracle.pipeline(batch.logits, batch.oracle_params(), bf16=batch.bf16, masks=masks,
                           row_has_mask=batch.row_has_mask, rows=rows)


def run_oracle_parallel(batch: workloads.Batch, rows=None, workers=None):
    """run_oracle over row chunks in threads (the oracle's C calls release the
    GIL and share no state); the same records, in row order."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    rows = np.arange(batch.B) if rows is None else np.asarray(rows)
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = [c for c in np.array_split(rows, workers * 4) if len(c)]
    params = batch.oracle_params()
    oracle.sample_row(np.zeros(4, np.float32), T=1.0)   # load the library once
    def one(c):
        return oracle.pipeline(batch.logits, params, bf16=batch.bf16, masks=batch.masks,
                               row_has_mask=batch.row_has_mask, rows=c)[0]
    with ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(one, chunks))
    return np.concatenate(parts)


def record_parity(label, stats):
    """Print the parity counts of a case and, when CDS_PARITY_RECORD names a
    file, append them to it as one JSON line (the flagged fraction per case
    is part of the parity report)."""
    import json
    import os
    n, nf, nfm = stats
    line = {"case": label, "rows": int(n), "flagged": int(nf),
            "flagged_fraction": nf / max(n, 1), "flagged_mismatch": int(nfm)}
    print("[parity] " + json.dumps(line), flush=True)
    path = os.environ.get("CDS_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


def compare(batch, gpu, ref, rows=None, *, lp_tol=1e-5, label=""):
    """Element-wise comparison; returns (n_rows, n_flagged, n_flagged_mismatch).
    Raises AssertionError with a description of every unexplained row."""
    ids, lp, st = gpu
    rows = np.arange(batch.B) if rows is None else np.asarray(rows)
    bad = []
    n_flag = n_flag_mm = 0
    for k, r in enumerate(rows):
        o = ref[k]
        if st[r] != o["status"]:
            bad.append(f"row {r}: status gpu={st[r]} oracle={o['status']}")
            continue
        if o["status"] == oracle.STATUS_INVALID:
            if ids[r] != -1 or lp[r] != -np.inf:
                bad.append(f"row {r}: INVALID but id={ids[r]} lp={lp[r]}")
            continue
        if o["status"] == oracle.STATUS_OVERFLOW:
            if ids[r] != -1 or not np.isnan(lp[r]):
                bad.append(f"row {r}: OVERFLOW but id={ids[r]} lp={lp[r]}")
            continue
        flagged = bool(o["flags"] & oracle.F_EXCUSE)
        n_flag += flagged
        if ids[r] != o["id"]:
            if flagged:
                n_flag_mm += 1
                continue
            bad.append(f"row {r}: id gpu={ids[r]} oracle={o['id']} (T={batch.temperature[r]}, "
                       f"k={batch.top_k[r]}, p={batch.top_p[r]}, min_p={batch.min_p[r]}, "
                       f"n3={o['n3']}, flags={o['flags']}, keys={o['best_key']:.9f}/"
                       f"{o['second_key']:.9f})")
            continue
        # within lp_tol, or one fp32 spacing where that is coarser (|lp| >= 128)
        tol = max(lp_tol, float(np.spacing(np.float32(abs(o["logprob"])))))
        if not abs(float(lp[r]) - o["logprob"]) <= tol:
            bad.append(f"row {r}: logprob gpu={lp[r]!r} oracle={o['logprob']!r}")
    assert not bad, f"{label}: {len(bad)} unexplained rows:\n" + "\n".join(bad[:20])
    return len(rows), n_flag, n_flag_mm
