"""Benchmark of the sampling step on one MI355X.

One step = the whole hot path on one batch: sampler_pack_params (host
validation + flags + async H2D of the packed parameters), the transforms and
bitmask when the workload has them, and sampler_sample.  Default workload:
B=192, V=151936 fp32 decode batch (greedy on a quarter of the rows, top-k /
top-p / min-p mixes on the rest), seeded synthetic logits.  Three distinct
input sets rotate so the 117 MB working set of a step does not stay in the
256 MB Infinity Cache between steps.

Prints one JSON line: metric and value, a roofline object for
sample_kernel (algorithmic HBM bytes per launch over its HIP-event launch
time, against 8 TB/s) and a cpu_baseline object (the CPU oracle timed on a
bounded sample of the same workload).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled rows/sec and achieved HBM GB/s at B=192, V=151936 fp32 (1 GPU)"
PEAK_HBM_GBS = 8000.0
ROW_PARAM_BYTES = 64   # packed per-row record read by the scan kernel
ROW_OUT_BYTES = 12     # id + logprob + status written per row


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="c2", choices=["c2", "c3", "c4", "c5a", "c5b"])
    ap.add_argument("--sets", type=int, default=3, help="rotating input sets")
    ap.add_argument("--cpu-rows", type=int, default=2304,
                    help="rows of the workload the oracle is timed on (cpu_baseline)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--algo", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (the "
                         "reference point for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}), flush=True)


WORKLOAD_FILES = {"c2": "c2_decode", "c3": "c3_penalties", "c4": "c4_grammar",
                  "c5a": "c5a_spec_greedy", "c5b": "c5b_spec_topk"}


def kernel_sources_digest():
    import hashlib
    h = hashlib.sha256()
    for f in ("kernels.hip", "device_common.h", "layout.h"):
        with open(os.path.join(ROOT, "constrained_decoding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config):
    """HBM bytes per sample_kernel launch from the committed FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when that summary is missing
    or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{WORKLOAD_FILES[config]}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("sample_kernel ") and ":" in ln:
                k, v = ln.split(":", 1)
                fields[k.split()[1]] = v.strip()
    if fields.get("traffic_sources_sha256") != kernel_sources_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(batch):
    """Bytes the method must move once per step: one read of the logits, the
    mask words of masked rows, the penalised tokens' read+write plus their
    ids, the bias entries, per-row params and outputs."""
    elem = 2 if batch.bf16 else 4
    n = batch.B * batch.V * elem
    if batch.masks is not None:
        rows = batch.B if batch.row_has_mask is None else int(batch.row_has_mask.sum())
        n += rows * ((batch.V + 31) // 32) * 4
    if batch.hist_indptr is not None:
        n += int(batch.hist_indptr[-1]) * 4
        uniq = sum(len(np.unique(batch.hist(r))) for r in range(batch.B))
        n += uniq * 8
    if batch.bias_indptr is not None:
        n += int(batch.bias_indptr[-1]) * (8 + 8)
    n += batch.B * (ROW_PARAM_BYTES + ROW_OUT_BYTES)
    return n


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by rows or by vocabulary)", file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import constrained_decoding_amd as cds
    import workloads

    make = workloads.CONFIGS[args.config]
    sets = []
    for s in range(args.sets):
        if args.config in ("c5a", "c5b"):
            b = make()
            if s:
                b.seed = b.seed + np.uint64(s)
        else:
            b = make(salt=s)
        sets.append(b)
    b0 = sets[0]
    B, V = b0.B, b0.V

    def dev_logits(b):
        if b.bf16:
            return torch.from_numpy(np.ascontiguousarray(b.logits).view(np.int16)) \
                .view(torch.bfloat16).cuda()
        return torch.from_numpy(b.logits).cuda()

    work = [dev_logits(b) for b in sets]
    masks = [None if b.masks is None else torch.from_numpy(b.masks).cuda() for b in sets]
    rhm = [None if b.row_has_mask is None else torch.from_numpy(b.row_has_mask).cuda()
           for b in sets]
    transforms = b0.rep is not None or b0.bias_indptr is not None
    ws = cds.Workspace(B, V)
    outs = (torch.empty(B, dtype=torch.int32, device="cuda"),
            torch.empty(B, dtype=torch.float32, device="cuda"),
            torch.empty(B, dtype=torch.int32, device="cuda"))
    cds.set_algo(args.algo)

    host_kw = []
    for b in sets:
        kw = dict(top_k=b.top_k, top_p=b.top_p, min_p=b.min_p, seed=b.seed, offset=b.offset)
        if b.rep is not None:
            kw.update(repetition_penalty=b.rep, frequency_penalty=b.freq,
                      presence_penalty=b.pres, hist_indptr=b.hist_indptr, hist_ids=b.hist_ids)
        if b.bias_indptr is not None:
            kw.update(bias_indptr=b.bias_indptr, bias_ids=b.bias_ids, bias_vals=b.bias_vals)
        host_kw.append(kw)

    def step(i, ev=None):
        j = i % len(sets)
        b = sets[j]
        pk = cds.PackedBatch(B, V, b.temperature, **host_kw[j])
        if transforms:
            cds.apply_transforms(pk, work[j])
        if ev is not None:
            cds.time_next(0, ev[0], ev[1])
        cds.sample(pk, work[j], bitmask=masks[j], row_has_mask=rhm[j], workspace=ws, out=outs)
        return pk

    # The transforms write their (few hundred per row) tokens in place, so a
    # step re-applies them to the previous step's output: the same work, on
    # values that drift; no copy enters the timed region.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps, inputs resident in HBM
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    kern_ms = float(np.mean([a.elapsed_time(z) for a, z in evs]))

    alg = algorithmic_bytes(b0)
    scan_bytes = B * V * (2 if b0.bf16 else 4) + B * ROW_PARAM_BYTES
    if b0.masks is not None:
        rows = B if b0.row_has_mask is None else int(b0.row_has_mask.sum())
        scan_bytes += rows * ((V + 31) // 32) * 4
    achieved = scan_bytes / (kern_ms * 1e-3) / 1e9
    rows_per_s = B * args.steps / elapsed

    cpu = None
    if not args.no_cpu:
        import oracle
        n_rows = args.cpu_rows
        done = 0
        t0 = time.perf_counter()
        k = 0
        while done < n_rows:
            b = sets[k % len(sets)]
            take = min(B, n_rows - done)
            oracle.pipeline(b.logits, b.oracle_params(), bf16=b.bf16, masks=b.masks,
                            row_has_mask=b.row_has_mask, rows=range(take))
            done += take
            k += 1
        cpu_s = time.perf_counter() - t0
        cpu = {"value": round(done / cpu_s, 3), "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} rows ({k} steps' worth, rotating the {len(sets)} input sets) "
                         f"of the same workload, single-threaded, {cpu_s:.1f} s"}

    names = {"c2": "decode B=192 V=151936 fp32, mixed greedy/top-k/top-p/min-p",
             "c3": "penalties+bias B=192 V=151936 fp32, T=0.8 top_p=0.95",
             "c4": "grammar bitmask B=192 V=151936 bf16, 96 masked rows, T=0.7 top_p=0.9",
             "c5a": "spec-verify 64x8=512 rows V=151936 fp32, all greedy",
             "c5b": "spec-verify 64x8=512 rows V=151936 fp32, T=1 top_k=50"}
    line = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if b0.bf16 else "f32",
        "data": "synthetic (seeded; stands in for GLM-5.3 decode logits)",
        "config": {"workload": names[args.config], "B": B, "V": V, "input_sets": len(sets),
                   "algo": "fast" if args.algo == 0 else "row-exact"},
        "pipeline_gbs": round(alg / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "sample_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(args.config),
                     "kernel_us": round(kern_ms * 1e3, 2), "bytes_per_launch": scan_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
