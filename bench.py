"""Benchmark of the sampling step on one MI355X.

One step = the whole hot path on one batch: sampler_pack_params (host
validation + flags + packing + async H2D of the parameter block, on a copy
stream so that it overlaps the previous step's kernels), the transforms
kernel when the workload has penalties or bias, and sampler_sample (the
fused sampling kernel, with the grammar bitmask fused into its loads when the
workload has one).  Default workload: B=192, V=151936 fp32 decode batch
(greedy on a quarter of the rows, top-k / top-p / min-p mixes on the rest),
seeded synthetic logits.  Three distinct input sets rotate so that the 117 MB
working set of a step does not stay in the 256 MB Infinity Cache between
steps.

Prints one JSON line: metric and value (rows/s over the whole timed region),
a roofline object for sample_kernel (algorithmic HBM bytes per launch over
its HIP-event launch time, taken on every eighth launch of the timed region,
against 8 TB/s; median, p10 and p90 of the timed launches; a warm figure from
steps that reuse one input set), the host time of a step and of its
parameter pack, and a
cpu_baseline object (the CPU oracle timed on a bounded sample of the same
workload on all host cores, with the single-thread figure beside it).
"""
import argparse
import ctypes as ct
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled rows/sec and achieved HBM GB/s at B=192, V=151936 fp32 (1 GPU)"
PEAK_HBM_GBS = 8000.0
ROW_PARAM_BYTES = 64   # packed per-row record read by the sampling kernel
ROW_OUT_BYTES = 12     # id + logprob + status written per row
MAX_CPU_WORKERS = 16   # host threads for the oracle baseline: one GPU's share of the host


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="c2", choices=["c2", "c3", "c4", "c5a", "c5b"])
    ap.add_argument("--sets", type=int, default=3, help="rotating input sets")
    ap.add_argument("--warm-steps", type=int, default=50,
                    help="extra steps on one input set (warm Infinity Cache figure)")
    ap.add_argument("--cpu-rows", type=int, default=2304,
                    help="rows of the workload the oracle is timed on (cpu_baseline)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--algo", type=int, default=0)
    ap.add_argument("--upload", choices=["auto", "side", "same"], default="auto",
                    help="parameter upload on a side stream (overlapping the previous "
                         "step) or on the compute stream; auto: the side stream for "
                         "blocks over 64 KB (measured: it pays for c3's 434 KB block, "
                         "and stalls the host for mid-size blocks such as c5's 41 KB)")
    ap.add_argument("--outputs", action="store_true",
                    help="time the further-outputs call (sampler_logprobs: top-20 and 4 "
                         "named-token logprobs per row, the support sets of every 12th "
                         "row) on the workload instead of the sampling step")
    ap.add_argument("--spec", action="store_true",
                    help="spec-verify workloads (c5a, c5b): add speculative verification "
                         "(sampler_spec_accept, drafts = each row's most likely token) to "
                         "the step and report emitted tokens/s")
    ap.add_argument("--shards", type=int, default=0, metavar="TP",
                    help="time vocabulary-parallel sampling (sampler_shard_pass / merge) "
                         "with the vocabulary split into TP shards, every shard on this GPU")
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


KERNEL_SOURCES = {
    "sample_kernel": ("kernels.hip", "exact_path.h", "device_common.h", "layout.h"),
    "outputs_kernel": ("outputs.hip", "exact_path.h", "device_common.h", "layout.h", "kernels.h"),
    "shard_pass_kernel": ("shard.hip", "exact_path.h", "device_common.h", "layout.h", "kernels.h"),
}


def kernel_sources_digest(kernel="sample_kernel"):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "constrained_decoding_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config, kernel="sample_kernel"):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when that summary is missing
    or was taken on different kernel sources."""
    name = WORKLOAD_FILES[config] + {"sample_kernel": "", "outputs_kernel": "_outputs",
                                     "shard_pass_kernel": "_shards"}[kernel]
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith(kernel + " ") and ":" in ln:
                k, v = ln.split(":", 1)
                fields[k.split()[1]] = v.strip()
    if fields.get("traffic_sources_sha256") != kernel_sources_digest(kernel):
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


WORKLOAD_NAMES = {
    "c2": "decode B=192 V=151936 fp32, mixed greedy/top-k/top-p/min-p",
    "c3": "penalties+bias B=192 V=151936 fp32, T=0.8 top_p=0.95",
    "c4": "grammar bitmask B=192 V=151936 bf16, 96 masked rows, T=0.7 top_p=0.9",
    "c5a": "spec-verify 64x8=512 rows V=151936 fp32, all greedy",
    "c5b": "spec-verify 64x8=512 rows V=151936 fp32, T=1 top_k=50"}

# the further-outputs request the --outputs leg times on every input set
OUT_TOP_N = 20           # top logprobs per row
OUT_NAMED = 4            # named tokens per row
OUT_MASK_EVERY = 12      # every 12th row returns its support set ...
OUT_MASK_CAP = 40000     # ... with room for this many tokens


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sets, n_rows):
    """The oracle as it stands on a bounded sample of the workload: rows taken
    in order from the rotating input sets, once on one thread and once spread
    over the host cores (threads: the oracle's C calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    B = sets[0].B
    work = []
    done = k = 0
    while done < n_rows:
        take = min(B, n_rows - done)
        work.append((k % len(sets), np.arange(take)))
        done += take
        k += 1
    params = [b.oracle_params() for b in sets]

    def run(j, rows):
        b = sets[j]
        oracle.pipeline(b.logits, params[j], bf16=b.bf16, masks=b.masks,
                        row_has_mask=b.row_has_mask, rows=rows)

    oracle.sample_row(np.zeros(4, np.float32), T=1.0)   # load the library first
    one_rows = max(1, n_rows // 4)                        # single thread: a quarter
    t0 = time.perf_counter()
    left = one_rows
    for j, rows in work:
        if left <= 0:
            break
        run(j, rows[:left])
        left -= len(rows)
    t1 = time.perf_counter() - t0
    workers = max(1, min(MAX_CPU_WORKERS, len(os.sched_getaffinity(0))))
    chunks = [(j, c) for j, rows in work for c in np.array_split(rows, workers) if len(c)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda jc: run(*jc), chunks))
    tn = time.perf_counter() - t0
    return {"value": round(done / tn, 3), "unit": "rows/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} rows ({k} steps' worth, rotating the {len(sets)} input sets) "
                      f"of the same workload, row-parallel over {workers} threads, "
                      f"{tn:.1f} s",
            "single_thread": {"value": round(one_rows / t1, 3), "unit": "rows/s", "cores": 1,
                              "sample": f"the first {one_rows} of those rows, {t1:.1f} s"}}


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

    if args.outputs:
        bench_outputs(args)
        return
    if args.shards:
        bench_shards(args)
        return

    import constrained_decoding_amd as cds
    from constrained_decoding_amd import _binding as bd
    import workloads

    sets = [workloads.input_set(args.config, s) for s in range(args.sets)]
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
    spec = None
    if args.spec:
        if args.config not in ("c5a", "c5b"):
            raise SystemExit("--spec needs a spec-verify workload (c5a or c5b)")
        n_pos = 8
        n_req = B // n_pos
        drafts = [torch.from_numpy(workloads.spec_drafts(b, n_pos)).cuda() for b in sets]
        spec = dict(n_req=n_req, k=n_pos - 1, drafts=drafts,
                    tokens=torch.empty((n_req, n_pos), dtype=torch.int32, device="cuda"),
                    count=torch.empty(n_req, dtype=torch.int32, device="cuda"),
                    rollback=torch.empty(n_req, dtype=torch.int32, device="cuda"),
                    ev=(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)),
                    emitted=[])

    # The host parameter arrays of each input set (what a serving loop hands
    # over each step), and a ring of parameter slots -- a device block, a
    # pinned staging buffer and their events -- deep enough that a slot's
    # previous step has long finished when it comes round again (a copy that
    # has to wait on unfinished kernels stalls the host inside the enqueue).
    host = []
    for b in sets:
        kw = dict(top_k=b.top_k, top_p=b.top_p, min_p=b.min_p, seed=b.seed, offset=b.offset)
        if b.rep is not None:
            kw.update(repetition_penalty=b.rep, frequency_penalty=b.freq,
                      presence_penalty=b.pres, hist_indptr=b.hist_indptr, hist_ids=b.hist_ids)
        if b.bias_indptr is not None:
            kw.update(bias_indptr=b.bias_indptr, bias_ids=b.bias_ids, bias_vals=b.bias_vals)
        host.append(bd._HostArrays(B, V, b.temperature, **kw))
    nbytes = max(h.bytes_bound() for h in host)
    if args.upload == "auto":
        args.upload = "side" if nbytes > (64 << 10) else "same"
    # (events are made once per slot and recorded again each time round: the
    # step allocates nothing)
    ring = [dict(d_buf=torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
                 staging=torch.empty(nbytes, dtype=torch.uint8, pin_memory=True),
                 batch=bd.Batch(), copied=torch.cuda.Event(), used=torch.cuda.Event(),
                 fresh=True) for _ in range(8)]
    compute = torch.cuda.current_stream()
    copy_s = torch.cuda.Stream() if args.upload == "side" else compute
    lib = bd.lib
    mask_args = [(None, 0, None) if masks[j] is None else
                 (masks[j].data_ptr(), masks[j].stride(0),
                  None if rhm[j] is None else rhm[j].data_ptr()) for j in range(len(sets))]
    dtype = cds.DTYPE_BF16 if b0.bf16 else cds.DTYPE_F32
    out_ptrs = tuple(t.data_ptr() for t in outs)
    pack_s, step_s = [], []
    # everything a step passes through ctypes, made once
    host_refs = [ct.byref(h.hp) for h in host]
    work_args = [(w.data_ptr(), w.stride(0)) for w in work]
    copy_h, compute_h = copy_s.cuda_stream, compute.cuda_stream
    opts = bd.Options(size=ct.sizeof(bd.Options), algo=args.algo)
    opts_ref = ct.byref(opts)
    for hs in ring:
        hs.update(batch_ref=ct.byref(hs["batch"]), d_ptr=hs["d_buf"].data_ptr(),
                  s_ptr=hs["staging"].data_ptr())

    def step(i, ev=None, j=None):
        t_in = time.perf_counter()
        j = i % len(sets) if j is None else j
        hs = ring[i % len(ring)]
        # the staging buffer and the device block are reused: the previous copy
        # out of the staging buffer must have run, and the previous kernels that
        # read the device block must be done before the copy overwrites it
        if not hs["fresh"]:
            hs["copied"].synchronize()
            if copy_s is not compute:
                copy_s.wait_event(hs["used"])
        hs["fresh"] = False
        t0 = time.perf_counter()
        rc = lib.sampler_pack_params(host_refs[j], hs["d_ptr"], nbytes, hs["s_ptr"], copy_h,
                                     hs["batch_ref"])
        pack_s.append(time.perf_counter() - t0)
        if rc != 0:
            raise cds.SamplerError(rc, "sampler_pack_params")
        hs["copied"].record(copy_s)
        if copy_s is not compute:
            compute.wait_event(hs["copied"])
        wp, wld = work_args[j]
        if transforms:
            rc = lib.sampler_apply_transforms(hs["batch_ref"], wp, wld, compute_h)
            if rc != 0:
                raise cds.SamplerError(rc, "sampler_apply_transforms")
        mp, mld, rp = mask_args[j]
        if ev is not None:
            opts.start_event, opts.stop_event = ev[0].cuda_event, ev[1].cuda_event
        else:
            opts.start_event = opts.stop_event = None
        rc = lib.sampler_sample_ex(hs["batch_ref"], wp, dtype, wld, mp, mld, rp, *out_ptrs,
                                   ws.ptr, ws.nbytes, compute_h, opts_ref)
        if rc != 0:
            raise cds.SamplerError(rc, "sampler_sample_ex")
        if spec is not None:
            rc = lib.sampler_spec_accept(spec["n_req"], spec["k"], out_ptrs[0], out_ptrs[2],
                                         spec["drafts"][j].data_ptr(), None,
                                         spec["tokens"].data_ptr(), spec["count"].data_ptr(),
                                         spec["rollback"].data_ptr(), compute_h)
            if rc != 0:
                raise cds.SamplerError(rc, "sampler_spec_accept")
        hs["used"].record(compute)
        step_s.append(time.perf_counter() - t_in)

    # The transforms write their (few hundred per row) tokens in place, so a
    # step re-applies them to the previous step's output: the same work, on
    # values that drift; no copy enters the timed region.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if spec is not None:
        # tokens each input set emits (the draws are deterministic), and the
        # verification kernel's own time
        for j in range(len(sets)):
            step(j, j=j)
            torch.cuda.synchronize()
            spec["emitted"].append(int(spec["count"].sum().item()))
        acc = []
        for _ in range(20):
            spec["ev"][0].record()
            rc = lib.sampler_spec_accept(spec["n_req"], spec["k"], out_ptrs[0], out_ptrs[2],
                                         spec["drafts"][0].data_ptr(), None,
                                         spec["tokens"].data_ptr(), spec["count"].data_ptr(),
                                         spec["rollback"].data_ptr(), compute_h)
            spec["ev"][1].record()
            torch.cuda.synchronize()
            acc.append(spec["ev"][0].elapsed_time(spec["ev"][1]) * 1e3)
        spec["accept_us"] = float(np.median(acc))
    pack_s.clear()
    step_s.clear()

    # timed region: K whole steps, inputs resident in HBM.  The kernel's own
    # time comes from HIP events the library records right around the launch,
    # on every TIME_EVERY-th step of the region: a timing event pair costs the
    # step ~10 us of queue time on this runtime, which timing every launch
    # would add to the step rate it measures.
    TIME_EVERY = 8
    timed = list(range(0, args.steps, TIME_EVERY))
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in timed}
    for e in evs.values():             # create the HIP events outside the timed region
        e[0].record()
        e[1].record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    kern = np.array([a.elapsed_time(z) for a, z in evs.values()]) * 1e3   # us
    host_pack_us = float(np.mean(pack_s)) * 1e6
    host_step_us = float(np.mean(step_s)) * 1e6

    # warm figure: the same input set every step (its 117 MB can stay in the
    # Infinity Cache); reported beside, never as the value
    warm = None
    if args.warm_steps > 0:
        wevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.warm_steps)]
        for e in wevs:
            e[0].record()
            e[1].record()
        torch.cuda.synchronize()
        for i in range(args.warm_steps):
            step(i, wevs[i], j=0)
        torch.cuda.synchronize()
        warm = float(np.median([a.elapsed_time(z) for a, z in wevs])) * 1e3

    alg = algorithmic_bytes(b0)
    scan_bytes = B * V * (2 if b0.bf16 else 4) + B * ROW_PARAM_BYTES
    if b0.masks is not None:
        rows = B if b0.row_has_mask is None else int(b0.row_has_mask.sum())
        scan_bytes += rows * ((V + 31) // 32) * 4
    kern_mean = float(np.mean(kern))
    achieved = scan_bytes / (kern_mean * 1e-6) / 1e9
    rows_per_s = B * args.steps / elapsed

    cpu = None if args.no_cpu else cpu_baseline(sets, args.cpu_rows)

    names = WORKLOAD_NAMES
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
        "host_pack_us": round(host_pack_us, 2),
        "host_step_us": round(host_step_us, 2),
        "param_upload": args.upload,
        "roofline": {"bound": "hbm", "kernel": "sample_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(args.config),
                     "kernel_us": round(kern_mean, 2),
                     "kernel_launches_timed": len(kern),
                     "kernel_us_p10_p50_p90": [round(float(np.percentile(kern, q)), 2)
                                               for q in (10, 50, 90)],
                     "kernel_us_warm_p50": None if warm is None else round(warm, 2),
                     "bytes_per_launch": scan_bytes},
        "cpu_baseline": cpu,
    }
    if spec is not None:
        emitted = float(np.mean([spec["emitted"][i % len(sets)] for i in range(args.steps)]))
        line["metric"] = (f"emitted tokens/sec of the spec-verify step ({spec['n_req']} requests x "
                          f"{spec['k'] + 1} rows, V={V}, 1 GPU)")
        line["value"] = round(emitted * args.steps / elapsed, 1)
        line["unit"] = "tokens/s"
        line["config"]["workload"] += "; speculative verification, drafts = rows' modes"
        line["spec"] = {"requests": spec["n_req"], "drafts_per_request": spec["k"],
                        "emitted_per_step": emitted,
                        "emitted_per_set": spec["emitted"],
                        "rows_per_s": round(rows_per_s, 1),
                        "accept_kernel_us": round(spec["accept_us"], 2)}
    print(json.dumps(line), flush=True)


def bench_outputs(args):
    """The further-outputs call (sampler_logprobs) on the workload, two
    requests timed apart: every row asks for its top-20 logprobs, the
    logprobs of 4 named tokens and the chosen token's logprob (the value and
    the roofline); every 12th row returns its support set with room for 40000
    tokens, from the thresholds the sampling call returned (the "support"
    object).  The sampling step runs once per input set before the timed
    region (its ids are the chosen tokens, its thresholds the support sets').  One JSON line in
    the form of the sampling step's, for outputs_kernel."""
    import torch

    import constrained_decoding_amd as cds
    from constrained_decoding_amd import _binding as bd
    import workloads

    sets = [workloads.input_set(args.config, s) for s in range(args.sets)]
    b0 = sets[0]
    B, V = b0.B, b0.V
    rng = np.random.default_rng(20261202)
    named = [[rng.integers(0, V, OUT_NAMED) for _ in range(B)] for _ in sets]
    mask_rows = np.arange(0, B, OUT_MASK_EVERY, dtype=np.int32)
    R = len(mask_rows)
    d_mask_rows = torch.from_numpy(mask_rows).cuda()
    top_n = torch.full((B,), OUT_TOP_N, dtype=torch.int32, device="cuda")
    # outputs, shared by the input sets
    o_next = torch.empty(B, dtype=torch.float32, device="cuda")
    o_tidx = torch.empty((B, OUT_TOP_N), dtype=torch.int32, device="cuda")
    o_tval = torch.empty((B, OUT_TOP_N), dtype=torch.float32, device="cuda")
    o_tok = torch.empty(B * OUT_NAMED, dtype=torch.float32, device="cuda")
    o_mids = torch.empty((R, OUT_MASK_CAP), dtype=torch.int32, device="cuda")
    o_mlp = torch.empty((R, OUT_MASK_CAP), dtype=torch.float32, device="cuda")
    o_mlen = torch.empty(R, dtype=torch.int32, device="cuda")
    o_msel = torch.empty(R, dtype=torch.float32, device="cuda")
    o_mst = torch.empty(R, dtype=torch.int32, device="cuda")
    out_rows = bd.LogprobOutputs(
        size=ct.sizeof(bd.LogprobOutputs), next_token_logprobs=o_next.data_ptr(),
        top_logprobs_idx=o_tidx.data_ptr(), top_logprobs_val=o_tval.data_ptr(),
        token_ids_logprobs=o_tok.data_ptr())
    out_sup = bd.LogprobOutputs(
        size=ct.sizeof(bd.LogprobOutputs), mask_token_ids=o_mids.data_ptr(),
        mask_support_logprobs=o_mlp.data_ptr(), mask_lengths=o_mlen.data_ptr(),
        mask_selected_logprobs=o_msel.data_ptr(), mask_statuses=o_mst.data_ptr())
    ws_need = int(bd.lib.sampler_logprobs_workspace_bytes(B, V, OUT_TOP_N, R))
    ws_buf = torch.empty(ws_need + 256, dtype=torch.uint8, device="cuda")
    ws_ptr = ws_buf.data_ptr() + (-ws_buf.data_ptr()) % 256
    keep, calls = [], {"rows": [], "support": []}
    for j, b in enumerate(sets):
        if b.bf16:
            x = torch.from_numpy(np.ascontiguousarray(b.logits).view(np.int16)) \
                .view(torch.bfloat16).cuda()
        else:
            x = torch.from_numpy(b.logits).cuda()
        kw = dict(top_k=b.top_k, top_p=b.top_p, min_p=b.min_p, seed=b.seed, offset=b.offset)
        if b.rep is not None:
            kw.update(repetition_penalty=b.rep, frequency_penalty=b.freq,
                      presence_penalty=b.pres, hist_indptr=b.hist_indptr, hist_ids=b.hist_ids)
        if b.bias_indptr is not None:
            kw.update(bias_indptr=b.bias_indptr, bias_ids=b.bias_ids, bias_vals=b.bias_vals)
        pk = cds.PackedBatch(B, V, b.temperature, **kw)
        if b.rep is not None or b.bias_indptr is not None:
            cds.apply_transforms(pk, x)
        m = None if b.masks is None else torch.from_numpy(b.masks).cuda()
        rh = None if b.row_has_mask is None else torch.from_numpy(b.row_has_mask).cuda()
        cut = torch.empty(B, dtype=torch.float32, device="cuda")
        ids, _, _ = cds.sample(pk, x, bitmask=m, row_has_mask=rh, cut=cut)
        indptr, flat = cds.csr(named[j])
        d_ind = torch.from_numpy(indptr).cuda()
        d_tok = torch.from_numpy(flat.astype(np.int32)).cuda()
        req_rows = bd.LogprobRequest(size=ct.sizeof(bd.LogprobRequest), basis=cds.LOGPROB_SAMPLED,
                                     selected=ids.data_ptr(), top_n_max=OUT_TOP_N,
                                     top_n=top_n.data_ptr(), token_indptr=d_ind.data_ptr(),
                                     token_ids=d_tok.data_ptr(), workspace=ws_ptr,
                                     workspace_bytes=ws_need)
        req_sup = bd.LogprobRequest(size=ct.sizeof(bd.LogprobRequest), basis=cds.LOGPROB_SAMPLED,
                                    selected=ids.data_ptr(), n_mask_rows=R,
                                    mask_rows=d_mask_rows.data_ptr(), mask_cap=OUT_MASK_CAP,
                                    cuts=cut.data_ptr(), workspace=ws_ptr,
                                    workspace_bytes=ws_need)
        keep.append((x, pk, m, rh, ids, cut, d_ind, d_tok, req_rows, req_sup))
        base = (ct.byref(pk.batch), x.data_ptr(), x.stride(0),
                None if m is None else m.data_ptr(), 0 if m is None else m.stride(0),
                None if rh is None else rh.data_ptr())
        calls["rows"].append(base + (ct.byref(req_rows), ct.byref(out_rows)))
        calls["support"].append(base + (ct.byref(req_sup), ct.byref(out_sup)))
    dtype = cds.DTYPE_BF16 if b0.bf16 else cds.DTYPE_F32
    compute_h = torch.cuda.current_stream().cuda_stream
    lib = bd.lib

    def launch(kind, j):
        br, xp, ld, mp, mld, rp, rq, oq = calls[kind][j]
        rc = lib.sampler_logprobs(br, xp, dtype, ld, mp, mld, rp, rq, oq, compute_h)
        if rc != 0:
            raise cds.SamplerError(rc, "sampler_logprobs")

    # support entries written per launch (for the algorithmic bytes)
    sup_entries = []
    for j in range(len(sets)):
        launch("support", j)
        torch.cuda.synchronize()
        sup_entries.append(int(o_mlen.sum().item()))

    def timed(kind):
        for i in range(args.warmup):
            launch(kind, i % len(sets))
        torch.cuda.synchronize()
        every = 4
        evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for i in range(0, args.steps, every)}
        for e in evs.values():
            e[0].record()
            e[1].record()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev = evs.get(i)
            if ev:
                ev[0].record()
            launch(kind, i % len(sets))
            if ev:
                ev[1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        kern = np.array([a.elapsed_time(z) for a, z in evs.values()]) * 1e3   # us
        return elapsed, kern

    elapsed, kern = timed("rows")
    s_elapsed, s_kern = timed("support")

    elem = 2 if b0.bf16 else 4
    mwords = (V + 31) // 32 * 4
    mrows = 0 if b0.masks is None else (B if b0.row_has_mask is None else int(b0.row_has_mask.sum()))
    # per-row request: each row read once, its params, chosen id, named ids
    # and offsets in; chosen, top-N (id + value) and named logprobs out
    alg = B * V * elem + mrows * mwords + B * (ROW_PARAM_BYTES + 4) + B * OUT_NAMED * 4 + \
        (B + 1) * 8 + B * 4 + B * OUT_TOP_N * 8 + B * OUT_NAMED * 4
    # support request: each support row read once; ids and logprobs of the
    # support entries plus length, status and selected logprob out
    sup_mrows = 0 if b0.masks is None else int(
        (np.ones(B, bool) if b0.row_has_mask is None else b0.row_has_mask.astype(bool))[mask_rows].sum())
    s_alg = R * V * elem + sup_mrows * mwords + R * (ROW_PARAM_BYTES + 8) + R * 12 + \
        int(np.mean(sup_entries)) * 8
    kern_mean, s_mean = float(np.mean(kern)), float(np.mean(s_kern))
    achieved = alg / (kern_mean * 1e-6) / 1e9
    s_achieved = s_alg / (s_mean * 1e-6) / 1e9

    cpu = None if args.no_cpu else cpu_baseline_outputs(sets, named, args.cpu_rows // 4)
    line = {
        "metric": "rows/sec with further outputs (top-20 and 4 named-token logprobs and the "
                  "chosen token's logprob per row) at B=192, V=151936 (1 GPU)",
        "value": round(B * args.steps / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if b0.bf16 else "f32",
        "data": "synthetic (seeded; stands in for GLM-5.3 decode logits)",
        "config": {"workload": WORKLOAD_NAMES[args.config] + "; further outputs",
                   "B": B, "V": V, "input_sets": len(sets), "top_n": OUT_TOP_N,
                   "named_tokens_per_row": OUT_NAMED},
        "roofline": {"bound": "hbm", "kernel": "outputs_slice_kernel+outputs_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(args.config, "outputs_kernel"),
                     "kernel_us": round(kern_mean, 2),
                     "kernel_launches_timed": len(kern),
                     "kernel_us_p10_p50_p90": [round(float(np.percentile(kern, q)), 2)
                                               for q in (10, 50, 90)],
                     "bytes_per_launch": alg},
        "support": {"rows": R, "cap": OUT_MASK_CAP, "kernel_us": round(s_mean, 2),
                    "kernel_us_p10_p50_p90": [round(float(np.percentile(s_kern, q)), 2)
                                              for q in (10, 50, 90)],
                    "entries_per_launch": int(np.mean(sup_entries)),
                    "bytes_per_launch": s_alg, "achieved": round(s_achieved, 1),
                    "frac": round(s_achieved / PEAK_HBM_GBS, 4),
                    "rows_per_s": round(R * args.steps / s_elapsed, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_outputs(sets, named, n_rows):
    """The oracle's per-row further outputs (top-20, named tokens, chosen
    token) on a bounded sample of rows (in order, rotating the input sets),
    row-parallel over the host cores."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    B = sets[0].B
    work = []
    k = 0
    while len(work) < n_rows:
        j = k % len(sets)
        for r in range(min(B, n_rows - len(work))):
            work.append((j, r))
        k += 1
    params = [b.oracle_params() for b in sets]

    def one(jr):
        j, r = jr
        b, pr = sets[j], params[j]
        hist = pr.get("hist")
        bias = pr.get("bias")
        mk = None
        if b.masks is not None and (b.row_has_mask is None or b.row_has_mask[r]):
            mk = b.masks[r]
        z = oracle.transform_row(
            b.logits[r], hist_ids=None if hist is None or hist[r] is None or not len(hist[r])
            else np.asarray(hist[r], np.int32),
            rep=float(pr["rep"][r]) if "rep" in pr else 1.0,
            freq=float(pr["freq"][r]) if "freq" in pr else 0.0,
            pres=float(pr["pres"][r]) if "pres" in pr else 0.0,
            bias_ids=np.asarray([q[0] for q in bias[r]], np.int32) if bias and bias[r] else None,
            bias_vals=np.asarray([q[1] for q in bias[r]], np.float32) if bias and bias[r] else None,
            mask=mk, bf16=b.bf16)
        oracle.row_outputs(z, T=float(b.temperature[r]), top_k=int(b.top_k[r]),
                           top_p=float(b.top_p[r]), min_p=float(b.min_p[r]),
                           seed=int(b.seed[r]), offset=int(b.offset[r]), order=b.order,
                           n_top=OUT_TOP_N, token_ids=named[j][r], selected=0)

    oracle.sample_row(np.zeros(4, np.float32), T=1.0)   # load the library first
    workers = max(1, min(MAX_CPU_WORKERS, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, work))
    tn = time.perf_counter() - t0
    return {"value": round(len(work) / tn, 3), "unit": "rows/s", "cores": workers,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"transforms and further outputs of {len(work)} rows of the same "
                      f"workload (rotating the {len(sets)} input sets), row-parallel over "
                      f"{workers} threads, {tn:.1f} s"}


SHARD_PHASE_NAMES = ["stats", "top-k 1", "top-k 2", "top-k 3", "top-k 4", "top-p sums",
                     "top-p 1", "top-p 2", "top-p 3", "top-p 4", "race"]
SHARD_RECORD_BYTES = {"stats": 24, "top-p sums": 16, "race": 16}   # per row; histograms 2048


def bench_shards(args):
    """Vocabulary-parallel sampling on the workload with the vocabulary split
    into TP shards (multiples of 4 tokens) and every shard on this GPU: each
    step runs the phases the batch needs, each phase a pass over every shard
    and one merge.  HIP events around each whole step (the value) and around
    the stats phase's TP passes (the roofline: one pass over one shard).  A
    rank's own share (one shard's passes and the merges) is read from a
    kernel trace."""
    import torch

    import constrained_decoding_amd as cds
    from constrained_decoding_amd import _binding as bd
    import workloads

    TP = args.shards
    sets = [workloads.input_set(args.config, s) for s in range(args.sets)]
    b0 = sets[0]
    B, V = b0.B, b0.V
    step_w = (V // TP + 3) // 4 * 4
    bounds = [min(i * step_w, V) for i in range(TP)] + [V]
    prep = []
    for b in sets:
        if b.bf16:
            x = torch.from_numpy(np.ascontiguousarray(b.logits).view(np.int16)) \
                .view(torch.bfloat16).cuda()
        else:
            x = torch.from_numpy(b.logits).cuda()
        kw = dict(top_k=b.top_k, top_p=b.top_p, min_p=b.min_p, seed=b.seed, offset=b.offset,
                  filter_order=b.order)
        if b.rep is not None:
            kw.update(repetition_penalty=b.rep, frequency_penalty=b.freq,
                      presence_penalty=b.pres, hist_indptr=b.hist_indptr, hist_ids=b.hist_ids)
        if b.bias_indptr is not None:
            kw.update(bias_indptr=b.bias_indptr, bias_ids=b.bias_ids, bias_vals=b.bias_vals)
        pk = cds.PackedBatch(B, V, b.temperature, **kw)
        if b.rep is not None or b.bias_indptr is not None:
            cds.apply_transforms(pk, x)
        bits = None
        if b.masks is not None:
            w = b.masks.view(np.uint32)
            bits = ((w[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1) \
                .reshape(B, -1)[:, :V].astype(bool)
        shards = []
        for a0, a1 in zip(bounds[:-1], bounds[1:]):
            m = None
            if bits is not None:
                m = torch.from_numpy(workloads.pack_bitmask(
                    [np.flatnonzero(bits[r, a0:a1]) for r in range(B)], a1 - a0)).cuda()
            shards.append((x[:, a0:a1].contiguous(), a0, m))
        rhm = None if b.row_has_mask is None else torch.from_numpy(b.row_has_mask).cuda()
        prep.append((pk, shards, rhm))
        del x
    bufs = bd.ShardBuffers(B, [a1 - a0 for a0, a1 in zip(bounds[:-1], bounds[1:])])
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    lp = torch.empty(B, dtype=torch.float32, device="cuda")
    st = torch.empty(B, dtype=torch.int32, device="cuda")
    lib = bd.lib
    sp = torch.cuda.current_stream().cuda_stream
    phases = [int(lib.sampler_shard_phases(ct.byref(p[0].batch))) for p in prep]
    run = [ph for ph in range(bd.SHARD_PHASES) if (phases[0] >> ph) & 1]
    calls = []
    for pk, shards, rhm in prep:
        br = ct.byref(pk.batch)
        per = []
        for ph in run:
            passes = [(br, ph, xs.data_ptr(), cds.DTYPE_BF16 if b0.bf16 else cds.DTYPE_F32,
                       xs.stride(0), v0, xs.shape[1], None if m is None else m.data_ptr(),
                       0 if m is None else m.stride(0), None if rhm is None else rhm.data_ptr(),
                       bufs.state, bufs.offsets[p], sp)
                      for p, (xs, v0, m) in enumerate(shards)]
            merge = (br, ph, bufs.state, bufs.parts, bufs.n_records, ids.data_ptr(),
                     lp.data_ptr(), st.data_ptr(), sp)
            per.append((passes, merge))
        calls.append(per)

    def step(j, ev_step=None, ev_stats=None):
        if ev_step is not None:
            ev_step[0].record()
        for k, (passes, merge) in enumerate(calls[j]):
            if k == 0 and ev_stats is not None:
                ev_stats[0].record()
            for c in passes:
                rc = lib.sampler_shard_pass(*c)
                if rc != 0:
                    raise cds.SamplerError(rc, "sampler_shard_pass")
            if k == 0 and ev_stats is not None:
                ev_stats[1].record()
            rc = lib.sampler_shard_merge(*merge)
            if rc != 0:
                raise cds.SamplerError(rc, "sampler_shard_merge")
        if ev_step is not None:
            ev_step[1].record()

    for i in range(args.warmup):
        step(i % len(sets))
    torch.cuda.synchronize()
    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    evs = [(mk(), mk()) for _ in range(args.steps)]
    for a, z in evs:                   # create the HIP events outside the timed region
        for e in (*a, *z):
            e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % len(sets), *evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_us = np.array([a[0].elapsed_time(a[1]) for a, _ in evs]) * 1e3
    stats_us = np.array([z[0].elapsed_time(z[1]) for _, z in evs]) * 1e3 / TP
    elem = 2 if b0.bf16 else 4
    width = bounds[1] - bounds[0]
    shard_bytes = B * width * elem + B * ROW_PARAM_BYTES
    if b0.masks is not None:
        rows = B if b0.row_has_mask is None else int(b0.row_has_mask.sum())
        shard_bytes += rows * ((width + 31) // 32) * 4
    st_us = float(np.mean(stats_us))
    achieved = shard_bytes / (st_us * 1e-6) / 1e9
    # what the ranks would exchange per step if each folded its slices'
    # records into one per row first: an all-gather of those, or all-reduces
    # (sums) for the histogram rounds
    rec = [SHARD_RECORD_BYTES.get(SHARD_PHASE_NAMES[ph], 2048) for ph in run]
    exchange = sum(rec) * B * TP
    exchange_ar = sum(r for r in rec if r != 2048) * B * TP + sum(r for r in rec if r == 2048) * B
    cpu = None if args.no_cpu else cpu_baseline(sets, args.cpu_rows)
    line = {
        "metric": f"rows/sec of vocabulary-parallel sampling with the vocabulary split "
                  f"{TP} ways and every shard on one GPU, B={B}, V={V}",
        "value": round(B / (float(np.mean(step_us)) * 1e-6), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_us)) * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if b0.bf16 else "f32",
        "data": "synthetic (seeded; stands in for GLM-5.3 decode logits)",
        "config": {"workload": WORKLOAD_NAMES[args.config] + f"; vocabulary split {TP} ways",
                   "B": B, "V": V, "tp": TP, "shard_width": width, "input_sets": len(sets),
                   "phases": [SHARD_PHASE_NAMES[ph] for ph in run]},
        "step_us_p10_p50_p90": [round(float(np.percentile(step_us, q)), 2) for q in (10, 50, 90)],
        "wall_ms_per_step": round(elapsed * 1e3 / args.steps, 3),
        "exchange_allgather_bytes_per_step": exchange,
        "exchange_allreduce_hist_bytes_per_step": exchange_ar,
        "roofline": {"bound": "hbm", "kernel": "shard_pass_kernel (stats phase)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(args.config, "shard_pass_kernel"),
                     "kernel_us": round(st_us, 2), "bytes_per_launch": shard_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
