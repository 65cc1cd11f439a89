"""Benchmark of the integrity scan on one MI355X.

Default workload: the Llama-70B-shaped bf16 parameter list (723 tensors,
70,553,706,496 elements, 141.1 GB) scanned in a single pass and compared
against its stored fingerprint table -- the check run after every optimizer
step group and after a checkpoint restore.  One step = one fingerprint scan of
the whole list (scan launch + merge launch) plus the diff against the
stored table.  Inputs are resident in HBM before timing starts.

Also reported (same JSON line, "secondary"): the GPT-style ~0.96B fp32
parameter list with 3 replicas, one step = scan of the 3 replicas + strict-
majority compare.

Output: one JSON line with the metric, the roofline of the scan kernel
(algorithmic bytes per launch / launch time from HIP events on the launch
stream; beside it the same figure from the committed rocprofv3 trace of this
kernel source, and the HBM bytes from its committed counter passes) and the
oracle timed on this host's cores over the whole list, whose rows are the
stored table every timed step is diffed against.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fingerprint scan GB/s (and % of HBM peak) on ~1B fp32 and 70B bf16 param lists"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
# Everything the profiled fingerprint kernel and its launch plan are built from.
KERNEL_SOURCES = ["silent_corruption_detection_amd/csrc/scan.hip",
                  "silent_corruption_detection_amd/csrc/fingerprint_device.h",
                  "silent_corruption_detection_amd/csrc/scan_device.h",
                  "silent_corruption_detection_amd/csrc/plan.cpp",
                  "silent_corruption_detection_amd/csrc/sdc_internal.h"]


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload):
    """(HBM bytes per scan launch, cross-check) from the committed counter
    summary, if it was taken on the current kernel source; else (None, None).
    The bytes are FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what
    the same counter reads for an elementwise kernel of known size; the
    cross-check gives the read bytes from two independent counter sets (EA
    read requests by size, and DRAM read requests in 32-byte units) over the
    scaled FETCH_SIZE."""
    path = os.path.join(ROOT, "profiles", f"fingerprint_kernel_{workload}_pmc.json")
    if not os.path.exists(path):
        return None, None
    try:
        d = json.load(open(path))
    except ValueError:
        return None, None
    if d.get("kernel_hash") != kernel_hash():
        return None, None
    return d.get("hbm_bytes_per_launch"), d.get("read_cross_check")


def profiled_time(workload, total_bytes):
    """The scan kernel's average duration in the committed rocprofv3 kernel
    trace of the default benchmark, if it was taken on the current kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", f"fingerprint_kernel_{workload}_trace.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("kernel_hash") != kernel_hash():
        return None
    ms = (d["scan_avg_us"] + d.get("merge_avg_us", 0.0)) / 1000.0
    gbs = total_bytes / ms / 1e6
    return {"kernel_ms": round(ms, 4), "achieved": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "source": f"profiles/fingerprint_kernel_{workload}_trace.json (rocprofv3 "
                      "--kernel-trace --stats of bench.py, average over its launches)"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_plan(sdc, torch, tensors):
    """The plan (packing on the host + one upload), and its wall time in ms: a
    one-time cost per tensor list, reported beside the scan, not inside it."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    plan = sdc.sdc_plan_build(tensors)
    return plan, round((time.perf_counter() - t0) * 1000.0, 3)


def time_steps(step, K, W, stream):
    import torch
    for _ in range(W):
        step(None)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kernel_ms = sum(a.elapsed_time(b) for a, b in evs) / K
    return (t1 - t0) * 1000.0 / K, kernel_ms


def bench_c5(args, torch, sdc, W_):
    """The headline workload.  Before timing, the oracle computes the table
    stored at checkpoint time from the resident weights (all 723 tensors,
    the cpu_baseline leg); every timed step then scans the list and diffs the
    result against that table on the GPU, so each step re-checks parity.
    With --cpu-budget 0 the stored table is the GPU's own first scan."""
    import numpy as np
    log("bench: generating the Llama-70B bf16 list (141 GB) ...")
    w = W_.c5("cuda")
    plan, plan_ms = build_plan(sdc, torch, w.tensors)
    stream = torch.cuda.current_stream()
    out = sdc.sdc_fingerprint_plan(plan)
    torch.cuda.synchronize()
    cpu, match = None, None
    if args.cpu_budget > 0:
        cpu, ref = cpu_baseline(w, out, args.cpu_budget, sdc, torch)
        stored = torch.from_numpy(ref.view(np.int64)).to("cuda")  # the oracle's table
        match = int((sdc.rows_numpy(out) == ref).all(axis=1).sum())
    else:
        stored = out.clone()
    torch.cuda.synchronize()
    bad = []

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        sdc.sdc_fingerprint_plan(plan, out, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        d = sdc.sdc_fingerprint_diff(stored, out, idx_cap=16, stream=stream)
        if d["n_diff"]:
            bad.append(d)

    log("bench: timing ...")
    ms, kms = time_steps(step, args.steps, args.warmup, stream)
    if bad:
        raise RuntimeError(f"scan differs from the stored table: {bad[:2]}")
    if match is not None and match != plan.n_tensors:
        raise RuntimeError(f"only {match} of {plan.n_tensors} rows equal the oracle's")
    return w, plan, out, ms, kms, plan_ms, cpu, match


def bench_c2(args, torch, sdc, W_):
    log("bench: generating the GPT-style 0.96B fp32 list x 3 replicas ...")
    w = W_.c2("cuda")
    plan, plan_ms = build_plan(sdc, torch, w.tensors)
    stream = torch.cuda.current_stream()
    out = sdc.sdc_fingerprint_plan(plan)
    torch.cuda.synchronize()
    res = {}

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        sdc.sdc_fingerprint_plan(plan, out, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        res.update(sdc.sdc_majority_compare(out, w.R, w.T, stream=stream))

    ms, kms = time_steps(step, args.steps, args.warmup, stream)
    if res.get("suspects") != [w.injections[0]["replica"]]:
        raise RuntimeError(f"majority compare gave {res}")
    info = dict(workload="gpt_decoder_0.96b_fp32_3_replicas_majority", tensors=w.R * w.T,
                elements=plan.total_elems, bytes=plan.total_bytes, item_bytes=plan.item_bytes,
                ms_per_step=round(ms, 4), value=round(plan.total_bytes / ms / 1e6, 1),
                unit="GB/s", kernel_ms=round(kms, 4),
                kernel_frac_of_hbm_peak=round(plan.total_bytes / kms / 1e6 / HBM_PEAK_GBS, 4),
                plan_build_ms=plan_ms)
    del w, plan, out
    return info


def bench_other(args, torch, sdc, W_, name):
    """Timing of the other workloads (c1 replicas, c3 gradients + replay, c4
    small tensors): scan + the comparison each is for, and for c3 the
    NaN/Inf-count and squared-norm launches on their own."""
    w = W_.BUILDERS[name]("cuda")
    plan, plan_ms = build_plan(sdc, torch, w.tensors)
    stream = torch.cuda.current_stream()
    out = sdc.sdc_fingerprint_plan(plan)
    counts = torch.empty(max(plan.n_tensors, 1), dtype=torch.int64, device="cuda")
    total = torch.empty(1, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    T = w.T

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        sdc.sdc_fingerprint_plan(plan, out, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        if name == "c3":
            sdc.sdc_fingerprint_diff(out[:T], out[T:], stream=stream)
        else:
            sdc.sdc_majority_compare(out, w.R, w.T, stream=stream)

    ms, kms = time_steps(step, args.steps, args.warmup, stream)
    res = dict(workload=w.name, tensors=plan.n_tensors, elements=plan.total_elems,
               bytes=plan.total_bytes, item_bytes=plan.item_bytes, work_items=plan.n_items,
               ms_per_step=round(ms, 4), value=round(plan.total_bytes / ms / 1e6, 1), unit="GB/s",
               kernel_ms=round(kms, 4), kernel_gbs=round(plan.total_bytes / kms / 1e6, 1),
               kernel_frac_of_hbm_peak=round(plan.total_bytes / kms / 1e6 / HBM_PEAK_GBS, 4),
               plan_build_ms=plan_ms)
    if name == "c3":
        def nf_step(ev):
            if ev is not None:
                ev[0].record(stream)
            sdc.sdc_nonfinite(plan, counts, total, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        _, nkms = time_steps(nf_step, args.steps, args.warmup, stream)
        res.update(nonfinite_kernel_ms=round(nkms, 4),
                   nonfinite_gbs=round(plan.total_bytes / nkms / 1e6, 1),
                   nonfinite_total=int(total.item()))
        sq = torch.empty(max(plan.n_tensors, 1), dtype=torch.float64, device="cuda")
        sq_total = torch.empty(1, dtype=torch.float64, device="cuda")
        flag = torch.empty(1, dtype=torch.int32, device="cuda")

        def sq_step(ev):
            if ev is not None:
                ev[0].record(stream)
            sdc.sdc_sqnorm(plan, sq, sq_total, flag, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        _, skms = time_steps(sq_step, args.steps, args.warmup, stream)
        res.update(sqnorm_ms=round(skms, 4), sqnorm_gbs=round(plan.total_bytes / skms / 1e6, 1),
                   sqnorm_frac_of_hbm_peak=round(plan.total_bytes / skms / 1e6 / HBM_PEAK_GBS, 4),
                   sqnorm_flag=int(flag.item()))
    return res


def bench_recompute(args, torch, sdc, W_):
    """The recompute audit's scans (a second workload on the scan kernel): per
    step every checkpointed layer output of a Llama-70B micro-batch is scanned
    by the plan-free single-tensor path and compared on the device with the row
    stored at forward time -- one call per tensor, as the hook makes them.
    --act-split S cuts each output into S row blocks scanned by a call each
    (S = 8: 640 calls on 64 MiB), where the host's cost per call decides."""
    log("bench: generating 80 activation tensors [32768, 8192] bf16 (43 GB) ...")
    w = W_.recompute_acts("cuda")
    S = args.act_split
    if S < 1 or w.tensors[0].shape[0] % S:
        raise SystemExit(f"--act-split must divide {w.tensors[0].shape[0]}")
    tensors = [b for t in w.tensors for b in t.split(t.shape[0] // S)]
    T = len(tensors)
    stream = torch.cuda.current_stream()
    stored = torch.empty((T, 4), dtype=torch.int64, device="cuda")
    out = torch.empty_like(stored)
    mis = torch.zeros(T, dtype=torch.int32, device="cuda")
    # one-row views made once, as the audit holds them
    stored_rows, out_rows, mis_at = stored.split(1), out.split(1), mis.split(1)
    for k in range(T):
        sdc.sdc_fingerprint_tensor(tensors[k], out=stored_rows[k], stream=stream)
    # one workspace for all calls: they run in order on the one stream
    ws = torch.empty(sdc.sdc_tensor_ws_bytes(tensors[0]), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    host_s = []

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        t0 = time.perf_counter()
        for k in range(T):
            sdc.sdc_fingerprint_tensor(tensors[k], out=out_rows[k], ref=stored_rows[k],
                                       mismatch=mis_at[k], stream=stream, ws=ws)
        if ev is not None:
            host_s.append(time.perf_counter() - t0)
            ev[1].record(stream)

    ms, kms = time_steps(step, args.steps, args.warmup, stream)
    if int(mis.sum().item()) != 0 or not torch.equal(out, stored):
        raise RuntimeError("single-tensor scan is not reproducible")
    nbytes = sum(t.numel() * t.element_size() for t in tensors)
    enqueue_us = sorted(host_s)[len(host_s) // 2] / T * 1e6
    return dict(workload=w.name if S == 1 else f"{w.name}, each cut into {S} row blocks",
                tensors=T, tensor_bytes=tensors[0].numel() * tensors[0].element_size(),
                bytes=nbytes, calls_per_step=T, ms_per_step=round(ms, 4),
                value=round(nbytes / ms / 1e6, 1), unit="GB/s", per_call_us=round(ms / T * 1e3, 2),
                host_enqueue_us_per_call=round(enqueue_us, 2),
                kernel_ms=round(kms, 4), kernel_gbs=round(nbytes / kms / 1e6, 1),
                kernel_frac_of_hbm_peak=round(nbytes / kms / 1e6 / HBM_PEAK_GBS, 4),
                note=f"kernel_ms spans the step's {T} scan + compare launch pairs on the stream; "
                     "host_enqueue_us_per_call: the binding and library's host time per call "
                     "(median step)")


def read_reference(args, torch, sdc, gib=32):
    """Streaming-read reference in the same run: sdc_read_sum (the scan's load
    structure, one add per 32-bit word, partial sums merged by a second launch)
    over one `gib` GiB device buffer of random bits, timed with HIP events on
    the launch stream.  Returns None when the device lacks the free memory."""
    free, _ = torch.cuda.mem_get_info()
    nbytes = gib << 30
    if free < nbytes + (2 << 30):
        log(f"bench: read reference skipped ({free / 2**30:.1f} GiB free)")
        return None
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    out = torch.empty(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(sdc.sdc_read_sum_ws_bytes(nbytes), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        sdc.sdc_read_sum(buf, out=out, ws=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    log("bench: timing the streaming-read reference ...")
    _, kms = time_steps(step, args.steps, args.warmup, stream)
    del buf, ws
    torch.cuda.empty_cache()
    gbs = nbytes / kms / 1e6
    return {"kernel": "read_sum_kernel (+ read_merge_kernel)", "bytes": nbytes, "kernel_ms": round(kms, 4),
            "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "note": "sum of the 32-bit words of one buffer, read with the scan's load structure "
                    "for lists of large items (1 MiB per workgroup, one workgroup per CU, "
                    "non-pipelined rounds of non-temporal 16-byte loads, 8 per lane: the fastest "
                    "depth for a pure read; partial sums merged by a second launch).  A reference "
                    "measured in the same run, not an upper bound: over its buffer of random words "
                    "it measured 0-1.2 % below the scan over the model's 141 GB list in the same runs"}


def usable_cores(cap=16):
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, cap))


def cpu_baseline(w, out, budget_s, sdc, torch):
    """The oracle (unchanged, single-threaded C) timed on this host, over the
    same list the GPU scans.  (1) The whole list, every tensor one oracle
    call, on every usable host core at once (at most 16): the main thread
    copies tensor after tensor into pinned host buffers, each copied tensor
    goes to the thread pool at once, so the copies overlap the oracle's work;
    its rows are the stored table.  value = bytes / wall time of that run,
    with the copy time reported on its own.  (2) One thread, over whole
    tensors in list order until budget_s seconds of oracle time.  Every row is
    checked against the GPU's first scan."""
    import numpy as np
    from oracle import BF16, fingerprint
    from oracle.device_lists import rows_of_device_tensors
    rows = sdc.rows_numpy(out)
    cores = usable_cores()
    log(f"bench: the oracle over all {len(w.tensors)} tensors on {cores} threads ...")
    ref, st = rows_of_device_tensors(w.tensors, threads=cores)
    okm = int((ref == rows).all(axis=1).sum())

    order = list(range(1, w.T - 2)) + [0, w.T - 2, w.T - 1]
    spent, nbytes, nel, n, ok = 0.0, 0, 0, 0, True
    for k in order:
        h = w.tensors[k].detach().reshape(-1).view(torch.uint8).cpu().numpy()
        t0 = time.perf_counter()
        r = fingerprint(h, BF16)
        spent += time.perf_counter() - t0
        ok &= bool(np.array_equal(np.array(r, dtype=np.uint64), rows[k]))
        nbytes += h.nbytes
        nel += w.tensors[k].numel()
        n += 1
        del h
        if spent >= budget_s:
            break
    single = {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": 1,
              "elements_per_s": round(nel / spent, 1), "rows_match_gpu": ok,
              "sample": f"{n} whole tensors in list order ({nbytes / 1e9:.2f} GB), {spent:.1f} s"}
    gb = st["bytes"] / 1e9
    cpu = {"value": round(st["bytes"] / st["wall_s"] / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": (f"the whole list: all {len(w.tensors)} tensors ({st['elements']} elements, "
                      f"{gb:.2f} GB), the single-threaded C oracle once per tensor on {cores} "
                      f"threads at once, fed by device-to-host copies into pinned buffers that "
                      f"overlap it; value = bytes / wall time ({st['wall_s']:.1f} s) including "
                      f"the copies"),
           "tensors": len(w.tensors), "elements_per_s": round(st["elements"] / st["wall_s"], 1),
           "wall_s": round(st["wall_s"], 3), "d2h_s": round(st["d2h_s"], 3),
           "d2h_gbs": round(gb / st["d2h_s"], 2) if st["d2h_s"] > 0 else None,
           "compute_s": round(st["busy_s"], 3),
           "compute_gbs_per_core": round(gb / st["busy_s"], 4) if st["busy_s"] > 0 else None,
           "rows_match_gpu": f"{okm}/{len(w.tensors)}",
           "single_thread": single}
    return cpu, ref


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=5.0,
                    help="seconds of the single-threaded oracle sample of the CPU baseline "
                         "(0: skip the CPU baseline, including the oracle's stored table)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5", "recompute"],
                    help="c5 (default) prints the benchmark line; the others print their "
                         "own timing object")
    ap.add_argument("--act-split", type=int, default=1,
                    help="recompute workload: scan each activation as this many row blocks")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(each GPU would scan its own replica and exchange only a small all-gather of "
              "fingerprint tables, which this library does not implement)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import silent_corruption_detection_amd as sdc
    import workloads as W_

    torch.cuda.set_device(0)
    if args.calib_copy_mib:
        # an elementwise kernel (not a memcpy): reads n bytes, writes n bytes
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        log(f"bench: calibration copy (bitwise_not) of {n} bytes done")
        del src, dst
    if args.workload != "c5":
        if args.workload == "c2":
            res = bench_c2(args, torch, sdc, W_)
        elif args.workload == "recompute":
            res = bench_recompute(args, torch, sdc, W_)
        else:
            res = bench_other(args, torch, sdc, W_, args.workload)
        print(json.dumps(res), flush=True)
        return
    secondary = None
    if not args.no_secondary:
        secondary = bench_c2(args, torch, sdc, W_)
        torch.cuda.empty_cache()
    w, plan, out, ms, kms, plan_ms, cpu, match = bench_c5(args, torch, sdc, W_)
    del w
    torch.cuda.empty_cache()
    total_bytes = plan.total_bytes
    achieved = total_bytes / kms / 1e6  # GB/s
    traffic, traffic_check = traffic_from_profile("llama70b_bf16")
    ref_read = read_reference(args, torch, sdc)
    value = total_bytes / ms / 1e6
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u64",
        "data": "synthetic",
        "config": {"workload": "llama70b_bf16_param_list_single_pass_vs_stored_table",
                   "data_dtype": "bf16", "tensors": plan.n_tensors, "elements": plan.total_elems,
                   "bytes": total_bytes, "item_bytes": plan.item_bytes, "work_items": plan.n_items,
                   "step": "fingerprint scan + merge of split rows + diff against the stored table",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_read_cross_check": traffic_check,
                     "kernel": "fingerprint_kernel (+ merge_rows_kernel)",
                     "kernel_ms": round(kms, 4), "kernel_hash": kernel_hash(),
                     "timing": "HIP events on the launch stream, this run",
                     "profiled": profiled_time("llama70b_bf16", total_bytes),
                     "frac_of_read_reference": (round(achieved / ref_read["gbs"], 4)
                                                if ref_read else None)},
        "read_reference": ref_read,
        "elements_per_s": round(plan.total_elems / ms * 1e3, 1),
        "plan_build_ms": plan_ms,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "rows_match_oracle": (f"{match}/{plan.n_tensors}" if match is not None else None),
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
