#!/usr/bin/env python3
"""Benchmark of the fused cross-entropy hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 5] [--gpus 1]
                    [--smoothing all|others] [--reduction none|mean|sum]

A step is one pass of the whole path over one batch of synthetic input
already resident in HBM: for the default workload (4 x 2048 rows of 128000
BF16 logits, label smoothing 0.1, mean over the 7782 non-ignored rows) that is
one ce_fwd_bwd_fused call, one kernel launch (the first workgroups count the
non-ignored rows; every workgroup reads its part of the logits once and writes
the gradient over it; the workgroup that starts last sums the mean).
--smoothing and --reduction run the same step with smoothing over the other
V-1 classes or another reduction.  The call overwrites its
input with the gradient, so each timed step works on its own copy of the
logits from a pool in HBM, refreshed from the generated batch just before the
timed region: every timed step sees the logits as generated, never a previous
step's gradient (on this chip the kernel's duration depends on the values it
reads, since it runs near the power limit).  Warmup steps reuse the pool.

Printed: one JSON line with the whole-step throughput (formula bytes
N*V*b read + N*V*b written, per step), the roofline of the step's dominant
kernel (its own average duration from HIP events recorded by the library on
the same stream) and every main kernel's duration and rate, HBM traffic from
committed rocprofv3 counter runs when they match the current kernel source,
each step timed alone with cold caches (median and min), and the FP64 oracle
timed on a bounded sample of rows on the host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused CE fwd+bwd achieved HBM GB/s (% of peak) and rows/sec at V=128000 bf16"
PEAK_GBPS = 8000.0  # MI355X HBM3E peak, AMD public specification
KERNEL_SRC = os.path.join(ROOT, "vocab_cross_entropy_amd", "csrc", "ce_kernels.hip")
PMC_FILE = os.path.join(ROOT, "profiles", "fused_bf16_v128000_pmc.json")


def kernel_source_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_profiles(workload_name: str):
    """HBM bytes per launch of the fused kernel from committed rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE) of this workload, each scaled by what the
    same counter reads for a plain copy kernel of known size.  None when no
    counter file covers the workload or the kernel source changed since."""
    import glob

    found = []
    for path in sorted(glob.glob(os.path.join(os.path.dirname(PMC_FILE), "*_pmc.json"))):
        try:
            with open(path) as f:
                pmc = json.load(f)
        except (OSError, ValueError):
            continue
        if pmc.get("workload") == workload_name:
            found.append(pmc)
    if not found:
        return None, "no counter file for this workload"
    pmc = found[0]
    if pmc.get("kernel_source_sha256") != kernel_source_sha():
        return None, "kernel changed since the counters were taken"
    c = pmc["copy"]
    fetch_scale = c["bytes"] / (c["fetch_kib"] * 1024.0)
    write_scale = c["bytes"] / (c["write_kib"] * 1024.0)
    t = pmc["fetch_kib"] * 1024.0 * fetch_scale + pmc["write_kib"] * 1024.0 * write_scale
    return t, f"fetch x{fetch_scale:.3f}, write x{write_scale:.3f} (copy calibration)"


def _counter_rows(outdir: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} from a rocprofv3 --pmc csv output directory."""
    import csv
    import glob

    files = glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {outdir}")
    out = {}
    for path in files:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = (path, r["Dispatch_Id"])
                name, v = out.get(k, (r["Kernel_Name"], 0.0))
                out[k] = (name, v + float(r["Counter_Value"]))
    return out


def write_pmc_json(args):
    """The counter file of the fused kernel on a workload: the median FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of its launches, and of the benchmark's full-size input copies (the calibration: a copy of
    known size), stamped with the kernel source's sha256."""
    import statistics

    import workloads

    w = workloads.WORKLOADS[args.workload]
    dt = args.dtype or ("bf16" if "bf16" in w.name else "f32")
    if args.dtype:
        other = "_bf16" if args.dtype == "f32" else "_f32"
        name = w.name.replace(other, f"_{args.dtype}") if other in w.name else w.name
    else:
        name = w.name
    eb = 2 if dt == "bf16" else 4
    copy_bytes = w.rows * w.V * eb
    vals = {}
    for counter, d in (("FETCH_SIZE", args.pmc_json[0]), ("WRITE_SIZE", args.pmc_json[1])):
        rows = _counter_rows(d, counter)
        fused = [v for n, v in rows.values() if "k_fused<" in n]
        copies = [v for n, v in rows.values() if "copyBuffer" in n]
        if not fused or not copies:
            raise SystemExit(f"{d}: no k_fused or copy dispatches with {counter}")
        kname = sorted({n for n, _ in rows.values() if "k_fused<" in n})
        vals[counter] = (statistics.median(fused), statistics.median(sorted(copies)[len(copies) // 2:]), kname)
    kernel = vals["FETCH_SIZE"][2][0]
    kernel = kernel[kernel.index("k_fused<"):kernel.index(">", kernel.index("k_fused<")) + 1]
    pmc = {
        "workload": name,
        "kernel": kernel,
        "kernel_source_sha256": kernel_source_sha(),
        "fetch_kib": vals["FETCH_SIZE"][0],
        "write_kib": vals["WRITE_SIZE"][0],
        "copy": {"bytes": copy_bytes, "fetch_kib": vals["FETCH_SIZE"][1], "write_kib": vals["WRITE_SIZE"][1]},
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -d {args.pmc_json[0]} -o pmc --output-format csv -- python -u bench.py "
            f"--workload {args.workload} --steps 3 --warmup 1 --no-cpu-baseline",
            f"rocprofv3 --pmc WRITE_SIZE -d {args.pmc_json[1]} -o pmc --output-format csv -- python -u bench.py "
            f"--workload {args.workload} --steps 3 --warmup 1 --no-cpu-baseline",
            f"python bench.py --workload {args.workload} --pmc-json {args.pmc_json[0]} {args.pmc_json[1]}",
        ],
    }
    out = os.path.join(os.path.dirname(PMC_FILE), f"fused_{dt}_v{w.V}_pmc.json")
    with open(out, "w") as f:
        json.dump(pmc, f, indent=1)
        f.write("\n")
    t, note = traffic_from_profiles(name)
    print(json.dumps({"written": out, "traffic_bytes_per_launch": t, "note": note}))


def device_info(torch, dev) -> dict:
    """What the runtime reports of the device the step ran on; the peak HBM
    rate used as the roofline's denominator is the published figure."""
    pr = torch.cuda.get_device_properties(dev)
    info = {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count,
            "total_memory_bytes": pr.total_memory, "l2_cache_bytes": getattr(pr, "L2_cache_size", None),
            "lds_per_workgroup_bytes": getattr(pr, "shared_memory_per_block", None),
            "wave_size": getattr(pr, "warp_size", None), "peak_hbm_GBps_published": PEAK_GBPS}
    return info


def cpu_baseline(w, inputs, sample_rows: int, reduction: str, smoothing: str):
    """The FP64 oracle (as it is) on the first `sample_rows` rows: loss and
    gradient, the same work per row as the GPU step."""
    import numpy as np

    import oracle
    import workloads

    orc = oracle.default()
    N = w.rows
    rows = np.arange(N if sample_rows <= 0 else min(sample_rows, N), dtype=np.int64)
    n_valid = orc.count_valid(inputs.targets)
    g = None if reduction == "none" else 1.0
    if w.shards > 1:  # the shard form: per-shard statistics, their combine, per-shard gradients
        bounds = workloads.shard_bounds(w.V, w.shards)
        shards = [inputs.logits[..., a:c].contiguous() for a, c in bounds]
    t0 = time.perf_counter()
    for b in range(0, rows.size, 256):
        blk = rows[b:b + 256]
        if w.shards > 1:
            st = np.stack([orc.shard_stats(sh, inputs.targets, a, w.V, rows=blk) for sh, (a, c) in zip(shards, bounds)])
            _, lse = orc.shard_combine(st, inputs.targets, w.V, w.alpha, rows=blk, smoothing=smoothing)
            for sh, (a, c) in zip(shards, bounds):
                orc.shard_grad(sh, inputs.targets, a, w.V, lse, w.alpha, reduce_loss=reduction, g=g, rows=blk,
                               n_valid=n_valid, smoothing=smoothing)
        else:
            orc.loss_rows(inputs.logits, inputs.targets, w.alpha, rows=blk, smoothing=smoothing)
            orc.grad_rows(inputs.logits, inputs.targets, w.alpha, reduce_loss=reduction, g=g, rows=blk,
                          n_valid=n_valid, smoothing=smoothing)
    dt = time.perf_counter() - t0
    nbytes = 2 * rows.size * w.V * w.elem_bytes
    return {
        "value": nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": orc.max_threads(),
        "kind": "oracle",
        "sample": (f"all {N} rows" if rows.size == N else f"first {rows.size} of {N} rows")
                  + f" of the step's logits (loss + gradient, FP64{', shard form' if w.shards > 1 else ''}), {dt:.2f} s wall",
        "rows_per_s": rows.size / dt,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--pool", type=int, default=0,
                    help="device copies of the input (HBM); 0 = one per timed step, as memory allows")
    ap.add_argument("--cpu-sample-rows", type=int, default=0, help="rows the CPU oracle is timed on (0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-chunks", type=int, default=0, help="tuning: force the fused kernel's split")
    ap.add_argument("--smoothing", choices=["all", "others"], default="all",
                    help="label smoothing a/V over all classes (default) or a/(V-1) over the other classes")
    ap.add_argument("--reduction", choices=["none", "mean", "sum"], default=None,
                    help="loss reduction (default: the workload's own)")
    ap.add_argument("--split", action="store_true",
                    help="unsharded workloads: ce_forward then ce_backward_inplace in place of the fused call")
    ap.add_argument("--fused-shards", action="store_true",
                    help="shard workloads: one ce_shards_fwd_bwd_fused launch in place of the three-call flow")
    ap.add_argument("--dtype", choices=["bf16", "f32"], default=None,
                    help="the workload's logits in this dtype instead of its own (same shape and recipe)")
    ap.add_argument("--vocab", type=int, default=0,
                    help="tuning: the workload's recipe with this many columns (the metric's workload is unchanged "
                         "otherwise)")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as HIP graph replays (one captured step per input copy), without the "
                         "host's per-call cost")
    ap.add_argument("--phases", action="store_true",
                    help="time the main kernel's phases per workgroup with the phase-stamped library build "
                         "(libce_phases.so) and print their summary instead of the benchmark line")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--linear", action="store_true",
                    help="time the chunked linear head + cross-entropy (ce_linear_cross_entropy) instead")
    ap.add_argument("--hidden", type=int, default=4096, help="--linear: hidden size D")
    ap.add_argument("--chunk-rows", type=int, default=0, help="--linear: rows per chunk (0: automatic)")
    ap.add_argument("--tune", action="store_true", help="--linear: ce_linear_tune before the timed steps")
    ap.add_argument("--gemm", choices=["auto", "native", "library"], default="auto",
                    help="--linear: the products' engine (the library's MFMA kernel or hipBLASLt)")
    ap.add_argument("--pmc-json", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="no GPU work: from the rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE output directories of "
                         "two runs of this benchmark (same workload), write the counter file "
                         "profiles/fused_<dtype>_v<V>_pmc.json that the benchmark line's roofline.traffic reads")
    args = ap.parse_args()
    if args.pmc_json:
        return write_pmc_json(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the multi-GPU "
              "(vocabulary- or row-sharded) path is not implemented here; each GPU would run its own rows or shards",
              file=sys.stderr)
        sys.exit(2)

    if args.phases:
        os.environ["VCE_PHASE_CLOCK"] = "1"  # the binding then loads libce_phases.so

    import torch

    import vocab_cross_entropy_amd as vce
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.linear:
        return bench_linear(args, torch, vce, workloads, dev)
    w = workloads.WORKLOADS[args.workload]
    if args.dtype:
        dt = torch.bfloat16 if args.dtype == "bf16" else torch.float32
        if dt != w.dtype:
            other = "_bf16" if args.dtype == "f32" else "_f32"
            name = w.name.replace(other, f"_{args.dtype}") if other in w.name else f"{w.name}_{args.dtype}"
            w = dataclasses.replace(w, dtype=dt, name=name)
    if args.vocab:
        w = w.scaled(V=args.vocab, name=w.name.replace(f"_v{w.V}_", f"_v{args.vocab}_"))
    t_gen = time.perf_counter()
    inputs = workloads.generate(w)
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] generated {w.name} in {gen_s:.1f} s", file=sys.stderr, flush=True)

    N, V, b = w.rows, w.V, w.elem_bytes
    red = args.reduction or ("mean" if w.reduce_loss else "none")
    sm = args.smoothing
    formula_bytes = 2 * N * V * b  # N*V*b read + N*V*b gradient written

    phys_dev = inputs.logits_phys.to(dev)
    targets_dev = inputs.targets_phys.to(dev)
    view = (lambda p: p.transpose(0, 1)) if w.swapped else (lambda p: p)
    t_view = view(targets_dev)
    want = args.pool if args.pool > 0 else args.steps
    free_b, _ = torch.cuda.mem_get_info(dev)
    fit = int(0.6 * free_b) // max(1, phys_dev.numel() * phys_dev.element_size())
    P = max(1, min(want, fit))
    if P < args.steps:
        print(f"[bench] pool of {P} copies < {args.steps} steps: some timed steps reuse a gradient",
              file=sys.stderr, flush=True)
    pool = [phys_dev.clone() for _ in range(P)] if w.calls != "shard" else None
    torch.cuda.synchronize()

    loss = torch.empty(1 if red != "none" else N, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int32, device=dev)
    calls_per_step = 1
    calls = w.calls
    if calls == "shard" and args.fused_shards:
        calls = "shard_fused"
    if calls == "fused" and args.split:
        calls = "split"
    if calls == "fused":
        ws = torch.empty(vce.ce_workspace_bytes(view(pool[0]), w.alpha, red, split_chunks=args.split_chunks),
                         dtype=torch.uint8, device=dev)

        def step(p):
            vce.ce_fwd_bwd_fused(view(p), t_view, w.alpha, red, loss=loss, n_valid=n_valid, ws=ws,
                                 split_chunks=args.split_chunks, smoothing=sm)
    elif calls == "split":  # forward, then the backward from its lse and lse_aux hand-off
        ws = torch.empty(vce.ce_workspace_bytes(view(pool[0]), w.alpha, red), dtype=torch.uint8, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        aux = torch.empty((N, 2), dtype=torch.float32, device=dev)
        g = torch.ones(N if red == "none" else 1, dtype=torch.float32, device=dev)
        calls_per_step = 2

        def step(p):
            x = view(p)
            vce.ce_forward_ex(x, t_view, w.alpha, red, loss=loss, lse=lse, lse_aux=aux, n_valid=n_valid, ws=ws,
                              smoothing=sm)
            vce.ce_backward_inplace_ex(x, t_view, lse, aux, w.alpha, red, grad_out=g, n_valid=n_valid,
                                       smoothing=sm)
    elif calls == "shard_fused":  # vocabulary shards, every shard read once in one launch
        bounds = workloads.shard_bounds(V, w.shards)
        pool = [[phys_dev[..., a:c].contiguous() for a, c in bounds] for _ in range(P)]
        ws = torch.empty(vce.ce_shards_workspace_bytes(pool[0], w.alpha, red, smoothing=sm), dtype=torch.uint8,
                         device=dev)

        def step(shards):
            vce.ce_shards_fwd_bwd_fused([view(x) for x in shards], t_view, w.alpha, red, loss=loss,
                                        n_valid=n_valid, ws=ws, smoothing=sm)
    else:  # vocabulary shards: S partial-stat calls, one combine, S backward calls
        bounds = workloads.shard_bounds(V, w.shards)
        pool = [[phys_dev[..., a:c].contiguous() for a, c in bounds] for _ in range(P)]
        stats = torch.empty((len(bounds), N, 4), dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        aux = torch.empty((N, 2), dtype=torch.float32, device=dev)
        ws = torch.empty(vce.ce_combine_workspace_bytes(N, red), dtype=torch.uint8, device=dev)
        g = torch.ones(N if red == "none" else 1, dtype=torch.float32, device=dev)
        calls_per_step = 2 * len(bounds)

        def step(shards):
            for s, (a, c) in enumerate(bounds):
                vce.ce_shard_partial_stats(shards[s], t_view, a, V, stats=stats[s])
            vce.ce_shard_combine_ex(stats, t_view, V, w.alpha, red, loss=loss, lse=lse, lse_aux=aux,
                                    n_valid=n_valid, ws=ws, smoothing=sm)
            for s, (a, c) in enumerate(bounds):
                vce.ce_backward_inplace_ex(shards[s], t_view, lse, aux, w.alpha, red, grad_out=g,
                                           n_valid=n_valid, vocab_start=a, vocab_total=V, smoothing=sm)

    def restore(p):
        """One pool copy back to the generated logits."""
        if isinstance(p, list):
            for (a, c), sh in zip(bounds, p):
                sh.copy_(phys_dev[..., a:c])
        else:
            p.copy_(phys_dev)

    def refresh():
        """Every pool copy back to the generated logits (outside any timed region)."""
        for p in pool:
            restore(p)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        step(pool[i % P])
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    refresh()
    if args.phases:
        return phase_profile(args, torch, vce, w, calls, step, pool, restore, bounds if calls.startswith("shard")
                             else None, t_view, red, sm, dev)

    timed = step
    if args.graph:
        # one captured step per input copy (their pointers differ); each replay
        # takes a fresh tag from the workspace, so replays are full calls
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for p in pool:
                captured = torch.cuda.CUDAGraph()
                with torch.cuda.graph(captured, stream=cap):
                    step(p)
                graphs.append(captured)
        torch.cuda.current_stream().wait_stream(cap)
        for captured in graphs:  # a first launch of each (its upload), outside the timed region
            captured.replay()
        refresh()
        by_id = {id(p): gr for p, gr in zip(pool, graphs)}
        timed = lambda p: by_id[id(p)].replay()  # noqa: E731

    # the timed steps: nothing but the calls themselves between the two events
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        timed(pool[i % P])
    e1.record()
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    step_ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] timed {args.steps} steps: {step_ms * 1e3:.1f} us/step (host {1e6 * (h1 - h0) / args.steps:.1f})",
          file=sys.stderr, flush=True)
    # the same steps again, on refreshed copies, with the library recording HIP
    # events around each call's main kernel on the call's stream, for the
    # kernel's own duration
    refresh()
    with vce.Profiler(args.steps * calls_per_step) as prof:
        for i in range(args.steps):
            step(pool[i % P])
        torch.cuda.synchronize()

    # each step timed alone with the caches cold: before it (outside its
    # events) its logits are restored and a 512 MiB scratch buffer is written,
    # more than the L2s and the 256 MB Infinity Cache hold
    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(args.steps):
        restore(pool[i % P])
        evict.fill_(i & 0xFF)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        step(pool[i % P])
        c1.record()
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    cold.sort()
    del pool, evict
    torch.cuda.empty_cache()

    # plain device copy of the same byte count, for context (achievable read+write rate)
    flat = phys_dev.view(-1)
    dst = torch.empty_like(flat)
    for _ in range(3):
        dst.copy_(flat)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        dst.copy_(flat)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * flat.numel() * flat.element_size() / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
    del dst
    # and an in-place elementwise pass over the same bytes (read, then write to the same addresses;
    # the generated logits on the device are not used after this)
    for _ in range(3):
        flat.neg_()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        flat.neg_()
    c1.record()
    torch.cuda.synchronize()
    inplace_gbps = 2 * flat.numel() * flat.element_size() / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
    # the library's reference pass over the same bytes (ce_stream_reference: a plain one-pass kernel with
    # the fused kernel's own 16-byte non-temporal buffer loads and stores), in place and as a copy
    def ref_rate(dst):
        for _ in range(3):
            vce.ce_stream_reference(flat, dst)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record()
        for _ in range(10):
            vce.ce_stream_reference(flat, dst)
        r1.record()
        torch.cuda.synchronize()
        return 2 * flat.numel() * flat.element_size() / (r0.elapsed_time(r1) / 10 * 1e-3) / 1e9
    stream_inplace_gbps = stream_copy_gbps = None
    if (flat.numel() * flat.element_size()) % 16 == 0:
        stream_inplace_gbps = ref_rate(None)
        dst = torch.empty_like(flat)
        stream_copy_gbps = ref_rate(dst)
        del dst

    # each call's main kernel: its average duration over the event pass and
    # the algorithmic bytes one launch moves (read + written, formula N*V*b
    # per pass over the logits or a shard)
    main_ms = prof.ms
    if calls == "fused":
        layout = [("k_fused", formula_bytes)]
    elif calls == "shard_fused":
        layout = [("k_fused_shards", formula_bytes)]
    elif calls == "split":
        layout = [("k_stats (ce_forward)", N * V * b), ("k_backward (ce_backward_inplace)", 2 * N * V * b)]
    else:
        layout = ([("k_stats (ce_shard_partial_stats)", N * (c - a) * b) for a, c in bounds]
                  + [("k_backward (shard)", 2 * N * (c - a) * b) for a, c in bounds])
    kernels = {}
    for k, (name, nbytes) in enumerate(layout):
        ms = main_ms[k::len(layout)]
        if not ms:
            continue
        ent = kernels.setdefault(name, {"launches": 0, "total_ms": 0.0, "bytes": 0})
        ent["launches"] += len(ms)
        ent["total_ms"] += sum(ms)
        ent["bytes"] += nbytes * len(ms)
    kernel_summary = {name: {"avg_us": round(1e3 * e["total_ms"] / e["launches"], 2),
                             "algorithmic_bytes_per_launch": e["bytes"] // e["launches"],
                             "GBps": round(e["bytes"] / (e["total_ms"] * 1e-3) / 1e9, 1)}
                      for name, e in kernels.items()}
    roofline = None
    if kernels:
        # the dominant kernel: the largest share of the step's kernel time
        dom = max(kernels, key=lambda n: kernels[n]["total_ms"])
        e = kernels[dom]
        k_ms = e["total_ms"] / e["launches"]
        per_launch = e["bytes"] // e["launches"]
        achieved = per_launch / (k_ms * 1e-3) / 1e9
        traffic, traffic_note = (traffic_from_profiles(w.name) if dom == "k_fused"
                                 else (None, "counters are collected for the fused kernel only"))
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                    "kernel": dom, "kernel_avg_us": round(k_ms * 1e3, 2),
                    "algorithmic_bytes": per_launch, "traffic_note": traffic_note}

    value = formula_bytes / (step_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {**w.describe(), "io_dtype": "bf16" if w.elem_bytes == 2 else "f32", "calls": calls,
                   "reduction": red, "smoothing": sm,
                   "split_chunks": args.split_chunks, "pool": P, "fresh_inputs": P >= args.steps,
                   "graph": bool(args.graph)},
        "rows_per_s": round(N / (step_ms * 1e-3), 1),
        "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
        "formula_bytes_per_step": formula_bytes,
        "copy_ref_GBps": round(copy_gbps, 1),
        "inplace_ref_GBps": round(inplace_gbps, 1),
        "stream_ref_GBps": None if stream_inplace_gbps is None else {
            "in_place": round(stream_inplace_gbps, 1), "copy": round(stream_copy_gbps, 1),
            "frac_of_in_place": round(value / stream_inplace_gbps, 4)},
        "roofline": roofline,
        "kernels": kernel_summary,
        "cold_steps": {"median_us": round(1e3 * cold[len(cold) // 2], 2), "min_us": round(1e3 * cold[0], 2),
                       "n": len(cold), "evict_bytes": 512 << 20,
                       "note": "each step timed alone after restoring its logits and writing 512 MiB of scratch"},
        "cpu_baseline": None,
        "device": device_info(torch, dev),
    }
    if calls in ("split", "shard"):
        moved = 3 * N * V * b
        out["moved_bytes_per_step"] = moved
        out["moved_GBps"] = round(moved / (step_ms * 1e-3) / 1e9, 1)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_sample_rows, red, sm)
    line = json.dumps(out)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")
    print(line, flush=True)


PHASES_FUSED = ["start -> chunk loads issued", "loads + max pass", "sum pass", "partner exchange",
                "gradient + stores issued", "target store + loss publish"]
PHASES_STATS = ["start -> first batch issued", "loads + max (all batches)", "reduction + outputs"]


def _phase_summary(st, names, tick_us, chunks=1):
    """Per-phase means over the records that reached every stamp, the item
    time, the launch's span, the spread of start times and the mean number
    of records in flight (sum of item times / span)."""
    import numpy as np

    n = len(names) + 1
    full = np.all(st[:, :n] != 0, axis=1)
    t = st[full, :n].astype(np.float64) * tick_us
    t0 = st[st[:, 0] != 0, 0].astype(np.float64) * tick_us
    ends = [st[:, n - 1][st[:, n - 1] != 0].astype(np.float64) * tick_us]
    if st.shape[1] > 7 and np.any(st[:, 7]):
        ends.append(st[:, 7][st[:, 7] != 0].astype(np.float64) * tick_us)
    end = max(e.max() for e in ends)
    span = end - t0.min()
    d = np.diff(t, axis=1)
    item = t[:, -1] - t[:, 0]
    out = {"records": int(st.shape[0]), "timed_records": int(full.sum()), "span_us": round(span, 2),
           "start_spread_us": round(t0.max() - t0.min(), 2),
           "tail_after_last_start_us": round(end - t0.max(), 2),
           "item_us_mean": round(float(item.mean()), 3), "item_us_p90": round(float(np.percentile(item, 90)), 3),
           "in_flight_mean": round(float(item.sum() / span), 1) if span > 0 else None,
           "phases_us_mean": {nm: round(float(d[:, i].mean()), 3) for i, nm in enumerate(names)}}
    if st.shape[1] > 7 and np.any(st[:, 7]):
        last = st[st[:, 7] != 0]
        out["finish_us"] = round(float((last[:, 7] - last[:, 6]).mean() * tick_us), 3)
    if chunks > 1 and st.shape[0] % chunks == 0:
        # split rows: how far apart a row's chunks start, and finish their sums (the exchange waits for the last)
        rows = st.reshape(-1, chunks, 8).astype(np.float64) * tick_us
        ok = np.all(rows[:, :, :4] > 0, axis=(1, 2))
        rows = rows[ok]
        out["row_chunk_start_spread_us"] = round(float((rows[:, :, 0].max(1) - rows[:, :, 0].min(1)).mean()), 3)
        out["row_chunk_sum_done_spread_us"] = round(float((rows[:, :, 3].max(1) - rows[:, :, 3].min(1)).mean()), 3)
        out["row_chunk_loads_done_spread_us"] = round(float((rows[:, :, 2].max(1) - rows[:, :, 2].min(1)).mean()), 3)
    return out


def phase_profile(args, torch, vce, w, calls, step, pool, restore, bounds, t_view, red, sm, dev):
    """Phase stamps of the main kernel: the real-time counter (100 MHz) read by
    thread 0 of every workgroup at its phase boundaries, from the
    phase-stamped build of the same sources, over --steps launches on fresh
    copies of the logits; the summary is the mean over launches."""
    import ctypes

    import numpy as np

    tick_us = 0.01  # the 100 MHz real-time counter
    N = w.rows
    buf = torch.zeros((N * 64 * 8,), dtype=torch.int64, device=dev)  # up to 64 workgroups per row, 8 stamps each
    lib = vce.lib
    summaries = []
    kernel_ms = []
    if calls in ("fused", "shard_fused"):
        names, kernel = PHASES_FUSED, "k_fused_shards" if calls == "shard_fused" else "k_fused"
    elif calls == "shard":
        names, kernel = PHASES_STATS, "k_stats (ce_shard_partial_stats, shard 0)"
    else:
        names, kernel = PHASES_STATS, "k_stats (ce_forward_ex)"
    for i in range(args.steps):
        p = pool[i % len(pool)]
        restore(p)
        buf.zero_()
        torch.cuda.synchronize()
        lib.ce_phase_clock(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 8)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if calls in ("fused", "shard_fused"):
            step(p)
        elif calls == "shard":
            a, c = bounds[0]
            vce.ce_shard_partial_stats(p[0], t_view, a, w.V, stats=torch.empty((N, 4), device=dev))
        else:
            vce.ce_forward_ex(p.transpose(0, 1) if w.swapped else p, t_view, w.alpha, red, smoothing=sm)
        e1.record()
        torch.cuda.synchronize()
        lib.ce_phase_clock(None, 0)
        kernel_ms.append(e0.elapsed_time(e1))
        st = buf.view(-1, 8).cpu().numpy().view(np.uint64)
        st = st[np.any(st != 0, axis=1)]
        chunks = st.shape[0] // N if calls in ("fused", "shard_fused") and st.shape[0] % N == 0 else 1
        summaries.append(_phase_summary(st, names, tick_us, chunks))
    keys = ["span_us", "start_spread_us", "tail_after_last_start_us", "item_us_mean", "item_us_p90", "in_flight_mean"]
    mean = {k: round(float(np.mean([s_[k] for s_ in summaries])), 3) for k in keys}
    mean["phases_us_mean"] = {nm: round(float(np.mean([s_["phases_us_mean"][nm] for s_ in summaries])), 3)
                              for nm in names}
    for k in ("finish_us", "row_chunk_start_spread_us", "row_chunk_loads_done_spread_us",
              "row_chunk_sum_done_spread_us"):
        if k in summaries[0]:
            mean[k] = round(float(np.mean([s_[k] for s_ in summaries])), 3)
    out = {"phases": True, "workload": w.name, "kernel": kernel, "calls": calls, "launches": len(summaries),
           "records_per_launch": summaries[0]["records"], "timed_records": summaries[0]["timed_records"],
           "event_us_mean": round(1e3 * float(np.mean(kernel_ms)), 2), "mean": mean,
           "note": "stamps from the phase-stamped build (libce_phases.so): its kernels carry the stamps' "
                   "extra registers and stores; event_us brackets the call on its stream"}
    line = json.dumps(out)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")
    print(line, flush=True)


def cpu_baseline_linear(h, W, t, alpha, reduction, smoothing, n_rows):
    """The FP64 oracle (as it is) for the head + loss of the first `n_rows`
    rows: logits, loss, dh and those rows' share of dW (6 n D V flops)."""
    import oracle

    orc = oracle.default()
    hs = h[:n_rows].cpu()
    ts = t[:n_rows].cpu()
    Wc = W.cpu()
    t0 = time.perf_counter()
    orc.linear_ce(hs, Wc, ts, alpha, reduce_loss=reduction, smoothing=smoothing,
                  n_valid=int((t != -100).sum().item()))
    dt = time.perf_counter() - t0
    flops = 6.0 * n_rows * W.shape[1] * W.shape[0]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": orc.max_threads(), "kind": "oracle",
            "sample": f"first {n_rows} of {h.shape[0]} rows (logits, loss, dh, their dW share; FP64), {dt:.2f} s wall"}


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak, AMD public specification
PEAK_F32_TFLOPS = 157.3    # MI355X FP32 matrix peak


def bench_linear(args, torch, vce, workloads, dev):
    """The language-model head and its loss over row chunks: one step is one
    ce_linear_cross_entropy call (logits GEMM, fused cross-entropy, dh and dW
    GEMMs for every chunk) on 4 x 2048 rows, D = --hidden, V = 128000, BF16,
    label smoothing 0.1, mean over the non-ignored rows.  Synthetic inputs:
    h ~ N(0, 1), W ~ N(0, (2 / sqrt(D))^2), so the logits have a standard
    deviation near 2 as in the 128000-column cross-entropy workload."""
    w5 = workloads.WORKLOADS[5]
    N, D, V = w5.rows, args.hidden, w5.V
    g = torch.Generator(device="cpu").manual_seed(4321)
    h = torch.randn((N, D), generator=g).to(torch.bfloat16).to(dev)
    W = (torch.randn((V, D), generator=g) * (2.0 / D ** 0.5)).to(torch.bfloat16).to(dev)
    t = torch.randint(0, V, (N,), generator=g)
    t[torch.randperm(N, generator=g)[:w5.n_ignored]] = -100
    t = t.to(dev)
    red = args.reduction or "mean"
    nb, chunk = vce.ce_linear_workspace_bytes(h, W, red, args.chunk_rows, w5.alpha, smoothing=args.smoothing)
    ws = vce.ce_workspace_init(torch.empty(nb, dtype=torch.uint8, device=dev))
    loss = torch.empty(1 if red != "none" else N, dtype=torch.float32, device=dev)
    dh = torch.empty_like(h)
    dw = torch.empty((V, D), dtype=torch.float32, device=dev)
    n = torch.empty(1, dtype=torch.int32, device=dev)
    if args.tune:
        t_tune = time.perf_counter()
        vce.ce_linear_tune(h, W, red, dh=dh, dw=dw, chunk_rows=args.chunk_rows, ws=ws, label_smoothing=w5.alpha,
                           smoothing=args.smoothing, gemm=args.gemm)
        print(f"[bench] tuned the GEMMs in {time.perf_counter() - t_tune:.1f} s", file=sys.stderr, flush=True)

    def step():
        vce.ce_linear_cross_entropy(h, W, t, w5.alpha, red, loss=loss, n_valid=n, dh=dh, dw=dw, ws=ws,
                                    chunk_rows=args.chunk_rows, smoothing=args.smoothing, gemm=args.gemm)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / args.steps
    nchunks = (N + chunk - 1) // chunk
    with vce.Profiler(args.steps * nchunks) as prof:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
    ce_ms = sum(prof.ms) / args.steps          # the fused cross-entropy kernels of one step
    flops = 6.0 * N * D * V                     # logits, dh and dW products
    gemm_ms = step_ms - ce_ms                   # the GEMMs and the two small count/finish kernels
    ws_bytes = ws.numel()
    out = {
        "metric": "chunked linear head + cross-entropy fwd+bwd: TFLOP/s of its three GEMMs, step time",
        "value": round(flops / (step_ms * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"linear_ce_n{N}_d{D}_v{V}_bf16", "rows": N, "hidden": D, "vocab": V,
                   "chunk_rows": chunk, "chunks": nchunks, "reduction": red, "smoothing": args.smoothing,
                   "tuned": bool(args.tune), "gemm": args.gemm,
                   "native_products": vce.ce_linear_gemm_plan(h, W, args.gemm),
                   "label_smoothing": w5.alpha},
        "roofline": {"bound": "mfma", "achieved": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "the three products (native MFMA kernel for the products in native_products, bit 0 "
                               "logits, 1 dh, 2 dW; hipBLASLt for the rest): step time minus the fused "
                               "cross-entropy kernels"},
        "cross_entropy": {"us_per_step": round(ce_ms * 1e3, 1), "share": round(ce_ms / step_ms, 4),
                          "GBps": round(2 * N * V * 2 / (ce_ms * 1e-3) / 1e9, 1)},
        "memory": {"workspace_bytes": ws_bytes, "full_logits_bytes": N * V * 2},
        "loss": float(loss[0].item()) if red != "none" else None,
        "device": device_info(torch, dev),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_linear(h, W, t, w5.alpha, red, args.smoothing, n_rows=4)
    line = json.dumps(out)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")
    print(line, flush=True)


if __name__ == "__main__":
    main()
