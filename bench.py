#!/usr/bin/env python3
"""Throughput of the fused guided denoising step on one MI355X.

One bench step = one sampler step of the large bf16 workload: 256 samples,
latent 16x128x128 stored in bf16 (fp32 arithmetic), 2 feathered regional
conds + uncond per sample, 8 guidance buckets on a linear 2.0 -> 1.2 curve,
mixed per-sample progress over a 50-step log-linear Euler schedule.  Each
step is one fused launch (guided_step_dplan) that builds the step's bucket
plan on the device -- bucket ids, scales, uncond decisions, the stable
(bucket, sample) order, offsets and rows -- and advances every sample, all
inside libbcg's native loop (--plan host: the plan is built on the host and
uploaded instead; --graph G: runs of G launches replay a captured graph).
Progress is steady-state continuous batching (sample i at step
(start_i + k) mod 50), so every launch is full and mixes all 8 buckets.
With --replicas R > 1, R independent batches are served round-robin, which
keeps the working set (R x 128 MiB) beyond the 256 MB last-level cache so
every launch streams from HBM.

Prints one JSON line (metric, value in latent element-steps/s, roofline of
the guided_step kernel against 8 TB/s HBM, and the CPU oracle's rate).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "latent element-steps/sec on 1 GPU + achieved HBM GB/s as % of peak"
PEAK_HBM_GBS = 8000.0
# the bench kernel's device code and its launch shape (a traffic record is
# void once any of them changes)
KERNEL_SOURCES = ["bcg_step_impl.h", "bcg_device.h", "bcg_plan_dev.h", "bcg_launch.h", "bcg_step_bf16_nt.hip",
                  "bcg_step_bf16_queue.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "guided_step_large_bf16_traffic.json")


WEIGHT_SOURCES = ["bcg_weight.hip", "bcg_device.h", "bcg_launch.h"]


def weight_traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"weight_patch_{workload}_traffic.json")


def kernel_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bucketed_classifier_free_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def bytes_per_element(spec) -> float:
    """Algorithmic HBM bytes per latent element-step of guided_step: read x,
    write x', plus x_orig and a mask shared by the C channels when inpainting."""
    es = 2 if spec.dtype == "bf16" else 4
    b = 2 * es
    if spec.inpaint:
        b += es + 4.0 / spec.C
    return b


def cpu_baseline(inp, seconds: float):
    """The float64 oracle's step function on a bounded sample of the workload."""
    import numpy as np
    from oracle import definition as D
    sp = inp.spec
    sig, table, cov = D.run_setup(inp)
    x = D.init_latent(inp, sig, sp.dtype)
    t = inp.start_step.astype(np.int64)
    plan = D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov)
    elems = 0
    done = 0
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        ti = int(t[i])
        D.step(x[i], float(sig[ti]), float(sig[ti + 1]), float(plan["scale"][i]),
               D.sample_params(inp, i), sp.sampler)
        elems += sp.C * sp.H * sp.W
        done += 1
        i = (i + 1) % sp.n
    dt = time.perf_counter() - t0
    return {"value": elems / dt, "unit": "element-steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} sample-steps of {sp.name} (float64 NumPy definition, one thread; "
                      f"{len(os.sched_getaffinity(0))} cores available), {dt:.1f} s"}


def _oracle_worker(job):
    """One process of the parallel oracle baseline: its own copy of the seeded
    inputs, the float64 step on its share of the samples for `seconds`."""
    import dataclasses
    import numpy as np
    import workloads as W
    from oracle import definition as D
    name, nb, idx, seconds = job
    sp = W.config(name)
    if nb:
        sp = dataclasses.replace(sp, num_buckets=nb)
    inp = W.make_inputs(sp)
    sig, table, cov = D.run_setup(inp)
    x = D.init_latent(inp, sig, sp.dtype)
    t = inp.start_step.astype(np.int64)
    plan = D.build_plan(t, sp.steps, sp.num_buckets, table, inp.cfg_override, cov)
    elems = done = 0
    t0 = time.perf_counter()
    q = 0
    while time.perf_counter() - t0 < seconds:
        i = idx[q % len(idx)]
        ti = int(t[i])
        D.step(x[i], float(sig[ti]), float(sig[ti + 1]), float(plan["scale"][i]),
               D.sample_params(inp, i), sp.sampler)
        elems += sp.C * sp.H * sp.W
        done += 1
        q += 1
    return elems, done, time.perf_counter() - t0


def cpu_parallel(spec, nb, seconds: float, workers: int):
    """The same oracle step sharded over `workers` fresh processes (samples dealt
    round-robin), started before this process touches the GPU."""
    import multiprocessing as mp
    jobs = [(spec.name, nb, list(range(w, spec.n, workers)), seconds) for w in range(workers)]
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_oracle_worker, jobs)
    elems = sum(r[0] for r in res)
    rate = sum(r[0] / r[2] for r in res)
    return {"value": rate, "unit": "element-steps/s", "cores": workers, "kind": "oracle",
            "sample": f"{sum(r[1] for r in res)} sample-steps of {spec.name} over {workers} processes "
                      f"(float64 NumPy definition, one thread each), {seconds:.0f} s each, {elems} element-steps"}


def copy_probe(mib: int, iters: int):
    """Plain device copy of a known size (counter scale reference)."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    print(json.dumps({"copy_probe_mib": mib, "ms": ms, "GBps": 2 * mib * (1 << 20) / ms / 1e6}))


def _counter_means(path, counter, last=0):
    """Mean per dispatch of a counter, per kernel name (over the last `last`
    dispatches of each kernel when last > 0: the timed launches, after the
    warm-up's)."""
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    out = {}
    for k, d in acc.items():
        v = [d[i] for i in sorted(d)]
        v = v[-last:] if last > 0 else v
        out[k] = sum(v) / len(v)
    return out


def traffic_from_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib, workload,
                          kernel="guided_step_kernel", sources=None, last=0):
    """Per-launch HBM bytes of a kernel (guided_step by default) from two
    rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each
    scaled by what the same counter reads for a plain device copy of copy_mib
    MiB."""
    copy_bytes = copy_mib * (1 << 20)
    pick = lambda d, key: max((v for k, v in d.items() if key in k), default=None)
    cf = pick(_counter_means(copy_fetch_csv, "FETCH_SIZE"), "copyBuffer")
    cw = pick(_counter_means(copy_write_csv, "WRITE_SIZE"), "copyBuffer")
    f = pick(_counter_means(fetch_csv, "FETCH_SIZE", last), kernel)
    w = pick(_counter_means(write_csv, "WRITE_SIZE", last), kernel)
    rf, rw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    return {"workload": workload, "kernel": kernel, "kernel_hash": kernel_hash(sources),
            "fetch_kib_raw": f, "write_kib_raw": w, "copy_fetch_kib_raw": cf,
            "copy_write_kib_raw": cw, "copy_mib": copy_mib, "dispatches": last or "all",
            "fetch_scale": rf, "write_scale": rw,
            "bytes_per_launch": f * 1024 * rf + w * 1024 * rw}


def rows_bench(inp, args):
    """Steady state of the materialised-branch update: guided_step_rows reads
    each batch's model-output rows in the layout of that step's device-built
    plan.  By default the launch also builds the batch's next plan
    (guided_step_rows_dplan: the plan of step m+1 is due before the model's
    forward of step m+1, i.e. after the update of step m); --rows-plan separate
    builds each step's plan in its own launch (bcg_plan_device) first.  The rows
    are synthetic and resident (one buffer per batch and evaluation: no model
    runs here); the uncond rows of samples whose uncond branch is skipped are
    neither produced nor read."""
    import numpy as np
    import torch
    from bucketed_classifier_free_amd import GuidedSampler, api
    from bucketed_classifier_free_amd import _lib as L
    spec = inp.spec
    s = GuidedSampler.from_inputs(inp, wrap=True)
    n, R = spec.n, max(1, args.replicas)
    heun = spec.sampler == "heun"
    evals = 2 if heun else 1
    x = torch.empty((R, n, spec.C, spec.H, spec.W), dtype=s.tdtype, device="cuda")
    for r in range(R):
        s.init_state(x[r])
    g = torch.Generator(device="cuda")
    g.manual_seed(spec.seed)
    pred = torch.randn((R, evals, 2 * n, spec.C, spec.H, spec.W), generator=g, device="cuda").to(s.tdtype)
    dbuf = torch.empty((n, spec.C, spec.H, spec.W), dtype=torch.float32, device="cuda") if heun else None
    xt = torch.empty_like(x[0]) if heun else None
    fused = args.rows_plan == "fused"
    # step indices: three buffers per batch (step m's, read by its update, while
    # the fused plan of step m+1 reads m+1's and writes m+2's); two plans per batch
    steps_state = torch.empty((R, 3, n), dtype=torch.int32, device="cuda")
    steps_state[:, 0] = torch.from_numpy(s.step_indices(0)).cuda()
    plans = [[api.device_plan_arrays(n, s.nb) for _ in range(2)] for _ in range(R)]
    hint = L.BCG_CACHE_STREAM if R > 1 else L.BCG_CACHE_KEEP
    opt = dict(x_orig=s.d_x_orig, mask=s.d_mask, cache_hint=hint)
    pkw = dict(cfg_override=s.d_override, covered=s.d_covered, wrap=True, bucket_cfg_end=s.d_table_end)

    def build_plan(r, m):  # the plan of batch r's step m, in its own launch
        api.bcg_plan_device(s.steps, s.d_table, steps_state[r, m % 3], step_out=steps_state[r, (m + 1) % 3],
                            out=plans[r][m & 1], **pkw)

    if fused:
        for r in range(R):
            build_plan(r, 0)

    def step(k):
        r, m = k % R, k // R
        if not fused:
            build_plan(r, m)
        pl = plans[r][m & 1]
        rows = dict(order=pl["order"], step_idx=steps_state[r, m % 3], scale=pl["scale"],
                    uncond_row=pl["uncond_row"], cond_row=pl["cond_row"])
        first = dict(phase="heun_predict", d=dbuf) if heun else dict(phase="euler")
        out0 = xt if heun else x[r]
        if fused:
            nxt = api.device_plan(s.steps, s.d_table, steps_state[r, (m + 1) % 3],
                                  step_out=steps_state[r, (m + 2) % 3], out=plans[r][(m + 1) & 1], **pkw)
            api.guided_step_rows_dplan(x[r], out0, pred[r, 0], s.d_sigmas, n_active=n, plan=nxt,
                                       **first, **rows, **opt)
        else:
            api.guided_step_rows(x[r], out0, pred[r, 0], s.d_sigmas, n_active=n, **first, **rows, **opt)
        if heun:
            api.guided_step_rows(x[r], x[r], pred[r, 1], s.d_sigmas, n_active=n, phase="heun_correct",
                                 d=dbuf, x_tilde=xt, **rows, **opt)

    # Whole steps replayed from a graph of G steps: G is a multiple of the
    # step-buffer period 6R, so replays continue the sequence.
    G = 6 * R * max(1, -(-16 // (6 * R)))
    for k in range(G):
        step(k)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(G):
            step(k)
    reps = max(1, args.steps // G)
    for _ in range(max(1, args.warmup // G)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not torch.isfinite(x.float()).all():
        raise RuntimeError("non-finite state after the timed steps")
    nsteps = reps * G
    step_ms = e0.elapsed_time(e1) / nsteps
    # bytes per element-step: x read + x' write, the cond row, the uncond rows of the samples
    # that keep them (the skip set does not change between steps here), per evaluation
    p0 = s.plan(0)
    keep = p0.n_uncond / max(p0.n_active, 1)
    es = 2 if spec.dtype == "bf16" else 4
    if heun:  # predictor: x, C, U, writes x~ and d; corrector: x, d, C, U, writes x'
        bpe = (es + es + keep * es + es + 4) + (es + 4 + es + keep * es + es)
    else:
        bpe = es + es + keep * es + es
    if spec.inpaint:
        bpe += evals * (es + 4.0 / spec.C)
    elems = n * spec.C * spec.H * spec.W
    achieved = bpe * elems / (step_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "materialised-branch guided update, latent element-steps/sec on 1 GPU",
        "value": elems * nsteps / wall, "unit": "element-steps/s", "n_gpus": 1,
        "steps": nsteps, "warmup": G * max(1, args.warmup // G), "ms_per_step": wall * 1e3 / nsteps,
        "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": spec.name, "batch": n, "latent": [spec.C, spec.H, spec.W],
                   "storage": spec.dtype, "sampler": spec.sampler, "replicas": R,
                   "uncond_rows_kept": keep,
                   "plan": ("device, the next step's built in the update's launch" if fused
                            else "device (its own launch before the update)"),
                   "graph_steps": G},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None},
        "kernel": {"name": "guided_step_rows", "calls_per_step": evals,
                   "avg_us_per_step": step_ms * 1e3, "bytes_per_element_step": bpe,
                   "timing": "events around the graph replays; a step is the update launch(es) and "
                             "the plan (in the first update launch, or its own launch), so achieved "
                             "GB/s is a lower bound for the update"}}),
        flush=True)


def weight_cpu_baseline(inp, seconds: float):
    """The weight-patch oracle (float64 definition of the patched rows, then
    the float32 order and the store) on consecutive blocks of 64 rows."""
    from oracle import weight_patch as P
    from workloads import weights as WW
    sp = inp.spec
    t0 = time.perf_counter()
    done = 0
    r = 0
    while time.perf_counter() - t0 < seconds:
        r1 = min(r + 64, sp.rows)
        pats, specs = [], []
        for pd in inp.patches:
            ps = pd.spec
            a, b = max(r, ps.offset), min(r1, ps.offset + pd.rows)
            if a >= b:
                continue
            one = WW.PatchSpec(ps.kind, a - r, b - a, ps.rank, ps.strength_patch, ps.strength_model, ps.dtype)
            specs.append(one)
            k0, k1 = a - ps.offset, b - ps.offset
            pats.append(WW.PatchData(one, b - a, None if pd.diff is None else pd.diff[k0:k1],
                                     None if pd.up is None else pd.up[k0:k1], pd.down))
        sub = WW.WeightInputs(WW.WeightSpec(sp.name, r1 - r, sp.cols, sp.w_dtype, sp.out_dtype, tuple(specs),
                                            sp.rounding, sp.sr_seed, sp.seed), inp.w[r:r1], pats)
        acc = P.reference32(sub)
        P.reference(sub)
        if sp.rounding == "stochastic" and sp.out_dtype == "bf16":
            P.sr_bf16(acc, sp.sr_seed, base=r * sp.cols)
        else:
            P.store(acc, sp.out_dtype)
        done += (r1 - r) * sp.cols
        r = r1 % sp.rows
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "weight elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{done // sp.cols} rows of {sp.name} in blocks of 64 (float64 definition, float32 "
                      f"order and store, NumPy, one thread), {el:.1f} s"}


def weight_bench(name, args, cpu=None):
    """One weight_patch launch per step over resident inputs: the weight, its
    patch tensors and the output, replicated R times (rotated per launch) so
    the 256 MB last-level cache cannot hold them between launches; launches
    captured in a graph and timed with HIP events around its replays."""
    import torch
    from bucketed_classifier_free_amd import WeightPatch, weight_patch
    from workloads import weights as WW
    sp = WW.weight_config(name)
    if args.rounding:
        import dataclasses
        sp = dataclasses.replace(sp, rounding=args.rounding)
    inp = WW.make_weight_inputs(sp)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    R = max(1, args.replicas)
    reps = []
    for _ in range(R):
        w = torch.from_numpy(inp.w).cuda().to(tdt[sp.w_dtype])
        out = torch.empty(w.shape, dtype=tdt[sp.out_dtype], device="cuda")
        pats = []
        for pd in inp.patches:
            ps = pd.spec
            if ps.kind == "diff":
                pats.append(WeightPatch(ps.strength_patch, ps.strength_model, ps.offset,
                                        diff=torch.from_numpy(pd.diff).cuda().to(tdt[ps.dtype])))
            else:
                pats.append(WeightPatch(ps.strength_patch, ps.strength_model, ps.offset,
                                        up=torch.from_numpy(pd.up).cuda().to(torch.bfloat16),
                                        down=torch.from_numpy(pd.down).cuda().to(torch.bfloat16)))
        reps.append((w, out, pats))

    def launch(k):
        w, out, pats = reps[k % R]
        weight_patch(w, out, pats, rounding=sp.rounding, seed=sp.sr_seed + k)

    G = R * max(1, -(-16 // R))
    for k in range(G):
        launch(k)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(G):
            launch(k)
    nrep = max(1, args.steps // G)
    for _ in range(max(1, args.warmup // G)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(nrep):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not all(torch.isfinite(r[1].float()).all() for r in reps):
        raise RuntimeError("non-finite weights after the timed launches")
    n = nrep * G
    launch_ms = e0.elapsed_time(e1) / n
    elems = sp.rows * sp.cols
    es = {"f32": 4, "bf16": 2}
    alg = elems * (es[sp.w_dtype] + es[sp.out_dtype])
    flops = 0
    for pd in inp.patches:
        ps = pd.spec
        if ps.kind == "diff":
            alg += pd.rows * sp.cols * es[ps.dtype]
        else:
            alg += 2 * (pd.rows * ps.rank + ps.rank * sp.cols)
            flops += 2 * pd.rows * sp.cols * ps.rank
    achieved = alg / (launch_ms * 1e-3) / 1e9
    traffic = None
    tf = weight_traffic_file(sp.name)
    if os.path.exists(tf) and not args.rounding:
        with open(tf) as fh:
            tr = json.load(fh)
        if tr.get("kernel_hash") == kernel_hash(WEIGHT_SOURCES) and tr.get("workload") == sp.name:
            traffic = tr.get("bytes_per_launch")
    out = {
        "metric": "weight elements patched/sec on 1 GPU",
        "value": elems * n / wall, "unit": "weight elements/s", "n_gpus": 1, "steps": n,
        "warmup": G * max(1, args.warmup // G), "ms_per_step": wall * 1e3 / n,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": sp.name, "weight": [sp.rows, sp.cols], "w_dtype": sp.w_dtype,
                   "out_dtype": sp.out_dtype, "rounding": sp.rounding,
                   "patches": [{"kind": p.kind, "offset": p.offset, "rows": d.rows, "rank": p.rank,
                                "strength_patch": p.strength_patch, "strength_model": p.strength_model}
                               for p, d in zip(sp.patches, inp.patches)],
                   "replicas": R, "graph_launches": G},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "kernel": {"name": "weight_patch", "avg_launch_us": launch_ms * 1e3,
                   "kernel_hash": kernel_hash(WEIGHT_SOURCES),
                   "timing": f"HIP events around replays of a {G}-launch graph",
                   "algorithmic_bytes_per_launch": alg, "lowrank_flops_per_launch": flops,
                   "mfma_tflops": flops / (launch_ms * 1e-3) / 1e12},
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def trajectory(inp, args):
    """Whole trajectories end to end: latent init and every step of the
    schedule (device plans, the steps replayed from one captured graph, one
    batch in place), counting the active samples of each launch only."""
    import numpy as np
    import torch
    from bucketed_classifier_free_amd import GuidedSampler
    spec = inp.spec
    s = GuidedSampler.from_inputs(inp)
    x = s.alloc_state()
    starts = inp.start_step.astype(np.int64)
    launches = int(spec.steps - starts.min())
    G = launches  # one graph replay per trajectory
    loop = s.native_loop(x, device_plan=True, graph_launches=G)
    t = starts[:, None] + np.arange(launches)[None, :]
    elems = int(((t >= 0) & (t < spec.steps)).sum()) * spec.C * spec.H * spec.W
    reps = max(1, args.steps // launches)
    for _ in range(2):  # warm-up trajectories
        s.init_state(x)
        loop.run(0, launches)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        s.init_state(x)
        loop.run(0, launches)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    if not torch.isfinite(x.float()).all():
        raise RuntimeError("non-finite state after the trajectories")
    loop.close()
    print(json.dumps({
        "metric": "full-trajectory latent element-steps/sec on 1 GPU (init + every step, active samples only)",
        "value": elems / wall, "unit": "element-steps/s", "n_gpus": 1, "trajectories": reps,
        "ms_per_trajectory": wall * 1e3, "launches": launches, "higher_is_better": True,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.n, "latent": [spec.C, spec.H, spec.W],
                   "storage": spec.dtype, "sampler": spec.sampler, "schedule_steps": spec.steps,
                   "buckets": spec.num_buckets, "regions": spec.regions, "inpaint": spec.inpaint,
                   "plan": "device", "graph_launches": G}}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="large_bf16")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-workers", type=int, default=-1,
                    help="processes of the parallel oracle baseline (-1: the affinity cores, at most 16; 0: off)")
    ap.add_argument("--buckets", type=int, default=0, help="override the workload's bucket count")
    ap.add_argument("--rows-plan", choices=("fused", "separate"), default="fused",
                    help="with --rows: the next step's plan built in the update's launch (fused) or "
                         "each step's plan in its own launch first (separate)")
    ap.add_argument("--rows", action="store_true",
                    help="materialised branches: time guided_step_rows on model-output rows laid out "
                         "by a device-built plan (both Heun calls for a Heun workload)")
    ap.add_argument("--trajectory", action="store_true",
                    help="time whole trajectories (latent init + every step, active samples only) "
                         "instead of the steady state")
    ap.add_argument("--weight-patch", default="", metavar="WORKLOAD",
                    help="time weight_patch on a weight workload (workloads/weights.py) instead")
    ap.add_argument("--rounding", choices=("nearest", "stochastic"), default="",
                    help="bf16 rounding of the weight workload (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--upload-batch", type=int, default=8)
    ap.add_argument("--async-upload", type=int, default=0)
    ap.add_argument("--plan", choices=("device", "host"), default="device")
    ap.add_argument("--join-front", type=int, default=-1, metavar="J",
                    help="continuous batching: joins of a step dispatched first (-1: the loop's default)")
    ap.add_argument("--queue", type=int, default=512, metavar="Q",
                    help="continuous batching (device plans): the batch's slots are refilled from an "
                         "endless queue over a pool of Q requests (0: every finished slot restarts "
                         "at step 0 from its own latent instead)")
    ap.add_argument("--records", type=int, default=1,
                    help="device plans: each launch's plan writes the next step's sample records")
    ap.add_argument("--graph", type=int, default=40, metavar="G",
                    help="device plans: the timed launches run as replays of a captured graph of "
                         "min(G, --steps) launches (0 = direct launches)")
    ap.add_argument("--counter-last", type=int, default=0, metavar="N",
                    help="--traffic-from: average the kernel's counters over its last N dispatches (the timed "
                         "launches of the counted run; 0: all)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write the traffic record from rocprofv3 --pmc counter CSVs and exit")
    args = ap.parse_args()
    if args.traffic_from and args.weight_patch:
        kern = "patch_stream" if "diff" in args.weight_patch else "patch_lowrank"
        rec = traffic_from_counters(*args.traffic_from, 256, args.weight_patch, kern, WEIGHT_SOURCES,
                                    args.counter_last)
        with open(weight_traffic_file(args.weight_patch), "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec))
        return
    if args.traffic_from:
        rec = traffic_from_counters(*args.traffic_from, 256, args.workload, last=args.counter_last)
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path keeps every sample on one device and its "
              "multi-GPU form (sample-sharded, no per-step communication) is not built; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import workloads as W

    if args.weight_patch:
        from workloads import weights as WW
        wcpu = None
        if not args.no_cpu_baseline:  # before anything touches the GPU
            wcpu = weight_cpu_baseline(WW.make_weight_inputs(WW.weight_config(args.weight_patch)),
                                       min(args.cpu_seconds, 10.0))
        import torch
        from bucketed_classifier_free_amd import load
        load()
        torch.cuda.set_device(0)
        weight_bench(args.weight_patch, args, wcpu)
        return

    spec = W.config(args.workload)
    if args.buckets:
        spec = dataclasses.replace(spec, num_buckets=args.buckets)
    inp = W.make_inputs(spec) if not args.copy_probe else None
    cpu = None
    if not args.no_cpu_baseline and not args.copy_probe and not args.trajectory and not args.rows:
        # the oracle legs run before anything here touches the GPU
        cpu = cpu_baseline(inp, args.cpu_seconds)
        workers = args.cpu_workers if args.cpu_workers >= 0 else min(16, len(os.sched_getaffinity(0)))
        if workers > 1:
            cpu["parallel"] = cpu_parallel(spec, args.buckets, min(args.cpu_seconds, 10.0), workers)

    import numpy as np
    import torch

    from bucketed_classifier_free_amd import GuidedSampler, load

    load()
    if args.copy_probe:
        copy_probe(args.copy_probe, 50)
        return
    torch.cuda.set_device(0)
    if args.trajectory:
        trajectory(inp, args)
        return
    if args.rows:
        rows_bench(inp, args)
        return
    R = max(1, args.replicas)
    dev_plan = args.plan == "device"
    queue = dev_plan and args.queue > 0
    if queue:
        # the request pool: the workload's draws for Q requests (the first n
        # start in the slots at their mixed start steps)
        if args.queue < spec.n:
            raise SystemExit("--queue must be at least the batch size")
        s = GuidedSampler.from_inputs(W.make_inputs(dataclasses.replace(spec, n=args.queue)))
        x = torch.empty((R, spec.n, spec.C, spec.H, spec.W), dtype=s.tdtype, device="cuda")
    else:
        s = GuidedSampler.from_inputs(inp, wrap=True)
        x = torch.empty((R, spec.n, spec.C, spec.H, spec.W), dtype=s.tdtype, device="cuda")
        for r in range(R):
            s.init_state(x[r])
    # one graph replay covers up to G launches of the timed run
    G = min(args.graph, args.steps) if dev_plan else 0
    loop = s.native_loop(x if R > 1 else x[0], upload_batch=args.upload_batch,
                         async_upload=bool(args.async_upload), device_plan=dev_plan,
                         graph_launches=G, records=bool(args.records) or queue,
                         slots=spec.n if queue else None, ring=queue,
                         join_front=None if args.join_front < 0 else args.join_front)
    loop.run(0, args.warmup)
    torch.cuda.synchronize()
    elems_per_launch = spec.n * spec.C * spec.H * spec.W  # every sample active (steady state)
    t0 = time.perf_counter()
    launch_ms = loop.run(args.warmup, args.steps, timing=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    replayed, direct = loop.last_run()
    if not torch.isfinite(x.float()).all():
        raise RuntimeError("non-finite state after the timed steps")

    if not launch_ms > 0:
        raise RuntimeError("no launch was timed (--steps must be >= 1)")
    value = elems_per_launch * args.steps / wall
    bpe = bytes_per_element(spec)
    alg_bytes = bpe * elems_per_launch
    joins = 0
    if queue:
        # a joining request reads its fp32 noise (4 B per element) instead of
        # the slot's state: slot i's request finishes every `steps` launches of
        # its replica, first after steps - start_i of them
        st0 = s.start[:spec.n].astype(np.int64)
        for k in range(args.warmup, args.warmup + args.steps):
            m = k // R  # the replica's own launch index
            first = spec.steps - st0
            joins += int(((m >= first) & ((m - first) % spec.steps == 0)).sum())
        es = 2 if spec.dtype == "bf16" else 4
        alg_bytes += (4 - es) * spec.C * spec.H * spec.W * joins / args.steps
    achieved = alg_bytes / (launch_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        if tr.get("kernel_hash") == kernel_hash() and tr.get("workload") == spec.name:
            traffic = tr.get("bytes_per_launch")
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "element-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.n, "latent": [spec.C, spec.H, spec.W],
                   "storage": spec.dtype, "sampler": spec.sampler, "schedule_steps": spec.steps,
                   "buckets": spec.num_buckets, "regions": spec.regions,
                   "progress": ("continuous batching: slots refilled from an endless queue over "
                                f"{args.queue} requests ({joins} joins in the timed launches)" if queue
                                else "mixed, steady state (finished slots restart at step 0)"),
                   "replicas": R, "plan": args.plan},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "kernel": {"name": "guided_step", "avg_launch_us": launch_ms * 1e3,
                   "timing": (f"one pair of HIP events on the launch stream around all {args.steps} timed "
                              f"launches ({replayed} inside replays of a {G}-launch graph, {direct} "
                              f"launched directly); mean per launch, gaps between launches included"),
                   "launches_replayed": replayed, "launches_direct": direct,
                   "algorithmic_bytes_per_launch": alg_bytes, "bytes_per_element_step": bpe,
                   "element_steps_per_s_kernel_only": elems_per_launch / (launch_ms * 1e-3),
                   "kernel_hash": kernel_hash()},
    }
    if dev_plan:
        out["config"]["graph_launches"] = G
    else:
        out["config"].update(plan_upload_batch=args.upload_batch, async_upload=bool(args.async_upload))
    if cpu is not None:
        out["cpu_baseline"] = cpu
    loop.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
