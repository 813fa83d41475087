#!/usr/bin/env python3
"""Benchmark of the heterogeneous batched LoRA path on one MI355X.

One step = one apply over every projection of the workload for the whole token
batch (plan on the host into pinned memory, then the fused launches; a run of
same-shape projections goes through one slora_apply_multi, --per-projection: one
slora_apply each), adapters already resident in HBM. The default workload is the
Llama-7B-shape decode batch:
256 decode tokens, one 4096 -> 4096 projection, Zipf(1.0) routing over 1000
adapters with ranks in {8, 16, 32, 64}, fp16.

Steps rotate over --instances independent copies of the workload (own pool, own
pages, own x / y), about 0.5 GiB each, so the 256 MB Infinity Cache cannot hold
the weights of the instance being timed: the kernels read adapter pages from HBM.

Printed: one JSON line on stdout: tokens/s, the roofline of the dominant kernel
from HIP events the launches record (with p10/p50/p90 of its launch durations), a
plain device copy as a reachable-bandwidth reference, the CPU oracle's rate on the
host cores, the adapter fetch rate beside a copy-engine host-to-device copy of the
same bytes, and GPU / host facts. With the default decode workload the same line
carries a `prefill` record: the prefill SGMV batch (64 requests, q/k/v/o 4096 ->
4096, bf16) timed the same way, with the HBM and MFMA fractions of its launch.
Every instance's workspace status is read after the timed steps; a fused launch
whose wait gave up makes the run exit with status 3. Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16
METRIC = "LoRA tokens/s + % peak HBM (decode MBGMV), % MFMA peak (prefill SGMV)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(wl, proj, call):
    """Per-kernel algorithmic bytes and flops of one apply of projection `proj`, split by
    the family the library's own plan (slora_plan_inspect) gives each group of tokens.

    Weights of every distinct adapter a family uses are read once by that family's
    kernels; x is read once, y0 read and y written once per routed token. Intermediates
    (v), page tails and work lists are not counted."""
    from heterogeneous_lora_amd import _lib
    p = wl.projections[proj]
    e = 2
    groups, _ = _lib.plan_inspect(call)
    out = {}
    for fam_id, f in ((0, "mbgmv"), (1, "sgmv")):
        g = groups[groups[:, 0] == fam_id] if len(groups) else np.zeros((0, 5), np.int32)
        T = int(g[:, 2].sum())
        rank_of = {int(row[3]): int(row[4]) for row in g}  # adapters by first page-table entry
        r_sum = sum(rank_of.values())
        tok_r = int((g[:, 2].astype(np.int64) * g[:, 4].astype(np.int64)).sum())
        out[f + "_shrink"] = dict(bytes=int(r_sum * p.d_in * e + T * p.d_in * e),
                                  flops=int(2 * tok_r * p.d_in), tokens=T, adapters=len(rank_of))
        out[f + "_expand"] = dict(bytes=int(r_sum * p.d_out * e + 2 * T * p.d_out * e),
                                  flops=int(2 * tok_r * p.d_out), tokens=T, adapters=len(rank_of))
        out[f + "_fused"] = {k: out[f + "_shrink"][k] + out[f + "_expand"][k] for k in ("bytes", "flops")}
        out[f + "_fused"].update(tokens=T, adapters=len(rank_of))
    # both families in one launch (a call with decode groups and segments in one launch)
    out["mixed_fused"] = {k: out["mbgmv_fused"][k] + out["sgmv_fused"][k]
                          for k in ("bytes", "flops", "tokens", "adapters")}
    for f in ("sgmv_shrink", "sgmv_expand", "sgmv_fused", "mixed_fused"):
        out[f]["mfma_flops"] = out["sgmv_" + f.split("_")[1] if f.startswith("sgmv") else "sgmv_fused"]["flops"]
    return out


def launch_work(alg, groups):
    """Algorithmic [bytes, flops, matrix-core flops] of every timed interval a step has,
    per kernel id, from the per-projection figures of algorithmic(): one interval per
    projection and kernel id, except a slora_apply_multi's, which covers its group of
    projections (both families in one interval, multi_fused)."""
    per = {}
    for g in groups:
        if len(g) > 1:
            fam = [sum(alg[p][f][q] for p in g for f in ("mbgmv_fused", "sgmv_fused")) for q in ("bytes", "flops")]
            per.setdefault("multi_fused", []).append(fam + [sum(alg[p]["sgmv_fused"]["flops"] for p in g)])
        else:
            for k, a in alg[g[0]].items():
                per.setdefault(k, []).append([a["bytes"], a["flops"], a.get("mfma_flops", 0)])
    return per


def projection_groups(wl, multi):
    """Projections one step applies together: with multi, runs of consecutive projections
    of one shape (one slora_apply_multi each); otherwise one projection per call."""
    groups = []
    for p, pr in enumerate(wl.projections):
        if multi and groups and (wl.projections[groups[-1][0]].d_in, wl.projections[groups[-1][0]].d_out) == (pr.d_in, pr.d_out):
            groups[-1].append(p)
        else:
            groups.append([p])
    return groups


# Source files each kernel family is compiled from (a counter summary is void once they change).
KERNEL_SOURCES = {
    fam: [f"heterogeneous_lora_amd/csrc/{src}.hip", "heterogeneous_lora_amd/csrc/mbgmv_dev.h",
          "heterogeneous_lora_amd/csrc/device_common.h", "heterogeneous_lora_amd/csrc/internal.h"]
    for fam, src in (("mbgmv", "mbgmv"), ("sgmv", "sgmv"), ("mixed", "sgmv"), ("multi", "sgmv"))
}


def sources_sha256(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel.split("_")[0]]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(kernel, workload):
    """HBM traffic per launch from a committed rocprofv3 PMC summary, or None when the
    summary is missing or the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("sources_sha256") != sources_sha256(kernel):
        return None
    return d.get("traffic_bytes_per_launch")


def calib_copy(nbytes, reps):
    """Plain copies of known size, the reference the byte counters are scaled by: `reps`
    launches of torch's elementwise kernel computing dst = src * 1 over nbytes (ordinary
    loads and stores), then `reps` device-to-device copies (the runtime's copy kernel)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": nbytes, "launches": reps}), flush=True)


def _pmc_mean_kib(path, match, counter):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if match in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {match!r} in {path}")
    return float(np.mean(vals)), len(vals)


def pmc_summary(a):
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) of a kernel and of the
    calibration copy into HBM bytes per launch; writes profiles/pmc_<kernel>_<workload>.json."""
    fk, fn = _pmc_mean_kib(a.fetch_csv, a.match, "FETCH_SIZE")
    wk, wn = _pmc_mean_kib(a.write_csv, a.match, "WRITE_SIZE")
    cfk, _ = _pmc_mean_kib(a.calib_fetch_csv, a.calib_match, "FETCH_SIZE")
    cwk, _ = _pmc_mean_kib(a.calib_write_csv, a.calib_match, "WRITE_SIZE")
    f_scale = a.calib_bytes / (cfk * 1024.0)
    w_scale = a.calib_bytes / (cwk * 1024.0)
    out = {
        "kernel": a.kernel, "workload": a.workload,
        "sources": KERNEL_SOURCES[a.kernel.split("_")[0]], "sources_sha256": sources_sha256(a.kernel),
        "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
        "dispatches": [fn, wn],
        "calib_copy_bytes": a.calib_bytes,
        "calib_fetch_kib": round(cfk, 1), "calib_write_kib": round(cwk, 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "traffic_bytes_per_launch": int(fk * 1024 * f_scale + wk * 1024 * w_scale),
        "commands": a.commands.split(" ;; ") if a.commands else [],
    }
    path = os.path.join(ROOT, "profiles", f"pmc_{a.kernel}_{a.workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def oracle_threads():
    """Threads the oracle baseline runs on: every core this process may use, capped at the
    CPU share one job gets on the GPU host (16 cores per GPU; OMP_NUM_THREADS says so there)."""
    aff = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return max(1, min(aff, share)), aff


def cpu_baseline(wl, budget_s, threads=None, single_thread_s=0.0):
    """The oracle (fp64 C loops, threads over tokens) on the host cores, on the same
    workload: full steps while they fit the budget, else a token sample. With
    single_thread_s > 0, also one thread alone on a token sample for about that long."""
    import oracle
    if threads is None:
        threads, aff = oracle_threads()
    else:
        aff = len(os.sched_getaffinity(0))
    T = wl.n_tokens
    ids = np.concatenate([np.repeat(wl.seg_adapter, np.diff(wl.seg_offsets)), wl.token_adapter])
    work = sum(int(wl.ranks[a]) * (p.d_in + p.d_out) for a in ids if a >= 0 for p in wl.projections)

    def prepare(n_threads, budget):
        # a token sample when one full step would not fit the budget (cost ~ rank * (d_in + d_out))
        est_s = work / (1.5e8 * n_threads)
        n_eval = T if est_s < budget / 4 else max(16, int(T * (budget / 4) / est_s))
        ev = np.sort(np.random.default_rng(0).choice(T, size=n_eval, replace=False)) if n_eval < T else None
        prepared = []
        for proj in range(len(wl.projections)):
            p = wl.projections[proj]
            need = sorted(set(int(a) for a in (ids if ev is None else ids[ev]) if a >= 0 and wl.ranks[a] > 0))
            adapters = {a: wl.adapter(a, proj) for a in need}
            pool, pt, base = oracle.build_pool(adapters, wl.n_adapters, p.d_in, p.d_out,
                                               wl.page_elems, wl.dtype, np.random.default_rng(proj))
            prepared.append(dict(dtype=wl.dtype, d_in=p.d_in, d_out=p.d_out, x=wl.x(proj),
                                 y0=wl.y0(proj), pool=pool, page_elems=wl.page_elems, page_table=pt,
                                 base=base, rank=wl.ranks, scale=wl.scales, seg_offsets=wl.seg_offsets,
                                 seg_adapter=wl.seg_adapter, token_adapter=wl.token_adapter,
                                 eval_tokens=ev, n_threads=n_threads))
        return prepared, ev

    def timed(prepared, ev, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            for kw in prepared:
                oracle.lora(**kw)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 10000:
                break
        n = T if ev is None else ev.size
        sample = (f"{reps} full steps ({T} tokens x {len(wl.projections)} projections)" if ev is None
                  else f"{reps} x {ev.size} of {T} tokens (seeded sample) x {len(wl.projections)} projections")
        return reps * n / el, sample, el

    prepared, ev = prepare(threads, budget_s)
    value, sample, el = timed(prepared, ev, budget_s)
    out = {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": sample, "seconds": round(el, 3), "host_affinity_cores": aff,
           "cpu_model": cpu_model()}
    if single_thread_s > 0:
        prepared, ev = prepare(1, single_thread_s)
        v1, s1, e1 = timed(prepared, ev, single_thread_s)
        out["single_thread"] = {"value": v1, "unit": "tokens/s", "cores": 1, "sample": s1,
                                "seconds": round(e1, 3)}
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def device_info():
    """GPU name, CU count, peak engine and memory clocks (hipDeviceGetAttribute through the
    HIP runtime torch loaded), ROCm / torch versions."""
    import ctypes
    import torch
    props = torch.cuda.get_device_properties(0)
    info = {"gpu": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count,
            "hip_runtime": torch.version.hip, "torch": torch.__version__}
    try:
        hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        for key, attr in (("sclk_peak_mhz", 5), ("mclk_peak_mhz", 60)):  # ClockRate, MemoryClockRate (kHz)
            v = ctypes.c_int(0)
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0:
                info[key] = v.value // 1000
    except OSError:
        pass
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    return info


def copy_reference(dev, nbytes=256 << 20, reps=10):
    """A plain device-to-device copy of nbytes (torch's copy kernel), timed with events on the
    current stream: GB/s counting the bytes read and written (2 * nbytes per copy)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ms = float(np.median(ts))
    return {"bytes": nbytes, "ms": round(ms, 4), "gbps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def h2d_reference(dev, nbytes, reps=5):
    """Copy-engine host-to-device rate: nbytes from pinned host memory (hipMemcpyAsync)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ms = float(np.median(ts))
    return {"bytes": nbytes, "ms": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 2)}


def pct(a, q):
    return round(float(np.percentile(np.asarray(a), q)), 3) if len(a) else None


def run_workload(wl, policy, n_inst, steps, warmup, event_every, pct_steps, dev, overlap_steps=0,
                 variant="paged", multi=True):
    """Time `steps` steps (every projection applied once, rotating over n_inst instances)
    after `warmup` untimed ones. multi (paged variant): projections of one shape go
    through one slora_apply_multi, otherwise one slora_apply each. Returns the measured
    figures; exits non-zero if a fused call's wait gave up in any of them (its results
    would not be valid)."""
    import torch
    from heterogeneous_lora_amd import _lib, runtime
    T = wl.n_tokens
    n_proj = len(wl.projections)
    groups = projection_groups(wl, multi and variant != "gathered")
    active = [int(a) for a in wl.active_adapters()]
    log(f"[bench] {wl.name}: {wl.description}")
    log(f"[bench] {T} tokens, {len(active)} active adapters, {n_proj} projection(s), {n_inst} instance(s)")
    store = runtime.HostStore(wl, active)
    host_io = [(wl.x(p), wl.y0(p)) for p in range(n_proj)]
    insts, fetch_ms = [], []
    _lib.timing_enable(True)  # the fetch kernels of the instances' setup are timed too
    _lib.timing_read_all()
    for i in range(n_inst):
        inst = runtime.PagedLoRA(wl, device=dev, store=store, pool_seed=wl.pool_seed + i,
                                 ordered=variant == "split")
        fetch_ms.append(inst.fetch_ms)
        calls = [inst.call(p, policy) for p in range(n_proj)]
        io = [(runtime._dev_i16(x, inst.device), runtime._dev_i16(y0, inst.device)) for x, y0 in host_io]
        if variant == "gathered":
            need = max(_lib.gathered_workspace_size(c) for c in calls)
        else:
            need = max(_lib.workspace_size_multi([calls[p] for p in g]) if len(g) > 1
                       else _lib.workspace_size(calls[g[0]]) for g in groups)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        insts.append((inst, calls, io, ws))
        log(f"[bench] instance {i} ready (fetch {inst.fetch_ms:.2f} ms)")
    del host_io
    _lib.timing_enable(False)
    fnames, fms_all = _lib.timing_read_all()
    fetch_kernel_ms = [m for n, m in zip(fnames, fms_all) if n == "fetch"]
    fetch_bytes = sum(int(wl.ranks[a]) * (p.d_in + p.d_out) * 2 for a in active for p in wl.projections)

    stream = torch.cuda.current_stream(dev)
    bound = [[inst.bind_apply_multi([calls[p] for p in g], [io[p][0] for p in g], [io[p][1] for p in g],
                                    ws, stream) if len(g) > 1 else
              inst.bind_apply(calls[g[0]], io[g[0]][0], io[g[0]][1], ws, stream, gathered=variant == "gathered")
              for g in groups] for inst, calls, io, ws in insts]

    def step(i):
        for run in bound[i % len(bound)]:
            run()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    _lib.timing_enable(True)  # creates the event pairs the timed launches use
    _lib.timing_enable(False)
    _lib.timing_read_all()  # start from an empty record
    # HIP events recorded by the launch itself bracket every kernel of one step in
    # `event_every` (recording costs the host a few microseconds per launch, which would
    # otherwise pace the loop)
    ev = max(1, min(event_every, steps // 4))  # and at least 4 timed steps
    t0 = time.perf_counter()
    for i in range(steps):
        if i % ev == 0:
            _lib.timing_enable(True)
            step(i)
            _lib.timing_enable(False)
        else:
            step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    names, ms = _lib.timing_read_all()
    wall = t1 - t0
    # then pct_steps more steps with every launch timed, for the spread of kernel durations
    _lib.timing_enable(True)
    for i in range(pct_steps):
        step(i)
    _lib.timing_enable(False)
    torch.cuda.synchronize()
    pnames, pms = _lib.timing_read_all()
    overlap = None
    if overlap_steps and len(insts) >= 2:
        # apply kernels while an adapter fetch runs on a side stream: the last instance's
        # adapters are fetched again (same bytes into its own pages) while the other
        # instances run overlap_steps steps with every launch timed
        tgt = insts[-1][0]
        side = torch.cuda.Stream(device=dev)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        side.wait_stream(stream)
        f0.record(side)
        rows = [tgt.store.ptrs(a, n_proj) for a in tgt.adapters]
        tgt.pool.fetch_many_async(tgt.adapters, [r[0] for r in rows], [r[1] for r in rows],
                                  side.cuda_stream, None)
        f1.record(side)
        _lib.timing_enable(True)
        t2 = time.perf_counter()
        for i in range(overlap_steps):
            for run in bound[i % (len(bound) - 1)]:
                run()
        _lib.timing_enable(False)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        onames, oms = _lib.timing_read_all()
        f_ms = f0.elapsed_time(f1)
        dom_o = max(set(onames), key=lambda k: sum(m for n, m in zip(onames, oms) if n == k))
        during = np.array([m for n, m in zip(onames, oms) if n == dom_o]) * 1e3
        alone = np.array([m for n, m in zip(pnames, pms) if n == dom_o]) * 1e3
        overlap = {"kernel": dom_o, "steps": overlap_steps,
                   "apply_us_p50_alone": pct(alone, 50), "apply_us_p50_during_fetch": pct(during, 50),
                   "apply_us_p90_during_fetch": pct(during, 90),
                   "step_us_during_fetch": round((t3 - t2) / overlap_steps * 1e6, 2),
                   "fetch_bytes": fetch_bytes, "fetch_ms": round(f_ms, 3),
                   "fetch_gbps_during_apply": round(fetch_bytes / (f_ms * 1e-3) / 1e9, 2),
                   "steps_inside_fetch": int(min(overlap_steps, f_ms * 1e-3 / max((t3 - t2) / overlap_steps, 1e-9)))}
        log(f"[bench] apply during a side-stream fetch: {json.dumps(overlap)}")
    bad = [i for i, (_, _, _, ws) in enumerate(insts) if _lib.workspace_status(ws.data_ptr(), stream.cuda_stream)]
    if bad:
        print(f"bench.py: a fused launch gave up waiting in instance(s) {bad}: results invalid",
              file=sys.stderr)
        sys.exit(3)

    ms_per_step = wall / steps * 1e3
    value = T * steps / wall
    log(f"[bench] {steps} steps in {wall:.4f} s: {ms_per_step * 1e3:.1f} us/step, {value:.4g} tokens/s")
    alg = [algorithmic(wl, p, insts[0][1][p]) for p in range(n_proj)]
    per = launch_work(alg, groups)
    kernels = {}
    for k in sorted(set(names)):
        d = np.array([m for n, m in zip(names, ms) if n == k])
        dp = np.array([m for n, m in zip(pnames, pms) if n == k]) * 1e3
        # the paged kernels' algorithmic work; the gathered variant's copy and its padded
        # products have no such figure of their own (0)
        work = np.mean(per[k], axis=0) if variant == "paged" and k in per else np.zeros(3)
        per_launch_bytes, per_launch_flops, mfma_flops = (float(v) for v in work)
        avg_s = float(d.mean()) * 1e-3
        kernels[k] = {"launches": int(d.size), "avg_us": round(avg_s * 1e6, 3),
                      "p10_us": pct(dp, 10), "p50_us": pct(dp, 50), "p90_us": pct(dp, 90),
                      "pct_launches": int(dp.size),
                      "algorithmic_bytes": int(per_launch_bytes),
                      "gbps": round(per_launch_bytes / avg_s / 1e9, 1),
                      "tflops": round(per_launch_flops / avg_s / 1e12, 3),
                      "mfma_tflops": round(mfma_flops / avg_s / 1e12, 3)}
    n_timed = (steps + ev - 1) // ev
    kern_total_s = float(np.sum(ms)) * 1e-3 / n_timed
    step_bytes = sum(kv["algorithmic_bytes"] * kv["launches"] for kv in kernels.values()) / n_timed
    if variant != "paged":  # the same function: the paged path's algorithmic bytes per step
        step_bytes = sum(a[f]["bytes"] for a in alg for f in ("mbgmv_fused", "sgmv_fused"))
    log(f"[bench] kernels: {json.dumps(kernels)}")
    log(f"[bench] all kernels of a step: {kern_total_s * 1e6:.1f} us, "
        f"{step_bytes / kern_total_s / 1e9:.0f} GB/s algorithmic")
    fms = float(np.median(fetch_ms))
    out = dict(value=value, ms_per_step=ms_per_step, kernels=kernels, event_every=ev,
               step_kernel_us=round(kern_total_s * 1e6, 2),
               step_algorithmic_gbps=round(step_bytes / kern_total_s / 1e9, 1),
               fetch={"bytes": fetch_bytes, "ms": round(fms, 3),
                      "gbps": round(fetch_bytes / (fms * 1e-3) / 1e9, 2),
                      "kernel_ms": round(float(np.median(fetch_kernel_ms)), 3) if fetch_kernel_ms else None,
                      "kernel_gbps": round(fetch_bytes / (float(np.median(fetch_kernel_ms)) * 1e-3) / 1e9, 2)
                      if fetch_kernel_ms else None},
               active=len(active), workspace_status="clean", fetch_overlap=overlap)
    for inst, *_ in insts:
        inst.close()
    return out


def capacity_ablation(steps=400, seed=0, fractions=(0.25, 0.5, 0.75)):
    """Unified paging against separate adapter and KV memory (host simulation of the
    scheduler, no GPU): the same request trace through slora_sched with one pool of
    196,608 pages (the mixed 13B batch's pool, 5120-element pages) holding adapters and
    KV, and with the same pages split into an adapter pool and a KV pool. A layer's
    q/k/v/o adapters take rank x 8 pages, a token's KV 2 pages (K and V of one layer).
    Requests arrive Poisson(24) per step, adapters Zipf(0.8) over 2000 with ranks U{8..128},
    prompts U{16..256}, outputs U{64..512} tokens."""
    from heterogeneous_lora_amd import _lib
    fake = 0x7F0000000000
    total, P, d = 196608, 5120, 5120
    rng = np.random.default_rng(seed)
    ranks = rng.choice(np.array([8, 16, 32, 64, 128]), size=2000)
    p = np.arange(1, 2001, dtype=np.float64) ** -0.8
    p /= p.sum()
    trace = []
    for step in range(steps):
        for _ in range(int(rng.poisson(24))):
            a = int(rng.choice(2000, p=p))
            trace.append((step, a, int(ranks[a]), int(rng.integers(16, 257)), int(rng.integers(64, 513))))

    def run(split_frac):
        if split_frac is None:
            kv = _lib.Pool(fake, total, P, "f16", seed)
            ap = kv
        else:
            na = int(total * split_frac)
            ap = _lib.Pool(fake, na, P, "f16", seed, ordered=True)
            kv = _lib.Pool(fake, total - na, P, "f16", seed)
        res = _lib.Residency(ap, [d] * 4, [d] * 4)
        sch = _lib.Scheduler(kv, res, 2, 16384, 1024)
        out = dict(tokens=0, prefill_tokens=0, decode_tokens=0, finished=0, aborted_pool_full=0,
                   adapter_fetches=0, adapter_evictions=0, running_sum=0, fetch_bytes=0)
        at = 0
        for step in range(steps):
            while at < len(trace) and trace[at][0] == step:
                _, a, r, pl, mx = trace[at]
                sch.submit(at, a, r, pl, mx)
                at += 1
            b = sch.step()
            out["tokens"] += b["n_tokens"]
            out["prefill_tokens"] += int(b["seg_offsets"][-1])
            out["decode_tokens"] += b["token_adapter"].size
            out["finished"] += b["finished"].size
            out["aborted_pool_full"] += int((b["abort_reason"] == _lib.ABORT_POOL_FULL).sum())
            out["adapter_fetches"] += b["fetch"].size
            out["adapter_evictions"] += b["evicted"].size
            out["fetch_bytes"] += int(sum(int(ranks[a]) * 8 * P * 2 for a in b["fetch"]))
            out["running_sum"] += b["n_running"]
        out["mean_running"] = round(out.pop("running_sum") / steps, 1)
        out["waiting_at_end"] = b["n_waiting"]
        sch.destroy()
        res.destroy()
        kv.destroy()
        if ap is not kv:
            ap.destroy()
        return out

    rows = {"unified": run(None)}
    for f in fractions:
        rows[f"split adapters {int(f * 100)}%"] = run(f)
    return {"steps": steps, "requests": len(trace), "pool_pages": total, "results": rows}


def roofline_of(kernels, workload, kernel=None):
    dom = kernel or max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    dk = kernels[dom]
    r = {"bound": "hbm", "kernel": dom, "achieved": dk["gbps"], "peak": HBM_PEAK_GBPS,
         "unit": "GB/s", "frac": round(dk["gbps"] / HBM_PEAK_GBPS, 4),
         "traffic": load_traffic(dom, workload)}
    if dk.get("mfma_tflops"):  # the segment (matrix-core) part of the kernel's work
        r["mfma_tflops"] = dk["mfma_tflops"]
        r["mfma_frac"] = round(dk["mfma_tflops"] / MFMA_BF16_PEAK_TFLOPS, 5)
    return r


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_7b")
    ap.add_argument("--policy", default="auto", choices=["auto", "mbgmv", "sgmv"])
    ap.add_argument("--active", type=int, default=0,
                    help="mlp_asym only: number of active adapters (tokens per adapter = 4096 / this)")
    ap.add_argument("--instances", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode_7b only: skip the prefill_sgmv sub-record")
    ap.add_argument("--pct-steps", type=int, default=64,
                    help="extra steps, every launch timed, for the p10/p50/p90 kernel durations")
    ap.add_argument("--per-projection", action="store_true",
                    help="one slora_apply per projection, instead of one slora_apply_multi per "
                         "run of same-shape projections")
    ap.add_argument("--variant", default="paged", choices=["paged", "gathered", "split"],
                    help="paged: slora_apply on the unified pool; gathered: slora_apply_gathered "
                         "(adapters copied out and padded, then a padded batched GEMM); split: "
                         "slora_apply with the adapters alone in an ordered pool")
    ap.add_argument("--capacity-ablation", action="store_true",
                    help="only the host simulation of unified against split pools (no GPU)")
    ap.add_argument("--overlap-steps", type=int, default=64,
                    help="steps timed while a side-stream adapter fetch runs (0: skip)")
    ap.add_argument("--event-every", type=int, default=16,
                    help="time the kernels of one step in this many with HIP events (each timed "
                         "launch costs the host ~8 us; 1 in 16 keeps the timed loop within ~1%% "
                         "of an untimed one on the decode batch)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="BYTES",
                    help="only run the plain copy the byte counters are calibrated with")
    ap.add_argument("--pmc-summary", action="store_true",
                    help="only summarize rocprofv3 FETCH_SIZE / WRITE_SIZE runs (no GPU)")
    for opt in ("kernel", "workload", "match", "fetch-csv", "write-csv", "calib-match",
                "calib-fetch-csv", "calib-write-csv", "commands"):
        ap.add_argument(f"--{opt}", default="")
    ap.add_argument("--calib-bytes", type=int, default=0)
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: each GPU would own its pool and serve its own "
              "requests, with no exchange between GPUs on this path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        calib_copy(args.calib_copy, 20)
        return
    if args.capacity_ablation:
        print(json.dumps(capacity_ablation(args.steps)), flush=True)
        return

    import torch
    import workloads
    from heterogeneous_lora_amd import _lib

    _lib.load()
    policy = {"auto": 0, "mbgmv": 1, "sgmv": 2}[args.policy]
    wl = workloads.make(args.config, **({"n_active": args.active} if args.active else {}))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dinfo = device_info()
    log(f"[bench] device: {dinfo}")
    main_run = run_workload(wl, policy, args.instances, args.steps, args.warmup, args.event_every,
                            args.pct_steps, dev, overlap_steps=args.overlap_steps if args.variant == "paged" else 0,
                            variant=args.variant, multi=not args.per_projection)
    roofline = roofline_of(main_run["kernels"], wl.name)
    copy_ref = copy_reference(dev)
    roofline["copy_gbps"] = copy_ref["gbps"]
    roofline["frac_of_copy"] = round(roofline["achieved"] / copy_ref["gbps"], 4)
    fetch = dict(main_run["fetch"])
    h2d = h2d_reference(dev, fetch["bytes"])
    fetch["h2d_copy_engine_gbps"] = h2d["gbps"]
    fetch["frac_of_h2d"] = round(fetch["gbps"] / h2d["gbps"], 4)
    if fetch.get("kernel_gbps"):
        fetch["kernel_frac_of_h2d"] = round(fetch["kernel_gbps"] / h2d["gbps"], 4)

    prefill = None
    if args.config == "decode_7b" and not args.no_prefill and args.variant == "paged":
        pw = workloads.make("prefill_sgmv")
        pr = run_workload(pw, 0, 2, max(10, min(args.steps, 40)), max(2, min(args.warmup, 5)),
                          args.event_every, min(args.pct_steps, 16), dev, multi=not args.per_projection)
        prefill = {"workload": pw.name, "value": round(pr["value"], 1), "unit": "tokens/s",
                   "ms_per_step": round(pr["ms_per_step"], 5), "tokens": pw.n_tokens,
                   "projections": len(pw.projections), "instances_rotated": 2,
                   "kernels": pr["kernels"], "step_kernel_us": pr["step_kernel_us"],
                   "step_algorithmic_gbps": pr["step_algorithmic_gbps"],
                   "roofline": {k: roofline_of(pr["kernels"], pw.name, k) for k in pr["kernels"]},
                   "workspace_status": pr["workspace_status"]}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(wl, args.cpu_seconds,
                           single_thread_s=min(3.0, args.cpu_seconds) if wl.name in ("tiny_decode", "decode_7b") else 0.0)
        log(f"[bench] oracle: {cpu}")

    rec = {
        "metric": METRIC, "value": round(main_run["value"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_run["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.n_tokens, "projections": len(wl.projections),
                   "shape": [[p.d_in, p.d_out] for p in wl.projections],
                   "active_adapters": main_run["active"], "policy": args.policy,
                   "variant": args.variant,
                   "projection_calls": "per projection" if args.per_projection else
                                       "one slora_apply_multi per run of same-shape projections",
                   "instances_rotated": args.instances, "accumulate": "f32",
                   "page_elems": wl.page_elems, "pool_pages": wl.n_pages},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": main_run["kernels"],
        "kernel_timing": f"HIP events recorded by the launch at kernel start and end, on the launch "
                         f"stream, for every kernel of 1 step in {main_run['event_every']}; p10/p50/p90 "
                         f"from {args.pct_steps} further steps with every launch timed",
        "step_kernel_us": main_run["step_kernel_us"],
        "step_algorithmic_gbps": main_run["step_algorithmic_gbps"],
        "workspace_status": main_run["workspace_status"],
        "copy_reference": copy_ref,
        "fetch": fetch,
        "fetch_overlap": main_run["fetch_overlap"],
        "prefill": prefill,
        "device": dinfo,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
