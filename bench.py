#!/usr/bin/env python3
"""Throughput of the SPA-Cache cached layer step on one MI355X.

Workload (default "llada-layer"): one LLaDA-8B-shaped layer, bf16, B=1, N=1024 tokens, d=4096,
32 heads x 128, SwiGLU FFN 12288, singular proxy rank r=128, rho=0.25 -> k=256 rows per step,
random-init weights with a planted power-law Value spectrum, hidden states drifting over 8 steps.
A step is one cached layer step: proxy GEMM, cosine + proxy-cache update, Top-k, RMSNorm gather,
QKV GEMM with K/V scatter, sparse-query attention, W_o + residual, RMSNorm, gate/up + SwiGLU,
W_down + residual scattered into H^c. Inputs are resident in HBM before timing starts.

Prints one JSON line: value = layer-steps/s (B x layers x steps / time); extra fields give the
tokens/s projection, the speedup over a full recompute of the same layer, per-kernel times from
HIP events recorded between the kernels, the roofline of the dominant kernel, and the CPU oracle
baseline on the host cores.
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # dense fp32 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_work(name, s, M):
    """Algorithmic bytes (operands read once, outputs written once) and flops of one GEMM kernel."""
    e = 2 if s.dtype == "bf16" else 4
    d, dq, dkv, F = s.d_model, s.d_q, s.d_kv, s.d_ffn
    if name == "qkv_gemm_scatter":
        n, kk = dq + 2 * dkv, d
    elif name == "wo_gemm_residual":
        n, kk = d, dq
    elif name == "gate_up_gemm_swiglu":
        n, kk = 2 * F, d
    elif name == "down_gemm_scatter":
        n, kk = d, F
    else:
        return None
    flops = 2.0 * M * n * kk
    out_cols = F if name == "gate_up_gemm_swiglu" else n
    extra_in = M * d * e if name in ("wo_gemm_residual", "down_gemm_scatter") else 0   # residual rows
    byts = (M * kk + n * kk + M * out_cols) * e + extra_in
    return byts, flops


KERNEL_SOURCES = {
    "gemm": ("adaptive_hidden_state_amd/csrc/gemm.hip", "adaptive_hidden_state_amd/csrc/common.hpp",
             "adaptive_hidden_state_amd/csrc/launch.hpp"),
}


def kernel_source_hash(family):
    """sha256 over the sources that define a kernel family (to tell whether counters are current)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary of this kernel and workload, or None
    when there is none or the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    try:
        if fields["source_sha256"] != kernel_source_hash(fields["family"]):
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize_profile(trace_csv=None, counter_csvs=()):
    """Text summary of rocprofv3 CSV output: per (kernel, grid, phase) dispatch count and average /
    median duration from a --kernel-trace run, and per (kernel, grid, phase) average counter values from
    --pmc runs. phase: "step" for dispatches after a Top-k (the cached step), "full" after a cosine pass
    without one (the full recompute, or spa_identify), "-" before either; in dispatch order."""
    import csv
    import statistics

    def short(name):
        name = re.sub(r"^void ", "", name)
        name = re.sub(r"\(.*$", "", name)
        return name.replace("unsigned short", "bf16").replace("spa::", "")

    def grid_of(row):
        if "Grid_Size" in row:
            return int(row["Grid_Size"]), int(row["Workgroup_Size"])
        g = int(row["Grid_Size_X"]) * int(row["Grid_Size_Y"]) * int(row["Grid_Size_Z"])
        wg = int(row["Workgroup_Size_X"]) * int(row["Workgroup_Size_Y"]) * int(row["Workgroup_Size_Z"])
        return g, wg

    def phased(rows):
        """(row, phase) in dispatch order."""
        phase, out = "-", []
        for row in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
            name = short(row["Kernel_Name"])
            if name.startswith(("cosine_topk_kernel", "topk_kernel")):
                phase = "step"
            elif name.startswith("proxy_cosine_kernel"):
                phase = "full"
            out.append((row, phase))
        return out

    out = []
    if trace_csv:
        groups = {}
        with open(trace_csv) as f:
            for row, phase in phased(list(csv.DictReader(f))):
                g, wg = grid_of(row)
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0
                groups.setdefault((short(row["Kernel_Name"]), g // wg, wg, phase), []).append(dur)
        out.append(f"{'kernel':58s} {'workgroups':>10s} {'wg':>5s} {'phase':>5s} {'calls':>6s} {'avg_us':>9s} "
                   f"{'med_us':>9s}")
        for (name, nwg, wg, ph), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{name[:58]:58s} {nwg:10d} {wg:5d} {ph:>5s} {len(v):6d} {sum(v) / len(v):9.2f} "
                       f"{statistics.median(v):9.2f}")
    for path in counter_csvs:
        groups = {}
        with open(path) as f:
            rows = list(csv.DictReader(f))
        for row, phase in phased(rows):
            g, wg = grid_of(row)
            groups.setdefault((short(row["Kernel_Name"]), g // wg, wg, phase, row["Counter_Name"]), []).append(
                float(row["Counter_Value"]))
        out.append("")
        out.append(f"{'kernel':58s} {'workgroups':>10s} {'wg':>5s} {'phase':>5s} {'counter':>12s} {'calls':>6s} "
                   f"{'avg':>14s}")
        for (name, nwg, wg, ph, cn), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{name[:58]:58s} {nwg:10d} {wg:5d} {ph:>5s} {cn:>12s} {len(v):6d} {sum(v) / len(v):14.1f}")
    return "\n".join(out)


def gpu_info():
    """The device's name, arch, compute units and shader clocks (sysfs DPM table: the highest level and
    the level current at the time of the call), for the bench line."""
    import glob
    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"name": torch.cuda.get_device_name(0) or getattr(p, "name", ""),
            "arch": getattr(p, "gcnArchName", ""), "compute_units": int(p.multi_processor_count)}
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                lv = [ln.split() for ln in f.read().splitlines() if "Mhz" in ln]
        except OSError:
            continue
        mhz = [int(x[1].lower().replace("mhz", "")) for x in lv if len(x) >= 2]
        cur = [int(x[1].lower().replace("mhz", "")) for x in lv if len(x) >= 3 and x[-1] == "*"]
        if mhz:
            info["sclk_max_mhz"] = max(mhz)
            info["sclk_now_mhz"] = cur[0] if cur else None
            break
    return info


def kernel_work(name, s, k):
    """Algorithmic bytes and flops of one kernel of the cached step (inputs read once, outputs written
    once), for the per-kernel HBM / MFMA fractions."""
    e = 2 if s.dtype == "bf16" else 4
    rows, M = s.batch * s.n_tokens, s.batch * k
    if name == "proxy_gemm":
        return (rows * s.d_model + s.rank * s.d_model) * e + rows * s.rank * 4, 2.0 * rows * s.d_model * s.rank
    if name == "proxy_cosine":
        return rows * s.rank * 4 * 3 + rows * 4, 6.0 * rows * s.rank
    if name == "cosine_topk":     # the cosine pass plus the Top-k (scores re-read, indices written)
        return rows * s.rank * 4 * 3 + rows * 4 * 2 + M * 4, 6.0 * rows * s.rank
    if name == "topk":
        return rows * 4 + M * 4, 0.0
    if name == "attention":
        kv = 2 * s.batch * s.n_kv_heads * s.n_tokens * s.head_dim * e
        return kv + 2 * M * s.d_q * e, 4.0 * M * s.n_q_heads * s.n_tokens * s.head_dim
    return gemm_work(name, s, M)


def cpu_baseline(wl, w, w_r, xs, k, seconds, threads=None):
    """The oracle's cached layer step timed on the host cores (bounded sample); threads: limit the BLAS
    thread pool to that many threads (None: the pool as configured)."""
    if threads is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads, user_api="blas"):
            return cpu_baseline(wl, w, w_r, xs, k, seconds)
    import numpy as np
    import oracle
    s = wl.shape
    threads = blas_threads()
    kc, vc = oracle.kv_project(xs[0], w, s.head_dim, s.norm_eps, s.dtype)
    pc = oracle.proxy(xs[0], w_r).astype(np.float32).astype(np.float64)
    cache = oracle.LayerCache(kc, vc, np.asarray(xs[0], np.float64), pc)
    done, t0 = 0, time.perf_counter()
    while True:
        cache, _, _ = oracle.cached_layer_step(xs[1 + done % (len(xs) - 1)], w, w_r, cache, k, s.head_dim,
                                               s.norm_eps, s.dtype)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= 64:
            break
    return {"value": done / el, "unit": "layer-steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} cached layer steps of {wl.name} (B={s.batch}, N={s.n_tokens}, d={s.d_model}, "
                      f"k={k}) by the NumPy float64 oracle, {el:.1f} s"}


def roofline_of(byts, flops, us, peak_flops):
    """Roofline record of one kernel: its nearer bound (HBM bytes or MFMA flops) and the fraction."""
    dur_s = us * 1e-6
    if byts / (PEAK_HBM_GBS * 1e9) >= flops / (peak_flops * 1e12):
        roof = {"bound": "hbm", "achieved": byts / dur_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / dur_s / 1e12, "peak": peak_flops, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    return roof


def per_kernel_fractions(per_us, work, peak_flops):
    out = {}
    for n, us in per_us.items():
        if n not in work:
            continue
        byts, flops = work[n]
        out[n] = {"us": round(us, 2), "GB/s": round(byts / us / 1e3, 1),
                  "hbm_frac": round(byts / us / 1e3 / PEAK_HBM_GBS, 4),
                  "TFLOP/s": round(flops / us / 1e6, 1), "mfma_frac": round(flops / us / 1e6 / peak_flops, 4)}
    return out


IDENTIFY_KERNELS = ("proxy_gemm", "cosine_topk", "proxy_cosine", "topk")


def identification_summary(per_us, work, ms_step, target_us=None):
    """The update identification (proxy projection, cosine, Top-k) against its roofline target: its
    event-bracketed time, share of the step, algorithmic bytes and the fraction of HBM peak they
    reach (target 0.6); target_us: a time target for the whole identification, if one applies."""
    names = [n for n in IDENTIFY_KERNELS if n in per_us and n in work]
    if not names:
        return None
    us = sum(per_us[n] for n in names)
    byts = sum(work[n][0] for n in names)
    out = {"kernels": names, "us": round(us, 2), "share_of_step": round(us / (ms_step * 1e3), 4),
           "algorithmic_bytes": byts, "GB/s": round(byts / us / 1e3, 1),
           "hbm_frac": round(byts / us / 1e3 / PEAK_HBM_GBS, 4), "hbm_frac_target": 0.6}
    if target_us is not None:
        out["target_us"] = target_us
    return out


def dominant_roofline(per_us, work, peak_flops, workload):
    """Roofline of the longest GEMM (the dominant kernel of every workload here)."""
    dom = max((n for n in per_us if n in work and n in GEMM_KERNELS), key=lambda n: per_us[n])
    byts, flops = work[dom]
    roof = roofline_of(byts, flops, per_us[dom], peak_flops)
    roof["traffic"] = measured_traffic(dom, workload)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = byts
    roof["algorithmic_flops"] = flops
    roof["mfma_frac"] = flops / (per_us[dom] * 1e-6) / 1e12 / peak_flops
    return roof


def ideal_floor_us(work, peak_flops):
    """Sum over kernels of max(bytes / HBM peak, flops / MFMA peak): no schedule can beat it."""
    return sum(max(b / (PEAK_HBM_GBS * 1e3), f / (peak_flops * 1e6)) for b, f in work.values())


GEMM_KERNELS = ("qkv_gemm_scatter", "wo_gemm_residual", "gate_up_gemm_swiglu", "down_gemm_scatter")
STEP_KERNELS = ("proxy_gemm", "cosine_topk") + GEMM_KERNELS[:1] + ("attention",) + GEMM_KERNELS[1:]
SPLIT_IDENTIFY = ("proxy_gemm", "proxy_cosine", "topk") + GEMM_KERNELS[:1] + ("attention",) + GEMM_KERNELS[1:]


def step_kernels(s):
    """Kernel names of one cached step: the Top-k runs inside the cosine kernel up to 8192 hidden rows."""
    return STEP_KERNELS if s.batch * s.n_tokens <= 8192 else SPLIT_IDENTIFY


def base_line(args, wl, s, value, unit, ms_step, steps, warmup, data):
    return {
        "metric": "tokens/s & layer-steps/s (8B-shape, N=1024, r=128) + % HBM/MFMA peak",
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": data,
    }


def timed_blocks(step, first, steps, blocks, run_range=None):
    """Time exactly `steps` consecutive steps first, first + 1, ... as `blocks` consecutive blocks of
    (nearly) equal size, with an event on the current stream between blocks and a synchronize before
    the first and after the last; a block runs step(i) for each of its steps, or run_range(i, n) when
    given (n steps from step i). Returns the median over the blocks of the time per step (ms) and the
    per-block values."""
    import numpy as np
    import torch
    nb = max(1, min(blocks, steps))
    sizes = [steps // nb + (1 if b < steps % nb else 0) for b in range(nb)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    i = first
    evs[0].record()
    for b, n in enumerate(sizes):
        if run_range is not None:
            run_range(i, n)
            i += n
        else:
            for _ in range(n):
                step(i)
                i += 1
        evs[b + 1].record()
    torch.cuda.synchronize()
    per = [evs[b].elapsed_time(evs[b + 1]) / sizes[b] for b in range(nb)]
    return float(np.median(per)), per


def block_stats(per, ms):
    """Summary of a timed_blocks result for the bench line."""
    return {"blocks": len(per), "ms_per_step_blocks": [round(v, 5) for v in per],
            "ms_per_step_mean": round(sum(per) / len(per), 5),
            "spread": round((max(per) - min(per)) / ms, 4) if ms > 0 else None}


def timed_kernels(spa, calls, reps):
    """Per-kernel durations (us, median over reps) of a sequence of spa_layer_step_timed calls;
    `calls(ev)` runs one pass and returns [(name, ms), ...] summed over its layers."""
    import numpy as np
    ev = spa.HipEvents(24)
    per = {}
    for _ in range(reps):
        tot = {}
        for name, ms in calls(ev):
            tot[name] = tot.get(name, 0.0) + ms
        for name, ms in tot.items():
            per.setdefault(name, []).append(ms)
    ev.close()
    return {n: 1000.0 * float(np.median(v)) for n, v in per.items()}


def run_layer(args, wl):
    """One layer of a workload, cached steps over rotating layer instances, graph-replayed."""
    import numpy as np
    import torch

    import adaptive_hidden_state_amd as spa
    import synth

    s = wl.shape.replace(rope_theta=wl.arch_rope_theta) if args.arch else wl.shape
    k = int(spa.spa_budget(1, 1, wl.rho, wl.rho, wl.rho, s.n_tokens)[1][0])
    steps = args.steps or 200
    warmup = 10 if args.warmup is None else args.warmup

    log(f"[bench] generating {wl.name} weights and inputs")
    t = time.time()
    w = synth.layer_weights(wl)
    if args.arch:
        w["rope_theta"] = s.rope_theta
    w_r = synth.to_storage(spa.singular_proxy_from_factors(w["v_lambda"], w["v_right"], s.rank, w["g_attn"]), s.dtype)
    xs, _ = synth.drift_sequence(wl)
    log(f"[bench] inputs ready in {time.time() - t:.1f} s")

    # R independent layer instances (weights, caches, inputs at distinct addresses), visited in turn, so
    # that no step finds the previous step's data in the 256 MB Infinity Cache (one cycle streams > 1 GB)
    R = max(1, args.instances)
    dw0 = spa.upload_weights(w, w_r, s.dtype)
    dws = [dw0] + [spa.DeviceWeights(*(t.clone() if t is not None else None for t in dw0)) for _ in range(R - 1)]
    tdt = spa.torch_dtype(s.dtype)
    xd0 = [torch.from_numpy(x).to("cuda", tdt).contiguous() for x in xs]
    xds = [xd0] + [[t.clone() for t in xd0] for _ in range(R - 1)]
    caches = [spa.alloc_cache(s) for _ in range(R)]
    ws = spa.alloc_workspace(s, s.n_tokens)
    idx = torch.empty(s.batch, k, dtype=torch.int32, device="cuda")
    scores = torch.empty(s.batch, s.n_tokens, dtype=torch.float32, device="cuda")
    n_in = len(xd0) - 1
    for r in range(R):
        spa.spa_layer_full(s, dws[r], caches[r], xds[r][0], ws)
    torch.cuda.synchronize()

    def which(i):  # step i -> (instance, input step)
        return i % R, 1 + (i // R) % n_in

    def eager_step(i):
        r, j = which(i)
        spa.spa_layer_step(s, dws[r], caches[r], xds[r][j], k, spa.SPA_PROXY_WRITE_ALL, idx, scores, ws)

    # the vanilla full recompute of the same layer (the "Baseline 100%" path, every token updated), into
    # caches of its own, for the speedup; timed the same way as the cached step
    scratch = [spa.alloc_cache(s) for _ in range(R)]

    def eager_full(i):
        r, j = which(i)
        spa.spa_layer_full(s, dws[r], scratch[r], xds[r][j], ws)

    # Captured HIP graphs (every launch of a step is stream-ordered and allocation-free, so a step is
    # capturable as is): one per (instance, input step), and one per window of R consecutive steps
    # (the R instances in turn, from any starting step), as a denoising step's graph holds the steps of
    # every layer. Step i's work depends only on i mod R n_in. A range of steps replays the R-step
    # graphs while whole windows fit and the one-step graphs for the rest.
    G = R if args.graph_group else 1
    period = R * n_in
    graphs = graphs_full = groups = groups_full = None
    if args.graph:
        graphs = capture(args, [lambda i=i: eager_step(i) for i in range(period)])
        graphs_full = capture(args, [lambda i=i: eager_full(i) for i in range(period)])
        if G > 1 and graphs is not None:
            groups = capture(args, [lambda w=w: [eager_step(i) for i in range(w, w + R)] for w in range(period)])
            groups_full = capture(args, [lambda w=w: [eager_full(i) for i in range(w, w + R)] for w in range(period)])

    step = range_runner(graphs, groups, eager_step, R, n_in)
    full = range_runner(graphs_full, groups_full, eager_full, R, n_in)
    step(0, warmup)
    full(0, warmup)
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} cached layer steps ({'graphs of %d steps' % (G if groups else 1) if graphs else 'eager'}, "
        f"{R} instances, {args.blocks} blocks)")
    ms_step, per_step = timed_blocks(None, warmup, steps, args.blocks, run_range=step)
    log(f"[bench] timing {steps} full recomputes")
    ms_full, per_full = timed_blocks(None, warmup, steps, args.blocks, run_range=full)
    del scratch, graphs_full, groups_full

    # per-kernel durations: HIP events between the kernels of the same step sequence
    it = iter(range(10 ** 9))

    def one(ev):
        r, j = which(next(it))
        return spa.spa_layer_step_timed(s, dws[r], caches[r], xds[r][j], k, spa.SPA_PROXY_WRITE_ALL, idx, scores,
                                        ws, ev)

    per_us = timed_kernels(spa, one, max(10, min(steps, 50)))
    peak_flops = PEAK_BF16_TFLOPS if s.dtype == "bf16" else PEAK_FP32_TFLOPS
    work = {n: kernel_work(n, s, k) for n in step_kernels(s)}

    line = base_line(args, wl, s, s.batch / (ms_step * 1e-3), "layer-steps/s", ms_step, steps, warmup,
                     "synthetic (seeded random-init weights with a planted Value spectrum; drifting N(0,1) "
                     "hidden states)")
    line["config"] = {"workload": wl.name, "batch": s.batch, "n_tokens": s.n_tokens, "d_model": s.d_model,
                      "n_q_heads": s.n_q_heads, "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                      "d_ffn": s.d_ffn, "rank": s.rank, "rho": wl.rho, "k": k, "rope_theta": s.rope_theta}
    line["tokens_per_s_projected"] = round(16 * s.batch / (32 * ms_step * 1e-3), 2)
    line["full_recompute_ms"] = round(ms_full, 5)
    line["speedup_vs_full"] = round(ms_full / ms_step, 3)
    line["ideal_floor_ms"] = round(ideal_floor_us(work, peak_flops) / 1e3, 5)
    line["per_kernel_us"] = {n: round(v, 2) for n, v in per_us.items()}
    line["per_kernel_roofline"] = per_kernel_fractions(per_us, work, peak_flops)
    line["timing"] = {"graphs": graphs is not None, "instances": R,
                      "steps_per_graph": G if groups is not None else 1, **block_stats(per_step, ms_step),
                      "full_recompute": block_stats(per_full, ms_full),
                      "note": "ms_per_step = median over the blocks of the timed steps (steps_per_graph consecutive "
                              "steps, one per layer instance, per graph launch; the full recompute likewise); "
                              "per-kernel us from HIP events recorded between kernels on the launch stream"}
    line["roofline"] = dominant_roofline(per_us, work, peak_flops, wl.name)
    line["identification"] = identification_summary(per_us, work, ms_step, 10.0 if wl.name == "llada-layer" else None)
    line["gpu"] = gpu_info()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(wl, w, np.asarray(w_r, np.float64), xs, k, args.cpu_seconds)
        log("[bench] timing the CPU oracle on one core")
        line["cpu_baseline_1core"] = cpu_baseline(wl, w, np.asarray(w_r, np.float64), xs, k, args.cpu_seconds,
                                                  threads=1)
    else:
        line["cpu_baseline"] = None
    return line


def range_runner(single, windows, eager, R, n_in):
    """run(i0, n): steps i0 .. i0 + n - 1 of the rotation (step i = instance i mod R at input step
    1 + (i div R) mod n_in, which depends only on i mod R n_in), replaying windows[i mod R n_in] (a graph
    of steps i .. i + R - 1) while a whole window fits, else single[i mod R n_in] (a graph of step i),
    else eager(i)."""
    period = R * n_in

    def run(i0, n):
        i, end = i0, i0 + n
        while i < end:
            if windows is not None and i + R <= end:
                windows[i % period].replay()
                i += R
                continue
            if single is not None:
                single[i % period].replay()
            else:
                eager(i)
            i += 1
    return run


def capture(args, fns):
    """One captured HIP graph per callable (each a stream-ordered, allocation-free sequence of library
    calls), after one eager pass of all of them on a side stream; None if capture is unavailable."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for f in fns:
                f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for f in fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                f()
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs
    except Exception as exc:  # fall back to eager launches
        log(f"[bench] graph capture unavailable ({exc}); timing eager launches")
        return None


def host_weights(w):
    """float32 host copies of a device weight dict (inputs of the CPU oracle baseline)."""
    import numpy as np
    return {key: (v.float().cpu().numpy() if hasattr(v, "device") else np.asarray(v))
            for key, v in w.items() if key.startswith(("w_", "g_", "b_"))}


def run_stack(args, wl):
    """A multi-layer stack: every denoising step unmasks u tokens (fresh embedding rows at their
    positions of the layer-0 input) and runs the cached step of every layer, layer l reading layer
    l-1's output cache; k_l from the piecewise-Gaussian budget (or its mean, uniform)."""
    import numpy as np
    import torch

    import adaptive_hidden_state_amd as spa
    import synth

    s = wl.shape
    if args.identifier == "full":
        s = s.replace(rank=s.d_kv)
    elif args.rank:
        s = s.replace(rank=args.rank)
    bias = args.arch and wl.arch_qkv_bias
    if args.arch:
        s = s.replace(rope_theta=wl.arch_rope_theta)
    L, B, N = wl.n_layers, s.batch, s.n_tokens
    u = args.unmask or wl.unmask_per_step  # tokens unmasked per denoising step (parallel decoding: more)
    if u < 1 or u > N:
        raise SystemExit(f"--unmask must be in 1..{N}")
    rho_p, l_p, rho_1, rho_L = wl.budget
    rhos, ks = spa.spa_budget(L, l_p, rho_p, rho_1, rho_L, N)
    if args.budget == "uniform":
        mean = float(np.mean(rhos))
        ks = spa.spa_budget(1, 1, mean, mean, mean, N)[1] * L
    steps = args.steps or N // u
    warmup = 4 if args.warmup is None else args.warmup
    tdt = spa.torch_dtype(s.dtype)

    log(f"[bench] generating {L} {wl.name} layers on the device")
    t0 = time.time()
    pair = synth.haar_pair(wl, s)
    layers = []
    for l in range(L):
        w = synth.layer_weights_device(wl, l + 1, pair, shape=s, qkv_bias=bias)
        if args.identifier == "full":   # the full-dimension Value identifier: W_r = W_v diag(g_attn) = W_v
            w_r = w["w_v"]
        else:
            w_r = spa.singular_proxy_from_factors(w["v_lambda"], w["v_right"], s.rank, w["g_attn"]).to(tdt)
        layers.append(spa.upload_weights(w, w_r, s.dtype))
        del w, w_r
    torch.cuda.synchronize()
    pos, rows = synth.unmask_schedule(wl, s, per_step=u)
    rows_neg = -rows
    x0 = synth.normal_device((B, N, s.d_model), wl.config_id, 0, synth.STREAM_X0, dtype=s.dtype)
    x_buf = x0.clone()
    caches = [spa.alloc_cache(s) for _ in range(L)]
    ws = spa.alloc_workspace(s, N)
    idx = torch.empty(B, max(ks), dtype=torch.int32, device="cuda")
    scores = torch.empty(B, N, dtype=torch.float32, device="cuda")
    t_sched = pos.shape[0]
    log(f"[bench] {L} layers ready in {time.time() - t0:.1f} s; k_l = {ks}")

    def feed(t):  # unmask the step's u positions (every second pass over the schedule flips the rows' sign)
        c, j = divmod(t, t_sched)
        x_buf.index_copy_(1, pos[j], rows[j] if c % 2 == 0 else rows_neg[j])

    def chain(full):
        x = x_buf
        for l in range(L):
            if full:
                spa.spa_layer_full(s, layers[l], caches[l], x, ws)
            else:
                spa.spa_layer_step(s, layers[l], caches[l], x, ks[l], spa.SPA_PROXY_WRITE_ALL, idx, scores, ws)
            x = caches[l].h

    chain(True)  # warm-up at step 0 (every layer fully computed)
    torch.cuda.synchronize()
    graphs = capture(args, [lambda: chain(False)]) if args.graph else None

    def step(t):
        feed(t)
        if graphs is not None:
            graphs[0].replay()
        else:
            chain(False)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} denoising steps x {L} layers ({'graph' if graphs else 'eager'}, "
        f"{args.blocks} blocks)")
    ms_step, per_step = timed_blocks(step, warmup, steps, args.blocks)

    def one(ev):
        feed(warmup + steps)
        x, res = x_buf, []
        for l in range(L):
            res += spa.spa_layer_step_timed(s, layers[l], caches[l], x, ks[l], spa.SPA_PROXY_WRITE_ALL, idx,
                                            scores, ws, ev)
            x = caches[l].h
        return res

    per_us = timed_kernels(spa, one, 3)
    peak_flops = PEAK_BF16_TFLOPS
    work = {}
    for n in step_kernels(s):
        b = f = 0.0
        for kl in ks:
            bb, ff = kernel_work(n, s, kl)
            b, f = b + bb, f + ff
        work[n] = (b, f)

    # Parallel decoding: of the u positions a denoising step unmasks (fresh embedding rows at layer 0),
    # how many each layer's update set recomputes (one untimed step per u, from the current caches)
    coverage = {}
    for uu in sorted({16, 64, 256, u}):
        if uu > N:
            continue
        pos_u, _ = synth.unmask_schedule(wl, s, per_step=uu)
        # fresh rows (a stream of their own), so every one of the uu positions changes
        fresh = synth.normal_device((B, uu, s.d_model), wl.config_id, 100 + uu, synth.STREAM_DRIFT, dtype=s.dtype)
        x_buf.index_copy_(1, pos_u[0], fresh)
        unmasked = set(pos_u[0].tolist())
        x, frac = x_buf, []
        for l in range(L):
            spa.spa_layer_step(s, layers[l], caches[l], x, ks[l], spa.SPA_PROXY_WRITE_ALL, idx, scores, ws)
            sel = idx.view(-1)[:B * ks[l]].view(B, ks[l]).cpu().numpy()
            frac.append(float(np.mean([len(unmasked & set(sel[b].tolist())) / uu for b in range(B)])))
            x = caches[l].h
        coverage[str(uu)] = {"per_layer": [round(f, 4) for f in frac], "mean": round(float(np.mean(frac)), 4),
                             "min": round(min(frac), 4)}
    torch.cuda.synchronize()

    # vanilla decoding: every layer fully recomputed at every step (the same unmasking copy, graph-replayed
    # like the cached step); it overwrites the caches, so it is timed last
    graphs_full = capture(args, [lambda: chain(True)]) if args.graph else None

    def full_step(t):
        feed(t)
        if graphs_full is not None:
            graphs_full[0].replay()
        else:
            chain(True)

    n_full = max(args.blocks, min(steps, 8))
    full_step(warmup + steps + 1)
    log(f"[bench] timing {n_full} full recomputes of the stack")
    ms_full, per_full = timed_blocks(full_step, warmup + steps + 2, n_full, args.blocks)

    line = base_line(args, wl, s, u * B / (ms_step * 1e-3), "tokens/s", ms_step, steps, warmup,
                     "synthetic (seeded random-init layers with a planted Value spectrum, drawn on the device; "
                     "N(0,1) embeddings, u fresh rows per denoising step; layers chained)")
    line["config"] = {"workload": wl.name, "n_layers": L, "batch": B, "n_tokens": N, "d_model": s.d_model,
                      "n_q_heads": s.n_q_heads, "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                      "d_ffn": s.d_ffn, "rank": s.rank, "identifier": args.identifier, "budget": args.budget,
                      "rope_theta": s.rope_theta, "qkv_bias": bias,
                      "rho_peak_lpeak_first_last": list(wl.budget), "k_per_layer": ks,
                      "mean_k": round(float(np.mean(ks)), 2), "unmask_per_step": u}
    line["layer_steps_per_s"] = round(L * B / (ms_step * 1e-3), 2)
    line["full_recompute_ms"] = round(ms_full, 5)
    line["speedup_vs_full"] = round(ms_full / ms_step, 3)
    line["ideal_floor_ms"] = round(ideal_floor_us(work, peak_flops) / 1e3, 5)
    line["per_kernel_us"] = {n: round(v, 2) for n, v in per_us.items()}
    line["per_kernel_roofline"] = per_kernel_fractions(per_us, work, peak_flops)
    line["unmasked_rows_in_update_set"] = coverage
    line["timing"] = {"graphs": graphs is not None, "instances": 1, **block_stats(per_step, ms_step),
                      "full_recompute": block_stats(per_full, ms_full),
                      "note": "ms_per_step = median over the blocks of one denoising step through all layers (the "
                              "unmasking copy included); per-kernel us summed over the layers of one step"}
    line["roofline"] = dominant_roofline(per_us, work, peak_flops, wl.name)
    line["identification"] = identification_summary(per_us, work, ms_step)
    line["gpu"] = gpu_info()
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle over the first denoising steps of every layer")
        line["cpu_baseline"] = cpu_baseline_stack(wl, s, pair, ks, x0, pos, rows, args.cpu_steps, args.identifier,
                                                  bias)
    return line


def cpu_baseline_stack(wl, s, pair, ks, x0, pos, rows, n_steps, identifier, bias=False):
    """The oracle over the first n_steps denoising steps of the whole stack, on its own chain: every
    layer's warm-up from the step-0 embeddings (untimed), then each step unmasks its positions in the
    layer-0 input and runs the cached step of every layer, layer l reading layer l-1's output (timed)."""
    import numpy as np
    import oracle
    import adaptive_hidden_state_amd as spa
    import synth
    L = len(ks)
    threads = blas_threads()
    layers = []
    for l in range(L):   # host copies of the layers' weights (the same seeded draws as the GPU's)
        w = synth.layer_weights_device(wl, l + 1, pair, shape=s, qkv_bias=bias)
        if identifier == "full":
            w_r = w["w_v"].float().cpu().numpy().astype(np.float64)
        else:
            w_r = spa.singular_proxy_from_factors(w["v_lambda"], w["v_right"], s.rank, w["g_attn"])
            w_r = synth.to_storage(w_r.cpu().numpy(), s.dtype).astype(np.float64)
        wh = host_weights(w)
        wh["rope_theta"] = s.rope_theta
        layers.append((wh, w_r))
        del w
    emb = x0.float().cpu().numpy().astype(np.float64)
    caches, x = [], emb
    t0 = time.perf_counter()
    for l in range(L):
        wh, w_r = layers[l]
        caches.append(oracle.warmup(x, wh, w_r, s.head_dim, s.norm_eps, s.dtype))
        x = caches[l].h
    warm_s = time.perf_counter() - t0
    done, el = 0, 0.0
    for t in range(n_steps):
        emb = emb.copy()
        emb[:, pos[t].cpu().numpy()] = rows[t].float().cpu().numpy()
        x = emb
        t0 = time.perf_counter()
        for l in range(L):
            wh, w_r = layers[l]
            caches[l], _, _ = oracle.cached_layer_step(x, wh, w_r, caches[l], ks[l], s.head_dim, s.norm_eps,
                                                       s.dtype)
            x = caches[l].h
            done += 1
        el += time.perf_counter() - t0
    return {"value": done / el, "unit": "layer-steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the first {n_steps} denoising steps of {wl.name} through all {L} layers (k_l = the "
                      f"budget's, B={s.batch}, N={s.n_tokens}, d={s.d_model}) by the NumPy float64 oracle on its "
                      f"own chain: {done} cached layer steps in {el:.1f} s (warm-up of every layer, untimed: "
                      f"{warm_s:.1f} s)",
            "tokens_per_s": round(len(pos[0]) * s.batch * n_steps / el, 4)}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        return os.cpu_count() or 1


def run_batched(args, wl):
    """The batched stress workload: one layer of the llada shape at B sequences of N tokens, over a
    sweep of proxy ranks and budgets; rho = 1 also times the vanilla full recompute."""
    import numpy as np
    import torch

    import adaptive_hidden_state_amd as spa
    import synth

    s0 = wl.shape
    B, N = s0.batch, s0.n_tokens
    ranks = args.ranks or [64, 128, 512]
    rhos = [0.08, 0.16, 0.25, 1.0]
    steps = args.steps or wl.steps
    warmup = 2 if args.warmup is None else args.warmup
    tdt = spa.torch_dtype(s0.dtype)

    log(f"[bench] generating {wl.name} weights and {wl.steps} drift steps on the device")
    pair = synth.haar_pair(wl, s0)
    w = synth.layer_weights_device(wl, 0, pair, shape=s0)
    base = spa.upload_weights(w, spa.singular_proxy_from_factors(w["v_lambda"], w["v_right"], s0.rank,
                                                                 w["g_attn"]).to(tdt), s0.dtype)
    w_rs = {r: spa.spa_pack_weight(spa.singular_proxy_from_factors(w["v_lambda"], w["v_right"], r,
                                                                   w["g_attn"]).to(tdt).contiguous())
            for r in ranks}
    wh = host_weights(w) if not args.no_cpu_baseline else None
    v_lam, v_right = w["v_lambda"], w["v_right"]
    del w
    xs = synth.drift_sequence_device(wl, s0)
    n_in = len(xs) - 1
    sweep, head = [], None
    peak_flops = PEAK_BF16_TFLOPS
    for r in ranks:
        s = s0.replace(rank=r)
        dw = base._replace(w_r=w_rs[r])
        cache = spa.alloc_cache(s)
        ws = spa.alloc_workspace(s, N)
        scores = torch.empty(B, N, dtype=torch.float32, device="cuda")
        for rho in rhos:
            k = int(spa.spa_budget(1, 1, rho, rho, rho, N)[1][0])
            idx = torch.empty(B, k, dtype=torch.int32, device="cuda")
            spa.spa_layer_full(s, dw, cache, xs[0], ws)

            def step(i):
                spa.spa_layer_step(s, dw, cache, xs[1 + i % n_in], k, spa.SPA_PROXY_WRITE_ALL, idx, scores, ws)

            for i in range(warmup):
                step(i)
            torch.cuda.synchronize()
            ms, per = timed_blocks(step, warmup, steps, args.blocks)
            work = {n: kernel_work(n, s, k) for n in step_kernels(s)}
            floor = ideal_floor_us(work, peak_flops) / 1e3
            pt = {"rank": r, "rho": rho, "k": k, "ms_per_step": round(ms, 4),
                  "layer_steps_per_s": round(B / (ms * 1e-3), 2), "ideal_floor_ms": round(floor, 4),
                  "floor_frac": round(floor / ms, 4), "spread": block_stats(per, ms)["spread"]}
            if rho == 1.0:
                def full(i):
                    spa.spa_layer_full(s, dw, cache, xs[1 + i % n_in], ws)

                ms_f, per_f = timed_blocks(full, 0, steps, args.blocks)
                pt["full_recompute_ms"] = round(ms_f, 4)
            log(f"[bench] {pt}")
            sweep.append(pt)
            if r == s0.rank and rho == wl.rho:
                it = iter(range(10 ** 9))

                def one(ev):
                    return spa.spa_layer_step_timed(s, dw, cache, xs[1 + next(it) % n_in], k,
                                                    spa.SPA_PROXY_WRITE_ALL, idx, scores, ws, ev)

                per_us = timed_kernels(spa, one, 5)
                head = (ms, k, per_us, work)
        del cache, ws
    ms_step, k, per_us, work = head
    full = {p["rank"]: p["full_recompute_ms"] for p in sweep if p["rho"] == 1.0}
    line = base_line(args, wl, s0, B / (ms_step * 1e-3), "layer-steps/s", ms_step, steps, warmup,
                     "synthetic (seeded random-init layer with a planted Value spectrum, drawn on the device; "
                     "N(0,1) hidden states, 15% drifting rows per sequence and step)")
    line["config"] = {"workload": wl.name, "batch": B, "n_tokens": N, "d_model": s0.d_model,
                      "n_q_heads": s0.n_q_heads, "n_kv_heads": s0.n_kv_heads, "head_dim": s0.head_dim,
                      "d_ffn": s0.d_ffn, "rank": s0.rank, "rho": wl.rho, "k": k,
                      "sweep": {"rank": ranks, "rho": rhos}}
    line["full_recompute_ms"] = full.get(s0.rank)
    line["speedup_vs_full"] = round(full[s0.rank] / ms_step, 3) if s0.rank in full else None
    line["ideal_floor_ms"] = round(ideal_floor_us(work, peak_flops) / 1e3, 5)
    line["sweep"] = sweep
    line["per_kernel_us"] = {n: round(v, 2) for n, v in per_us.items()}
    line["per_kernel_roofline"] = per_kernel_fractions(per_us, work, peak_flops)
    line["timing"] = {"graphs": False, "instances": 1, "blocks": args.blocks,
                      "note": "eager launches (steps of milliseconds); every ms_per_step is the median over the "
                              "blocks of its timed steps; per-kernel us at the headline point"}
    line["roofline"] = dominant_roofline(per_us, work, peak_flops, wl.name)
    line["identification"] = identification_summary(per_us, work, ms_step)
    line["gpu"] = gpu_info()
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on one sequence")
        line["cpu_baseline"] = cpu_baseline_sequence(wl, s0, wh, v_lam, v_right, xs, args.cpu_seconds)
    return line


def cpu_baseline_sequence(wl, s0, wh, v_lam, v_right, xs, seconds):
    """The oracle's cached step of one sequence of the batched workload (rank and rho of the
    headline point), within a bounded time."""
    import numpy as np
    import oracle
    import adaptive_hidden_state_amd as spa
    import synth
    s = s0.replace(batch=1)
    k = int(spa.spa_budget(1, 1, wl.rho, wl.rho, wl.rho, s.n_tokens)[1][0])
    w_r = synth.to_storage(spa.singular_proxy_from_factors(v_lam, v_right, s.rank, None).cpu().numpy(),
                           s.dtype).astype(np.float64)
    x = [xs[j][:1].float().cpu().numpy().astype(np.float64) for j in range(len(xs))]
    kc, vc = oracle.kv_project(x[0], wh, s.head_dim, s.norm_eps, s.dtype)
    pc = oracle.proxy(x[0], w_r).astype(np.float32).astype(np.float64)
    cache = oracle.LayerCache(kc, vc, x[0].copy(), pc)
    done, t0 = 0, time.perf_counter()
    while True:
        cache, _, _ = oracle.cached_layer_step(x[1 + done % (len(x) - 1)], wh, w_r, cache, k, s.head_dim,
                                               s.norm_eps, s.dtype)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": done / el, "unit": "layer-steps/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{done} cached steps of one sequence of {wl.name} (N={s.n_tokens}, d={s.d_model}, "
                      f"r={s.rank}, k={k}) by the NumPy float64 oracle, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200 layer steps; the schedule's denoising steps for a stack; "
                         "16 for the batched sweep)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="llada-layer",
                    choices=["llada-layer", "tiny-f32", "llada-stack", "dream-stack", "batched-stress"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-steps", type=int, default=2,
                    help="stacks: denoising steps through every layer that the CPU oracle baseline runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--instances", type=int, default=4,
                    help="independent layer instances visited in turn (defeats Infinity-Cache reuse)")
    ap.add_argument("--no-graph", dest="graph", action="store_false", help="time eager launches")
    ap.add_argument("--graph-per-step", dest="graph_group", action="store_false",
                    help="layer workloads: one graph launch per step (default: the steps of the R instances "
                         "in one graph, as a denoising step's graph holds every layer)")
    ap.add_argument("--blocks", type=int, default=5,
                    help="the timed steps run as this many consecutive blocks; ms_per_step is their median")
    ap.add_argument("--budget", choices=["adaptive", "uniform"], default="adaptive",
                    help="stacks: piecewise-Gaussian rho(l), or its mean on every layer")
    ap.add_argument("--rank", type=int, default=None, help="stacks: proxy rank r")
    ap.add_argument("--identifier", choices=["proxy", "full"], default="proxy",
                    help="stacks: singular proxy, or the full Value projection (r = d_kv)")
    ap.add_argument("--ranks", type=int, nargs="*", default=None, help="batched sweep: proxy ranks")
    ap.add_argument("--arch", action="store_true",
                    help="the real layers' attention terms: rotary embedding (LLaDA theta 5e5, Dream 1e6) and "
                         "Dream's q/k/v biases")
    ap.add_argument("--unmask", type=int, default=None,
                    help="stacks: tokens unmasked per denoising step (default 16 LLaDA, 64 Dream)")
    ap.add_argument("--summarize-trace", metavar="CSV", help="summarise a rocprofv3 kernel_trace.csv and exit")
    ap.add_argument("--summarize-counters", metavar="CSV", nargs="*", default=[],
                    help="summarise rocprofv3 counter_collection.csv files and exit")
    args = ap.parse_args()
    if args.summarize_trace or args.summarize_counters:
        print(summarize_profile(args.summarize_trace, args.summarize_counters))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import adaptive_hidden_state_amd as spa
    import synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    spa.load_library()
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    if wl.n_layers > 1:
        line = run_stack(args, wl)
    elif wl.name == "batched-stress":
        line = run_batched(args, wl)
    else:
        line = run_layer(args, wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
