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
    """Text summary of rocprofv3 CSV output: per (kernel, grid) dispatch count and average/median
    duration from a --kernel-trace run, and per (kernel, grid) average counter values from --pmc runs."""
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

    out = []
    if trace_csv:
        groups = {}
        with open(trace_csv) as f:
            for row in csv.DictReader(f):
                g, wg = grid_of(row)
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0
                groups.setdefault((short(row["Kernel_Name"]), g // wg, wg), []).append(dur)
        out.append(f"{'kernel':64s} {'workgroups':>10s} {'wg':>5s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s}")
        for (name, nwg, wg), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{name[:64]:64s} {nwg:10d} {wg:5d} {len(v):6d} {sum(v) / len(v):9.2f} "
                       f"{statistics.median(v):9.2f}")
    for path in counter_csvs:
        groups = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                g, wg = grid_of(row)
                groups.setdefault((short(row["Kernel_Name"]), g // wg, wg, row["Counter_Name"]), []).append(
                    float(row["Counter_Value"]))
        out.append("")
        out.append(f"{'kernel':64s} {'workgroups':>10s} {'wg':>5s} {'counter':>12s} {'calls':>6s} {'avg':>14s}")
        for (name, nwg, wg, cn), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{name[:64]:64s} {nwg:10d} {wg:5d} {cn:>12s} {len(v):6d} {sum(v) / len(v):14.1f}")
    return "\n".join(out)


def kernel_work(name, s, k):
    """Algorithmic bytes and flops of one kernel of the cached step (inputs read once, outputs written
    once), for the per-kernel HBM / MFMA fractions."""
    e = 2 if s.dtype == "bf16" else 4
    rows, M = s.batch * s.n_tokens, s.batch * k
    if name == "proxy_gemm":
        return (rows * s.d_model + s.rank * s.d_model) * e + rows * s.rank * 4, 2.0 * rows * s.d_model * s.rank
    if name == "proxy_cosine":
        return rows * s.rank * 4 * 3 + rows * 4, 6.0 * rows * s.rank
    if name == "topk":
        return rows * 4 + M * 4, 0.0
    if name == "attention":
        kv = 2 * s.batch * s.n_kv_heads * s.n_tokens * s.head_dim * e
        return kv + 2 * M * s.d_q * e, 4.0 * M * s.n_q_heads * s.n_tokens * s.head_dim
    return gemm_work(name, s, M)


def cpu_baseline(wl, w, w_r, xs, k, seconds):
    """The oracle's cached layer step timed on the host cores (bounded sample)."""
    import numpy as np
    import oracle
    s = wl.shape
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llada-layer", choices=["llada-layer", "tiny-f32"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--instances", type=int, default=4,
                    help="independent layer instances visited in turn (defeats Infinity-Cache reuse)")
    ap.add_argument("--no-graph", dest="graph", action="store_false", help="time eager launches")
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

    import numpy as np
    import torch

    import adaptive_hidden_state_amd as spa
    import synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    spa.load_library()
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    s = wl.shape
    k = int(spa.spa_budget(1, 1, wl.rho, wl.rho, wl.rho, s.n_tokens)[1][0])
    M = s.batch * k

    log(f"[bench] generating {wl.name} weights and inputs")
    t = time.time()
    w = synth.layer_weights(wl)
    w_r = synth.to_storage(spa.singular_proxy_from_factors(w["v_lambda"], w["v_right"], s.rank, w["g_attn"]), s.dtype)
    xs, _ = synth.drift_sequence(wl)
    log(f"[bench] inputs ready in {time.time() - t:.1f} s")

    # R independent layer instances (weights, caches, inputs at distinct addresses), visited in turn, so
    # that no step finds the previous step's data in the 256 MB Infinity Cache (one cycle streams > 1 GB)
    R = max(1, args.instances)
    dw0 = spa.upload_weights(w, w_r, s.dtype)
    dws = [dw0] + [spa.DeviceWeights(*(t.clone() for t in dw0)) for _ in range(R - 1)]
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

    # vanilla full recompute of the same layer (the "Baseline 100%" path), for the speedup
    scratch = [spa.alloc_cache(s) for _ in range(R)]
    for r in range(R):
        spa.spa_layer_full(s, dws[r], scratch[r], xds[r][1], ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_full = 4 * R
    e0.record()
    for i in range(n_full):
        spa.spa_layer_full(s, dws[i % R], scratch[i % R], xds[i % R][1 + (i // R) % n_in], ws)
    e1.record()
    torch.cuda.synchronize()
    ms_full = e0.elapsed_time(e1) / n_full
    del scratch

    def which(i):  # step i -> (instance, input step)
        return i % R, 1 + (i // R) % n_in

    def eager_step(i):
        r, j = which(i)
        spa.spa_layer_step(s, dws[r], caches[r], xds[r][j], k, spa.SPA_PROXY_WRITE_ALL, idx, scores, ws)

    # one captured HIP graph per (instance, input step); every launch of a step is stream-ordered and
    # allocation-free, so the step is capturable as is
    graphs = None
    if args.graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for i in range(R * n_in):
                    eager_step(i)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graphs = []
            for i in range(R * n_in):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    eager_step(i)
                graphs.append(g)
            torch.cuda.synchronize()
        except Exception as exc:  # fall back to eager launches
            log(f"[bench] graph capture unavailable ({exc}); timing eager launches")
            graphs = None

    def step(i):
        if graphs is not None:
            r, j = which(i)
            graphs[r * n_in + (j - 1)].replay()
        else:
            eager_step(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} cached layer steps ({'graphs' if graphs else 'eager'}, {R} instances)")
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-kernel durations: HIP events between the kernels of the same step sequence
    ev = spa.HipEvents(24)
    per = {}
    n_prof = max(10, min(args.steps, 50))
    for i in range(n_prof):
        r, j = which(i)
        res = spa.spa_layer_step_timed(s, dws[r], caches[r], xds[r][j], k, spa.SPA_PROXY_WRITE_ALL, idx, scores,
                                       ws, ev)
        seen = {}
        for name, ms in res:
            seen[name] = seen.get(name, 0.0) + ms
        for name, ms in seen.items():
            per.setdefault(name, []).append(ms)
    ev.close()
    per_us = {n: 1000.0 * float(np.median(v)) for n, v in per.items()}

    peak_flops = PEAK_BF16_TFLOPS if s.dtype == "bf16" else PEAK_FP32_TFLOPS
    per_kernel = {}
    for n, us in per_us.items():
        wk = kernel_work(n, s, k)
        if wk is None:
            continue
        byts, flops = wk
        per_kernel[n] = {"us": round(us, 2), "GB/s": round(byts / us / 1e3, 1),
                         "hbm_frac": round(byts / us / 1e3 / PEAK_HBM_GBS, 4),
                         "TFLOP/s": round(flops / us / 1e6, 1),
                         "mfma_frac": round(flops / us / 1e6 / peak_flops, 4)}

    # roofline of the dominant kernel
    dom = max((n for n in per_us if gemm_work(n, s, M)), key=lambda n: per_us[n])
    byts, flops = gemm_work(dom, s, M)
    dur_s = per_us[dom] * 1e-6
    hbm_bound = byts / (PEAK_HBM_GBS * 1e9) >= flops / (peak_flops * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": byts / dur_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / dur_s / 1e12, "peak": peak_flops, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, wl.name)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = byts
    roof["algorithmic_flops"] = flops
    roof["mfma_frac"] = flops / dur_s / 1e12 / peak_flops

    value = s.batch / (ms_step * 1e-3)
    line = {
        "metric": "tokens/s & layer-steps/s (8B-shape, N=1024, r=128) + % HBM/MFMA peak",
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded random-init weights with a planted Value spectrum; drifting N(0,1) hidden states)",
        "config": {"workload": wl.name, "batch": s.batch, "n_tokens": s.n_tokens, "d_model": s.d_model,
                   "n_q_heads": s.n_q_heads, "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                   "d_ffn": s.d_ffn, "rank": s.rank, "rho": wl.rho, "k": k},
        "tokens_per_s_projected": round(16 * s.batch / (32 * ms_step * 1e-3), 2),
        "full_recompute_ms": round(ms_full, 5),
        "speedup_vs_full": round(ms_full / ms_step, 3),
        "per_kernel_us": {n: round(v, 2) for n, v in per_us.items()},
        "per_kernel_roofline": per_kernel,
        "timing": {"graphs": graphs is not None, "instances": R,
                   "note": "per-kernel us from HIP events recorded between kernels on the launch stream"},
        "roofline": roof,
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        import oracle  # noqa: F401  (test infrastructure, only for this baseline leg)
        w_r64 = np.asarray(w_r, np.float64)
        line["cpu_baseline"] = cpu_baseline(wl, w, w_r64, xs, k, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
