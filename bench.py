"""Benchmark of one GPU's expert-parallel MoE FFN share on MI355X.

A step is one pass of the whole path over one batch of synthetic input:
routing + dispatch layout (moe_dispatch_layout), the persistent fused FFN
(moe_ffn_forward: Linear-1 + SwiGLU, Linear-2 + weighted combine stores) and
the source-side reduction of the combine slots (moe_combine_check with
y_local, in bf16 by default: the model's activation format). Inputs are
resident in HBM before the timed region starts.

Prints one JSON line. ``value`` is TFLOP/s of the algorithmic FLOPs
(6*H*I per routed row) over the whole step, for the schedule named in
config.schedule; per-schedule FFN-only timings (paired, A-B-C-D-D-C-B-A
order, for Expert-Wave with the automatic waves and with one wave,
Interleaved and the schedule planner's recommendation, with the planner's
predictions beside them), the mean shader clock over the mainloops (from the
kernel's task trace) and the roofline of the dominant kernel ride along, with
the CPU oracle (float32) timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import moe_inputs as mi  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
FFN_KERNELS = {"bf16": "moe_ffn_bf16", "fp8": "moe_ffn_fp8", "w4a8": "moe_ffn_w4a8"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


KERNEL_SOURCES = {"bf16": "ffn_bf16.hip", "fp8": "ffn_fp8.hip", "w4a8": "ffn_w4a8.hip"}


def kernel_source_hash(dtype: str) -> str:
    """Hash of the sources one dtype's FFN kernel is built from (its own file,
    the shared device helpers and the schedules)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_expert_ffn_persistent_amd", "csrc")
    for name in (KERNEL_SOURCES[dtype], "ffn_common.hpp", "sched.hpp"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_counts(wl, R: int, active: int):
    H, I = wl.hidden, wl.inter
    flops = 6.0 * H * I * R
    sw = {"bf16": 2.0, "fp8": 1.0, "w4a8": 0.5}[wl.dtype]     # bytes per weight element
    sx = 2.0 if wl.dtype == "bf16" else 1.0                     # per x and h element
    weight_bytes = active * 3.0 * H * I * sw
    x_bytes = R * H * sx
    h_bytes = 2.0 * R * I * sx
    comb_bytes = R * H * 2.0
    scale_bytes = 0.0
    if wl.dtype == "fp8":
        scale_bytes = active * 3.0 * (H // 128) * (I // 128) * 4 + R * (H // 128) * 4 \
            + 2.0 * R * (I // 128) * 4
    elif wl.dtype == "w4a8":     # one E8M0 byte per 32 elements
        scale_bytes = active * 3.0 * H * I / 32 + R * H / 32 + 2.0 * R * I / 32
    return flops, weight_bytes + x_bytes + h_bytes + comb_bytes + scale_bytes, dict(
        weights=weight_bytes, x=x_bytes, h=h_bytes, combine=comb_bytes, scales=scale_bytes)


def host_info() -> dict:
    """CPU model, BLAS vendor and the threads BLAS runs with."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"cpu_model": model,
            "blas": ",".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in blas})) or "unknown",
            "threads": max([i.get("num_threads", 1) for i in blas] or [1]),
            "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_baseline(inp, seconds_budget: float):
    """Time the CPU oracle (its float32 setting: the same code in single
    precision) on a bounded sample: routing and layout over all tokens, then
    the expert FFN and weighted combine for as many local experts (in order)
    as fit the budget. When every local expert fits, the whole workload is
    run again while the budget lasts and the median time is reported."""
    from oracle import moe_oracle as mo
    wl = inp.wl
    info = host_info()
    t0 = time.perf_counter()
    n_exp = 0
    rows = 0
    while n_exp < wl.num_local:
        n_exp = min(wl.num_local, max(1, n_exp * 2))
        t1 = time.perf_counter()
        res = mo.run(inp, block_m=128, experts=n_exp, float_type=np.float32)
        dt = time.perf_counter() - t1
        rows = int(res.layout.row_offset[n_exp])
        # the next sample (twice the experts; its time estimated from its
        # routed rows) must end within the budget
        next_rows = int(res.layout.row_offset[min(wl.num_local, 2 * n_exp)])
        del res
        if n_exp < wl.num_local and time.perf_counter() - t0 + dt * max(1.0, next_rows / max(rows, 1)) > seconds_budget:
            break
    times = [dt]
    while n_exp == wl.num_local and time.perf_counter() - t0 + 1.2 * dt < seconds_budget:
        t1 = time.perf_counter()
        mo.run(inp, block_m=128, experts=n_exp, float_type=np.float32)
        times.append(time.perf_counter() - t1)
    dt = statistics.median(times)
    flops = 6.0 * wl.hidden * wl.inter * rows
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(info["threads"]),
            "kind": "oracle",
            "sample": f"{wl.name}: routing+layout of all {wl.num_tokens} tokens, expert FFN and "
                      f"combine of local experts 0..{n_exp - 1} ({rows} routed rows), float32 "
                      f"numpy, {dt:.2f} s (median of {len(times)})",
            "cpu_model": info["cpu_model"], "blas": info["blas"],
            "affinity_cores": info["affinity_cores"]}


def trace_clock(ffn, call, wall_khz: int):
    """Mean shader clock (MHz) over the mainloops of one traced FFN call:
    shader-clock cycles (trace words 6..7) over wall-clock ticks (words 2..4)
    of every task."""
    import torch
    from moe_expert_ffn_persistent_amd import _lib
    cap = 512
    tr = torch.zeros((ffn.plan.grid, cap, _lib.TRACE_WORDS), dtype=torch.int32, device=ffn.device)
    call(trace=tr, trace_capacity=cap)
    torch.cuda.synchronize()
    t = tr.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    t = t.reshape(-1, _lib.TRACE_WORDS)
    t = t[t[:, 0] != 0]
    cyc = (t[:, 7] - t[:, 6]) & 0xFFFFFFFF
    wall = (t[:, 4] - t[:, 2]) & 0xFFFFFFFF
    ok = wall > 0
    if not ok.any():
        return None
    return round(float(cyc[ok].sum()) / float(wall[ok].sum()) * wall_khz / 1e3, 1)


def rocm_version() -> str:
    try:
        return open("/opt/rocm/.info/version").read().strip()
    except OSError:
        return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_skew", choices=sorted(mi.WORKLOADS),
                    help="default: the largest single-GPU configuration by FLOPs (the "
                         "DeepSeek-V3-shaped share with Zipf-skewed routing, 8 x 2048 tokens)")
    ap.add_argument("--schedule", default="interleaved", choices=["interleaved", "expert_wave", "auto"],
                    help="auto: the schedule planner's recommendation for the workload's routing, "
                         "resolved once before the timed region")
    ap.add_argument("--pairs", type=int, default=10,
                    help="A-B-B-A rounds of the schedule comparison (0: none, e.g. under a profiler, so that "
                         "only the headline schedule is launched)")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--tokens-per-slice", type=int, default=0,
                    help="run the workload's shapes at another batch size (workload name gets @T<n>)")
    ap.add_argument("--lead-d", type=int, default=0)
    ap.add_argument("--y-dtype", default="bf16", choices=["bf16", "fp32"],
                    help="element type of the reduced output y_local")
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported here "
              "(one process, one MI355X). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    wl = mi.get_workload(args.workload)
    if args.tokens_per_slice > 0:
        wl = wl.with_tokens(args.tokens_per_slice)
    t_gen = time.perf_counter()
    inp = mi.make_inputs(wl, workers=min(16, os.cpu_count() or 1))   # before any GPU call
    t_gen = time.perf_counter() - t_gen

    import torch

    from moe_expert_ffn_persistent_amd import MoeExpertFFN
    dev = torch.device("cuda:0")
    S, T, H, k = wl.num_slices, wl.tokens_per_slice, wl.hidden, wl.top_k

    def up(a):
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    logits = up(inp.logits)
    bias = None if inp.bias is None else up(inp.bias)
    x = up(inp.x.reshape(S, T, H))
    xs = None if inp.x_scale is None else up(inp.x_scale.reshape(S, T, -1))
    w1, w2 = up(inp.w1), up(inp.w2)
    w1s = None if inp.w1_scale is None else up(inp.w1_scale)
    w2s = None if inp.w2_scale is None else up(inp.w2_scale)
    comb = torch.empty((S, T, k, H), dtype=torch.int16, device=dev)
    y = torch.empty((wl.num_tokens, H), dtype=torch.bfloat16 if args.y_dtype == "bf16" else torch.float32,
                    device=dev)
    x_sl = [x[s] for s in range(S)]
    xs_sl = None if xs is None else [xs[s] for s in range(S)]
    c_sl = [comb[s] for s in range(S)]

    ffn = MoeExpertFFN(S, T, wl.num_experts, k, wl.local_begin, wl.num_local, H, wl.inter,
                       dtype=wl.dtype, schedule=args.schedule, tile=args.tile,
                       lead_d=args.lead_d, device=dev)
    stream = torch.cuda.current_stream()

    def ffn_call(cfg):
        ffn.forward(x_sl, w1, w2, c_sl, x_scales=xs_sl, w1_scales=w1s, w2_scales=w2s, **cfg)

    def step(cfg, ev=None):
        ffn.layout(logits=logits, bias=bias)
        if ev is not None:
            ev[0].record(stream)
        ffn_call(cfg)
        if ev is not None:
            ev[1].record(stream)
        ffn.combine_check(c_sl, y=y)

    ffn.layout(logits=logits, bias=bias)
    torch.cuda.synchronize()
    totals = ffn.layout_bufs.totals.cpu().numpy()
    R, P, max_rows, active = (int(v) for v in totals)
    flops, alg_bytes, byte_parts = algorithmic_counts(wl, R, active)
    # schedule planner for this routing (host model; reads the layout's counts)
    pred = ffn.predict_schedule(schedule="interleaved", lead_d=args.lead_d)
    rec = pred["recommended"]
    rec_cfg = {"schedule": rec["schedule"], "lead_d": rec["lead_d"],
               "experts_per_wave": rec["experts_per_wave"]}
    head_cfg = rec_cfg if args.schedule == "auto" else {"schedule": args.schedule}

    for _ in range(args.warmup):
        step(head_cfg)
    torch.cuda.synchronize()
    ffn.check_status()   # raises on a latched device error

    # ---- timed region: exactly K steps of the headline schedule ----
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(head_cfg, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ffn_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = wall * 1e3 / args.steps
    ffn.check_status()

    # ---- the same step captured once in a HIP graph and replayed (after
    # the timed region; the headline figures above are the eager step) ----
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(head_cfg)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(head_cfg)
        graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = round((time.perf_counter() - t1) * 1e3 / args.steps, 4)
        del graph
    except RuntimeError as err:   # reported, not fatal: the eager step is the measurement
        graph_ms = f"capture failed: {err}"[:200]
    ffn.check_status()

    # ---- paired schedule comparison, FFN only, A-B-C-C-B-A: both orders
    # with their default parameters, and the planner's recommendation ----
    arms = {"expert_wave": {"schedule": "expert_wave"}, "interleaved": {"schedule": "interleaved"},
            "expert_wave_one_wave": {"schedule": "expert_wave", "experts_per_wave": wl.num_local},
            "recommended": rec_cfg}
    # the recommendation is timed as an arm of its own only when it is not
    # one of the fixed configurations (Expert-Wave with one wave is a
    # planner candidate too)
    same_as = None
    if rec_cfg["schedule"] == "interleaved" and rec_cfg["lead_d"] == ffn.plan.lead_d:
        same_as = "interleaved"
    elif rec_cfg["schedule"] == "expert_wave" and rec_cfg["experts_per_wave"] == 0:
        same_as = "expert_wave"
    elif rec_cfg["schedule"] == "expert_wave" and rec_cfg["experts_per_wave"] >= wl.num_local:
        same_as = "expert_wave_one_wave"
    if same_as:
        del arms["recommended"]
    per = {a: [] for a in arms}
    order = list(arms)
    for r in range(args.pairs):
        seq = order if r % 2 == 0 else order[::-1]
        for arm in seq:
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            ffn_call(arms[arm])
            b_.record(stream)
            b_.synchronize()
            per[arm].append(a_.elapsed_time(b_))
    sched_out = {}
    for s_, v in per.items():
        if not v:
            continue
        med = statistics.median(v)
        sched_out[s_] = {"ffn_us_median": round(med * 1e3, 2), "ffn_us_min": round(min(v) * 1e3, 2),
                         "tflops": round(flops / (med * 1e-3) / 1e12, 2),
                         "hbm_gbs": round(alg_bytes / (med * 1e-3) / 1e9, 1)}
    speedup = speedup_best = None
    if args.pairs > 0:
        speedup = statistics.median(per["expert_wave"]) / statistics.median(per["interleaved"])
        best_wave = min(statistics.median(per["expert_wave"]), statistics.median(per["expert_wave_one_wave"]))
        speedup_best = best_wave / statistics.median(per["interleaved"])
    sclk = trace_clock(ffn, lambda **kw: ffn_call(dict(head_cfg, **kw)), ffn.plan.wall_clock_khz)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    plan = ffn.plan
    # W4A8 runs e2m1 x e4m3 MFMAs, which issue at the fp8 rate
    peak_flops = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP8_TFLOPS
    ffn_avg_s = statistics.mean(ffn_ms) * 1e-3
    t_mfma = flops / (peak_flops * 1e12)
    t_hbm = alg_bytes / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE)).get(wl.name)
            if tr and tr.get("kernel_hash") == kernel_source_hash(wl.dtype):
                traffic = tr.get("bytes_per_launch")
        except (ValueError, OSError):
            traffic = None
    if bound == "hbm":
        achieved = alg_bytes / ffn_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        achieved = flops / ffn_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4), "traffic": traffic}
    roof.update({"kernel": FFN_KERNELS[wl.dtype], "avg_launch_us": round(ffn_avg_s * 1e6, 2),
                 "algorithmic_bytes": alg_bytes, "algorithmic_flops": flops,
                 "bytes_parts": byte_parts,
                 "mfma_frac": round(flops / ffn_avg_s / 1e12 / peak_flops, 4),
                 "hbm_frac": round(alg_bytes / ffn_avg_s / 1e9 / PEAK_HBM_GBS, 4)})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)

    out = {
        "metric": "MoE FFN TFLOP/s (L1+L2+combine) on 1 MI355X, % of MFMA peak, per schedule",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded normal inputs, random-init expert weights)",
        "config": {"workload": wl.name, "schedule": args.schedule, "schedule_config": head_cfg, "slices": S,
                   "tokens_per_slice": T, "experts": wl.num_experts, "top_k": k, "y_dtype": args.y_dtype,
                   "local_experts": wl.num_local, "hidden": H, "inter": wl.inter,
                   "routed_rows": R, "sched_rows": P, "max_rows_per_expert": max_rows,
                   "active_experts": active, "tile": plan.tile, "block_m": plan.block_m,
                   "block_n": plan.block_n1, "grid": plan.grid, "lead_d": plan.lead_d,
                   "r_expert": round(max_rows / (wl.num_tokens * k / wl.num_experts), 3)},
        "pct_of_mfma_peak": round(100 * flops / (ms_per_step * 1e-3) / 1e12 / peak_flops, 2),
        "ffn_only_ms": round(statistics.mean(ffn_ms), 4),
        "graph_ms_per_step": graph_ms,
        "ffn_ms_p50_p90": [round(float(np.percentile(ffn_ms, 50)), 4), round(float(np.percentile(ffn_ms, 90)), 4)],
        "per_schedule": sched_out,
        "speedup_interleaved_over_wave": None if speedup is None else round(speedup, 4),
        "speedup_interleaved_over_best_wave": None if speedup_best is None else round(speedup_best, 4),
        "sclk_mhz_mainloop": sclk,
        "rocm": rocm_version(),
        "torch": torch.__version__,
        "planner": {
            "recommended": rec_cfg,
            "predicted_units": {"expert_wave": round(pred["candidates"][0]["makespan"], 1),
                                "interleaved": round(pred["given"]["makespan"], 1),
                                "recommended": round(rec["makespan"], 1),
                                "lower_bound": round(pred["lower_bound"], 1)},
            "predicted_hbm_gb": {"expert_wave": round(pred["candidates"][0]["hbm_bytes"] / 1e9, 3),
                                 "interleaved": round(pred["given"]["hbm_bytes"] / 1e9, 3),
                                 "recommended": round(rec["hbm_bytes"] / 1e9, 3),
                                 "compulsory": round(pred["given"]["unique_bytes"] / 1e9, 3)},
            "predicted_wave_over_interleaved": round(pred["candidates"][0]["makespan"]
                                                     / max(pred["given"]["makespan"], 1e-9), 4),
            "measured_wave_over_interleaved": None if speedup is None else round(speedup, 4),
            "recommended_is": same_as,
            "measured_recommended_over_interleaved": None if args.pairs <= 0 else round(
                statistics.median(per[same_as or "recommended"]) / statistics.median(per["interleaved"]), 4),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
