"""The store path behind the Linear-2 epilogue on this GPU, in the terms of the
X-Stage paper (section 3, "Characterizing and Modeling X-Stage"; section 4.2).

The paper models remote stores with three platform quantities: the
backpressure-free issue time T_iss0 of a burst, the effective drain rate R
and the effective outstanding capacity Q. On one GPU the combine stores are
scattered stores to local HBM; this module calibrates the same quantities for
them with ``moe_store_burst_probe`` and reads the per-tile store spans of the
FFN kernel from its task trace (words 4, 5 and 8: mainloop end, stores
issued, stores completed).

The model functions are plain restatements of the paper's equations (Eq. 1-7,
14, 15) and are pinned by tests on synthetic data. The probe driver and
``tile_spans`` only marshal arguments and reduce time stamps; every store is
made by the HIP kernels.

Run ``python -m moe_expert_ffn_persistent_amd.xstage [--workload dsv3]`` on a
GPU: it prints one JSON object with the calibration, the gap sweep against
the model, and the span table of both schedules.
"""
from __future__ import annotations

import argparse
import json
import sys
from dataclasses import dataclass

import numpy as np

KIB = 1024


# ---------------------------------------------------------------- model ----
# V in bytes, times in microseconds, R in bytes per microsecond.

def t_iss(G, V, t0, R):
    """Sender-visible issue time of a periodic burst (Eq. 3)."""
    return np.maximum(t0, V / R - G)


def t_period(G, V, t0, R):
    """Start-to-start period of periodic bursts: issue plus gap (Eq. 2), and
    at least the drain time V/R (Eq. 1)."""
    return np.maximum(t0 + G, V / R)


def delta_t_iss(G, V, t0, R):
    """Backpressure overhead of the issue (Eq. 4)."""
    return np.maximum(0.0, V / R - G - t0)


def g_star(V, t0, R):
    """Shortest gap that recovers the backpressure-free issue time (Eq. 5)."""
    return np.maximum(0.0, V / R - t0)


def q_peak0(V, t0, R):
    """Outstanding volume at the end of an unconstrained isolated burst (Eq. 6)."""
    return np.maximum(0.0, V - R * t0)


def t_iss_isolated(V, t0, R, Q):
    """Issue time of an isolated burst with a finite capacity Q (Eq. 7)."""
    return np.maximum(t0, (V - Q) / R)


def fit_drain_rate(V, T) -> float:
    """R from drain-dominated zero-gap periods T = V / R (least squares
    through the origin, section 3.3)."""
    V = np.asarray(V, float)
    T = np.asarray(T, float)
    return float((V * V).sum() / (V * T).sum())


def fit_capacity(V, T_iso, t0, R, knee: float = 1.25):
    """Q from isolated bursts beyond the knee, where T_iso = (V - Q) / R
    (Eq. 7): the median of V - R * T_iso over the points whose issue time
    exceeds `knee` times their backpressure-free issue time t0 (a scalar or
    one value per point); None if no point does."""
    V = np.asarray(V, float)
    T = np.asarray(T_iso, float)
    sel = T > knee * np.broadcast_to(np.asarray(t0, float), T.shape)
    if not sel.any():
        return None
    return float(np.median(V[sel] - R * T[sel]))


def interleave_sufficient(n1, n2, V, t0, R, T_l1, T_l2) -> bool:
    """Condition 1 of section 4.2 (Eq. 14): the natural gap of the interleaved
    cycle covers the drain of its bursts, n2 V <= R (n2 (T_iss0 + T_L2) + n1 T_L1)."""
    return n2 * V <= R * (n2 * (t0 + T_l2) + n1 * T_l1)


def critical_stall(T_rs, T_cover):
    """Part of a tile's store span that reaches the compute critical path (Eq. 15)."""
    return np.maximum(0.0, np.asarray(T_rs, float) - np.asarray(T_cover, float))


# ------------------------------------------------------------- the probe ---

def _wrap(d):
    """Differences of low-32-bit clock stamps."""
    return (np.asarray(d, np.int64) + (1 << 32)) % (1 << 32)


def burst_concurrency(start, end) -> np.ndarray:
    """For each interval [start, end) of integer ticks (one per producer and
    burst; the intervals of one producer do not overlap), the mean number of
    intervals open over it, itself included: the number of producers issuing
    alongside it, so that (this count) x B is the aggregate burst volume V of
    the paper's model. Intervals of zero length count the intervals open at
    their start."""
    s = np.asarray(start, np.int64).ravel()
    e = np.maximum(np.asarray(end, np.int64).ravel(), s)
    lo = s.min()
    s, e = s - lo, e - lo
    n = int(e.max()) + 2
    diff = np.zeros(n, np.int64)
    np.add.at(diff, s, 1)
    np.add.at(diff, e, -1)
    open_ = np.cumsum(diff)[:-1]                 # intervals open during tick t
    pre = np.concatenate([[0], np.cumsum(open_)])
    width = e - s
    mean = np.where(width > 0, (pre[e] - pre[s]) / np.maximum(width, 1), open_[s] + (width == 0))
    return mean.reshape(np.shape(start))


@dataclass
class BurstRun:
    K: int
    B: int
    gap_us: float
    control: bool
    t_iss: np.ndarray      # [K, bursts] us
    t_period: np.ndarray   # [K, bursts - 1] us
    kernel_us: float       # launch to completion, every store drained
    window_us: float       # first burst start to last burst issued, over producers
    k_eff: np.ndarray      # [K, bursts] producers issuing alongside each burst

    @property
    def V(self) -> int:
        return self.K * self.B

    def drained_rate(self) -> float:
        """Bytes per microsecond over the whole launch: every store of every
        burst has left the chip's buffers once the kernel has completed."""
        return self.V * self.t_iss.shape[1] / self.kernel_us

    def steady(self, skip: int = 2):
        """Mean issue time and period over producers and bursts after the
        first `skip`: means, not medians, so that bursts x period is the
        producers' issue time (backpressure stalls are few and long)."""
        return (float(np.mean(self.t_iss[:, skip:])),
                float(np.mean(self.t_period[:, skip:])) if self.t_period.shape[1] > skip else float("nan"))

    def v_eff(self, skip: int = 2) -> float:
        """Aggregate burst volume in flight: mean concurrency x B."""
        return float(np.mean(self.k_eff[:, skip:])) * self.B


def wall_clock_khz() -> int:
    from . import _lib
    s = _lib.MoeShape(1, 1, 1, 1, 0, 1, 256, 128, 0)
    return _lib.ffn_plan(s, _lib.MoeSchedParams()).wall_clock_khz


class Prober:
    """Runs moe_store_burst_probe on one device with a reusable destination."""

    def __init__(self, dst_bytes: int = 1 << 30, device="cuda"):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.dst = torch.empty(dst_bytes, dtype=torch.uint8, device=self.device)
        self.khz = wall_clock_khz()

    def run(self, K: int, B: int, gap_us: float = 0.0, bursts: int = 10, control: bool = False,
            row_bytes: int = 512) -> BurstRun:
        from . import _lib
        torch = self.torch
        stamps = torch.zeros(K * bursts * 2, dtype=torch.int32, device=self.device)
        prm = _lib.MoeBurstParams(K, B, bursts, row_bytes, 1 if control else 0, int(gap_us * 1000))
        stream = torch.cuda.current_stream(self.device)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        _lib.store_burst_probe(prm, self.dst.data_ptr(), self.dst.numel(), stamps.data_ptr(),
                               stream.cuda_stream)
        ev1.record(stream)
        torch.cuda.synchronize(self.device)
        st = stamps.cpu().numpy().astype(np.int64).reshape(K, bursts, 2) & 0xFFFFFFFF
        us = 1e3 / self.khz
        rel = _wrap(st - st[:, :, 0].min())
        return BurstRun(K, B, gap_us, control, _wrap(st[:, :, 1] - st[:, :, 0]) * us,
                        _wrap(st[:, 1:, 0] - st[:, :-1, 0]) * us, ev0.elapsed_time(ev1) * 1e3,
                        float(rel[:, :, 1].max() * us), burst_concurrency(rel[:, :, 0], rel[:, :, 1]))


def calibrate(pr: Prober, K: int = 256) -> dict:
    """Drain rate, backpressure-free issue time, capacity and a gap sweep
    compared with the model (sections 3.3-3.5).

    R is the drained rate of long zero-gap runs: bytes over launch-to-
    completion time, which includes every store reaching memory. T_iss0 of a
    burst is the issue time of the L2-resident control of the same K and B
    (no HBM drain behind it). The aggregate volume V of each burst is its
    measured concurrency (producers issuing alongside it) times B: the
    workgroups of one launch do not all issue at once."""
    out = {"K": K}
    pts, runs = [], {}
    for k in (K, 2 * K, 4 * K):
        for b_kib in (16, 32, 64, 128, 256):
            r = pr.run(k, b_kib * KIB, 0.0, bursts=24)
            c = pr.run(k, b_kib * KIB, 0.0, bursts=24, control=True)
            runs[(k, b_kib * KIB)] = (r, c)
            ti, tp = r.steady()
            pts.append({"K": k, "B": b_kib * KIB, "t_iss_us": ti, "t_period_us": tp,
                        "k_eff": r.v_eff() / r.B, "V_eff": r.v_eff(), "t_iss0_us": c.steady()[0],
                        "kernel_us": r.kernel_us, "drained_TBps": r.drained_rate() / 1e6,
                        "control_drained_TBps": c.drained_rate() / 1e6})
    long_runs = [p for p in pts if p["drained_TBps"] * p["kernel_us"] * 1e6 >= 2 ** 30]
    R = float(np.median([p["drained_TBps"] for p in long_runs])) * 1e6
    out["R_bytes_per_us"] = R
    out["R_TBps"] = R / 1e6
    for p in pts:   # Eq. 1 with the measured aggregate volume
        p["model_t_period_us"] = float(t_period(0.0, p["V_eff"], p["t_iss0_us"], R))
    out["zero_gap"] = pts
    # isolated bursts (gap well past the drain time) against the control
    iso = []
    for b_kib in (4, 8, 16, 32, 64, 128, 256, 512):
        gap = max(200.0, 3.0 * K * b_kib * KIB / R)
        r = pr.run(K, b_kib * KIB, gap, bursts=4)
        c = pr.run(K, b_kib * KIB, gap, bursts=4, control=True)
        iso.append({"B": b_kib * KIB, "gap_us": gap, "k_eff": r.v_eff(1) / r.B, "V_eff": r.v_eff(1),
                    "t_iss_us": float(np.mean(r.t_iss[:, 1:])), "t_iss0_us": float(np.mean(c.t_iss[:, 1:]))})
    Q = fit_capacity([p["V_eff"] for p in iso], [p["t_iss_us"] for p in iso],
                     [p["t_iss0_us"] for p in iso], R)
    for p in iso:
        p["q_peak0_bytes"] = float(q_peak0(p["V_eff"], p["t_iss0_us"], R))
        if Q is not None:
            p["model_t_iss_us"] = float(t_iss_isolated(p["V_eff"], p["t_iss0_us"], R, Q))
    out["isolated"] = {"K": K, "points": iso}
    out["Q_bytes"] = Q
    # gap sweep at the zero-gap point with the most backpressure
    best = max(pts, key=lambda p: p["t_iss_us"] / p["t_iss0_us"])
    Ks, Bs = best["K"], best["B"]
    V0 = best["V_eff"]
    sweep = {}
    for control in (False, True):
        rows = []
        for f in (0.0, 0.25, 0.5, 0.75, 1.0, 1.5, 2.0, 4.0):
            g = f * V0 / R
            r = pr.run(Ks, Bs, g, bursts=12, control=control)
            ti, tp = r.steady()
            rows.append({"gap_us": g, "t_iss_us": ti, "t_period_us": tp, "V_eff": r.v_eff()})
        sweep["control" if control else "scattered"] = rows
    # V of the period law is the volume every resident producer adds per
    # period, V0 from the zero-gap run (with a gap the producers spread their
    # issue over the period, so fewer issue at the same instant); T_iss0 at
    # each gap is the control's issue time at that gap
    for row, ctl in zip(sweep["scattered"], sweep["control"]):
        row["model_t_iss_us"] = float(t_iss(row["gap_us"], V0, ctl["t_iss_us"], R))
        row["model_t_period_us"] = float(t_period(row["gap_us"], V0, ctl["t_iss_us"], R))
    t0 = sweep["control"][-1]["t_iss_us"]
    knee = next((row["gap_us"] for row, ctl in zip(sweep["scattered"], sweep["control"])
                 if row["t_iss_us"] <= 1.1 * ctl["t_iss_us"]), None)
    out["gap_sweep"] = {"K": Ks, "B": Bs, "V0": V0, "t_iss0_us": t0, "g_star_us": float(g_star(V0, t0, R)),
                        "measured_knee_us": knee, **sweep}
    return out


# ------------------------------------------------- spans of the FFN kernel ---

def tile_spans(trace: np.ndarray, khz: int) -> dict:
    """Per-task spans from an FFN task trace [G, cap, MOE_TRACE_WORDS]:
    Linear-2 sender-visible store span T_RS (words 5 - 4), drain lag after
    the issue (words 8 - 5), mainloop times, and the mean number of Linear-2
    store spans in flight alongside each one, itself included (K_act)."""
    tr = trace.astype(np.int64) & 0xFFFFFFFF
    used = tr[tr[:, :, 0] != 0xFFFFFFFF]
    if not len(used):
        return {}
    us = 1e3 / khz
    base = used[:, 2].min()
    rel = lambda c: _wrap(used[:, c] - base) * us
    kind = used[:, 0] & 3
    start, ready, main_end, issued, done = rel(2), rel(3), rel(4), rel(5), rel(8)
    l2 = kind == 2
    t_rs = (issued - main_end)[l2]
    lag = (done - issued)[l2]
    a, b = main_end[l2], issued[l2]
    # Linear-2 store spans in flight alongside each one, itself included
    k_act = burst_concurrency(np.round(a * khz / 1e3), np.round(b * khz / 1e3))
    pct = lambda x, q: float(np.percentile(x, q)) if len(x) else float("nan")
    # natural gap of each workgroup between its Linear-2 bursts: from one
    # tile's stores issued to the next Linear-2 tile's mainloop end (the
    # work that separates two bursts of one producer, section 3.2's G)
    gaps = []
    for g in range(trace.shape[0]):
        t = tr[g][tr[g][:, 0] != 0xFFFFFFFF]
        t = t[(t[:, 0] & 3) == 2]
        if len(t) > 1:
            gaps.append(_wrap(t[1:, 4] - t[:-1, 5]) * us)
    gaps = np.concatenate(gaps) if gaps else np.zeros(0)
    return {
        "l2_tiles": int(l2.sum()),
        "l2_gap_us": {"median": pct(gaps, 50), "p10": pct(gaps, 10)},
        "t_rs_us": {"median": pct(t_rs, 50), "p90": pct(t_rs, 90), "max": pct(t_rs, 100)},
        "drain_lag_us": {"median": pct(lag, 50), "p90": pct(lag, 90)},
        "k_act": {"median": pct(k_act, 50), "p90": pct(k_act, 90)},
        "mainloop_us": {"l1": pct((main_end - ready)[kind == 1], 50), "l2": pct((main_end - ready)[l2], 50)},
        # Linear-1 epilogue: SwiGLU, h stores completed and published
        "l1_epilogue_us": {"median": pct((issued - main_end)[kind == 1], 50),
                           "p90": pct((issued - main_end)[kind == 1], 90)},
        # task start to operands ready (Linear-2: the wait for h)
        "ready_wait_us": {"l1": pct((ready - start)[kind == 1], 50), "l2": pct((ready - start)[l2], 50)},
        "span_us": float((done.max() if len(done) else 0.0)),
    }


def ffn_spans(workload: str = "dsv3") -> dict:
    """Task traces of both schedules on a full-size workload."""
    import os
    import torch

    import moe_inputs as mi
    from . import MoeExpertFFN, _lib
    wl = mi.get_workload(workload)
    inp = mi.make_inputs(wl, workers=min(16, os.cpu_count() or 1))
    dev = torch.device("cuda:0")
    S, T, H, k = wl.num_slices, wl.tokens_per_slice, wl.hidden, wl.top_k
    up = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    x = up(inp.x.reshape(S, T, H))
    xs = None if inp.x_scale is None else up(inp.x_scale.reshape(S, T, -1))
    w1, w2 = up(inp.w1), up(inp.w2)
    w1s = None if inp.w1_scale is None else up(inp.w1_scale)
    w2s = None if inp.w2_scale is None else up(inp.w2_scale)
    comb = torch.empty((S, T, k, H), dtype=torch.int16, device=dev)
    ffn = MoeExpertFFN(S, T, wl.num_experts, k, wl.local_begin, wl.num_local, H, wl.inter,
                       dtype=wl.dtype, device=dev)
    ffn.layout(logits=up(inp.logits), bias=None if inp.bias is None else up(inp.bias))
    G, cap = ffn.plan.grid, 512
    out = {"workload": wl.name, "tile": ffn.plan.tile, "block_m": ffn.plan.block_m,
           "block_n": ffn.plan.block_n2, "n1": ffn.plan.n1_tiles, "n2": ffn.plan.n2_tiles,
           "combine_bytes_per_tile": ffn.plan.block_m * ffn.plan.block_n2 * 2}
    for sched in ("expert_wave", "interleaved"):
        trace = torch.full((G, cap, _lib.TRACE_WORDS), -1, dtype=torch.int32, device=dev)
        for _ in range(2):   # the second run is the one kept
            trace.fill_(-1)
            ffn.forward([x[s] for s in range(S)], w1, w2, [comb[s] for s in range(S)],
                        x_scales=None if xs is None else [xs[s] for s in range(S)],
                        w1_scales=w1s, w2_scales=w2s, schedule=sched, trace=trace, trace_capacity=cap)
            torch.cuda.synchronize()
        out[sched] = tile_spans(trace.cpu().numpy(), ffn.plan.wall_clock_khz)
    return out


def model_checks(cal: dict, spans: dict) -> dict:
    """Eq. 14 and Eq. 15 for each schedule of one workload. The stores of a
    Linear-2 tile are issued by the workgroup that computed it, with nothing
    else to hide them behind (T_cover = 0), so the whole sender-visible span
    T_RS reaches the critical path."""
    # T_iss0 = 0 makes Eq. 14 hardest to meet: the check is conservative
    R, t0 = cal["R_bytes_per_us"], 0.0
    checks = {}
    for sched in ("expert_wave", "interleaved"):
        s = spans.get(sched)
        if not s:
            continue
        V = s["k_act"]["median"] * spans["combine_bytes_per_tile"]
        t_rs = s["t_rs_us"]["median"]
        checks[sched] = {
            "V_aggregate_bytes": V,
            "drain_limited_span_us": V / R,
            "eq14_interleave_sufficient": bool(interleave_sufficient(
                spans["n1"], spans["n2"], V, t0, R, s["mainloop_us"]["l1"], s["mainloop_us"]["l2"])),
            "eq15_stall_us": float(critical_stall(t_rs, 0.0)),
            "stall_share_of_l2_tile": t_rs / (t_rs + s["mainloop_us"]["l2"]),
        }
    return checks


def stall_table(pr: "Prober", cal: dict, spans: dict, bursts: int = 8) -> dict:
    """Table 2 of the X-Stage paper for this GPU: per schedule, the Linear-2
    stall per tile that the store model predicts against the one the trace
    measures. The model's burst is one tile's combine rows (block_m rows of
    block_n bf16 values each) from K_act producers at once (the measured
    number of Linear-2 store spans in flight), separated by the measured
    natural gap G of a producer's Linear-2 bursts. Its backpressure-free
    issue time T_iss0 is the L2-resident control of the probe at exactly that
    K, B, row size and gap; Eq. 3 gives T_RS = max(T_iss0, V/R - G) with
    V = K_act B, and Eq. 15 the stall, max(0, T_RS - T_cover) with
    T_cover = 0 (the workgroup that computes a tile issues its stores before
    its next task). The probe's scattered run at the same K, B and G is the
    store path alone; the trace's T_RS adds the epilogue's own work (router
    weight, bf16 conversion, LDS staging)."""
    R = cal["R_bytes_per_us"]
    B = spans["combine_bytes_per_tile"]
    row = spans["block_n"] * 2
    out = {}
    for sched in ("expert_wave", "interleaved"):
        s = spans.get(sched)
        if not s:
            continue
        K = max(1, int(round(s["k_act"]["median"])))
        G = max(0.0, s["l2_gap_us"]["median"])
        ctl = pr.run(K, B, G, bursts=bursts, control=True, row_bytes=row)
        sca = pr.run(K, B, G, bursts=bursts, control=False, row_bytes=row)
        t0 = ctl.steady()[0]
        V = K * B
        pred = float(t_iss(G, V, t0, R))
        out[sched] = {"K_act": K, "B_bytes": B, "gap_us": G, "V_bytes": V, "V_over_R_us": V / R,
                      "t_iss0_us": t0, "backpressure_us": float(delta_t_iss(G, V, t0, R)),
                      "pred_t_rs_us": pred, "pred_stall_us": float(critical_stall(pred, 0.0)),
                      "probe_t_iss_us": sca.steady()[0],
                      "meas_stall_us": s["t_rs_us"]["median"], "meas_stall_p90_us": s["t_rs_us"]["p90"],
                      "epilogue_work_us": s["t_rs_us"]["median"] - sca.steady()[0]}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="dsv3", help="comma-separated workload names")
    ap.add_argument("--producers", type=int, default=256)
    ap.add_argument("--spans-only", action="store_true", help="skip the probe calibration")
    ap.add_argument("--calibration", help="reuse the calibration of an earlier run's JSON output")
    args = ap.parse_args(argv)
    if args.spans_only:
        out = {"workloads": {}}
        for name in args.workload.split(","):
            out["workloads"][name] = {"spans": ffn_spans(name)}
            print(f"[xstage] {name} done", file=sys.stderr, flush=True)
        print(json.dumps(out, default=float), flush=True)
        return 0
    pr = Prober()
    if args.calibration:
        cal = json.loads(open(args.calibration).read().strip().splitlines()[-1])["calibration"]
    else:
        cal = calibrate(pr, K=args.producers)
    print("[xstage] calibration done", file=sys.stderr, flush=True)
    out = {"calibration": cal, "workloads": {}}
    for name in args.workload.split(","):
        spans = ffn_spans(name)
        out["workloads"][name] = {"spans": spans, "model_checks": model_checks(cal, spans),
                                  "stall_table": stall_table(pr, cal, spans)}
        print(f"[xstage] {name} done", file=sys.stderr, flush=True)
    print(json.dumps(out, default=float), flush=True)


if __name__ == "__main__":
    sys.exit(main())
