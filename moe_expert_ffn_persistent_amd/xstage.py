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


@dataclass
class BurstRun:
    K: int
    B: int
    gap_us: float
    control: bool
    t_iss: np.ndarray      # [K, bursts] us
    t_period: np.ndarray   # [K, bursts - 1] us

    @property
    def V(self) -> int:
        return self.K * self.B

    def steady(self, skip: int = 2):
        """Median issue time and period over producers, after `skip` bursts."""
        return (float(np.median(self.t_iss[:, skip:])),
                float(np.median(self.t_period[:, skip:])) if self.t_period.shape[1] > skip else float("nan"))


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
        _lib.store_burst_probe(prm, self.dst.data_ptr(), self.dst.numel(), stamps.data_ptr(),
                               stream.cuda_stream)
        torch.cuda.synchronize(self.device)
        st = stamps.cpu().numpy().astype(np.int64).reshape(K, bursts, 2) & 0xFFFFFFFF
        us = 1e3 / self.khz
        return BurstRun(K, B, gap_us, control, _wrap(st[:, :, 1] - st[:, :, 0]) * us,
                        _wrap(st[:, 1:, 0] - st[:, :-1, 0]) * us)


def calibrate(pr: Prober, K: int = 256) -> dict:
    """Drain rate from zero-gap periodic bursts, isolated-burst floor and
    capacity knee, and a gap sweep compared with the model (sections 3.3-3.5).

    Every scattered run is paired with the L2-resident control of the same
    K and B, whose timing has no HBM drain behind it: a scattered period
    above its control's is backpressure, and only those points enter the fit
    of R (the drain-dominated regime of section 3.3)."""
    out = {"K": K}
    pts = []
    for k in (K, 2 * K, 4 * K):
        for b_kib in (16, 32, 64, 128, 256):
            r = pr.run(k, b_kib * KIB, 0.0, bursts=12)
            c = pr.run(k, b_kib * KIB, 0.0, bursts=12, control=True)
            ti, tp = r.steady()
            ci, cp = c.steady()
            pts.append({"K": k, "B": b_kib * KIB, "V": r.V, "t_iss_us": ti, "t_period_us": tp,
                        "control_t_period_us": cp, "rate_TBps": r.V / tp / 1e6})
    out["zero_gap"] = pts
    drain = [p for p in pts if p["V"] >= 8 * 1024 * KIB and p["t_period_us"] > 1.1 * p["control_t_period_us"]]
    out["drain_points"] = len(drain)
    if drain:
        R = fit_drain_rate([p["V"] for p in drain], [p["t_period_us"] for p in drain])
    else:   # issue-bound everywhere: the highest rate reached bounds R from below
        R = max(p["V"] / p["t_period_us"] for p in pts)
    out["R_bytes_per_us"] = R
    out["R_TBps"] = R / 1e6
    # the sweep runs at the point with the most backpressure
    best = max(pts, key=lambda p: p["t_period_us"] / p["control_t_period_us"])
    Ks, Bs = best["K"], best["B"]
    # isolated bursts (gap well past the drain time) against the control
    iso = []
    for b_kib in (4, 8, 16, 32, 64, 128, 256, 512):
        V = Ks * b_kib * KIB
        gap = max(200.0, 3.0 * V / R)
        r = pr.run(Ks, b_kib * KIB, gap, bursts=3)
        c = pr.run(Ks, b_kib * KIB, gap, bursts=3, control=True)
        iso.append({"B": b_kib * KIB, "V": V, "gap_us": gap, "t_iss_us": float(np.median(r.t_iss[:, 1:])),
                    "t_iss0_us": float(np.median(c.t_iss[:, 1:]))})
    out["isolated"] = {"K": Ks, "points": iso}
    out["Q_bytes"] = fit_capacity([p["V"] for p in iso], [p["t_iss_us"] for p in iso],
                                  [p["t_iss0_us"] for p in iso], R)
    # gap sweep at that point, scattered and control, gaps in units of V/R
    V = Ks * Bs
    sweep = {}
    for control in (False, True):
        rows = []
        for f in (0.0, 0.25, 0.5, 0.75, 1.0, 1.5, 2.0, 4.0):
            g = f * V / R
            r = pr.run(Ks, Bs, g, bursts=10, control=control)
            ti, tp = r.steady()
            rows.append({"gap_us": g, "t_iss_us": ti, "t_period_us": tp})
        sweep["control" if control else "scattered"] = rows
    t0 = float(np.median([r["t_iss_us"] for r in sweep["control"]]))
    for row in sweep["scattered"]:
        row["model_t_iss_us"] = float(t_iss(row["gap_us"], V, t0, R))
        row["model_t_period_us"] = float(t_period(row["gap_us"], V, t0, R))
    out["gap_sweep"] = {"K": Ks, "B": Bs, "V": V, "t_iss0_us": t0, "g_star_us": float(g_star(V, t0, R)),
                        **sweep}
    return out


# ------------------------------------------------- spans of the FFN kernel ---

def tile_spans(trace: np.ndarray, khz: int) -> dict:
    """Per-task spans from an FFN task trace [G, cap, MOE_TRACE_WORDS]:
    Linear-2 sender-visible store span T_RS (words 5 - 4), drain lag after
    the issue (words 8 - 5), mainloop times, and the number of other Linear-2
    store spans overlapping each one (K_act)."""
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
    # other Linear-2 store spans overlapping each one
    k_act = np.array([int(((a < b[i]) & (b > a[i])).sum()) - 1 for i in range(len(a))])
    pct = lambda x, q: float(np.percentile(x, q)) if len(x) else float("nan")
    return {
        "l2_tiles": int(l2.sum()),
        "t_rs_us": {"median": pct(t_rs, 50), "p90": pct(t_rs, 90), "max": pct(t_rs, 100)},
        "drain_lag_us": {"median": pct(lag, 50), "p90": pct(lag, 90)},
        "k_act": {"median": pct(k_act, 50), "p90": pct(k_act, 90)},
        "mainloop_us": {"l1": pct((main_end - ready)[kind == 1], 50), "l2": pct((main_end - ready)[l2], 50)},
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
    xs = None if inp.x_scale is None else up(inp.x_scale.reshape(S, T, H // 128))
    w1, w2 = up(inp.w1), up(inp.w2)
    w1s = None if inp.w1_scale is None else up(inp.w1_scale)
    w2s = None if inp.w2_scale is None else up(inp.w2_scale)
    comb = torch.empty((S, T, k, H), dtype=torch.int16, device=dev)
    ffn = MoeExpertFFN(S, T, wl.num_experts, k, wl.local_begin, wl.num_local, H, wl.inter,
                       dtype=wl.dtype, device=dev)
    ffn.layout(logits=up(inp.logits), bias=None if inp.bias is None else up(inp.bias))
    G, cap = ffn.plan.grid, 256
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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--producers", type=int, default=256)
    args = ap.parse_args(argv)
    pr = Prober()
    cal = calibrate(pr, K=args.producers)
    spans = ffn_spans(args.workload)
    # T_iss0 = 0 makes Eq. 14 hardest to meet: the check is conservative
    R, t0 = cal["R_bytes_per_us"], 0.0
    checks = {}
    for sched in ("expert_wave", "interleaved"):
        s = spans[sched]
        if not s:
            continue
        # the store spans in flight together: this one and the others overlapping it
        V = (s["k_act"]["median"] + 1) * spans["combine_bytes_per_tile"]
        checks[sched] = {
            "V_aggregate_bytes": V,
            "drain_limited_span_us": V / R,
            "eq14_interleave_sufficient": bool(interleave_sufficient(
                spans["n1"], spans["n2"], V, t0, R, s["mainloop_us"]["l1"], s["mainloop_us"]["l2"])),
        }
    print(json.dumps({"calibration": cal, "spans": spans, "model_checks": checks}, default=float), flush=True)


if __name__ == "__main__":
    sys.exit(main())
