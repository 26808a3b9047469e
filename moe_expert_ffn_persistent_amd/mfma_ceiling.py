"""The MFMA ceiling of this GPU under its power limit.

Runs moe_mfma_rate_probe with one workgroup (two wavefronts per SIMD) on
every compute unit, for each MFMA format, about 200 ms per run and four runs
each, and prints one JSON object: per run the rate in TFLOP/s, its fraction
of the dense figure at 2.4 GHz, the shader clock (s_memtime cycles over
s_memrealtime ticks of each workgroup's loop) and the FLOPs per clock per
SIMD.

    python -m moe_expert_ffn_persistent_amd.mfma_ceiling
"""
from __future__ import annotations

import argparse
import json

import numpy as np

from . import _lib

FLOP_PER_MFMA = {0: 32768.0, 1: 65536.0, 2: 131072.0}
NAMES = {0: "v_mfma_f32_32x32x16_bf16", 1: "v_mfma_scale_f32_16x16x128_f8f6f4 e4m3",
         2: "v_mfma_scale_f32_32x32x64_f8f6f4 e4m3"}
DENSE_TFLOPS = {0: 2516.6, 1: 5033.2, 2: 5033.2}   # MI355X dense figures at 2.4 GHz


def operands(fmt: int, seed: int = 7):
    """Random operand bytes: bf16 values of N(0,1) (format 0) or finite e4m3
    codes of magnitude 2^-8 .. 2^6 with random signs."""
    import torch
    rng = np.random.default_rng(seed + fmt)
    n = _lib.MFMA_PROBE_OPERAND_BYTES
    if fmt == 0:
        v = rng.standard_normal(n // 2).astype(np.float32)
        b = (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return torch.from_numpy(b.view(np.int16)).cuda()
    codes = rng.integers(0x08, 0x70, n, dtype=np.uint8) | (rng.integers(0, 2, n, dtype=np.uint8) << np.uint8(7))
    return torch.from_numpy(codes.astype(np.uint8)).cuda()


def wall_clock_khz() -> int:
    """The device wall-clock rate, from the library's plan of a tiny shape."""
    from . import make_params, make_shape
    plan = _lib.ffn_plan(make_shape(1, 16, 8, 2, 0, 2, 256, 128, "bf16"), make_params())
    return int(plan.wall_clock_khz)


def run(fmt: int, blocks: int, iters: int, ops, khz: int) -> dict:
    import torch
    stamps = torch.zeros(blocks * 2, dtype=torch.int64, device="cuda")
    sink = torch.empty(blocks * _lib.MFMA_PROBE_THREADS, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    _lib.mfma_rate_probe(fmt, blocks, iters, ops.data_ptr(), ops.numel() * ops.element_size(),
                         stamps.data_ptr(), sink.data_ptr(), stream.cuda_stream)
    b.record(stream)
    b.synchronize()
    ms = a.elapsed_time(b)
    st = stamps.view(blocks, 2).cpu().numpy().astype(np.float64)
    mhz = float(np.mean(st[:, 0] / np.maximum(st[:, 1], 1.0))) * khz / 1e3
    flops = blocks * 8 * iters * 16 * FLOP_PER_MFMA[fmt]
    tflops = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 3), "tflops": round(tflops, 1),
            "frac_of_dense": round(tflops / DENSE_TFLOPS[fmt], 4), "sclk_mhz": round(mhz, 0),
            "flop_per_clk_per_simd": round(flops / (ms * 1e-3) / (mhz * 1e6) / (blocks * 4), 0),
            "sink_finite": bool(np.isfinite(sink.cpu().numpy()).all())}


def main(argv=None):
    import torch
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--target-ms", type=float, default=200.0)
    ap.add_argument("--runs", type=int, default=4)
    args = ap.parse_args(argv)
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    khz = wall_clock_khz()
    out = {"blocks": blocks, "wavefronts_per_simd": 2, "formats": {}}
    for fmt in (0, 1, 2):
        ops = operands(fmt)
        probe = run(fmt, blocks, 2000, ops, khz)           # calibrates the loop count
        iters = max(1, int(2000 * args.target_ms / max(probe["ms"], 1e-3)))
        runs = [run(fmt, blocks, iters, ops, khz) for _ in range(args.runs)]
        out["formats"][NAMES[fmt]] = {"iters": iters, "runs": runs,
                                      "median_tflops": float(np.median([r["tflops"] for r in runs]))}
        print(f"[mfma] {NAMES[fmt]}: {runs[-1]}", flush=True)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
