"""The MFMA issue-rate probe through the C ABI (moe_mfma_rate_probe): short
runs of each format give positive clock stamps, a shader clock within the
GPU's range and finite accumulator sums, and bad arguments are refused
before anything is enqueued."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_persistent_amd import MoeError, _lib
from moe_expert_ffn_persistent_amd import mfma_ceiling as mc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_probe_runs_and_stamps(fmt):
    print(f"[mfma] probe format {fmt}", flush=True)
    khz = mc.wall_clock_khz()
    ops = mc.operands(fmt)
    r = mc.run(fmt, 8, 200, ops, khz)
    assert r["sink_finite"]
    assert 300 <= r["sclk_mhz"] <= 3000
    # no more than one MFMA's FLOPs per clock per SIMD at its format's rate
    assert 0 < r["flop_per_clk_per_simd"] <= (1024 if fmt == 0 else 2048) * 1.05


def test_probe_rejects_bad_arguments():
    ops = torch.zeros(_lib.MFMA_PROBE_OPERAND_BYTES, dtype=torch.uint8, device="cuda")
    stamps = torch.zeros(16, dtype=torch.int64, device="cuda")
    sink = torch.zeros(8 * _lib.MFMA_PROBE_THREADS, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for fmt, blocks, iters, nbytes in ((3, 8, 10, ops.numel()), (0, 0, 10, ops.numel()), (0, 8, 0, ops.numel()),
                                       (1, 8, 10, ops.numel() - 16)):
        with pytest.raises(MoeError):
            _lib.mfma_rate_probe(fmt, blocks, iters, ops.data_ptr(), nbytes, stamps.data_ptr(), sink.data_ptr(), s)
    assert (stamps.cpu().numpy() == 0).all()
