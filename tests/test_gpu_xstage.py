"""The store burst-gap probe through the C ABI (moe_store_burst_probe) and
the store spans of the FFN task trace, on the GPU."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_persistent_amd import MoeError, _lib
from moe_expert_ffn_persistent_amd import xstage as xs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def prober():
    return xs.Prober(dst_bytes=64 << 20)


@pytest.mark.parametrize("control", [False, True])
def test_probe_stamps_are_consistent(prober, control):
    print(f"[xstage] probe control={control}", flush=True)
    r = prober.run(K=64, B=16 * 1024, gap_us=0.0, bursts=6, control=control)
    assert r.t_iss.shape == (64, 6) and r.t_period.shape == (64, 5)
    assert (r.t_iss > 0).all() and (r.t_iss < 1e4).all()
    # a burst starts only after the previous one was issued
    assert (r.t_period >= r.t_iss[:, :-1] - 0.02).all()
    g = prober.run(K=64, B=16 * 1024, gap_us=30.0, bursts=4, control=control)
    assert (g.t_period >= 30.0).all()
    # the aggregate injection stays below any physical rate (50 TB/s)
    assert r.V / r.steady()[0] < 50e6


def test_probe_rejects_bad_sizes(prober):
    bad = [_lib.MoeBurstParams(0, 4096, 1, 512, 0, 0), _lib.MoeBurstParams(4, 1000, 1, 512, 0, 0),
           _lib.MoeBurstParams(4, 4096, 0, 512, 0, 0), _lib.MoeBurstParams(4, 4096, 1, 24, 0, 0),
           _lib.MoeBurstParams(4, 4096, 1, 48, 0, 0), _lib.MoeBurstParams(4, 8192, 1, 8192, 0, 0),
           _lib.MoeBurstParams(4, 4096, 1, 512, 0, -5)]
    stamps = torch.zeros(64, dtype=torch.int32, device="cuda")
    for prm in bad:
        with pytest.raises(MoeError):
            _lib.store_burst_probe(prm, prober.dst.data_ptr(), prober.dst.numel(), stamps.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(MoeError):   # the control region needs 256 KiB
        _lib.store_burst_probe(_lib.MoeBurstParams(4, 4096, 1, 512, 1, 0), small.data_ptr(), small.numel(),
                               stamps.data_ptr(), torch.cuda.current_stream().cuda_stream)
