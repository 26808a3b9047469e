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


def _burst_rows(i, nrows):
    """CPU replica of the probe's destination row of store index i: the
    high half of the 32 x 32-bit product of a multiplicative hash of i
    (mod 2^32) and the row count."""
    h = (np.asarray(i, np.uint64) * np.uint64(0x9E3779B1)) & np.uint64(0xFFFFFFFF)
    return ((h * np.uint64(nrows)) >> np.uint64(32)).astype(np.int64)


@pytest.mark.parametrize("row_bytes,control", [(512, False), (64, False), (4096, False), (512, True)])
def test_probe_writes_exactly_the_rows_it_names(row_bytes, control):
    # every (producer, burst, row) index i lands on row burst_row(i); column c
    # of it holds {producer, lane, 0x7f7f7f7f, 0} with lane = (r mod rows per
    # lane round) * columns per row + c; no other byte of the buffer changes
    K, B, bursts = (2, 8192, 2) if control else (12, 8192, 3)   # the control has 512 rows of 512 B
    dst_bytes = 4 << 20
    dst = torch.full((dst_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    stamps = torch.zeros(K * bursts * 2, dtype=torch.int32, device="cuda")
    print(f"[xstage] probe rows row_bytes={row_bytes} control={control}", flush=True)
    _lib.store_burst_probe(_lib.MoeBurstParams(K, B, bursts, row_bytes, 1 if control else 0, 0),
                           dst.data_ptr(), dst_bytes, stamps.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    nrows = (256 * 1024 if control else dst_bytes) // row_bytes
    rows = B // row_bytes
    cpr = row_bytes // 16
    rstep = 256 // cpr
    want = np.full(dst_bytes, 0xA5, np.uint8).view(np.int32).reshape(-1, row_bytes // 4)
    for p in range(K):
        for b in range(bursts):
            r_local = np.arange(rows)
            row = _burst_rows((p * bursts + b) * rows + r_local, nrows)
            for c in range(cpr):
                lane = (r_local % rstep) * cpr + c
                chunk = want[row, 4 * c:4 * c + 4]
                chunk[:, 0] = p
                chunk[:, 1] = lane
                chunk[:, 2] = 0x7F7F7F7F
                chunk[:, 3] = 0
                want[row, 4 * c:4 * c + 4] = chunk
    gv = got.view(np.int32).reshape(-1, row_bytes // 4)
    named = np.zeros(len(gv), bool)
    for p in range(K):
        for b in range(bursts):
            named[_burst_rows((p * bursts + b) * rows + np.arange(rows), nrows)] = True
    # rows nobody names are untouched, byte for byte
    assert (got.reshape(len(gv), -1)[~named] == 0xA5).all()
    # every named row holds the pattern of a store of the probe; rows named by
    # one store only hold exactly that store's {producer, lane}
    assert (gv[named][:, 2::4] == 0x7F7F7F7F).all() and (gv[named][:, 3::4] == 0).all()
    idx = np.concatenate([_burst_rows((p * bursts + b) * rows + np.arange(rows), nrows)
                          for p in range(K) for b in range(bursts)])
    once = np.bincount(idx, minlength=len(gv)) == 1
    assert once.sum() > 0.8 * named.sum()
    assert (gv[once] == want[once]).all()
