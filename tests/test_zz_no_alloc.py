"""The allocation-free FFN entry point (moe_ffn_forward_noalloc) against the
entry point with a caller-given workspace (moe_ffn_forward): same kernels, so
the combine rows must be bitwise identical, and within the bar of the oracle.
Two calls in a row on one stream, the second with a smaller input, so the
second runs on whatever the first left in the library's array; every dtype;
and a shape past the array's size is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as mo
from moe_expert_ffn_persistent_amd import _lib

from gpu_helpers import Uploaded, make_ffn, row_rel_err, run_forward

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp8": 5e-2, "w4a8": 8e-2}


def _wl(dtype, T, seed, **kw):
    base = dict(name="noalloc", num_slices=4, tokens_per_slice=T, num_experts=16, top_k=4, local_begin=2,
                num_local=6, hidden=512, inter=384, dtype=dtype, skew=False, seed=seed)
    base.update(kw)
    return mi.Workload(**base)


def _run_noalloc(ffn, up, **sched):
    ffn.forward_noalloc(up.x_slices, up.w1, up.w2, up.comb_slices, x_scales=up.x_scales,
                        w1_scales=up.w1s, w2_scales=up.w2s, **sched)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "w4a8"])
def test_noalloc_matches_workspace_entry_point_two_calls(dtype):
    big = _wl(dtype, 160, 7100)
    small = _wl(dtype, 37, 7101, hidden=256, inter=256, num_local=5, local_begin=0)
    cases = []
    for wl in (big, small):
        inp = mi.make_inputs(wl)
        up = Uploaded(inp)
        ffn = make_ffn(wl)
        ffn.layout(logits=up.logits, bias=up.bias)
        cases.append((wl, inp, up, ffn))
    # reference: the workspace entry point
    want = []
    for sched in ("interleaved", "expert_wave"):
        for wl, inp, up, ffn in cases:
            up.reset_combine()
            run_forward(ffn, up, schedule=sched)
            torch.cuda.synchronize()
            ffn.check_status()
            want.append(up.comb_all.clone())
    # the allocation-free entry point: the larger call, then the smaller one,
    # back to back on one stream, each schedule
    got = []
    for sched in ("interleaved", "expert_wave"):
        for wl, inp, up, ffn in cases:
            up.reset_combine()
        for wl, inp, up, ffn in cases:
            print(f"[noalloc] {dtype} {sched} T={wl.tokens_per_slice} H={wl.hidden} I={wl.inter} "
                  f"tile={ffn.plan.tile}", flush=True)
            _run_noalloc(ffn, up, schedule=sched)
        torch.cuda.synchronize()
        for wl, inp, up, ffn in cases:
            ffn.check_status()
            got.append(up.comb_all.clone())
    for a, b in zip(want, got):
        assert torch.equal(a, b)
    for wl, inp, up, ffn in cases:
        ref = mo.run(inp, block_m=16)
        C = up.combine_f64()
        assert (up.combine_bits()[~ref.written] == 0xFFFF).all()
        assert row_rel_err(C[ref.written], ref.C[ref.written]).max() <= TOL[dtype]


def test_noalloc_refuses_shapes_past_its_array():
    # the headline-sized share needs ~150 MB of h: refused on the host
    wl = mi.get_workload("dsv3")
    ffn = make_ffn(wl)
    assert ffn.plan.workspace_bytes > _lib.NOALLOC_WORKSPACE_BYTES
    x = [torch.zeros((wl.tokens_per_slice, wl.hidden), dtype=torch.int16, device="cuda")
         for _ in range(wl.num_slices)]
    comb = [torch.zeros((wl.tokens_per_slice, wl.top_k, wl.hidden), dtype=torch.int16, device="cuda")
            for _ in range(wl.num_slices)]
    w1 = torch.zeros((wl.num_local, 2 * wl.inter, wl.hidden), dtype=torch.int16, device="cuda")
    w2 = torch.zeros((wl.num_local, wl.hidden, wl.inter), dtype=torch.int16, device="cuda")
    with pytest.raises(_lib.MoeError) as err:
        ffn.forward_noalloc(x, w1, w2, comb)
    assert err.value.status == _lib.MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    ffn.check_status()
