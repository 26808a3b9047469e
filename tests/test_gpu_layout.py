"""GPU parity of routing and dispatch layout against the oracle: bit-exact
indices, counts and offsets; router weights within 1e-6."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as mo

pytestmark = pytest.mark.gpu

from gpu_helpers import dev, make_ffn, to_dev  # noqa: E402


def _check_layout(wl, lb, idx_ref, w_ref, block_m, routed=True):
    lay = mo.dispatch_layout(idx_ref, wl.local_begin, wl.num_local, block_m)
    idx = lb.topk_idx.cpu().numpy()
    assert (idx == idx_ref).all()
    if routed:
        assert np.abs(lb.topk_w.cpu().numpy() - w_ref).max() <= 1e-6
    R = lay.total_rows
    assert (lb.counts.cpu().numpy() == lay.counts).all()
    assert (lb.row_offset.cpu().numpy() == lay.row_offset).all()
    assert (lb.tile_offset.cpu().numpy() == lay.tile_offset).all()
    assert (lb.row_pair.cpu().numpy()[:R] == lay.row_pair).all()
    assert (lb.pair_row.cpu().numpy()[:wl.num_tokens * wl.top_k] == lay.pair_row).all()
    tot = lb.totals.cpu().numpy()
    assert tot[0] == R and tot[1] == lay.sched_rows
    assert tot[2] == lay.counts.max() and tot[3] == (lay.counts > 0).sum()
    # row weights are the slot weights of the routed pairs, bit for bit
    rw = lb.row_weight.cpu().numpy()[:R]
    assert (rw == lb.topk_w.cpu().numpy().reshape(-1)[lay.row_pair]).all()


@pytest.mark.parametrize("name", ["tiny", "dsv3", "dsv3_skew", "qwen3_decode", "qwen3_prefill",
                                  "dsv3_fp8", "dsv3_w4a8"])
def test_routing_and_layout_match_oracle(name):
    wl = mi.get_workload(name)
    if wl.dtype == "fp8":
        wl = mi.Workload(wl.name, wl.num_slices, wl.tokens_per_slice, wl.num_experts, wl.top_k,
                         wl.local_begin, wl.num_local, wl.hidden, wl.inter, "bf16", wl.skew,
                         wl.seed)
    print(f"[layout] workload={name}", flush=True)
    logits, bias = mi.make_logits(wl)
    idx_ref, w_ref = mo.route(logits, bias, wl.top_k)
    ffn = make_ffn(wl)
    lb = ffn.layout(logits=to_dev(logits), bias=None if bias is None else to_dev(bias))
    torch.cuda.synchronize()
    _check_layout(wl, lb, idx_ref, w_ref, ffn.plan.block_m)


@pytest.mark.parametrize("e0,L,k,E", [(5, 3, 4, 16), (0, 16, 16, 16), (15, 1, 1, 16), (7, 9, 3, 40)])
def test_layout_ragged_and_offset_local_ranges(e0, L, k, E):
    wl = mi.Workload("ragged", 3, 37, E, k, e0, L, 256, 128, "bf16", False, 4242)
    logits, _ = mi.make_logits(wl)
    logits[:20, e0] = 9.0        # pile some tokens onto one expert
    idx_ref, w_ref = mo.route(logits, None, k)
    ffn = make_ffn(wl)
    lb = ffn.layout(logits=to_dev(logits))
    torch.cuda.synchronize()
    _check_layout(wl, lb, idx_ref, w_ref, ffn.plan.block_m)


def test_layout_from_given_topk_and_ties():
    wl = mi.Workload("ties", 2, 50, 8, 3, 2, 4, 256, 128, "bf16", False, 99)
    logits = np.zeros((100, 8), np.float32)          # all equal: lowest indices win
    logits[50:, 6] = 1.0
    idx_ref, w_ref = mo.route(logits, None, 3)
    assert (idx_ref[:50] == [0, 1, 2]).all() and (idx_ref[50:] == [6, 0, 1]).all()
    ffn = make_ffn(wl)
    lb = ffn.layout(logits=to_dev(logits))
    torch.cuda.synchronize()
    _check_layout(wl, lb, idx_ref, w_ref, ffn.plan.block_m)
    # routing skipped: caller-provided top-k
    rng = np.random.default_rng(3)
    idx2 = np.stack([rng.permutation(8)[:3] for _ in range(100)]).astype(np.int32)
    w2 = rng.random((100, 3)).astype(np.float32)
    lb = ffn.layout(topk_idx=to_dev(idx2), topk_w=to_dev(w2))
    torch.cuda.synchronize()
    _check_layout(wl, lb, idx2, w2, ffn.plan.block_m, routed=False)


def test_routing_ties_across_lanes_and_slots():
    # 256 experts: lane l of the routing wavefront holds experts l, l+64, l+128
    # and l+192, so equal logits can tie within a lane (different slots) and
    # across lanes; -0 and +0 must tie; NaN sorts after every number and
    # -inf after every finite value (a stable sort of -z)
    wl = mi.Workload("ties256", 2, 32, 256, 8, 0, 32, 256, 128, "bf16", False, 7)
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((64, 256)).astype(np.float32)
    logits[:16] = 0.0
    logits[:16][rng.random((16, 256)) < 0.5] = -0.0          # mixed-sign zeros: experts 0..7 win
    logits[16:32] = -np.abs(logits[16:32]) - 1.0
    logits[16:32][:, [200, 136, 72, 8, 64, 128, 192, 0]] = 1.0
    for r in range(32, 48):
        cols = rng.choice(256, 12, replace=False)
        logits[r, cols[:6]] = np.nan
        logits[r, cols[6:]] = -np.inf
    logits[48:56, :250] = -np.inf                             # the finite six, then -inf by index
    idx_ref, w_ref = mo.route(logits, None, 8)
    assert (idx_ref[:16] == np.arange(8)).all()
    assert (idx_ref[16:32] == [0, 8, 64, 72, 128, 136, 192, 200]).all()
    assert (np.sort(idx_ref[48:56, :6], axis=1) == np.arange(250, 256)).all()
    assert (idx_ref[48:56, 6:] == [0, 1]).all()
    ffn = make_ffn(wl)
    lb = ffn.layout(logits=to_dev(logits))
    torch.cuda.synchronize()
    _check_layout(wl, lb, idx_ref, w_ref, ffn.plan.block_m)


def test_layout_empty_batch():
    wl = mi.Workload("empty", 2, 0, 8, 2, 0, 4, 256, 128, "bf16", False, 1)
    ffn = make_ffn(wl)
    lb = ffn.layout(logits=torch.zeros((0, 8), dtype=torch.float32, device=dev()))
    torch.cuda.synchronize()
    assert (lb.counts.cpu() == 0).all() and (lb.tile_offset.cpu() == 0).all()
    assert (lb.totals.cpu() == 0).all()
