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


@pytest.mark.parametrize("E", [256, 128])
def test_routing_ties_across_lanes_and_slots(E):
    # E = 256 (64 tokens: one wavefront per token, lane l holds experts l,
    # l+64, ...) and E = 128 (four tokens per wavefront, lane l of a token's
    # 16-lane row holds experts l, l+16, ...): equal logits tie within a lane
    # (different slots) and across lanes; -0 and +0 must tie; NaN sorts after
    # every number and -inf after every finite value (a stable sort of -z)
    wl = mi.Workload(f"ties{E}", 2, 32, E, 8, 0, 32, 256, 128, "bf16", False, 7)
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((64, E)).astype(np.float32)
    logits[:16] = 0.0
    logits[:16][rng.random((16, E)) < 0.5] = -0.0            # mixed-sign zeros: experts 0..7 win
    q = E // 4
    tie_cols = [0, 8, q, q + 8, 2 * q, 2 * q + 8, 3 * q, 3 * q + 8]
    logits[16:32] = -np.abs(logits[16:32]) - 1.0
    logits[16:32][:, tie_cols[::-1]] = 1.0
    for r in range(32, 48):
        cols = rng.choice(E, 12, replace=False)
        logits[r, cols[:6]] = np.nan
        logits[r, cols[6:]] = -np.inf
    logits[48:56, :E - 6] = -np.inf                           # the finite six, then -inf by index
    logits[56:64] = -np.abs(logits[56:64]) - 1.0
    logits[56:64][:, [49, 33, 17, 1, 48, 32, 16, 0]] = 2.0     # two lanes, four slots each
    idx_ref, w_ref = mo.route(logits, None, 8)
    assert (idx_ref[:16] == np.arange(8)).all()
    assert (idx_ref[16:32] == tie_cols).all()
    assert (np.sort(idx_ref[48:56, :6], axis=1) == np.arange(E - 6, E)).all()
    assert (idx_ref[48:56, 6:] == [0, 1]).all()
    assert (idx_ref[56:64] == [0, 1, 16, 17, 32, 33, 48, 49]).all()
    ffn = make_ffn(wl)
    lb = ffn.layout(logits=to_dev(logits))
    torch.cuda.synchronize()
    _check_layout(wl, lb, idx_ref, w_ref, ffn.plan.block_m)


def test_routing_sixteen_lane_rows_at_256_experts():
    # E = 256 with N >= 16384 takes the four-tokens-per-wavefront kernel:
    # ties, signed zeros, NaN and -inf in a batch large enough for it
    E = 256
    wl = mi.Workload("rows256", 8, 2048, E, 8, 0, 32, 256, 128, "bf16", False, 8)
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((wl.num_tokens, E)).astype(np.float32)
    logits[:1000] = 0.0
    logits[:1000][rng.random((1000, E)) < 0.5] = -0.0
    logits[1000:2000] = -np.abs(logits[1000:2000]) - 1.0
    logits[1000:2000][:, [49, 33, 17, 1, 48, 32, 16, 0]] = 2.0
    for r in range(2000, 3000):
        cols = rng.choice(E, 12, replace=False)
        logits[r, cols[:6]] = np.nan
        logits[r, cols[6:]] = -np.inf
    idx_ref, w_ref = mo.route(logits, None, 8)
    assert (idx_ref[:1000] == np.arange(8)).all()
    assert (idx_ref[1000:2000] == [0, 1, 16, 17, 32, 33, 48, 49]).all()
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
