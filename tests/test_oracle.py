"""Pins of the CPU oracle against facts fixed outside it: number-format
specifications, library routines, closed forms, hand-worked fixtures and
brute force. Every check runs on the CPU."""
import math
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows[key] = vals
    return rows


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def test_bf16_decode_ieee_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3F00, 0x7F7F, 0x0080, 0x0001, 0x4049],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 0.5, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -126, 2.0 ** -133,
            3.140625]
    got = mo.bf16_bits_to_f64(bits)
    assert list(got) == want


def test_bf16_decode_matches_torch_for_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = mo.bf16_bits_to_f64(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_decode_spec_values():
    # OCP 8-bit floating point specification, E4M3: max normal 448 (S.1111.110),
    # min normal 2^-6, min subnormal 2^-9, S.1111.111 is NaN.
    table = {0x00: 0.0, 0x80: -0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x77: 240.0, 0x40: 2.0}
    for c, v in table.items():
        assert mo.e4m3_to_f64(np.array([c], np.uint8))[0] == v, hex(c)
    assert np.isnan(mo.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = mo.e4m3_to_f64(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_generator_e4m3_encode_matches_torch_rounding():
    # the input generator's encoder (not oracle arithmetic, but both sides
    # consume its bytes): round-to-nearest-even, compared with torch's cast
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s
                        for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (mi.e4m3_encode(v) == ref).all()


def test_block_dequant_applies_the_right_scale():
    codes = np.full((256, 384), 0x38, np.uint8)       # every code is 1.0
    scales = np.arange(6, dtype=np.float32).reshape(2, 3) + 1
    v = mo.dequant_blocks(codes, scales, 128, 128)
    assert v[0, 0] == 1 and v[127, 127] == 1 and v[0, 128] == 2 and v[128, 0] == 4
    assert v[255, 383] == 6


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------

def test_route_full_topk_is_softmax():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((64, 16)).astype(np.float32)
    idx, w = mo.route(z, None, 16)
    sm = torch.softmax(torch.from_numpy(z.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(sm, idx, 1), rtol=1e-13, atol=0)


def test_route_invariants_and_bruteforce():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((300, 32)).astype(np.float32)
    z[:50, 3] = z[:50, 7]            # exact ties
    idx, w = mo.route(z, None, 4)
    for n in range(z.shape[0]):
        want = sorted(range(32), key=lambda e: (-float(z[n, e]), e))[:4]
        assert list(idx[n]) == want
        assert len(set(idx[n])) == 4
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)
    assert (np.diff(w, axis=1) <= 0).all()


def test_route_tie_goes_to_lower_index():
    z = np.array([[1.0, 3.0, 3.0, 2.0]], np.float32)
    idx, w = mo.route(z, None, 2)
    assert list(idx[0]) == [1, 2] and abs(w[0, 0] - 0.5) < 1e-15


def test_route_bias_enters_selection_and_weights():
    # z = 0 + bias: bias [0, ln 2, -inf-ish] -> picks expert 1 then 0, with
    # softmax weights 2/3 and 1/3
    z = np.zeros((1, 3), np.float32)
    b = np.array([0.0, math.log(2.0), -30.0], np.float32)
    idx, w = mo.route(z, b, 2)
    assert list(idx[0]) == [1, 0]
    np.testing.assert_allclose(w[0], [2 / 3, 1 / 3], rtol=1e-6)


# --------------------------------------------------------------------------
# Layout
# --------------------------------------------------------------------------

def test_layout_hand_worked_fixture():
    g = _read_golden("layout_small.txt")
    prm = dict(kv.split("=") for kv in g["params"])
    N, k, e0, L, bm = (int(prm[x]) for x in ("N", "k", "e0", "L", "block_m"))
    idx = np.array(g["topk_idx"], np.int32).reshape(N, k)
    lay = mo.dispatch_layout(idx, e0, L, bm)
    for name in ("counts", "row_offset", "tile_offset", "row_pair", "pair_row"):
        assert list(getattr(lay, name)) == [int(v) for v in g[name]], name


@pytest.mark.parametrize("name,bm", [("tiny", 16), ("dsv3", 256), ("qwen3_decode", 32)])
def test_layout_against_library_sort(name, bm):
    wl = mi.get_workload(name)
    logits, bias = mi.make_logits(wl)
    idx, _ = mo.route(logits, bias, wl.top_k)
    lay = mo.dispatch_layout(idx, wl.local_begin, wl.num_local, bm)
    flat = idx.reshape(-1).astype(np.int64) - wl.local_begin
    local = (flat >= 0) & (flat < wl.num_local)
    counts = np.bincount(flat[local], minlength=wl.num_local)
    assert (lay.counts == counts).all()
    assert (lay.row_offset == np.concatenate([[0], np.cumsum(counts)])).all()
    tiles = -(-counts // bm)
    assert (lay.tile_offset == np.concatenate([[0], np.cumsum(tiles)])).all()
    f_local = np.nonzero(local)[0]
    order = f_local[np.argsort(flat[local], kind="stable")]
    assert (lay.row_pair == order).all()
    # every local (token, slot) pair lands exactly once
    assert (lay.pair_row[lay.row_pair] == np.arange(lay.row_pair.size)).all()
    assert (lay.pair_row >= 0).sum() == local.sum()
    assert (lay.pair_row[~local] == -1).all()


def test_uniform_routing_mean_rows_per_expert():
    wl = mi.get_workload("dsv3")
    logits, _ = mi.make_logits(wl)
    idx, _ = mo.route(logits, None, wl.top_k)
    lay = mo.dispatch_layout(idx, 0, wl.num_local, 256)
    expect = wl.num_tokens * wl.top_k * wl.num_local / wl.num_experts
    assert abs(lay.total_rows - expect) < 4 * math.sqrt(expect)


# --------------------------------------------------------------------------
# Expert FFN and combine
# --------------------------------------------------------------------------

def test_swiglu_closed_form_elementwise():
    # H = I, gate = a*Id, up = Id, W2 = Id  ->  y = silu(a x) * x exactly
    H = 8
    a = 3.0
    W1 = np.concatenate([a * np.eye(H), np.eye(H)])
    W2 = np.eye(H)
    x = np.linspace(-2, 2, H)[None, :]
    y = mo.expert_ffn(x, W1, W2)[0]
    want = [(a * v) / (1 + math.exp(-a * v)) * v for v in x[0]]
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-15)


def test_expert_ffn_matches_torch_dense_mlp():
    rng = np.random.default_rng(2)
    H, I, M = 64, 48, 20
    x = rng.standard_normal((M, H))
    W1 = rng.standard_normal((2 * I, H)) * 0.1
    W2 = rng.standard_normal((H, I)) * 0.1
    t = lambda a: torch.from_numpy(a)
    g = torch.nn.functional.linear(t(x), t(W1[:I]))
    u = torch.nn.functional.linear(t(x), t(W1[I:]))
    ref = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, t(W2)).numpy()
    np.testing.assert_allclose(mo.expert_ffn(x, W1, W2), ref, rtol=1e-12, atol=1e-14)


def _bruteforce_slots(inp, idx, w):
    """Per token, per kept slot: evaluate the routed expert densely, with no
    dispatch. Returns C [N, k, H] (zero where not local)."""
    wl = inp.wl
    x = mo.decode_x(inp)
    experts = [mo.decode_expert(inp, e) for e in range(wl.num_local)]
    C = np.zeros((wl.num_tokens, wl.top_k, wl.hidden))
    for n in range(wl.num_tokens):
        for j in range(wl.top_k):
            e = int(idx[n, j]) - wl.local_begin
            if 0 <= e < wl.num_local:
                W1, W2 = experts[e]
                I = W2.shape[1]
                h = np.array([x[n] @ W1[i] for i in range(I)])
                u = np.array([x[n] @ W1[I + i] for i in range(I)])
                a = h / (1 + np.exp(-h)) * u
                C[n, j] = w[n, j] * np.array([a @ W2[o] for o in range(wl.hidden)])
    return C


def test_oracle_matches_bruteforce_tiny():
    wl = mi.get_workload("tiny").with_tokens(6)
    inp = mi.make_inputs(wl)
    r = mo.run(inp, block_m=16)
    C = _bruteforce_slots(inp, r.idx, r.w)
    scale = np.abs(C).max()
    assert scale > 0
    np.testing.assert_allclose(r.C, C, rtol=0, atol=1e-12 * scale)
    # dense-gating form of the per-token sum over this GPU's experts
    g = np.zeros((wl.num_tokens, wl.num_local))
    for n in range(wl.num_tokens):
        for j in range(wl.top_k):
            e = int(r.idx[n, j]) - wl.local_begin
            if 0 <= e < wl.num_local:
                g[n, e] += r.w[n, j]
    x = mo.decode_x(inp)
    y = np.zeros((wl.num_tokens, wl.hidden))
    for e in range(wl.num_local):
        W1, W2 = mo.decode_expert(inp, e)
        y += g[:, e:e + 1] * mo.expert_ffn(x, W1, W2)
    np.testing.assert_allclose(r.y_local, y, rtol=0, atol=1e-12 * np.abs(y).max())


def test_all_local_topk_equals_softmax_mixture():
    # L = E and k = E: y is the softmax-gated mixture of every expert
    base = mi.get_workload("tiny")
    wl = mi.Workload("mix", 1, 5, 4, 4, 0, 4, 32, 16, "bf16", False, 77)
    inp = mi.make_inputs(wl)
    r = mo.run(inp, block_m=8)
    p = torch.softmax(torch.from_numpy(inp.logits.astype(np.float64)), dim=1).numpy()
    x = mo.decode_x(inp)
    y = sum(p[:, e:e + 1] * mo.expert_ffn(x, *mo.decode_expert(inp, e)) for e in range(4))
    np.testing.assert_allclose(r.y_local, y, rtol=0, atol=1e-12 * np.abs(y).max())
    assert r.written.all()


def test_single_expert_k1_is_dense_mlp():
    # k = 1 and a bias that sends every token to local expert 0 with weight 1
    wl = mi.Workload("one", 2, 8, 4, 1, 0, 2, 64, 32, "bf16", False, 78)
    inp = mi.make_inputs(wl)
    inp.bias = np.array([50, 0, 0, 0], np.float32)
    r = mo.run(inp, block_m=16)
    assert (r.idx[:, 0] == 0).all() and (r.w == 1).all()
    x = torch.from_numpy(mo.decode_x(inp))
    W1, W2 = (torch.from_numpy(a) for a in mo.decode_expert(inp, 0))
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(x @ W1[:32].T) * (x @ W1[32:].T), W2).numpy()
    np.testing.assert_allclose(r.C[:, 0], ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r.y_local, ref, rtol=1e-12, atol=1e-15)


def test_nonlocal_slots_not_written_and_weights_scale_linearly():
    wl = mi.get_workload("tiny")
    inp = mi.make_inputs(wl)
    r = mo.run(inp, block_m=16)
    local = (r.idx >= wl.local_begin) & (r.idx < wl.local_begin + wl.num_local)
    assert (r.written == local).all()
    assert (r.C[~local] == 0).all()
    r2 = mo.run(inp, block_m=16, idx=r.idx, w=2 * r.w)
    assert (r2.C == 2 * r.C).all()


def test_fp8_oracle_uses_dequantized_inputs():
    wl = mi.Workload("f8", 1, 4, 8, 2, 0, 2, 256, 128, "fp8", False, 79)
    inp = mi.make_inputs(wl)
    r = mo.run(inp, block_m=16)
    x = mo.e4m3_to_f64(inp.x) * np.repeat(inp.x_scale, 128, axis=1)
    C = np.zeros_like(r.C)
    for n in range(4):
        for j in range(2):
            e = int(r.idx[n, j])
            if e < 2:
                W1 = mo.e4m3_to_f64(inp.w1[e]) * np.kron(inp.w1_scale[e], np.ones((128, 128)))
                W2 = mo.e4m3_to_f64(inp.w2[e]) * np.kron(inp.w2_scale[e], np.ones((128, 128)))
                g, u = x[n] @ W1[:128].T, x[n] @ W1[128:].T
                C[n, j] = r.w[n, j] * ((g / (1 + np.exp(-g)) * u) @ W2.T)
    np.testing.assert_allclose(r.C, C, rtol=0, atol=1e-12 * np.abs(C).max())
    # quantised activations stay within half of e4m3's largest step (32 units
    # of the block scale, in the binade [256, 448]) of the fp32 draw
    x32 = mi._normal(mi._children(wl.seed)[1], (4, 256))
    half_step = 16.0 * np.repeat(inp.x_scale.astype(np.float64), 128, axis=1)
    assert (np.abs(x - x32) <= half_step * (1 + 1e-6)).all()


def test_sampled_rows_match_full_oracle():
    wl = mi.get_workload("tiny")
    inp = mi.make_inputs(wl)
    r = mo.run(inp, block_m=16)
    pairs = np.nonzero(r.layout.pair_row >= 0)[0][::7]
    got = mo.row_outputs(inp, r.idx, r.w, pairs)
    want = r.C.reshape(-1, wl.hidden)[pairs]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13 * np.abs(want).max())


# --------------------------------------------------------------------------
# OCP MX formats (the W4A8 workload): e2m1 weights, e4m3 activations, E8M0
# block scales over 32 elements
# --------------------------------------------------------------------------

def test_e2m1_decode_spec_values():
    # OCP Microscaling Formats (MX) v1.0, FP4 E2M1: exponent bias 1, one
    # mantissa bit, no infinities or NaN
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = mo.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == want
    assert list(got[8:]) == [-v for v in want]


def test_e8m0_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = mo.e8m0_to_f64(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert mo.e8m0_to_f64(np.array([127, 128, 120], np.uint8)).tolist() == [1.0, 2.0, 2.0 ** -7]


def test_e2m1_packing_low_nibble_first():
    # bytes 0x21, 0xF7 hold codes 1, 2 (byte 0: low nibble first) and 7, 15
    vals = mo.e2m1_to_f64(mo.unpack_e2m1(np.array([[0x21, 0xF7]], np.uint8)))
    assert vals.tolist() == [[0.5, 1.0, 6.0, -6.0]]


def test_generator_e2m1_rounds_to_nearest_even_and_saturates():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.25, -2.9, 0.26])
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 0.0, -3.0, 0.5]
    assert mo.e2m1_to_f64(mi.e2m1_encode(v)).tolist() == want


def test_mx_quantisation_error_bounds():
    # the scale's exponent is floor(log2 amax) minus the element format's
    # largest exponent, so a block's amax maps into [4, 8) for e2m1 and
    # [256, 512) for e4m3: elements are within half a step of the draw, or
    # clamped to the largest magnitude (6, resp. 448)
    rng = np.random.default_rng(9)
    a = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 3)).astype(np.float32)
    p, s = mi.quantize_mx_e2m1(a)
    scale = np.repeat(mo.e8m0_to_f64(s), 32, axis=1)
    dq = mo.dequant_mx(mo.e2m1_to_f64(mo.unpack_e2m1(p)), s)
    amax = np.repeat(np.abs(a.reshape(64, 8, 32)).max(axis=2), 32, axis=1)
    assert ((amax / scale >= 4) & (amax / scale < 8)).all()
    err = np.abs(dq - a)
    clamped = np.abs(a) / scale > 6
    assert (err[~clamped] <= 1.0 * scale[~clamped] * (1 + 1e-9)).all()     # half of step 2 at [4, 6]
    assert (err[clamped] <= 2.0 * scale[clamped]).all()
    c, s8 = mi.quantize_mx_e4m3(a)
    scale8 = np.repeat(mo.e8m0_to_f64(s8), 32, axis=1)
    dq8 = mo.dequant_mx(mo.e4m3_to_f64(c), s8)
    rel = np.abs(dq8 - a) / np.abs(a)
    clamped8 = np.abs(a) / scale8 > 448
    big = (np.abs(a) / scale8 >= 2.0 ** -6) & ~clamped8         # normal e4m3 range
    assert (rel[big] <= 2.0 ** -4 * (1 + 1e-9)).all()
    assert (np.abs(dq8 - a)[clamped8] <= 64 * scale8[clamped8]).all()


def test_w4a8_oracle_uses_dequantized_inputs():
    wl = mi.Workload("w4", 1, 4, 8, 2, 0, 2, 256, 128, "w4a8", False, 81)
    inp = mi.make_inputs(wl)
    r = mo.run(inp, block_m=16)
    x = mo.e4m3_to_f64(inp.x) * np.kron(2.0 ** (inp.x_scale.astype(np.float64) - 127), np.ones(32))
    C = np.zeros_like(r.C)
    for n in range(4):
        for j in range(2):
            e = int(r.idx[n, j])
            if e < 2:
                def dq(p, s):
                    codes = np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[0], -1)
                    return mo.e2m1_to_f64(codes) * np.kron(2.0 ** (s.astype(np.float64) - 127),
                                                           np.ones(32))
                W1, W2 = dq(inp.w1[e], inp.w1_scale[e]), dq(inp.w2[e], inp.w2_scale[e])
                g, u = x[n] @ W1[:128].T, x[n] @ W1[128:].T
                C[n, j] = r.w[n, j] * ((g / (1 + np.exp(-g)) * u) @ W2.T)
    np.testing.assert_allclose(r.C, C, rtol=0, atol=1e-12 * np.abs(C).max())
    pairs = np.nonzero(r.layout.pair_row >= 0)[0]
    got = mo.row_outputs(inp, r.idx, r.w, pairs)
    np.testing.assert_allclose(got, r.C.reshape(-1, 256)[pairs], rtol=0, atol=1e-13 * np.abs(C).max())


def test_float32_setting_is_the_same_computation_in_single_precision():
    # the CPU baseline times run(float_type=float32); it must be the float64
    # definition up to single-precision rounding (the layout is shared)
    wl = mi.get_workload("tiny")
    inp = mi.make_inputs(wl)
    a = mo.run(inp, block_m=16)
    b = mo.run(inp, block_m=16, float_type=np.float32)
    assert b.C.dtype == np.float32 and b.y_local.dtype == np.float32
    assert (a.layout.row_pair == b.layout.row_pair).all()
    err = np.abs(b.C - a.C).max(axis=2) / np.maximum(np.abs(a.C).max(axis=2), 1e-30)
    assert err[a.written].max() < 1e-5
    assert (b.C[~a.written] == 0).all()
