"""Helpers for the GPU tests: upload seeded inputs, run the HIP path through
the C ABI binding, read results back. No arithmetic of the method here."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi

SENTINEL = -1   # int16 view of the bf16 pattern 0xFFFF


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


class Uploaded:
    def __init__(self, inp: mi.MoeInputs, separate_slices: bool = False):
        wl = inp.wl
        S, T, H = wl.num_slices, wl.tokens_per_slice, wl.hidden
        self.wl = wl
        self.logits = to_dev(inp.logits)
        self.bias = None if inp.bias is None else to_dev(inp.bias)
        x = inp.x.reshape(S, T, H)
        if separate_slices:
            self.x_slices = [to_dev(x[s].copy()) for s in range(S)]
        else:
            self.x_all = to_dev(x)
            self.x_slices = [self.x_all[s] for s in range(S)]
        self.x_scales = None
        if inp.x_scale is not None:
            xs = inp.x_scale.reshape(S, T, -1)
            self.xs_all = to_dev(xs)
            self.x_scales = [self.xs_all[s] for s in range(S)]
        self.w1 = to_dev(inp.w1)
        self.w2 = to_dev(inp.w2)
        self.w1s = None if inp.w1_scale is None else to_dev(inp.w1_scale)
        self.w2s = None if inp.w2_scale is None else to_dev(inp.w2_scale)
        self.comb_all = torch.full((S, T, wl.top_k, H), SENTINEL, dtype=torch.int16, device=dev())
        self.comb_slices = [self.comb_all[s] for s in range(S)]

    def reset_combine(self):
        self.comb_all.fill_(SENTINEL)

    def combine_f64(self) -> np.ndarray:
        """[N, k, H] float64 of the combine buffers (bf16 widened)."""
        u = self.comb_all.cpu().numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):
            return u.view(np.float32).astype(np.float64).reshape(
                self.wl.num_tokens, self.wl.top_k, self.wl.hidden)

    def combine_rows_bits(self, flat_pairs) -> np.ndarray:
        """[len(flat_pairs), H] uint16 of the selected (token, slot) rows,
        gathered on the device (the full buffer can be several GB)."""
        idx = torch.as_tensor(np.asarray(flat_pairs, dtype=np.int64), device=dev())
        rows = self.comb_all.reshape(-1, self.wl.hidden).index_select(0, idx)
        return rows.cpu().numpy().view(np.uint16)

    def combine_rows_f64(self, flat_pairs) -> np.ndarray:
        u = self.combine_rows_bits(flat_pairs).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):
            return u.view(np.float32).astype(np.float64)

    def combine_bits(self) -> np.ndarray:
        return self.comb_all.cpu().numpy().view(np.uint16).reshape(
            self.wl.num_tokens, self.wl.top_k, self.wl.hidden)


def make_ffn(wl: mi.Workload, **kw):
    from moe_expert_ffn_persistent_amd import MoeExpertFFN
    return MoeExpertFFN(wl.num_slices, wl.tokens_per_slice, wl.num_experts, wl.top_k,
                        wl.local_begin, wl.num_local, wl.hidden, wl.inter, dtype=wl.dtype, **kw)


def run_forward(ffn, up: Uploaded, **sched):
    ffn.forward(up.x_slices, up.w1, up.w2, up.comb_slices, x_scales=up.x_scales,
                w1_scales=up.w1s, w2_scales=up.w2s, **sched)


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row (last axis): max|got - ref| / max|ref|."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-30)
