"""MI355X (gfx950) persistent MoE expert FFN: Python binding.

PyTorch serves only as the device allocator and stream provider: every step
(routing, dispatch layout, Linear-1 + SwiGLU, Linear-2 + weighted combine
stores, combine reduction) runs in the HIP kernels of libmoe_ffn.so through
its C ABI (include/moe_ffn.h). If the library is missing, every call raises;
there is no host fallback.
"""
from __future__ import annotations

import dataclasses

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_FP8_E4M3, MOE_SCHED_EXPERT_WAVE, MOE_SCHED_INTERLEAVED, MOE_W4A8,
                   MoeError, MoeLayout, MoePlan, MoeSchedParams, MoeShape)

__all__ = ["MoeExpertFFN", "LayoutBuffers", "MoeError", "SCHEDULES", "make_shape", "prediction_dict",
           "make_params", "library", "check_layout_inputs", "check_combine_inputs"]

SCHEDULES = {"expert_wave": MOE_SCHED_EXPERT_WAVE, "interleaved": MOE_SCHED_INTERLEAVED}
SCHEDULE_NAMES = {v: k for k, v in SCHEDULES.items()}


def _estimate(e) -> dict:
    return {"schedule": SCHEDULE_NAMES[e.schedule], "lead_d": e.lead_d,
            "experts_per_wave": e.experts_per_wave, "makespan": e.makespan,
            "working_set": e.working_set, "hbm_bytes": e.hbm_bytes, "unique_bytes": e.unique_bytes}


def prediction_dict(pred) -> dict:
    """A moe_schedule_prediction as plain Python values."""
    return {"given": _estimate(pred.given), "recommended": _estimate(pred.recommended),
            "candidates": [_estimate(pred.candidates[i]) for i in range(pred.num_candidates)],
            "sched_rows": pred.sched_rows, "lower_bound": pred.lower_bound}
DTYPES = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "w4a8": MOE_W4A8}


def library():
    """The loaded ctypes library (raises if it has not been built)."""
    return _lib.load()


def make_shape(S, T, E, k, e0, L, H, I, dtype="bf16") -> MoeShape:
    return MoeShape(S, T, E, k, e0, L, H, I, DTYPES[dtype])


def make_params(schedule="interleaved", lead_d=0, experts_per_wave=0, grid=0, tile=0,
                timeout_ms=0, status=None, trace=None, trace_capacity=0,
                debug_skip_l1_row=-1) -> MoeSchedParams:
    return MoeSchedParams(SCHEDULES[schedule], lead_d, experts_per_wave, grid, tile, timeout_ms,
                          None if status is None else status.data_ptr(),
                          None if trace is None else trace.data_ptr(), trace_capacity,
                          debug_skip_l1_row)


def _need(t, what, nbytes, dtype=None, device_type="cuda"):
    """``t`` must be a contiguous tensor on ``device_type`` of at least
    ``nbytes`` bytes (and of ``dtype`` when given). The C ABI takes raw
    pointers, so a wrong tensor would let a kernel read or write past its
    end; this raises ValueError before anything is enqueued."""
    if t is None:
        raise ValueError(f"{what} is required")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what}: need dtype {dtype}, got {t.dtype}")
    if t.device.type != device_type or not t.is_contiguous():
        raise ValueError(f"{what}: need a contiguous {device_type} tensor")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what}: need at least {nbytes} bytes, got {t.numel() * t.element_size()}")


def check_layout_inputs(shape: MoeShape, logits=None, bias=None, topk_idx=None, topk_w=None,
                        device_type="cuda"):
    """Routing inputs of moe_dispatch_layout: fp32 logits [N, E] and an
    optional fp32 bias [E], or (without logits) int32 topk_idx and fp32
    topk_w [N, k]."""
    N = shape.num_slices * shape.tokens_per_slice
    E, k = shape.num_experts, shape.top_k
    if logits is not None:
        _need(logits, "logits", N * E * 4, torch.float32, device_type)
        if bias is not None:
            _need(bias, "expert bias", E * 4, torch.float32, device_type)
    else:
        if bias is not None:
            raise ValueError("an expert bias needs logits (it enters the routing)")
        _need(topk_idx, "topk_idx", N * k * 4, torch.int32, device_type)
        _need(topk_w, "topk_w", N * k * 4, torch.float32, device_type)


def check_combine_inputs(shape: MoeShape, combine_slices, y=None, report=None, device_type="cuda"):
    """Buffers of moe_combine_check: S combine slices of [T, k, H] 2-byte
    (bf16) elements, an optional fp32 or bf16 y_local [N, H] and int32
    report [4]."""
    S, T, k, H = shape.num_slices, shape.tokens_per_slice, shape.top_k, shape.hidden
    if len(combine_slices) != S:
        raise ValueError(f"need {S} combine slices, got {len(combine_slices)}")
    for t in combine_slices:
        if t is not None and t.element_size() != 2:
            raise ValueError("combine slices hold 2-byte (bf16) elements")
        _need(t, "combine slice", T * k * H * 2, None, device_type)
    if y is not None:
        if y.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError(f"y_local must be float32 or bfloat16, got {y.dtype}")
        _need(y, "y_local", S * T * H * y.element_size(), y.dtype, device_type)
    if report is not None:
        _need(report, "report", 16, torch.int32, device_type)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


@dataclasses.dataclass
class LayoutBuffers:
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    row_offset: torch.Tensor
    tile_offset: torch.Tensor
    row_pair: torch.Tensor
    row_weight: torch.Tensor
    pair_row: torch.Tensor
    totals: torch.Tensor
    scratch: torch.Tensor
    block_m: int

    @classmethod
    def allocate(cls, shape: MoeShape, block_m: int, device) -> "LayoutBuffers":
        N = shape.num_slices * shape.tokens_per_slice
        k, L = shape.top_k, shape.num_local_experts
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        nscr = max(1, _lib.layout_scratch_bytes(shape) // 4)
        return cls(torch.zeros((N, k), **i32), torch.zeros((N, k), **f32),
                   torch.zeros(L, **i32), torch.zeros(L + 1, **i32), torch.zeros(L + 1, **i32),
                   torch.zeros(max(1, N * k), **i32), torch.zeros(max(1, N * k), **f32),
                   torch.zeros(max(1, N * k), **i32), torch.zeros(4, **i32),
                   torch.zeros(nscr, **i32), block_m)

    def c_struct(self) -> MoeLayout:
        return MoeLayout(*(t.data_ptr() for t in (
            self.topk_idx, self.topk_w, self.counts, self.row_offset, self.tile_offset,
            self.row_pair, self.row_weight, self.pair_row, self.totals, self.scratch)),
            self.block_m)


class MoeExpertFFN:
    """One GPU's share of an MoE FFN layer: S source slices of T tokens,
    E global experts with top-k routing, local experts e0..e0+L-1, hidden H,
    intermediate I. Owns the layout buffers and the workspace; the caller
    owns inputs, weights and combine buffers."""

    def __init__(self, S, T, E, k, e0, L, H, I, dtype="bf16", schedule="interleaved",
                 lead_d=0, experts_per_wave=0, grid=0, tile=0, timeout_ms=0, device="cuda"):
        self.device = torch.device(device)
        self.shape = make_shape(S, T, E, k, e0, L, H, I, dtype)
        self.dtype = dtype
        self.defaults = dict(schedule=schedule, lead_d=lead_d, experts_per_wave=experts_per_wave,
                             grid=grid, tile=tile, timeout_ms=timeout_ms)
        with torch.cuda.device(self.device):
            self.plan = _lib.ffn_plan(self.shape, make_params(**self.defaults))
            self.layout_bufs = LayoutBuffers.allocate(self.shape, self.plan.block_m, self.device)
            self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
            self.workspace = torch.empty(self.plan.workspace_bytes, dtype=torch.uint8,
                                         device=self.device)
            _lib.workspace_init(self.workspace.data_ptr(), self.plan.workspace_bytes,
                                _stream(None))

    @property
    def num_tokens(self) -> int:
        return self.shape.num_slices * self.shape.tokens_per_slice

    def params(self, **over) -> MoeSchedParams:
        kw = dict(self.defaults)
        kw.update(over)
        kw.setdefault("status", self.status)
        if kw["schedule"] == "auto":   # resolved per call by predict_schedule
            kw["schedule"] = "interleaved"
        return make_params(**kw)

    def resolved_plan(self, **over) -> MoePlan:
        return _lib.ffn_plan(self.shape, self.params(**over))

    def layout(self, logits=None, bias=None, topk_idx=None, topk_w=None, stream=None):
        """Routing (from fp32 logits [N, E] and optional bias [E]) or given
        top-k (int32 idx and fp32 weights [N, k]), then the dispatch layout."""
        lb = self.layout_bufs
        check_layout_inputs(self.shape, logits, bias, topk_idx, topk_w, self.device.type)
        if logits is None:
            lb.topk_idx.copy_(topk_idx)
            lb.topk_w.copy_(topk_w)
        _lib.dispatch_layout(self.shape, None if logits is None else logits.data_ptr(),
                             None if bias is None else bias.data_ptr(), lb.c_struct(),
                             _stream(stream))
        return lb

    def predict_schedule(self, counts=None, **sched) -> dict:
        """The library's schedule planner (moe_predict_schedule) for the
        current routing: predicted makespan and weight working set of the
        configuration in ``sched`` and of each candidate order, and the
        recommended one. ``counts`` (rows per local expert) defaults to the
        layout's, copied to the host, which waits for the layout."""
        if counts is None:
            counts = self.layout_bufs.counts.cpu().tolist()
        knee_plan = self.resolved_plan(**dict(sched, lead_d=0))
        return prediction_dict(_lib.predict_schedule(self.shape, knee_plan, counts,
                                                     self.params(**sched)))

    def _check_buffers(self, x_slices, w1, w2, combine_slices, x_scales, w1_scales, w2_scales):
        """The C ABI takes raw pointers; check sizes here so that a mismatch
        (e.g. fp8 tensors given to a bf16 instance) raises instead of letting
        a kernel read past a buffer."""
        sh = self.shape
        S, T, L, H, I, k = (sh.num_slices, sh.tokens_per_slice, sh.num_local_experts, sh.hidden,
                            sh.inter, sh.top_k)
        elt = 2 if self.dtype == "bf16" else 1          # bytes per x element
        wpe = {"bf16": 2.0, "fp8": 1.0, "w4a8": 0.5}[self.dtype]   # bytes per weight element

        def need(t, nbytes, what):
            if t is None:
                raise ValueError(f"{what} is required")
            if (t.device.type != self.device.type or t.numel() * t.element_size() < nbytes
                    or not t.is_contiguous()):
                raise ValueError(f"{what}: need a contiguous device tensor of at least {nbytes} bytes")

        if len(x_slices) != S or len(combine_slices) != S:
            raise ValueError(f"need {S} x slices and {S} combine slices")
        for t in x_slices:
            if t.element_size() != elt:
                raise ValueError(f"x slices must have {elt}-byte elements for dtype {self.dtype}")
            need(t, T * H * elt, "x slice")
        for t in combine_slices:
            need(t, T * k * H * 2, "combine slice")
        for t, n, what in ((w1, L * 2 * I * H, "w1"), (w2, L * H * I, "w2")):
            if t.element_size() != elt:
                raise ValueError(f"{what} must have {elt}-byte elements for dtype {self.dtype}")
            need(t, int(n * wpe), what)
        if self.dtype != "bf16":
            if x_scales is None or len(x_scales) != S:
                raise ValueError(f"{self.dtype} needs one x-scale tensor per slice")
            if self.dtype == "fp8":   # fp32 per 1x128 (x) and 128x128 (weights) block
                xs_b, w1s_b, w2s_b = (T * (H // 128) * 4, L * (2 * I // 128) * (H // 128) * 4,
                                      L * (H // 128) * (I // 128) * 4)
            else:                     # one E8M0 byte per 1x32 block
                xs_b, w1s_b, w2s_b = T * (H // 32), L * 2 * I * (H // 32), L * H * (I // 32)
            for t in x_scales:
                need(t, xs_b, "x scales")
            need(w1_scales, w1s_b, "w1 scales")
            need(w2_scales, w2s_b, "w2 scales")

    def forward(self, x_slices, w1, w2, combine_slices, x_scales=None, w1_scales=None,
                w2_scales=None, stream=None, **sched):
        """Run Linear-1 + SwiGLU and Linear-2 + weighted combine stores for
        every local expert, in the schedule given by ``sched`` (defaults from
        the constructor). ``schedule="auto"`` runs the planner's recommendation
        for the current routing (predict_schedule; it waits for the layout)."""
        if self.num_tokens:
            self._check_buffers(x_slices, w1, w2, combine_slices, x_scales, w1_scales, w2_scales)
        if sched.get("schedule", self.defaults["schedule"]) == "auto":
            rec = self.predict_schedule(**{k: v for k, v in sched.items() if k != "schedule"})["recommended"]
            sched = dict(sched, schedule=rec["schedule"], lead_d=rec["lead_d"],
                         experts_per_wave=rec["experts_per_wave"])
        params = self.params(**sched)
        ptr = lambda t: None if t is None else t.data_ptr()
        _lib.ffn_forward(self.shape, self.layout_bufs.c_struct(),
                         [t.data_ptr() for t in x_slices],
                         None if x_scales is None else [t.data_ptr() for t in x_scales],
                         w1.data_ptr(), ptr(w1_scales), w2.data_ptr(), ptr(w2_scales),
                         [t.data_ptr() for t in combine_slices], self.workspace.data_ptr(),
                         self.plan.workspace_bytes, params, _stream(stream))

    def forward_noalloc(self, x_slices, w1, w2, combine_slices, x_scales=None, w1_scales=None,
                        w2_scales=None, stream=None, **sched):
        """forward() through moe_ffn_forward_noalloc: the workspace is the
        library's own per-GPU array instead of this instance's, so the call
        allocates nothing (shapes up to the array's size; larger ones raise
        MoeError with MOE_ERR_WORKSPACE_TOO_SMALL). Calls that overlap on one
        GPU share that array and race."""
        if self.num_tokens:
            self._check_buffers(x_slices, w1, w2, combine_slices, x_scales, w1_scales, w2_scales)
        params = self.params(**sched)
        ptr = lambda t: None if t is None else t.data_ptr()
        _lib.ffn_forward_noalloc(self.shape, self.layout_bufs.c_struct(),
                                 [t.data_ptr() for t in x_slices],
                                 None if x_scales is None else [t.data_ptr() for t in x_scales],
                                 w1.data_ptr(), ptr(w1_scales), w2.data_ptr(), ptr(w2_scales),
                                 [t.data_ptr() for t in combine_slices], params, _stream(stream))

    def combine_check(self, combine_slices, y=None, report=None, stream=None):
        """Source-side reduction of the local slots into ``y`` ([N, H]; the
        fp32 sum, or that sum rounded to bf16 when ``y`` is bfloat16) and,
        with ``report`` (int32 [4]), the sentinel audit; report[3] receives
        this instance's device status word."""
        check_combine_inputs(self.shape, combine_slices, y, report, self.device.type)
        _lib.combine_check(self.shape, self.layout_bufs.c_struct(),
                           [t.data_ptr() for t in combine_slices],
                           None if y is None else y.data_ptr(),
                           _lib.MOE_Y_BF16 if y is not None and y.dtype == torch.bfloat16 else _lib.MOE_Y_FP32,
                           self.status.data_ptr(),
                           None if report is None else report.data_ptr(), _stream(stream))

    def check_status(self, clear: bool = True) -> None:
        """Raise MoeError if a kernel of an earlier call recorded an error in
        the device status word (a Linear-2 tile that gave up waiting for its
        Linear-1 inputs leaves its combine rows unwritten). The library never
        clears the word, so one error stays latched until it is read here:
        ``clear`` resets it. Waits for the device first, as the word is only
        meaningful once the calls that write it have completed."""
        torch.cuda.synchronize(self.device)
        st = int(self.status.item())
        if st != 0:
            if clear:
                self.status.zero_()
            raise MoeError(st, "device status")
