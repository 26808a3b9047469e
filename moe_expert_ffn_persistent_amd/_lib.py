"""ctypes binding of libmoe_ffn.so (include/moe_ffn.h), argument marshalling
only. Every step of the path runs in the library's HIP kernels; nothing here
computes on the host."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_ffn.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE_TOO_SMALL = -3
MOE_ERR_HIP = -4
MOE_ERR_TIMEOUT = -5

MOE_BF16 = 0
MOE_FP8_E4M3 = 1
MOE_W4A8 = 2
MOE_SCHED_EXPERT_WAVE = 0
MOE_SCHED_INTERLEAVED = 1
MOE_MAX_SLICES = 64
MOE_Y_FP32 = 0
MOE_Y_BF16 = 1

# every symbol include/moe_ffn.h declares
EXPORTS = ("moe_abi_version", "moe_status_string", "moe_layout_scratch_bytes", "moe_ffn_plan",
           "moe_workspace_init", "moe_dispatch_layout", "moe_ffn_forward", "moe_combine_check",
           "moe_store_burst_probe", "moe_predict_schedule", "moe_ffn_forward_noalloc",
           "moe_mfma_rate_probe")
MFMA_PROBE_THREADS = 512
MFMA_PROBE_OPERAND_BYTES = 64 * 64 * 16 * 16
NOALLOC_WORKSPACE_BYTES = 64 << 20
NOALLOC_MAX_SCHED_ROWS = 16384

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p


class MoeShape(ctypes.Structure):
    _fields_ = [("num_slices", c_i32), ("tokens_per_slice", c_i32), ("num_experts", c_i32),
                ("top_k", c_i32), ("local_expert_begin", c_i32), ("num_local_experts", c_i32),
                ("hidden", c_i32), ("inter", c_i32), ("dtype", c_i32)]


class MoeLayout(ctypes.Structure):
    _fields_ = [("topk_idx", c_vp), ("topk_w", c_vp), ("counts", c_vp), ("row_offset", c_vp),
                ("tile_offset", c_vp), ("row_pair", c_vp), ("row_weight", c_vp),
                ("pair_row", c_vp), ("totals", c_vp), ("scratch", c_vp), ("block_m", c_i32)]


class MoeSchedParams(ctypes.Structure):
    _fields_ = [("schedule", c_i32), ("lead_d", c_i32), ("experts_per_wave", c_i32),
                ("grid", c_i32), ("tile", c_i32), ("timeout_ms", c_i32), ("status", c_vp),
                ("trace", c_vp), ("trace_capacity", c_i32), ("debug_skip_l1_row", c_i32)]


class MoePlan(ctypes.Structure):
    _fields_ = [("tile", c_i32), ("block_m", c_i32), ("block_n1", c_i32), ("block_n2", c_i32),
                ("n1_tiles", c_i32), ("n2_tiles", c_i32), ("grid", c_i32), ("lead_d", c_i32),
                ("max_sched_rows", c_i32), ("workspace_bytes", ctypes.c_size_t),
                ("wall_clock_khz", c_i32)]

TRACE_WORDS = 10
MAX_SCHEDULE_CANDIDATES = 8


class MoeScheduleEstimate(ctypes.Structure):
    _fields_ = [("schedule", c_i32), ("lead_d", c_i32), ("experts_per_wave", c_i32),
                ("makespan", ctypes.c_double), ("working_set", ctypes.c_double),
                ("hbm_bytes", ctypes.c_double), ("unique_bytes", ctypes.c_double)]


PLANNER_CACHE_BYTES = 256.0 * 1024 * 1024


class MoeSchedulePrediction(ctypes.Structure):
    _fields_ = [("given", MoeScheduleEstimate), ("recommended", MoeScheduleEstimate),
                ("candidates", MoeScheduleEstimate * MAX_SCHEDULE_CANDIDATES),
                ("num_candidates", c_i32), ("sched_rows", c_i32), ("lower_bound", ctypes.c_double)]


class MoeBurstParams(ctypes.Structure):
    _fields_ = [("producers", c_i32), ("bytes_per_burst", c_i32), ("bursts", c_i32),
                ("row_bytes", c_i32), ("control", c_i32), ("gap_ns", ctypes.c_int64)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load(path: str | None = None):
    """Load the HIP library (``LIB_PATH`` unless a path is given); raises if
    it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m moe_expert_ffn_persistent_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.moe_abi_version.restype = c_i32
    lib.moe_abi_version.argtypes = []
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [c_i32]
    lib.moe_layout_scratch_bytes.restype = ctypes.c_size_t
    lib.moe_layout_scratch_bytes.argtypes = [P(MoeShape)]
    lib.moe_ffn_plan.restype = c_i32
    lib.moe_ffn_plan.argtypes = [P(MoeShape), P(MoeSchedParams), P(MoePlan)]
    lib.moe_workspace_init.restype = c_i32
    lib.moe_workspace_init.argtypes = [c_vp, ctypes.c_size_t, c_vp]
    lib.moe_dispatch_layout.restype = c_i32
    lib.moe_dispatch_layout.argtypes = [P(MoeShape), c_vp, c_vp, P(MoeLayout), c_vp]
    lib.moe_ffn_forward.restype = c_i32
    lib.moe_ffn_forward.argtypes = [P(MoeShape), P(MoeLayout), P(c_vp), P(c_vp), c_vp, c_vp,
                                    c_vp, c_vp, P(c_vp), c_vp, ctypes.c_size_t,
                                    P(MoeSchedParams), c_vp]
    lib.moe_ffn_forward_noalloc.restype = c_i32
    lib.moe_ffn_forward_noalloc.argtypes = [P(MoeShape), P(MoeLayout), P(c_vp), P(c_vp), c_vp, c_vp,
                                            c_vp, c_vp, P(c_vp), P(MoeSchedParams), c_vp]
    lib.moe_combine_check.restype = c_i32
    lib.moe_combine_check.argtypes = [P(MoeShape), P(MoeLayout), P(c_vp), c_vp, c_i32, c_vp, c_vp, c_vp]
    lib.moe_store_burst_probe.restype = c_i32
    lib.moe_store_burst_probe.argtypes = [P(MoeBurstParams), c_vp, ctypes.c_size_t, c_vp, c_vp]
    lib.moe_mfma_rate_probe.restype = c_i32
    lib.moe_mfma_rate_probe.argtypes = [c_i32, c_i32, ctypes.c_int64, c_vp, ctypes.c_size_t, c_vp, c_vp, c_vp]
    lib.moe_predict_schedule.restype = c_i32
    lib.moe_predict_schedule.argtypes = [P(MoeShape), P(MoePlan), P(c_i32), P(MoeSchedParams),
                                         P(MoeSchedulePrediction)]
    _lib = lib
    return lib


def status_string(st: int) -> str:
    return load().moe_status_string(st).decode()


def check(st: int, what: str):
    if st != MOE_OK:
        raise MoeError(st, what)


def ptr_array(ptrs):
    arr = (c_vp * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def abi_version() -> int:
    return load().moe_abi_version()


def layout_scratch_bytes(shape: MoeShape) -> int:
    return load().moe_layout_scratch_bytes(ctypes.byref(shape))


def ffn_plan(shape: MoeShape, params: MoeSchedParams) -> MoePlan:
    plan = MoePlan()
    check(load().moe_ffn_plan(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(plan)),
          "moe_ffn_plan")
    return plan


def workspace_init(ws_ptr: int, nbytes: int, stream: int):
    check(load().moe_workspace_init(ws_ptr, nbytes, stream), "moe_workspace_init")


def dispatch_layout(shape, logits_ptr, bias_ptr, layout: MoeLayout, stream: int):
    check(load().moe_dispatch_layout(ctypes.byref(shape), logits_ptr, bias_ptr,
                                     ctypes.byref(layout), stream), "moe_dispatch_layout")


def ffn_forward(shape, layout, x_ptrs, xs_ptrs, w1, w1s, w2, w2s, comb_ptrs, ws, ws_bytes,
                params, stream):
    xs = ptr_array(xs_ptrs) if xs_ptrs is not None else None
    check(load().moe_ffn_forward(ctypes.byref(shape), ctypes.byref(layout), ptr_array(x_ptrs),
                                 xs, w1, w1s, w2, w2s, ptr_array(comb_ptrs), ws, ws_bytes,
                                 ctypes.byref(params), stream), "moe_ffn_forward")


def ffn_forward_noalloc(shape, layout, x_ptrs, xs_ptrs, w1, w1s, w2, w2s, comb_ptrs, params, stream):
    xs = ptr_array(xs_ptrs) if xs_ptrs is not None else None
    check(load().moe_ffn_forward_noalloc(ctypes.byref(shape), ctypes.byref(layout), ptr_array(x_ptrs),
                                         xs, w1, w1s, w2, w2s, ptr_array(comb_ptrs),
                                         ctypes.byref(params), stream), "moe_ffn_forward_noalloc")


def combine_check(shape, layout, comb_ptrs, y_ptr, y_dtype, status_ptr, report_ptr, stream):
    check(load().moe_combine_check(ctypes.byref(shape), ctypes.byref(layout),
                                   ptr_array(comb_ptrs), y_ptr, y_dtype, status_ptr, report_ptr, stream),
          "moe_combine_check")


def mfma_rate_probe(fmt: int, blocks: int, iters: int, operands_ptr: int, operand_bytes: int, stamps_ptr: int,
                    sink_ptr: int, stream: int):
    check(load().moe_mfma_rate_probe(fmt, blocks, iters, operands_ptr, operand_bytes, stamps_ptr, sink_ptr, stream),
          "moe_mfma_rate_probe")


def store_burst_probe(params: MoeBurstParams, dst_ptr: int, dst_bytes: int, stamps_ptr: int,
                      stream: int):
    check(load().moe_store_burst_probe(ctypes.byref(params), dst_ptr, dst_bytes, stamps_ptr, stream),
          "moe_store_burst_probe")


def predict_schedule(shape: MoeShape, plan: MoePlan, counts, params: MoeSchedParams | None):
    """counts: host sequence of L ints (rows of each local expert)."""
    arr = (c_i32 * max(1, len(counts)))(*[int(c) for c in counts])
    out = MoeSchedulePrediction()
    check(load().moe_predict_schedule(ctypes.byref(shape), ctypes.byref(plan), arr,
                                      None if params is None else ctypes.byref(params),
                                      ctypes.byref(out)), "moe_predict_schedule")
    return out
