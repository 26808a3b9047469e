"""Seeded synthetic inputs for one GPU's expert-parallel share of an MoE FFN.

This module is shared by the CPU oracle and the HIP path. It holds no step of
the method's arithmetic: no routing, no layout, no FFN and no combine. It only
draws seeded random numbers and packs them into the byte formats that both
sides receive (bf16 bit patterns; e4m3 bytes plus fp32 block scales; OCP MX
blocks of 32 elements: e2m1 weights packed two per byte, e4m3 activations,
each block with one E8M0 power-of-two scale).

Workload shapes follow the X-Stage paper's MegaMoE evaluation (section 5.1,
expert parallelism over eight ranks: eight source slices stand in for the
eight ranks) with model shapes chosen to match DeepSeek-V3 and Qwen3-MoE
expert FFNs, since the paper's own model table (Table 2) names shapes without
giving their dimensions.

Draw order per workload (numpy ``default_rng`` over one ``SeedSequence`` per
workload, one child stream per tensor and per expert, so any single expert's
weights can be regenerated on their own):
  1. router logits [N, E] ~ N(0, 1)            (child 0)
  2. activations x [N, H] ~ N(0, 1)            (child 1)
  3. W1[e] [2I, H] ~ N(0, 0.02^2), e = 0..L-1  (child 2, grandchild e)
  4. W2[e] [H, I]  ~ N(0, 0.02^2), e = 0..L-1  (child 3, grandchild e)
The skewed workload adds a per-expert bias 1.5 * ln p(e) to the logits, where
p is a Zipf(s=1.2) popularity over ranks 1..E and global expert e has rank
e + 1 (index order is popularity order, so the experts 0..L-1 owned by this
GPU are the hottest ones).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "MoeInputs", "make_inputs",
    "f32_to_bf16_bits", "quantize_e4m3_blocks", "e4m3_encode", "e2m1_encode",
    "quantize_mx_e4m3", "quantize_mx_e2m1",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_slices: int          # S: source slices (stand-ins for the EP ranks)
    tokens_per_slice: int    # T
    num_experts: int         # E: global experts
    top_k: int               # k
    local_begin: int         # e0: first local expert
    num_local: int           # L: local experts on this GPU
    hidden: int              # H
    inter: int               # I
    dtype: str               # "bf16", "fp8" (e4m3 with fp32 block scales) or
                             # "w4a8" (MX: e2m1 weights, e4m3 activations)
    skew: bool               # Zipf-biased router logits
    seed: int

    @property
    def num_tokens(self) -> int:
        return self.num_slices * self.tokens_per_slice

    def with_tokens(self, tokens_per_slice: int, name: str | None = None) -> "Workload":
        return dataclasses.replace(self, tokens_per_slice=tokens_per_slice,
                                   name=name or f"{self.name}@T{tokens_per_slice}")


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 8, 32, 32, 2, 0, 4, 256, 128, "bf16", False, 1001),
        Workload("dsv3", 8, 512, 256, 8, 0, 32, 7168, 2048, "bf16", False, 1002),
        Workload("dsv3_skew", 8, 2048, 256, 8, 0, 32, 7168, 2048, "bf16", True, 1003),
        Workload("dsv3_fp8", 8, 4096, 256, 8, 0, 32, 7168, 2048, "fp8", False, 1004),
        Workload("qwen3_decode", 8, 16, 128, 8, 0, 16, 4096, 1536, "bf16", False, 1005),
        Workload("qwen3_prefill", 8, 8192, 128, 8, 0, 16, 4096, 1536, "bf16", False, 1006),
        Workload("dsv3_w4a8", 8, 4096, 256, 8, 0, 32, 7168, 2048, "w4a8", False, 1007),
    ]
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even) and return
    the 16-bit patterns as uint16. Inputs are finite by construction."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Encode fp32 values as OCP FP8 E4M3 (the 'fn' variant: bias 7, no
    infinities, 0x7F/0xFF are NaN, largest finite 448), rounding to nearest
    with ties to even and saturating to +-448. Returns uint8 codes."""
    v = np.asarray(v, dtype=np.float32)
    sign = (np.signbit(v)).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(v).astype(np.float64), 448.0)
    # exponent of the binade the value falls in, clamped to the normal range;
    # below 2^-6 the spacing is the subnormal step 2^-9.
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    e = np.clip(e, -6, 8)
    step = 2.0 ** (e - 3)
    q = np.rint(a / step) * step          # np.rint rounds ties to even
    # rounding can carry into the next binade; recompute fields from q
    q = np.minimum(q, 448.0)
    code = np.zeros(v.shape, dtype=np.uint8)
    nz = q > 0
    qe = np.floor(np.log2(np.where(nz, q, 1.0)))
    normal = nz & (qe >= -6)
    sub = nz & ~normal
    mant_n = np.rint(q / 2.0 ** qe * 8.0 - 8.0).astype(np.int64)
    exp_n = (qe + 7).astype(np.int64)
    code = np.where(normal, (exp_n << 3) | mant_n, 0)
    code = np.where(sub, np.rint(q / 2.0 ** -9).astype(np.int64), code)
    return (code.astype(np.uint8) | sign)


def quantize_e4m3_blocks(a: np.ndarray, block_rows: int, block_cols: int):
    """Blockwise e4m3 quantization of a 2-D fp32 array: one fp32 scale per
    (block_rows x block_cols) block, scale = amax / 448, codes = e4m3(a/scale).
    Returns (codes uint8 [R, C], scales fp32 [ceil(R/br), ceil(C/bc)])."""
    a = np.asarray(a, dtype=np.float32)
    R, C = a.shape
    assert R % block_rows == 0 and C % block_cols == 0
    blk = a.reshape(R // block_rows, block_rows, C // block_cols, block_cols)
    amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = blk / scale[:, None, :, None]
    codes = e4m3_encode(q.reshape(R, C))
    return codes, scale


# OCP Microscaling (MX) formats: blocks of 32 consecutive elements along a
# row share one E8M0 scale 2^(byte - 127). The block exponent is
# floor(log2(amax)) minus the element format's largest exponent (2 for e2m1,
# whose largest value is 6 = 1.5 * 2^2; 8 for e4m3, 448 = 1.75 * 2^8), and
# elements are value / 2^exponent rounded to nearest-even in the element
# format, clamped to its largest magnitude. An all-zero block gets scale 1.
MX_BLOCK = 32
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Encode values as OCP FP4 E2M1 codes (sign bit 3, two exponent bits of
    bias 1, one mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), rounding
    to nearest with ties to the even code and saturating to +-6. Returns one
    code (0..15) per element as uint8."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[..., None] - _E2M1_GRID)              # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d <= best                                   # nearest, both codes on a tie
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    sign = np.signbit(v) & (idx > 0)
    return (idx | (sign.astype(np.int64) << 3)).astype(np.uint8)


def _mx_exponents(a: np.ndarray, emax: int) -> np.ndarray:
    """Per-block exponent for [R, C] values: [R, C/32] int."""
    R, C = a.shape
    assert C % MX_BLOCK == 0
    amax = np.abs(a.reshape(R, C // MX_BLOCK, MX_BLOCK)).max(axis=2).astype(np.float64)
    e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64) - emax
    return np.where(amax > 0, e, 0)


def quantize_mx_e4m3(a: np.ndarray):
    """MX e4m3 of a 2-D array: (codes uint8 [R, C], E8M0 scale bytes uint8 [R, C/32])."""
    a = np.asarray(a, dtype=np.float32)
    R, C = a.shape
    e = _mx_exponents(a, 8)
    q = a.astype(np.float64) / np.ldexp(1.0, np.repeat(e, MX_BLOCK, axis=1))
    codes = e4m3_encode(np.clip(q, -448.0, 448.0).astype(np.float32))
    return codes, (e + 127).astype(np.uint8)


def quantize_mx_e2m1(a: np.ndarray):
    """MX e2m1 of a 2-D array: (packed uint8 [R, C/2] with element 2i in the
    low nibble of byte i and 2i+1 in the high nibble, E8M0 scale bytes uint8
    [R, C/32])."""
    a = np.asarray(a, dtype=np.float32)
    R, C = a.shape
    e = _mx_exponents(a, 2)
    q = a.astype(np.float64) / np.ldexp(1.0, np.repeat(e, MX_BLOCK, axis=1))
    codes = e2m1_encode(q)
    packed = codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))
    return packed.astype(np.uint8), (e + 127).astype(np.uint8)


@dataclasses.dataclass
class MoeInputs:
    wl: Workload
    logits: np.ndarray            # fp32 [N, E]
    bias: np.ndarray | None       # fp32 [E] or None
    x: np.ndarray                 # bf16 bits uint16 [N, H], or e4m3 codes uint8 [N, H]
    x_scale: np.ndarray | None    # fp8: fp32 [N, H/128]; w4a8: E8M0 uint8 [N, H/32]
    w1: np.ndarray                # [L, 2I, H] bf16 bits or e4m3 codes; w4a8: packed
                                  # e2m1 uint8 [L, 2I, H/2]
    w1_scale: np.ndarray | None   # fp8: fp32 [L, 2I/128, H/128]; w4a8: E8M0 [L, 2I, H/32]
    w2: np.ndarray                # [L, H, I] (w4a8: [L, H, I/2] packed e2m1)
    w2_scale: np.ndarray | None   # fp8: fp32 [L, H/128, I/128]; w4a8: E8M0 [L, H, I/32]


def _children(seed: int):
    ss = np.random.SeedSequence(seed)
    return ss.spawn(4)


def zipf_bias(num_experts: int, s: float = 1.2, strength: float = 1.5) -> np.ndarray:
    ranks = np.arange(1, num_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    return (strength * np.log(p)).astype(np.float32)


def _normal(ss, shape, scale=1.0):
    g = np.random.default_rng(ss)
    out = g.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def make_logits(wl: Workload) -> tuple[np.ndarray, np.ndarray | None]:
    ch = _children(wl.seed)
    logits = _normal(ch[0], (wl.num_tokens, wl.num_experts))
    bias = zipf_bias(wl.num_experts) if wl.skew else None
    return logits, bias


def make_x(wl: Workload):
    ch = _children(wl.seed)
    x = _normal(ch[1], (wl.num_tokens, wl.hidden))
    if wl.dtype == "fp8":
        return quantize_e4m3_blocks(x, 1, 128)
    if wl.dtype == "w4a8":
        return quantize_mx_e4m3(x)
    return f32_to_bf16_bits(x), None


def make_expert_weights(wl: Workload, e: int):
    """Weights of local expert e (0-based within the local range)."""
    ch = _children(wl.seed)
    s1 = ch[2].spawn(wl.num_local)[e]
    s2 = ch[3].spawn(wl.num_local)[e]
    w1 = _normal(s1, (2 * wl.inter, wl.hidden), 0.02)
    w2 = _normal(s2, (wl.hidden, wl.inter), 0.02)
    if wl.dtype == "fp8":
        q1, s1_ = quantize_e4m3_blocks(w1, 128, 128)
        q2, s2_ = quantize_e4m3_blocks(w2, 128, 128)
        return q1, s1_, q2, s2_
    if wl.dtype == "w4a8":
        q1, s1_ = quantize_mx_e2m1(w1)
        q2, s2_ = quantize_mx_e2m1(w2)
        return q1, s1_, q2, s2_
    return f32_to_bf16_bits(w1), None, f32_to_bf16_bits(w2), None


_SHARED = {}


def _expert_job(args):
    """Draw expert e's weights into the arrays of _SHARED (fork workers see
    the parent's shared mappings, so nothing large is pickled)."""
    wl, e = args
    a, a_s, b, b_s = make_expert_weights(wl, e)
    _SHARED["w1"][e] = a
    _SHARED["w2"][e] = b
    if a_s is not None:
        _SHARED["w1s"][e] = a_s
        _SHARED["w2s"][e] = b_s
    return e


def _shared_array(shape, dtype):
    import mmap
    n = int(np.prod(shape)) * np.dtype(dtype).itemsize
    buf = mmap.mmap(-1, max(n, 1))   # anonymous MAP_SHARED: visible across fork
    return np.frombuffer(buf, dtype=dtype, count=int(np.prod(shape))).reshape(shape)


def make_inputs(wl: Workload, experts: int | None = None, workers: int = 1) -> MoeInputs:
    """Generate every input of a workload. ``experts`` limits how many local
    experts' weights are drawn (the rest are left zero) for quick host tests.
    ``workers`` > 1 draws the experts in that many forked processes (each
    expert has its own seed stream, so the result does not depend on it);
    call it before the process initialises a GPU."""
    logits, bias = make_logits(wl)
    x, xs = make_x(wl)
    L = wl.num_local
    wdt = np.uint16 if wl.dtype == "bf16" else np.uint8
    pack = 2 if wl.dtype == "w4a8" else 1      # e2m1: two elements per byte
    jobs = [(wl, e) for e in range(L if experts is None else min(experts, L))]
    parallel = workers > 1 and len(jobs) > 1
    alloc = _shared_array if parallel else (lambda shape, dt: np.zeros(shape, dt))
    w1 = alloc((L, 2 * wl.inter, wl.hidden // pack), wdt)
    w2 = alloc((L, wl.hidden, wl.inter // pack), wdt)
    w1s = w2s = None
    if wl.dtype == "fp8":
        w1s = alloc((L, 2 * wl.inter // 128, wl.hidden // 128), np.float32)
        w2s = alloc((L, wl.hidden // 128, wl.inter // 128), np.float32)
        w1s[...] = 1.0
        w2s[...] = 1.0
    elif wl.dtype == "w4a8":
        w1s = alloc((L, 2 * wl.inter, wl.hidden // MX_BLOCK), np.uint8)
        w2s = alloc((L, wl.hidden, wl.inter // MX_BLOCK), np.uint8)
        w1s[...] = 127
        w2s[...] = 127
    _SHARED.update(w1=w1, w2=w2, w1s=w1s, w2s=w2s)
    try:
        if parallel:
            import concurrent.futures as cf
            import multiprocessing as mp
            with cf.ProcessPoolExecutor(min(workers, len(jobs)), mp.get_context("fork")) as ex:
                list(ex.map(_expert_job, jobs))
        else:
            for j in jobs:
                _expert_job(j)
    finally:
        _SHARED.clear()
    return MoeInputs(wl, logits, bias, x, xs, w1, w1s, w2, w2s)
