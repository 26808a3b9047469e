"""CPU oracle for one GPU's expert-parallel share of a Mixture-of-Experts FFN.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the
HIP library and its Python binding) never calls it, and this module imports
nothing from the product path. It shares no code with it: the only common
dependency is the seeded input generator ``moe_inputs``, which holds none of
the method's arithmetic.

What it computes is the plain definition of the MoE FFN as the X-Stage paper
describes MegaMoE's dataflow (section 2.2, "MegaMoE Execution"): a router
selects k experts per token; each expert evaluates Linear-1 (hidden to
intermediate, gate and up projections), a SwiGLU activation and Linear-2
(intermediate back to hidden); Combine aggregates the top-k results with the
router weights. Restricted to the experts e0..e0+L-1 owned by one GPU, with
each weighted expert output stored in its own (token, top-k slot) entry of a
per-source-slice combine buffer, as the fused kernel's Linear-2 epilogue does.
The two scheduling orders of the paper (section 4.2, Algorithm 1) reorder
independent tiles only, so they do not change this result.

Precision: floating point is evaluated in float64. Two decisions that turn
floating point into integers are taken in float32, the precision of the
kernel: the biased router logit z = logit + bias, and the top-k selection on
z. Inputs are the exact bytes the GPU receives (bf16 bit patterns, e4m3
codes with their fp32 block scales, or OCP MX blocks: e2m1 weights and e4m3
activations with one E8M0 scale per 32 elements), decoded exactly.

Readings where the pages are silent (each is listed in the design notes):
  * top-k order: descending z, equal z broken by the lower expert index;
  * router weights: softmax over the k kept logits (equivalently, a full
    softmax renormalised over the kept experts); they sum to 1 per token;
  * SwiGLU: h = silu(gate) * up, silu(g) = g / (1 + exp(-g)); W1[e] rows
    0..I-1 are the gate projection, rows I..2I-1 the up projection; W2[e] is
    [H, I] (output-by-input, as a linear layer stores it);
  * the router weight multiplies the Linear-2 output of each routed row;
  * rows of one expert are ordered by ascending flat pair index f = n*k + j;
  * the intermediate activation h is kept in float64 here (the kernel rounds
    it to its storage type; the tolerance absorbs that).
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "e4m3_to_f64", "e2m1_to_f64", "e8m0_to_f64", "unpack_e2m1",
    "dequant_blocks", "dequant_mx", "route", "Layout",
    "dispatch_layout", "swiglu", "expert_ffn", "combine", "local_reduce",
    "OracleResult", "run",
]


# ---------------------------------------------------------------------------
# Exact decoding of the input formats
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32: widen by 16 zero bits."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN payloads widen as NaN
        return u32.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point, E4M3 ('fn': exponent bias 7, no infinities,
    S.1111.111 is NaN). Normal: (-1)^s * 2^(E-7) * (1 + M/8); subnormal
    (E = 0): (-1)^s * 2^-6 * (M/8)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    normal = s * np.ldexp(1.0 + M / 8.0, E - 7)
    sub = s * np.ldexp(M / 8.0, -6)
    out = np.where(E == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP 4-bit floating point E2M1 (MX specification): sign bit 3, exponent
    bits 2..1 with bias 1, mantissa bit 0, no infinities or NaN. Normal
    (E > 0): (-1)^s * 2^(E-1) * (1 + M/2); subnormal (E = 0): (-1)^s * M/2."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    E = (c >> 1) & 0x3
    M = c & 0x1
    return np.where(E == 0, s * M / 2.0, s * np.ldexp(1.0 + M / 2.0, E - 1))


def e8m0_to_f64(b: np.ndarray) -> np.ndarray:
    """OCP E8M0 scale: 2^(b - 127); 0xFF is NaN."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """Two e2m1 codes per byte along the last axis, element 2i in the low
    nibble of byte i: [..., C/2] bytes -> [..., C] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_mx(values: np.ndarray, scale_bytes: np.ndarray, block: int = 32) -> np.ndarray:
    """MX block scaling: element (r, c) times the E8M0 scale of block
    (r, c // block)."""
    s = np.repeat(e8m0_to_f64(scale_bytes), block, axis=-1)
    return np.asarray(values, np.float64) * s


def dequant_blocks(codes: np.ndarray, scales: np.ndarray, br: int, bc: int) -> np.ndarray:
    """Value = e4m3(code) * scale of the (br x bc) block holding it."""
    v = e4m3_to_f64(codes)
    R, C = v.shape
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), br, axis=0), bc, axis=1)
    return v * s[:R, :C]


# ---------------------------------------------------------------------------
# Routing (the router upstream of the fused kernel)
# ---------------------------------------------------------------------------

def route(logits: np.ndarray, bias: np.ndarray | None, k: int):
    """Top-k routing. z = logits + bias is formed in float32; experts are
    ranked by descending z with ties to the lower index (a stable sort of -z);
    the weights are a float64 softmax over the k kept z values.
    Returns (idx int32 [N, k], w float64 [N, k])."""
    z = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        z = (z + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    order = np.argsort(-z, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    zk = np.take_along_axis(z, idx, axis=1).astype(np.float64)
    ex = np.exp(zk - zk.max(axis=1, keepdims=True))
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w


# ---------------------------------------------------------------------------
# Dispatch layout: flattened row space of the local experts
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Layout:
    counts: np.ndarray        # int32 [L]   routed rows per local expert (M_e)
    row_offset: np.ndarray    # int32 [L+1] first row of expert e (unpadded)
    tile_offset: np.ndarray   # int32 [L+1] first scheduler row of e (O_e), padded to b_m
    row_pair: np.ndarray      # int32 [R]   flat pair f = n*k + j of each routed row
    pair_row: np.ndarray      # int32 [N*k] routed row of pair f, -1 if not local
    block_m: int

    @property
    def total_rows(self) -> int:
        return int(self.row_offset[-1])

    @property
    def sched_rows(self) -> int:
        return int(self.tile_offset[-1])


def dispatch_layout(idx: np.ndarray, e0: int, L: int, block_m: int) -> Layout:
    """Keep the pairs whose expert is local (e0 <= idx < e0 + L). Walk the
    pairs in ascending flat index f and append each to its expert's list, so
    rows of one expert come out in ascending f. Row offsets are the running
    sum of the counts; scheduler-row offsets (the paper's O_e in Algorithm 1)
    are the running sum of ceil(M_e / b_m), the per-expert M-tile count of the
    grouped-GEMM tile-count formula (the resource-management paper's Eq. 6)."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    per_expert = [[] for _ in range(L)]
    for f in range(flat.size):
        e = int(flat[f]) - e0
        if 0 <= e < L:
            per_expert[e].append(f)
    counts = np.array([len(r) for r in per_expert], dtype=np.int32)
    row_offset = np.zeros(L + 1, dtype=np.int32)
    tile_offset = np.zeros(L + 1, dtype=np.int32)
    for e in range(L):
        row_offset[e + 1] = row_offset[e] + counts[e]
        tile_offset[e + 1] = tile_offset[e] + (counts[e] + block_m - 1) // block_m
    row_pair = np.array([f for r in per_expert for f in r], dtype=np.int32)
    pair_row = np.full(flat.size, -1, dtype=np.int32)
    pair_row[row_pair] = np.arange(row_pair.size, dtype=np.int32)
    return Layout(counts, row_offset, tile_offset, row_pair, pair_row, block_m)


# ---------------------------------------------------------------------------
# Expert FFN and weighted combine
# ---------------------------------------------------------------------------

def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """SwiGLU (Shazeer 2020): silu(gate) * up with silu(g) = g * sigmoid(g)."""
    return gate / (1.0 + np.exp(-gate)) * up


def expert_ffn(X: np.ndarray, W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """Linear-1 (gate and up), SwiGLU, Linear-2 for one expert, float64.
    X [M, H], W1 [2I, H], W2 [H, I] -> Y [M, H]."""
    I = W2.shape[1]
    gate = X @ W1[:I].T
    up = X @ W1[I:].T
    return swiglu(gate, up) @ W2.T


def combine(w: np.ndarray, layout: Layout, Y: np.ndarray, N: int, k: int, H: int):
    """Weighted combine stores: slot (n, j) of the combine buffer receives
    w[n, j] * Y[row(n*k + j)] when pair n*k + j is local. Returns
    (C float64 [N, k, H] with zeros in unwritten slots, written bool [N, k])."""
    C = np.zeros((N * k, H), dtype=Y.dtype)
    written = layout.pair_row >= 0
    rows = layout.pair_row[written]
    C[written] = w.reshape(-1)[written][:, None] * Y[rows]
    return C.reshape(N, k, H), written.reshape(N, k)


def local_reduce(C: np.ndarray, written: np.ndarray) -> np.ndarray:
    """Source-side aggregation of this GPU's contributions: y[n] is the sum of
    the written slots of token n over ascending j."""
    N, k, H = C.shape
    y = np.zeros((N, H), dtype=C.dtype)
    for j in range(k):
        y += np.where(written[:, j:j + 1], C[:, j, :], 0.0)
    return y


@dataclasses.dataclass
class OracleResult:
    idx: np.ndarray
    w: np.ndarray
    layout: Layout
    Y: np.ndarray          # [R, H] per-row expert outputs (unweighted)
    C: np.ndarray          # [N, k, H] weighted combine slots
    written: np.ndarray    # [N, k]
    y_local: np.ndarray    # [N, H]


def decode_x_rows(inp, rows=slice(None)) -> np.ndarray:
    if inp.wl.dtype == "fp8":
        return dequant_blocks(inp.x[rows], inp.x_scale[rows], 1, 128)
    if inp.wl.dtype == "w4a8":
        return dequant_mx(e4m3_to_f64(inp.x[rows]), inp.x_scale[rows])
    return bf16_bits_to_f64(inp.x[rows])


def decode_x(inp) -> np.ndarray:
    return decode_x_rows(inp)


def decode_expert(inp, e: int):
    if inp.wl.dtype == "fp8":
        return (dequant_blocks(inp.w1[e], inp.w1_scale[e], 128, 128),
                dequant_blocks(inp.w2[e], inp.w2_scale[e], 128, 128))
    if inp.wl.dtype == "w4a8":
        return (dequant_mx(e2m1_to_f64(unpack_e2m1(inp.w1[e])), inp.w1_scale[e]),
                dequant_mx(e2m1_to_f64(unpack_e2m1(inp.w2[e])), inp.w2_scale[e]))
    return bf16_bits_to_f64(inp.w1[e]), bf16_bits_to_f64(inp.w2[e])


def run(inp, block_m: int = 128, idx=None, w=None, experts: int | None = None,
        float_type=np.float64) -> OracleResult:
    """The whole path: routing (unless idx/w are given), layout, per-expert
    FFN over the routed rows of each local expert, weighted combine and the
    source-side reduction. ``experts`` evaluates only the first that many
    local experts (a bounded sample for timing; other rows stay zero).
    ``float_type`` is the type of the FFN and combine arithmetic: float64 for
    parity; float32 only to time the plain fp32 CPU baseline (the same code in
    single precision)."""
    wl = inp.wl
    N, k, H = wl.num_tokens, wl.top_k, wl.hidden
    if idx is None:
        idx, w = route(inp.logits, inp.bias, k)
    lay = dispatch_layout(idx, wl.local_begin, wl.num_local, block_m)
    x = decode_x(inp).astype(float_type, copy=False)
    Y = np.zeros((lay.total_rows, H), dtype=float_type)
    for e in range(wl.num_local if experts is None else min(experts, wl.num_local)):
        r0, r1 = int(lay.row_offset[e]), int(lay.row_offset[e + 1])
        if r1 == r0:
            continue
        tokens = lay.row_pair[r0:r1] // k
        W1, W2 = (a.astype(float_type, copy=False) for a in decode_expert(inp, e))
        Y[r0:r1] = expert_ffn(x[tokens], W1, W2)
    C, written = combine(np.asarray(w, float_type), lay, Y, N, k, H)
    return OracleResult(idx, np.asarray(w, np.float64), lay, Y, C, written,
                        local_reduce(C, written))


def row_outputs(inp, idx, w, pairs, block_m: int = 128):
    """Expected combine rows for a sample of flat pairs (each must be local):
    w[f] * FFN_{idx[f]}(x[f // k]). Used for spot checks at full size, where
    the whole oracle would take too long."""
    wl = inp.wl
    k = wl.top_k
    x = decode_x(inp) if wl.dtype == "bf16" else None
    out = np.zeros((len(pairs), wl.hidden), dtype=np.float64)
    by_e = {}
    for i, f in enumerate(pairs):
        by_e.setdefault(int(idx.reshape(-1)[f]) - wl.local_begin, []).append(i)
    for e, ids in by_e.items():
        W1, W2 = decode_expert(inp, e)
        toks = [int(pairs[i]) // k for i in ids]
        X = decode_x_rows(inp, toks) if x is None else x[toks]
        Yr = expert_ffn(X, W1, W2)
        for r, i in enumerate(ids):
            out[i] = np.asarray(w, np.float64).reshape(-1)[pairs[i]] * Yr[r]
    return out
