// Persistent fused MoE expert FFN for gfx950 with W4A8 operands in the OCP
// Microscaling (MX) formats: weights e2m1 (4-bit, two per byte), activations
// e4m3, each block of 32 elements along K with one E8M0 (power-of-two)
// scale. The X-Stage paper evaluates its schedules at W4A8 and W8A8 (section
// 5.2.1); this kernel is the W4A8 variant of the fp8 kernel (ffn_fp8.hip),
// with the same task structure, schedules and epilogues. What differs:
//
//  - v_mfma_scale_f32_16x16x128_f8f6f4 with A = e2m1 weights (16 bytes per
//    lane) and B = e4m3 tokens (32 bytes per lane). Each lane's 32 K-values
//    are exactly one MX block, and the instruction applies the two blocks'
//    E8M0 scales itself: accumulators stay in the matrix core's fp32 chain
//    across the whole K loop, with no promotion on the VALU.
//  - A stage is one 128-wide K block: 64-byte weight rows, 128-byte token
//    rows and one scale word (four E8M0 bytes) per row, 42 KiB for a
//    192 x 256 tile, so three stages fit in LDS.
//  - Linear-1 quantises h to MX e4m3: per token and 32 columns, the scale
//    exponent is the smallest e with amax / 2^e <= 448 (no element clamps),
//    values are h / 2^e rounded to nearest-even. One wavefront holds exactly
//    one such block per token (32 h columns).
#include <hip/hip_runtime.h>

#include "ffn_common.hpp"
#include "internal.hpp"
#include "sched.hpp"

namespace moe {
namespace {

template <int TM_, int TN_, int WT_, int WF_, int NS_, int SP_ = MOE_ISSUE_SPREAD>
struct CfgMx {
  static constexpr int TM = TM_, TN = TN_, WT = WT_, WF = WF_, NS = NS_;
  static constexpr int NW = WT * WF;
  static constexpr int THREADS = 64 * NW;
  static constexpr int TT = TM / WT, FT = TN / WF;
  static constexpr int FB16 = FT / 16, TB16 = TT / 16;
  static constexpr int A_ROW = 64;                   // e2m1 bytes of a weight row per K block
  static constexpr int B_ROW = 128;                  // e4m3 bytes of a token row per K block
  static constexpr int A_BYTES = TN * A_ROW;
  static constexpr int B_OFF = A_BYTES;
  static constexpr int B_BYTES = TM * B_ROW;
  static constexpr int S_OFF = B_OFF + B_BYTES;      // scale words: weight rows, then token rows
  static constexpr int S_WORDS = 64 * NW;            // one four-byte copy per wavefront
  static constexpr int STAGE_BYTES = S_OFF + S_WORDS * 4;
  static constexpr int NIA = TN / 16 / NW;           // weight copies (16 rows of 64 B) per wavefront
  static constexpr int NIB = TM / 8 / NW;            // token copies (8 rows of 128 B)
  static constexpr int NI = NIA + NIB + 1;           // plus the scale-word copy
  static constexpr int NB = FB16 * TB16;             // MFMAs per wavefront per stage
  static constexpr int SP = SP_;
  // copy i of a stage is issued after MFMA issue_slot(i) of the stage before
  static constexpr int issue_slot(int i) { return i * NB * SP / (NI * 8); }
  static_assert(TN == 256, "an N-tile owns four 32-column h scale blocks, one per feature wavefront");
  static_assert(WF == 4 && FT == 64, "gate/up pairing: one 32-row gate and one 32-row up block per wavefront");
  static_assert(TT % 16 == 0 && TB16 >= 2, "token blocks");
  static_assert(TN % (16 * NW) == 0 && TM % (8 * NW) == 0, "copies split evenly over wavefronts");
  static_assert(TN + TM <= S_WORDS, "one scale word per row");
  static_assert(NS >= 2 && NI * (NS - 1) <= 63, "vmcnt range");
  static_assert(SP >= 1 && SP <= 8, "spread in eighths of the stage");
};

// Physical 16-byte chunk of logical chunk q (the K quarter lane group q
// reads) in 64-byte weight row r: q ^ ((r >> 2) & 3) ^ ((q & 1) << 1), a
// bijection of the row's 4 chunks. The row term alone spreads 16 rows of one
// chunk over all banks, but measured on MI355X (rocprofv3
// SQ_LDS_BANK_CONFLICT, an LDS probe of this read) the 128-bit reads of the
// four lane groups still conflict two ways; the (q & 1) << 1 term removes it.
__device__ __forceinline__ int wchunk_of(int r, int q) { return q ^ ((r >> 2) & 3) ^ ((q & 1) << 1); }
// logical chunk held by physical chunk p of weight row r (the inverse)
__device__ __forceinline__ int wlogical_chunk(int r, int p) {
  const int x = p ^ ((r >> 2) & 3);
  return x ^ ((x & 1) << 1);
}

template <class C>
struct TileMx {
  const char* asrc[C::NIA];   // this lane's weight-row chunk, stage 0
  const char* bsrc[C::NIB];   // token-row chunk, stage 0
  const char* ssrc;           // scale word of row (wave*64 + lane) (clamped), stage 0
  uint32_t ring;
  f32x4 acc[C::FB16][C::TB16];

  // Weight copy i of wavefront w fills rows [16j, 16j+16), j = w + NW*i, lane
  // l row 16j + l/4, physical chunk l%4 (logical chunk wlogical_chunk(row, l%4));
  // token copy i fills rows [8j, 8j+8), lane l row 8j + l/8, physical chunk
  // l%8 (logical l%8 ^ ((row>>1)&7)). Scale word q = 64w + lane: weight row
  // q, token row q - TN (rows past TN + TM repeat the last token row).
  template <class ARow, class BRow, class ASc, class BSc>
  __device__ __forceinline__ void setup(ARow arow, BRow brow, ASc asc, BSc bsc) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < C::NIA; ++i) {
      const int r = (wave + C::NW * i) * 16 + lane / 4;
      asrc[i] = arow(r) + (wlogical_chunk(r, lane & 3) << 4);   // lands at physical chunk lane % 4
    }
#pragma unroll
    for (int i = 0; i < C::NIB; ++i) {
      const int r = (wave + C::NW * i) * 8 + lane / 8;
      bsrc[i] = brow(r) + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    }
    const int q = wave * 64 + lane;
    ssrc = q < C::TN ? asc(q) : bsc(min(q - C::TN, C::TM - 1));
  }

  template <bool COH>
  __device__ __forceinline__ void issue_one(int i, int kt, uint32_t slot) {
    const int wave = threadIdx.x >> 6;
    if (i < C::NIA) {
      dma16<kCacheNormal>(asrc[i] + (size_t)kt * C::A_ROW, uni(slot + (wave + C::NW * i) * 1024));
    } else if (i < C::NIA + C::NIB) {
      const int ib = i - C::NIA;
      const uint32_t dst = uni(slot + C::B_OFF + (wave + C::NW * ib) * 1024);
      if (COH) dma16<kCoherent>(bsrc[ib] + (size_t)kt * C::B_ROW, dst);
      else dma16<kCacheNormal>(bsrc[ib] + (size_t)kt * C::B_ROW, dst);
    } else {
      // token scale words of h are written during this launch (COH); weight
      // scale words share the same copy instruction and take the same policy
      const uint32_t dst = uni(slot + C::S_OFF + wave * 256);
      if (COH) dma4<kCoherent>(ssrc + kt * 4, dst);
      else dma4<kCacheNormal>(ssrc + kt * 4, dst);
    }
  }

  // One 128-wide K block: 16x16x128 MFMAs, A = e2m1 weights, B = e4m3
  // tokens, each lane's E8M0 scale byte taken from its row's scale word.
  // Operand placement (checked on the GPU with one-hot and scaled operands):
  // the matrix core pairs e2m1 lane group q (lanes 16q..16q+15), its 32
  // values in nibble order, with e4m3 lane group q', bytes 0-15 / 16-31,
  // such that an A lane group reading K elements 32q..32q+31 of its row (one
  // MX block, scaled by that lane's byte) meets B lane groups that read
  // elements 16q'..16q'+15 and 64+16q'..64+16q'+15 of the token row; a B
  // lane's scale applies to MX block q' of the token row (elements
  // 32q'..32q'+31, which lanes 16q'.. hold across two lane groups).
  // Program order is fixed: the weight fragments of block i are read before
  // MFMA i, the next token block's fragment and scales while the current one
  // is multiplied, and the copies of a later stage between the MFMAs.
  template <bool COH>
  __device__ __forceinline__ void compute(const char* stage, int wf, int wt, int kt_next, uint32_t slot) {
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, q = lane >> 4;   // row within a block, 32-wide K quarter
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(stage + C::S_OFF);
    i32x8 af[C::FB16], bf[2];
    int sa[C::FB16], sb[2];
    auto afrag = [&](int i) {
      const int r = wf * C::FT + i * 16 + r16;
      const uint4 v = *reinterpret_cast<const uint4*>(stage + r * C::A_ROW + (wchunk_of(r, q) << 4));
      af[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      sa[i] = (int)(sw[r] >> (8 * q));
    };
    auto bfrag = [&](int j) {
      const int r = wt * C::TT + j * 16 + r16;
      const char* row = stage + C::B_OFF + r * C::B_ROW;
      const int swz = (r >> 1) & 7;
      const uint4 lo = *reinterpret_cast<const uint4*>(row + ((q ^ swz) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(row + (((q + 4) ^ swz) << 4));
      bf[j & 1] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sb[j & 1] = (int)(sw[C::TN + r] >> (8 * q));
    };
    bfrag(0);
    afrag(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
      const int j = b / C::FB16, i = b % C::FB16;   // token block, feature block
      if (b + 1 < C::FB16) afrag(b + 1);
      if (i == 0 && j + 1 < C::TB16) bfrag(j + 1);
      // formats: A 4 = e2m1, B 0 = e4m3; scale bytes in bits 7..0 (op_sel 0)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j & 1], acc[i][j], 4, 0, 0, sa[i],
                                                                   0, sb[j & 1]);
      // the scale-word and token-row copies of the stage go out before its
      // weight-row copies: the gathered token rows come back later (measured
      // on MI355X: 2.3% faster Interleaved, 3.3% Expert-Wave)
#pragma unroll
      for (int k = 0; k < C::NI; ++k)
        if (C::issue_slot(k) == b) issue_one<COH>(C::NI - 1 - k, kt_next, slot);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // K loop over nk 128-wide blocks through the NS-stage ring: stage kt is
  // awaited (own copies, then one workgroup barrier), then multiplied while
  // the copy of stage kt+NS-1 goes into the slot stage kt-1 used. The copy is
  // issued unconditionally (the last NS-1 stages re-copy stage nk-1 into
  // their free slot); those extra copies are awaited at the end, before the
  // epilogue reuses LDS.
  template <bool COH>
  __device__ __forceinline__ void mainloop(char* lds, int nk, int wf, int wt) {
#pragma unroll
    for (int i = 0; i < C::FB16; ++i)
#pragma unroll
      for (int j = 0; j < C::TB16; ++j) acc[i][j] = f32x4{};
    lds_barrier();
#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s) {
      const int ks = min(s, nk - 1);
#pragma unroll
      for (int i = 0; i < C::NI; ++i) issue_one<COH>(i, ks, ring + s * C::STAGE_BYTES);
    }
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
      vm_wait<C::NI * (C::NS - 2)>();   // stage kt has landed (later stages may not have)
      lds_barrier();
      const int nxt = min(kt + C::NS - 1, nk - 1);
      const int nslot = slot == 0 ? C::NS - 1 : slot - 1;
      compute<COH>(lds + slot * C::STAGE_BYTES, wf, wt, nxt, ring + nslot * C::STAGE_BYTES);
      slot = slot + 1 == C::NS ? 0 : slot + 1;
    }
    vm_wait<0>();
  }

  // Linear-1: blocks 0-1 of the wavefront are gate rows, 2-3 the matching up
  // rows (32-row interleave of W1's N-tile), so the wavefront holds 32 h
  // columns of each token: one MX block, whose amax is reduced within the
  // lane and across the lanes l, l^16, l^32, l^48 of a token column. The
  // e4m3 h tile and its scale bytes are staged in the ring and written as
  // whole 16-byte row pieces and one scale word per row.
  __device__ __forceinline__ void epi_l1(const FfnArgs& a, int p, int n, int j0, char* lds) {
    const int tid = opaque(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int wf = wave % C::WF, wt = wave / C::WF;
    const int r16 = lane & 15;
    constexpr int HROW = C::TN / 2;   // the N-tile's h columns, one byte each
    uint8_t* const hsc = reinterpret_cast<uint8_t*>(lds + C::TM * HROW);   // [TM][4] scale bytes
    static_assert(C::TM * HROW + C::TM * 4 <= C::NS * C::STAGE_BYTES, "h staging fits the ring");
    lds_barrier();   // every wavefront is past its last stage: the ring is free
#pragma unroll
    for (int j = 0; j < C::TB16; ++j) {
      float hv[2][4];
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float h = silu(acc[i][j][v]) * acc[i + 2][j][v];
          hv[i][v] = h;
          mx = fmaxf(mx, fabsf(h));
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // block exponent: the smallest e with amax / 2^e <= 448 (e4m3's
      // largest value), so no element is clamped; at least -127 (E8M0 byte
      // 0); an all-zero block gets exponent 0
      const int ebits = (int)((__float_as_uint(mx) >> 23) & 0xFF);
      int ex = mx > 0.f ? max(ebits - 127 - 8, -127) : 0;
      if (mx * __uint_as_float((uint32_t)(127 - ex) << 23) > 448.f) ++ex;
      const float inv = __uint_as_float((uint32_t)(127 - ex) << 23);   // 2^-ex
      const int tok_l = wt * C::TT + j * 16 + r16;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<uint32_t*>(lds + stage_off<HROW>(tok_l, wf * 32 + i * 16 + 4 * (lane >> 4))) =
            quant4(hv[i], inv);
      if (lane < 16) hsc[tok_l * 4 + wf] = (uint8_t)(ex + 127);
    }
    __syncthreads();
    char* hb = static_cast<char*>(a.h) + (size_t)p * C::TM * a.I + j0;
    constexpr int NCH = HROW / 16;
    for (int idx = tid; idx < C::TM * NCH; idx += C::THREADS) {
      const int row = idx / NCH, c = idx - row * NCH;
      const i32x4 v = *reinterpret_cast<const i32x4*>(lds + stage_off<HROW>(row, c * 16));
      // device scope: written through this XCD's L2 for the consuming XCD
      store16<kCoherent>(hb + (size_t)row * a.I + c * 16, v);
    }
    char* hs = reinterpret_cast<char*>(a.hs) + (size_t)p * C::TM * (a.I / 32) + n * 4;
    for (int row = tid; row < C::TM; row += C::THREADS)
      __hip_atomic_store(reinterpret_cast<uint32_t*>(hs + (size_t)row * (a.I / 32)),
                         reinterpret_cast<const uint32_t*>(hsc)[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Linear-2: bf16(w * acc) into the combine slot of each routed row, staged
  // in the ring and stored as whole 16-byte row pieces (row destinations
  // resolved once from the routed pairs fetch_rows copied to LDS).
  __device__ __forceinline__ void epi_l2(const FfnArgs& a, int n, int m, int Me, char* const* comb, char* lds,
                                         const int* pair_s, const float* wgt_s) {
    const int tid = opaque(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int wf = wave % C::WF, wt = wave / C::WF;
    const int r16 = lane & 15;
    constexpr int CROW = C::TN * 2;
    static_assert(C::TM * CROW + C::TM * (int)sizeof(char*) <= C::NS * C::STAGE_BYTES,
                  "combine staging and row destinations fit the ring");
    char** const rowdst = reinterpret_cast<char**>(lds + C::TM * CROW);
    const int rows = min(C::TM, Me - m * C::TM);   // padding rows are never stored
    lds_barrier();
    for (int row = tid; row < rows; row += C::THREADS) {
      const int f = pair_s[row];
      const int tok = f / a.k;
      const int slot = f - tok * a.k;
      const int s = tok / a.T;
      rowdst[row] = comb[s] + (((size_t)(tok - s * a.T) * a.k + slot) * a.H + (size_t)n * C::TN) * 2;
    }
#pragma unroll
    for (int j = 0; j < C::TB16; ++j) {
      const int tok_l = wt * C::TT + j * 16 + r16;
      const float w = wgt_s[tok_l];
#pragma unroll
      for (int i = 0; i < C::FB16; ++i) {
        const f32x4& v = acc[i][j];
        const uint64_t o = (uint64_t)pack_bf16x2(w * v[0], w * v[1]) |
                           ((uint64_t)pack_bf16x2(w * v[2], w * v[3]) << 32);
        *reinterpret_cast<uint64_t*>(lds + stage_off<CROW>(tok_l, (wf * C::FT + i * 16 + 4 * (lane >> 4)) * 2)) = o;
      }
    }
    __syncthreads();
    constexpr int NCH = CROW / 16;
    for (int idx = tid; idx < rows * NCH; idx += C::THREADS) {
      const int row = idx / NCH, c = idx - row * NCH;
      const i32x4 v = *reinterpret_cast<const i32x4*>(lds + stage_off<CROW>(row, c * 16));
      if (MOE_COMBINE_NT) store16<kStream>(rowdst[row] + c * 16, v);
      else store16<kCacheNormal>(rowdst[row] + c * 16, v);
    }
  }
};

struct MetaMx {
  Meta m;
  const char* xs[MOE_MAX_SLICES];
};

template <class C>
__global__ void __launch_bounds__(C::THREADS, 1) moe_ffn_w4a8(const FfnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[C::NS * C::STAGE_BYTES];
  __shared__ MetaMx metam;
  __shared__ int pair_s[C::TM];   // routed pair and router weight of each row of a
  __shared__ float wgt_s[C::TM];  // Linear-2 tile (fetch_rows)
  Meta& meta = metam.m;
  // with L2-cached h loads: drop lines an earlier launch left in this XCD's L2
  if (!MOE_H_COHERENT) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wf = wave % C::WF;
  const int wt = wave / C::WF;
  const int L = a.L, H = a.H, I = a.I, K = a.k, T = a.T;

  for (int i = tid; i <= L; i += C::THREADS) meta.tile_off[i] = a.tile_offset[i];
  for (int i = tid; i < a.S; i += C::THREADS) {
    meta.x[i] = static_cast<const char*>(a.x[i]);
    meta.comb[i] = static_cast<char*>(a.comb[i]);
    metam.xs[i] = reinterpret_cast<const char*>(a.xs[i]);
  }
  __syncthreads();
  if (tid == 0 && a.schedule == MOE_SCHED_EXPERT_WAVE)
    meta.nwaves = build_waves(meta.tile_off, L, a.N1, a.grid, a.experts_per_wave, meta.wave_exp);
  __syncthreads();
  const int P = uni(meta.tile_off[L]);
  const int G = a.grid;
  const int g = logical_instance(G, a.xcd_group, a.xcd_bx);

  InterleavedStream ist;
  ExpertWaveStream ews;
  const bool interleaved = a.schedule == MOE_SCHED_INTERLEAVED;
  if (interleaved) ist.init(g, G, P, a.N1, a.N2, a.lead_d);
  else ews.init(g, G, a.N1, a.N2, meta.tile_off, meta.wave_exp, uni(meta.nwaves));

  TileMx<C> tile;
  tile.ring = (uint32_t)(uintptr_t)lds;
  const char* w1b = static_cast<const char*>(a.w1);
  const char* w2b = static_cast<const char*>(a.w2);
  const char* w1sb = reinterpret_cast<const char*>(a.w1s);
  const char* w2sb = reinterpret_cast<const char*>(a.w2s);
  const char* hb = static_cast<const char*>(a.h);
  const char* hsb = reinterpret_cast<const char*>(a.hs);
  int seq = 0;
  for (;;) {
    const Task t = interleaved ? ist.next() : ews.next();
    if (t.kind == 0) break;
    const int p = uni(t.p), n = uni(t.n);
    const bool tracing = a.trace && seq < a.trace_cap;   // uniform
    uint32_t* rec = (tracing && tid == 0)
                        ? a.trace + ((size_t)g * a.trace_cap + seq) * kTraceWords
                        : nullptr;
    if (rec) {
      rec[0] = (uint32_t)t.kind | ((uint32_t)n << 2);
      rec[1] = (uint32_t)p;
      rec[2] = (uint32_t)wall_clock64();
      rec[6] = (uint32_t)__builtin_readcyclecounter();   // shader clock
      rec[9] = blockIdx.x;
    }
    ++seq;
    const int e = expert_of_row(meta.tile_off, L, p);
    const int m = p - uni(meta.tile_off[e]);
    const int r_base = uni(a.row_offset[e]);
    const int Me = uni(a.row_offset[e + 1]) - r_base;
    const bool l1 = t.kind == 1;
    if (l1) {
      if (p == a.debug_skip_row) continue;
    } else {
      if (tid == 0) {
        int ok = 1;
        if (__hip_atomic_load(a.l2_full + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.N1) {
          const long long t0 = wall_clock64();
          while (__hip_atomic_load(a.l2_full + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.N1) {
            __builtin_amdgcn_s_sleep(2);
            if (wall_clock64() - t0 > a.timeout_ticks) {
              ok = 0;
              if (a.status) __hip_atomic_store(a.status, (int)MOE_ERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          }
        }
        meta.flag = ok;
      }
      __syncthreads();
      const int ok = uni(meta.flag);
      __syncthreads();
      if (!ok) continue;
      fetch_rows<C>(a.row_pair + r_base, a.row_weight + r_base, m * C::TM, Me, pair_s, wgt_s, wave, lane);
    }
    if (rec) rec[3] = (uint32_t)wall_clock64();

    const int j0 = n * (C::TN / 2);
    if (l1) {
      // gate/up rows of W1[e] (32-row blocks alternate gate and up rows) and
      // the gathered token rows of x; padding rows repeat the last routed row
      auto wrow = [&](int q) {
        const int blk = q >> 5;
        return (size_t)e * 2 * I + ((blk & 1) ? I : 0) + j0 + (blk >> 1) * 32 + (q & 31);
      };
      auto tok_of = [&](int q) { return a.row_pair[r_base + min(m * C::TM + q, Me - 1)] / K; };
      tile.setup([&](int q) { return w1b + wrow(q) * (H / 2); },
                 [&](int q) {
                   const int tok = tok_of(q), s = tok / T;
                   return meta.x[s] + (size_t)(tok - s * T) * H;
                 },
                 [&](int q) { return w1sb + wrow(q) * (H / 32); },
                 [&](int q) {
                   const int tok = tok_of(q), s = tok / T;
                   return metam.xs[s] + (size_t)(tok - s * T) * (H / 32);
                 });
    } else {
      tile.setup([&](int q) { return w2b + ((size_t)e * H + n * C::TN + q) * (I / 2); },
                 [&](int q) { return hb + ((size_t)p * C::TM + q) * I; },
                 [&](int q) { return w2sb + ((size_t)e * H + n * C::TN + q) * (I / 32); },
                 [&](int q) { return hsb + ((size_t)p * C::TM + q) * (I / 32); });
    }
    const int nk = (l1 ? H : I) / 128;
    if (l1 || !MOE_H_COHERENT) tile.template mainloop<false>(lds, nk, wf, wt);
    else tile.template mainloop<true>(lds, nk, wf, wt);
    if (rec) {
      rec[4] = (uint32_t)wall_clock64();
      rec[7] = (uint32_t)__builtin_readcyclecounter();
    }

    if (l1) {
      tile.epi_l1(a, p, n, j0, lds);
      // publish: every wavefront's h stores have completed before the row
      // counter moves
      vm_wait<0>();
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(a.l2_full + p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (rec) rec[5] = rec[8] = (uint32_t)wall_clock64();
    } else {
      tile.epi_l2(a, n, m, Me, meta.comb, lds, pair_s, wgt_s);
      trace_store_span(tracing, rec);
    }
  }

  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(a.done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    meta.flag = prev == a.grid - 1;
  }
  __syncthreads();
  if (meta.flag) {
    for (int i = tid; i < P; i += C::THREADS)
      __hip_atomic_store(a.l2_full + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) __hip_atomic_store(a.done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// CfgMx<tokens, features, token waves, feature waves, ring stages, copy spread>
using CfgMxMain = CfgMx<192, 256, 2, 4, 3, 6>;   // 96 tokens x 64 features per wavefront

template <class C>
hipError_t launch(const FfnArgs& a, hipStream_t s) {
  moe_ffn_w4a8<C><<<a.grid, C::THREADS, 0, s>>>(a);
  return hipGetLastError();
}

template <class C>
hipError_t occupancy(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, moe_ffn_w4a8<C>, C::THREADS, 0);
}

}  // namespace

extern const TileInfo kW4a8Tiles[];
extern const int kNumW4a8Tiles;
const TileInfo kW4a8Tiles[] = {
    {31, MOE_W4A8, CfgMxMain::TM, CfgMxMain::TN, CfgMxMain::THREADS},
};
const int kNumW4a8Tiles = sizeof(kW4a8Tiles) / sizeof(kW4a8Tiles[0]);

hipError_t launch_ffn_w4a8(int id, const FfnArgs& a, hipStream_t s) {
  switch (id) {
    case 31: return launch<CfgMxMain>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t occupancy_ffn_w4a8(int id, int* n) {
  switch (id) {
    case 31: return occupancy<CfgMxMain>(n);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
