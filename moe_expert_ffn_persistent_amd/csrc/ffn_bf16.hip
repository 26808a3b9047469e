// Persistent fused MoE expert FFN for gfx950, bf16 inputs, fp32 accumulate.
//
// One launch runs every tile of one GPU's expert-parallel share (the X-Stage
// paper's MegaMoE kernel, section 2.2): Linear-1 tiles (gate and up
// projections over K = H, SwiGLU fused into the epilogue, h stored to the
// workspace and published through the per-row l2_full counter) and
// Linear-2 tiles (down projection over K = I after waiting for l2_full to
// reach N1; the epilogue multiplies each row by its router weight, rounds to
// bf16 and stores it into the (token, top-k slot) entry of the combine
// buffer of the token's source slice). The order of the tiles is the
// Expert-Wave order or Algorithm 1 (sched.hpp).
//
// CDNA4 mapping:
//  - MFMA v_mfma_f32_32x32x16_bf16. Weights are the MFMA A operand (rows =
//    output features), tokens the B operand (columns = tokens), so each lane
//    ends up holding one token and runs of 4 consecutive output features:
//    the epilogue writes 8-byte pieces and one router weight per lane.
//  - Both operands are K-contiguous in HBM (W[e] rows, x rows, h rows), so
//    global->LDS copies move 16-byte chunks and each MFMA lane reads one
//    16-byte chunk from LDS. Chunks are XOR-swizzled by row so that a
//    16-byte read of 16 consecutive rows touches 16 distinct bank groups.
//  - An NS-stage LDS ring filled by direct-to-LDS copies: the copy of stage
//    kt+NS-1 is issued between the MFMAs of stage kt (spread over the first
//    half of them), one workgroup barrier per stage.
//  - Linear-1 N-tiles interleave gate and up rows in 32-row blocks, so the
//    gate and up accumulators of one output column sit in the same lane.
//  - h and l2_full cross XCDs (each XCD has its own L2): the producer writes
//    h with device-scope (sc1) stores that go through its L2, waits for them
//    to complete, then bumps the counter with a device-scope atomic; the
//    consumer polls the counter with device-scope loads and copies h with
//    device-scope (sc1) loads, which are never served from a stale L2 line.
//    No whole-L2 write-back or invalidate is needed on either side.
//  - Copies move whole 128-byte row segments where the LDS budget allows
//    (BK = 64): measured on MI355X, 64-byte segments and the gathered token
//    rows that every N-tile of a row re-reads limit the weight stream long
//    before HBM does.
#include <hip/hip_runtime.h>

#include "ffn_common.hpp"
#include "internal.hpp"
#include "sched.hpp"

namespace moe {
namespace {


template <int TM_, int TN_, int WT_, int WF_, int BK_, int NS_, int SP_ = MOE_ISSUE_SPREAD,
          bool TF_ = false>
struct Cfg {
  static constexpr int TM = TM_;          // tokens per M-block (b_m)
  static constexpr int TN = TN_;          // features per N-tile (b_n)
  static constexpr int WT = WT_;          // wavefronts along tokens
  static constexpr int WF = WF_;          // wavefronts along features
  static constexpr int BK = BK_;          // K elements per stage
  static constexpr int NS = NS_;          // LDS ring stages
  static constexpr int NW = WT * WF;
  static constexpr int THREADS = 64 * NW;
  static constexpr int TT = TM / WT;      // tokens per wavefront
  static constexpr int FT = TN / WF;      // features per wavefront
  static constexpr int TB = TT / 32;      // 32-token MFMA blocks per wavefront
  static constexpr int FB = FT / 32;      // 32-feature MFMA blocks per wavefront
  static constexpr int ROW_BYTES = BK * 2;
  static constexpr int CPR = ROW_BYTES / 16;      // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;            // rows per 1 KiB DMA instruction
  // chunk c of row r is stored at chunk c ^ ((r >> SWZ_SHIFT) & SWZ_MASK): the
  // 16 lanes served per LDS clock (16-byte reads of rows r..r+15 at one
  // logical chunk) then hit 16 distinct 16-byte bank groups of the 256-byte
  // bank space
  static constexpr int SWZ_SHIFT = CPR == 8 ? 1 : 2;
  static constexpr int SWZ_MASK = CPR - 1;
  static constexpr int NI = (TN + TM) / RPI / NW; // DMA instructions per wavefront per stage
  static constexpr int NIW = TN / RPI / NW;       // of which weight rows (the first NIW)
  static constexpr int NM = (BK / 16) * (TT / 32) * (FT / 32);   // MFMAs per wavefront per stage
  // copy instruction i of a stage is issued after MFMA issue_slot(i) of the
  // stage before: spread evenly over the first SP/8 of the MFMAs (measured
  // per tile on MI355X: the HBM-bound 160 x 256 tile gains from spreading
  // the copies wider, the MFMA-bound 256 x 256 tiles from issuing earlier)
  static constexpr int SP = SP_;
  static_assert(SP >= 1 && SP <= 8, "spread in eighths of the stage");
  static constexpr int issue_slot(int i, int nm = NM) { return i * nm * SP / (NI * 8); }
  // TF: within a stage the token-row copies go out before the weight-row
  // copies (measured on MI355X: the HBM-bound 160 x 256 tile 1-2% faster,
  // the 256 x 256 tile 0.5-1.4% and the 32 x 128 decode tile 1.3% slower)
  static constexpr bool TF = TF_;
  static constexpr int copy_of(int o) { return TF ? NI - 1 - o : o; }
  static constexpr int A_BYTES = TN * ROW_BYTES;
  static constexpr int STAGE_BYTES = (TN + TM) * ROW_BYTES;
  // LDS: the copy ring, reused by the epilogue to stage a TM x TN bf16 tile
  static constexpr int LDS_BYTES = NS * STAGE_BYTES > TM * TN * 2 ? NS * STAGE_BYTES : TM * TN * 2;
  static_assert(TT % 32 == 0 && FT % 32 == 0, "wavefront tile must be a multiple of 32");
  static_assert(FB % 2 == 0, "gate/up pairing needs an even number of feature blocks");
  static_assert(CPR == 8 || CPR == 4, "rows of 64 or 128 bytes");
  static_assert(TN % RPI == 0 && TM % RPI == 0, "DMA instructions must not straddle operands");
  static_assert(((TN + TM) / RPI) % NW == 0, "DMA instructions must split evenly over wavefronts");
  static_assert(TN % (RPI * NW) == 0, "every wavefront copies weight rows in its first NIW instructions");
  static_assert(NS >= 2 && NI * (NS - 1) <= 63, "vmcnt range");
};

template <class C>
struct Tile {
  const char* src[C::NI];   // this lane's copy sources for stage 0
  f32x16 acc[C::FB][C::TB];
  uint32_t ring;            // LDS byte address of the ring

  // Copy sources: instruction i of wavefront w fills LDS rows
  // [j*RPI, (j+1)*RPI) of a stage, j = w + NW*i; lane l takes row
  // j*RPI + l/CPR and the logical chunk that lands at its physical slot.
  // Instructions below NIW take weight rows (wrow), the others token rows:
  // every token row's key (tkey, possibly a global load) is fetched before
  // any is used, so the loads overlap, then taddr maps keys to addresses.
  template <class WRow, class TKey, class TAddr>
  __device__ __forceinline__ void setup(WRow wrow, TKey tkey, TAddr taddr) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    int key[C::NI];
#pragma unroll
    for (int i = C::NIW; i < C::NI; ++i) key[i] = tkey((wave + C::NW * i) * C::RPI + lane / C::CPR - C::TN);
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      const int j = wave + C::NW * i;
      const int r = j * C::RPI + lane / C::CPR;
      const int c = (lane % C::CPR) ^ ((r >> C::SWZ_SHIFT) & C::SWZ_MASK);
      const char* base = i < C::NIW ? wrow(r) : taddr(key[i]);
      src[i] = base + c * 16;
    }
  }

  // One 1 KiB copy (instruction i of this wavefront) of the stage at byte
  // offset `off` of the rows into the ring slot at LDS address `slot`.
  // Instructions below NIW fill weight rows, the rest token rows; token rows
  // are h (written during this launch by other XCDs) when COH, copied with
  // device-scope loads.
  template <bool COH>
  __device__ __forceinline__ void issue_one(int i, size_t off, uint32_t slot) {
    const int wave = threadIdx.x >> 6;
    const uint32_t dst = uni(slot + (wave + C::NW * i) * 1024);
    if (i < C::NIW) dma16<MOE_WEIGHT_POLICY>(src[i] + off, dst);
    else if (COH) dma16<kCoherent>(src[i] + off, dst);
    else dma16<kCacheNormal>(src[i] + off, dst);
  }

  // fragment q of k-step ks: q < FB are weight (A) fragments, the rest token
  // (B) fragments; lane l reads row l%32 of its 32-row block, 16 bytes at
  // logical chunk 2*ks + l/32
  __device__ __forceinline__ void load_frag(const char* stage, int ks, int q, int wf, int wt,
                                            bf16x8 (&af)[C::FB], bf16x8 (&bf)[C::TB]) {
    const int lane = threadIdx.x & 63;
    const int r_lane = lane & 31;
    const int swz = (r_lane >> C::SWZ_SHIFT) & C::SWZ_MASK;
    const int chunk = ((2 * ks + (lane >> 5)) ^ swz) << 4;
    if (q < C::FB) {
      const int r = wf * C::FT + q * 32 + r_lane;
      af[q] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(stage + r * C::ROW_BYTES + chunk));
    } else {
      const int r = wt * C::TT + (q - C::FB) * 32 + r_lane;
      bf[q - C::FB] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(stage + C::A_BYTES + r * C::ROW_BYTES + chunk));
    }
  }

  // One stage of MFMAs with the copy of a later stage spread between them.
  // Program order is fixed: after MFMA m of k-step ks come the fragment reads
  // of k-step ks+1 assigned to m (register double buffering) and the copies
  // assigned to MFMA ks*NMF+m. Measured on MI355X, copies issued in one burst
  // hold the wavefront at the issue until the address unit drains them, so the
  // copy and the MFMAs of a stage run back to back; spread between the MFMAs
  // they overlap.
  // Only the first NTB token blocks are multiplied (the others hold padding
  // rows only); the copies are spread over the MFMAs that remain.
  template <bool COH, int NTB, bool COPY = true>
  __device__ __forceinline__ void compute(const char* stage, int wf, int wt, size_t off, uint32_t slot) {
    constexpr int KS = C::BK / 16;
    constexpr int NMF = C::FB * NTB;     // MFMAs per k-step
    constexpr int NL = C::FB + NTB;      // fragment reads per k-step
    static_assert(NTB >= 1 && NTB <= C::TB, "active token blocks");
    bf16x8 af[2][C::FB], bf[2][C::TB];
#pragma unroll
    for (int q = 0; q < NL; ++q) load_frag(stage, 0, q, wf, wt, af[0], bf[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        const int fb = m / NTB, tb = m % NTB;
        acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][fb], bf[cur][tb], acc[fb][tb], 0, 0, 0);
        if (ks + 1 < KS) {
#pragma unroll
          for (int q = 0; q < NL; ++q)
            if ((q < NMF ? q : NMF - 1) == m) load_frag(stage, ks + 1, q, wf, wt, af[cur ^ 1], bf[cur ^ 1]);
        }
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
          if (COPY && C::issue_slot(i, KS * NMF) == ks * NMF + m) issue_one<COH>(C::copy_of(i), off, slot);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Full K loop over nk stages of BK through an NS-stage LDS ring. Stage kt
  // is awaited (own copies, then one workgroup barrier, after which every
  // wavefront is also done with stage kt-1), then multiplied while the copy of
  // stage kt+NS-1 goes into the slot stage kt-1 used. The last NS-1 stages
  // have no later stage to copy and run a stage body without copies (chosen
  // outside the unrolled MFMA sequence, which no branch splits), so the
  // epilogue starts without waiting on a copy nobody reads. With fewer stages
  // than the ring holds, the prologue repeats the last stage into the spare
  // slots; those copies are older than the last stage's wait, which awaits
  // them all. acc starts at zero; token blocks NTB and up stay zero.
  // after_prologue runs once the prologue's copies are issued.
  template <bool COH, int NTB = C::TB, class Hook>
  __device__ __forceinline__ void mainloop(char* lds, int nk, int wf, int wt, Hook&& after_prologue) {
#pragma unroll
    for (int fb = 0; fb < C::FB; ++fb)
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) acc[fb][tb] = f32x16{};
    lds_barrier();   // every wavefront is done with the LDS of the previous tile
#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s) {
      const size_t off = (size_t)min(s, nk - 1) * C::ROW_BYTES;
#pragma unroll
      for (int i = 0; i < C::NI; ++i) issue_one<COH>(i, off, ring + s * C::STAGE_BYTES);
    }
    after_prologue();
    int slot = 0;
    const int nmain = nk - (C::NS - 1);   // stages that copy a later stage
    for (int kt = 0; kt < nmain; ++kt) {
      vm_wait<C::NI * (C::NS - 2)>();   // stage kt has landed (later stages may not have)
      lds_barrier();
      const int nslot = slot == 0 ? C::NS - 1 : slot - 1;
      compute<COH, NTB>(lds + slot * C::STAGE_BYTES, wf, wt, (size_t)(kt + C::NS - 1) * C::ROW_BYTES,
                        ring + nslot * C::STAGE_BYTES);
      slot = slot + 1 == C::NS ? 0 : slot + 1;
    }
    for (int kt = max(nmain, 0); kt < nk; ++kt) {
      vm_wait_ahead<C::NI, C::NS - 2>(nk - 1 - kt);   // copies of the later stages may be in flight
      lds_barrier();
      compute<COH, NTB, false>(lds + slot * C::STAGE_BYTES, wf, wt, 0, 0);
      slot = slot + 1 == C::NS ? 0 : slot + 1;
    }
  }
};

// token blocks multiplied for an M-block whose last token block is padding
template <class C>
constexpr int short_tb() { return C::WT == 1 && C::TB > 1 ? C::TB - 1 : C::TB; }

template <class C>
__global__ void __launch_bounds__(C::THREADS, 1) moe_ffn_bf16(const FfnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
  __shared__ Meta meta;
  // combine row destinations of the current Linear-2 task: past the staged
  // tile in the ring when there is room, else an array of their own
  constexpr bool kRowDstInRing = C::TM * C::TN * 2 + C::TM * (int)sizeof(char*) <= C::LDS_BYTES;
  __shared__ char* rowdst_s[kRowDstInRing ? 1 : C::TM];
  char** const rowdst = kRowDstInRing ? reinterpret_cast<char**>(lds + C::TM * C::TN * 2) : rowdst_s;
  __shared__ int pair_s[C::TM];
  __shared__ float wgt_s[C::TM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wf = wave % C::WF;
  const int wt = wave / C::WF;
  const int L = a.L, H = a.H, I = a.I, K = a.k, T = a.T;
  if (!MOE_H_COHERENT) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  for (int i = tid; i <= L; i += C::THREADS) meta.tile_off[i] = a.tile_offset[i];
  for (int i = tid; i < a.S; i += C::THREADS) {
    meta.x[i] = static_cast<const char*>(a.x[i]);
    meta.comb[i] = static_cast<char*>(a.comb[i]);
  }
  __syncthreads();
  if (tid == 0 && a.schedule == MOE_SCHED_EXPERT_WAVE)
    meta.nwaves = build_waves(meta.tile_off, L, a.N1, a.grid, a.experts_per_wave, meta.wave_exp);
  __syncthreads();
  const int P = uni(meta.tile_off[L]);
  // logical instance id: workgroups are dispatched round-robin over the 8
  // XCDs, so consecutive logical ids are placed on the same XCD (and share
  // its L2) when the grid is a multiple of 8
  const int G = a.grid;
  const int g = logical_instance(G, a.xcd_group, a.xcd_bx);

  InterleavedStream ist;
  ExpertWaveStream ews;
  const bool interleaved = a.schedule == MOE_SCHED_INTERLEAVED;
  if (interleaved) ist.init(g, G, P, a.N1, a.N2, a.lead_d);
  else ews.init(g, G, a.N1, a.N2, meta.tile_off, meta.wave_exp, uni(meta.nwaves));

  Tile<C> tile;
  tile.ring = (uint32_t)(uintptr_t)lds;
  // A Linear-1 task's row counter is published during the next task: after
  // a Linear-1 task's prologue copies are issued (the wait for the h stores
  // then overlaps their latency), before a Linear-2 task's dependency wait
  // (which may be on that very row), or after the last task. Publishing
  // waits for every wavefront's h stores to complete, then increments the
  // counter (row p_pub; seq_pub numbers that task's record).
  int p_pub = -1, seq_pub = 0;
  auto publish = [&]() {
    if (p_pub >= 0) {
      vm_wait<0>();
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(a.l2_full + p_pub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.trace && seq_pub < a.trace_cap && tid == 0)
        a.trace[((size_t)g * a.trace_cap + seq_pub) * kTraceWords + 8] = (uint32_t)wall_clock64();
      p_pub = -1;
    }
  };
  int seq = 0;
  for (;;) {
    const Task t = interleaved ? ist.next() : ews.next();
    if (t.kind == 0) break;
    const int p = uni(t.p), n = uni(t.n);
    // task record (thread 0 only): kind | n << 2, p, then wall-clock stamps
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
      publish();
      // ---- wait until every Linear-1 tile of row p has published h ----
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
      // h is read with device-scope (sc1) copies, which never hit a stale
      // line of this XCD's L2, so no L2 invalidate is needed here
      fetch_rows<C>(a.row_pair + r_base, a.row_weight + r_base, m * C::TM, Me, pair_s, wgt_s, wave, lane);
    }
    if (rec) rec[3] = (uint32_t)wall_clock64();

    // ---- operands of the task: one mainloop serves both GEMMs ----
    const int j0 = n * (C::TN / 2);   // Linear-1: first intermediate column
    if (l1) {
      // gate/up rows of W1[e] (32-row blocks alternate gate and up rows) and
      // the gathered token rows of x; padding rows repeat the last routed row
      const char* w1e = static_cast<const char*>(a.w1) + (size_t)e * 2 * I * H * 2;
      tile.setup(
          [&](int q) {
            const int blk = q >> 5;
            const int wrow = ((blk & 1) ? I : 0) + j0 + (blk >> 1) * 32 + (q & 31);
            return w1e + (size_t)wrow * H * 2;
          },
          [&](int q) { return a.row_pair[r_base + min(m * C::TM + q, Me - 1)]; },
          [&](int f) {
            const int tok = f / K;
            const int s = tok / T;
            return meta.x[s] + (size_t)(tok - s * T) * H * 2;
          });
    } else {
      // rows of W2[e] and the block's rows of h
      const char* w2e = static_cast<const char*>(a.w2) + (size_t)e * H * I * 2;
      const char* hb = static_cast<const char*>(a.h);
      tile.setup([&](int q) { return w2e + (size_t)(n * C::TN + q) * I * 2; }, [](int q) { return q; },
                 [&](int q) { return hb + ((size_t)p * C::TM + q) * I * 2; });
    }
    const int nk = (l1 ? H : I) / C::BK;
    // With one wavefront along the tokens, an M-block whose last 32-token
    // block holds only padding rows skips that block's MFMAs (an expert of
    // 101-128 rows in a 160-row block).
    const bool short_blk = C::WT == 1 && C::TB > 1 && Me - m * C::TM <= C::TM - 32;
    if (short_blk) {
      if (l1 || !MOE_H_COHERENT) tile.template mainloop<false, short_tb<C>()>(lds, nk, wf, wt, publish);
      else tile.template mainloop<true, short_tb<C>()>(lds, nk, wf, wt, publish);
    } else {
      if (l1 || !MOE_H_COHERENT) tile.template mainloop<false>(lds, nk, wf, wt, publish);
      else tile.template mainloop<true>(lds, nk, wf, wt, publish);
    }
    if (rec) {
      rec[4] = (uint32_t)wall_clock64();
      rec[7] = (uint32_t)__builtin_readcyclecounter();
    }

    // Epilogues stage the output tile in LDS (the ring is free once every
    // wavefront is past its last stage) and write whole rows: 16-byte stores,
    // a row's bytes contiguous, instead of 8-byte pieces scattered over 32 rows.
    lds_barrier();
    const int tid_e = opaque(tid), lane_e = tid_e & 63;
    if (l1) {
      // SwiGLU: h[p*TM + token][j0 .. j0 + TN/2) in bf16
      constexpr int HROW = C::TN;   // TN/2 columns x 2 bytes
      static_assert(C::TM * HROW <= C::LDS_BYTES, "h staging fits");
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) {
        const int tok_l = wt * C::TT + tb * 32 + (lane_e & 31);
#pragma unroll
        for (int fp = 0; fp < C::FB / 2; ++fp) {
          const int col0 = (wf * (C::FB / 2) + fp) * 32 + (lane_e >> 5) * 4;
          // one gate/up block pair at a time (accumulators held in AGPRs are
          // then read out block by block instead of all at once)
          f32x16 gate = tile.acc[2 * fp][tb], up = tile.acc[2 * fp + 1][tb];
          asm volatile("" : "+v"(gate), "+v"(up));
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = silu(gate[g4 * 4 + i]) * up[g4 * 4 + i];
            const uint64_t v = (uint64_t)pack_bf16x2(hv[0], hv[1]) |
                               ((uint64_t)pack_bf16x2(hv[2], hv[3]) << 32);
            *reinterpret_cast<uint64_t*>(lds + stage_off<HROW>(tok_l, (col0 + g4 * 8) * 2)) = v;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
      char* hb = static_cast<char*>(a.h) + ((size_t)p * C::TM * I + j0) * 2;
      constexpr int NCH = HROW / 16;
      for (int idx = tid_e; idx < C::TM * NCH; idx += C::THREADS) {
        const int row = idx / NCH, c = idx - row * NCH;
        const i32x4 v = *reinterpret_cast<const i32x4*>(lds + stage_off<HROW>(row, c * 16));
        // device scope: written through this XCD's L2 for the consuming XCD
        store16<kCoherent>(hb + (size_t)row * I * 2 + c * 16, v);
      }
      // published during the next task (or after the last one)
      p_pub = p;
      seq_pub = seq - 1;
      if (rec) rec[5] = (uint32_t)wall_clock64();
    } else {
      // weighted combine rows: bf16(w * acc), features n*TN .. n*TN + TN.
      // Destinations first (one row per thread, independent loads that
      // overlap the staging), so the store loop below waits on no load.
      constexpr int CROW = C::TN * 2;
      static_assert(C::TM * CROW <= C::LDS_BYTES, "combine staging fits");
      const int rows = min(C::TM, Me - m * C::TM);   // padding rows are never stored
      for (int row = tid_e; row < rows; row += C::THREADS) {
        const int f = pair_s[row];
        const int tok = f / K;
        const int j = f - tok * K;
        const int s = tok / T;
        rowdst[row] = meta.comb[s] + (((size_t)(tok - s * T) * K + j) * H + (size_t)n * C::TN) * 2;
      }
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) {
        const int tok_l = wt * C::TT + tb * 32 + (lane_e & 31);
        const float w = wgt_s[tok_l];
#pragma unroll
        for (int fb = 0; fb < C::FB; ++fb) {
          const int col0 = wf * C::FT + fb * 32 + (lane_e >> 5) * 4;
          // one block at a time (see the Linear-1 epilogue)
          f32x16 v = tile.acc[fb][tb];
          asm volatile("" : "+v"(v));
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const uint64_t o = (uint64_t)pack_bf16x2(w * v[g4 * 4 + 0], w * v[g4 * 4 + 1]) |
                               ((uint64_t)pack_bf16x2(w * v[g4 * 4 + 2], w * v[g4 * 4 + 3]) << 32);
            *reinterpret_cast<uint64_t*>(lds + stage_off<CROW>(tok_l, (col0 + g4 * 8) * 2)) = o;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
      constexpr int NCH = CROW / 16;
      for (int idx = tid_e; idx < rows * NCH; idx += C::THREADS) {
        const int row = idx / NCH, c = idx - row * NCH;
        char* dst = rowdst[row];
        const i32x4 v = *reinterpret_cast<const i32x4*>(lds + stage_off<CROW>(row, c * 16));
        if (MOE_COMBINE_NT) store16<kStream>(dst + c * 16, v);   // not re-read by this kernel
        else store16<kCacheNormal>(dst + c * 16, v);
      }
      trace_store_span(tracing, rec);
    }
  }

  publish();
  // ---- completion: the last workgroup to finish clears the counters ----
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

// Tile configurations (ids are part of the plan, stable within a build).
// Cfg<tokens, features, token waves, feature waves, BK, ring stages>
using CfgLarge = Cfg<256, 256, 2, 2, 32, 4>;   // 128x128 per wavefront: prefill-sized experts
using CfgMid = Cfg<192, 256, 2, 2, 32, 5>;     // 128x96: ~100-190 rows per expert, weights read once
using CfgSmall = Cfg<32, 128, 1, 2, 64, 3>;    // 64x32: decode-sized experts
using CfgTiny = Cfg<32, 64, 1, 1, 64, 4>;      // one wavefront, 64x32: twice the decode tasks
using CfgMid64 = Cfg<160, 256, 1, 4, 64, 3, 6, true>;   // 64x160, 128-byte rows per stage
using CfgLarge64 = Cfg<256, 256, 2, 2, 64, 2>;   // 128x128, 128-byte rows, two stages
using CfgLarge64w8 = Cfg<256, 256, 2, 4, 64, 2, 2>; // 64x128 per wavefront, eight wavefronts
using CfgLarge32w8 = Cfg<256, 256, 2, 4, 32, 4>; // as 7 with 64-byte rows and four stages
using CfgLarge32w8s3 = Cfg<256, 256, 2, 4, 32, 3>;

template <class C>
hipError_t launch(const FfnArgs& a, hipStream_t s) {
  moe_ffn_bf16<C><<<a.grid, C::THREADS, 0, s>>>(a);
  return hipGetLastError();
}

template <class C>
hipError_t occupancy(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, moe_ffn_bf16<C>, C::THREADS, 0);
}

}  // namespace

extern const TileInfo kBf16Tiles[];
extern const int kNumBf16Tiles;
const TileInfo kBf16Tiles[] = {
    {1, MOE_BF16, CfgLarge::TM, CfgLarge::TN, CfgLarge::THREADS},
    {2, MOE_BF16, CfgMid::TM, CfgMid::TN, CfgMid::THREADS},
    {3, MOE_BF16, CfgSmall::TM, CfgSmall::TN, CfgSmall::THREADS},
    {4, MOE_BF16, CfgTiny::TM, CfgTiny::TN, CfgTiny::THREADS},
    {5, MOE_BF16, CfgMid64::TM, CfgMid64::TN, CfgMid64::THREADS},
    {6, MOE_BF16, CfgLarge64::TM, CfgLarge64::TN, CfgLarge64::THREADS},
    {7, MOE_BF16, CfgLarge64w8::TM, CfgLarge64w8::TN, CfgLarge64w8::THREADS},
    {8, MOE_BF16, CfgLarge32w8::TM, CfgLarge32w8::TN, CfgLarge32w8::THREADS},
    {9, MOE_BF16, CfgLarge32w8s3::TM, CfgLarge32w8s3::TN, CfgLarge32w8s3::THREADS},
};
const int kNumBf16Tiles = sizeof(kBf16Tiles) / sizeof(kBf16Tiles[0]);

hipError_t launch_ffn_bf16(int id, const FfnArgs& a, hipStream_t s) {
  switch (id) {
    case 1: return launch<CfgLarge>(a, s);
    case 2: return launch<CfgMid>(a, s);
    case 3: return launch<CfgSmall>(a, s);
    case 4: return launch<CfgTiny>(a, s);
    case 5: return launch<CfgMid64>(a, s);
    case 6: return launch<CfgLarge64>(a, s);
    case 7: return launch<CfgLarge64w8>(a, s);
    case 8: return launch<CfgLarge32w8>(a, s);
    case 9: return launch<CfgLarge32w8s3>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t occupancy_ffn_bf16(int id, int* n) {
  switch (id) {
    case 1: return occupancy<CfgLarge>(n);
    case 2: return occupancy<CfgMid>(n);
    case 3: return occupancy<CfgSmall>(n);
    case 4: return occupancy<CfgTiny>(n);
    case 5: return occupancy<CfgMid64>(n);
    case 6: return occupancy<CfgLarge64>(n);
    case 7: return occupancy<CfgLarge64w8>(n);
    case 8: return occupancy<CfgLarge32w8>(n);
    case 9: return occupancy<CfgLarge32w8s3>(n);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
