// Persistent fused MoE expert FFN for gfx950 with e4m3 (OCP fp8) operands and
// fp32 block scales: x with one scale per 1x128 block, W1/W2 with one scale
// per 128x128 block (the fp8 workload of the X-Stage paper's MegaMoE
// evaluation, section 5.1, ran W8A8). Same task structure and schedules as
// the bf16 kernel (ffn_bf16.hip); what differs:
//
//  - MFMA with unit (2^0) MX scales: the fp32 block scales are not powers
//    of two, so they cannot ride in the MFMA. Each stage covers exactly one
//    128-wide K block. Tile8: two v_mfma_scale_f32_32x32x64_f8f6f4 per 32x32
//    output block accumulate a partial tile, which the VALU then adds into
//    the fp32 accumulator times (token scale x weight scale) of that block.
//    Tile8W: one v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 block covers
//    the whole K block, and each block is promoted right behind the matrix
//    core, which keeps the register budget of a 192 x 256 tile within eight
//    wavefronts (fewer copy bytes per FLOP than 128 x 256).
//  - Weight rows and token rows sit in two LDS rings, and one of them may be
//    a stage deeper (three stages against two is what 160 KiB holds at
//    192 x 256). The default tile gives the tokens the third stage: a token
//    stage is copied two stages ahead of use, a weight stage one.
//  - Token scales of the stage are copied into LDS next to the token rows
//    by four-byte direct-to-LDS copies; the weight scales of the task (two
//    128-row blocks) are staged in LDS once per task.
//  - Linear-1 writes h as e4m3 with one fp32 scale per token and 128 columns
//    (amax/448, values clamped to +-448, round to nearest even): a 256-wide
//    N-tile owns exactly one such block, the amax of a token row is reduced
//    across the two feature wavefronts through LDS.
//  - Linear-2 multiplies e4m3 W2 by e4m3 h with the same promotion; its
//    epilogue is the bf16 weighted combine store.
#include <hip/hip_runtime.h>

#include "ffn_common.hpp"
#include "internal.hpp"
#include "sched.hpp"

namespace moe {
namespace {

template <int TM_, int TN_, int WT_, int WF_, int NS_, bool WIDE_ = false, int SP_ = MOE_ISSUE_SPREAD,
          int XW_ = 0>
struct Cfg8 {
  static constexpr int TM = TM_, TN = TN_, WT = WT_, WF = WF_, NS = NS_;
  // ring depths: XW = 1 gives the weights one stage more than the tokens
  // (a weight stage is copied two stages ahead of use, a token stage one),
  // XW = -1 the tokens one stage more than the weights
  static constexpr int XW = XW_;
  static constexpr int NSW = NS + (XW > 0 ? 1 : 0), NST = NS + (XW < 0 ? 1 : 0);
  static_assert(XW >= -1 && XW <= 1, "one ring at most one stage deeper");
  // WIDE: 16x16x128 MFMAs (one per output block and K block), promoted
  // block by block between them (Tile8W); else 32x32x64 MFMAs (Tile8)
  static constexpr bool WIDE = WIDE_;
  static constexpr int NW = WT * WF;
  static constexpr int THREADS = 64 * NW;
  static constexpr int TT = TM / WT, FT = TN / WF;
  static constexpr int TB = TT / 32, FB = FT / 32;
  static constexpr int ROW_BYTES = 128;                 // one 128-element K block of e4m3
  static constexpr int CPR = 8, RPI = 8;
  static constexpr int NID = (TN + TM) / RPI / NW;      // operand copies per wavefront per stage
  static constexpr int NIW = TN / RPI / NW;             // of which weight rows (the first NIW)
  static constexpr int NI = NID + 1;                    // plus one token-scale copy
  static constexpr int NTC = NI - NIW;                  // token-row and token-scale copies
  // LDS: NSW weight stages of TN rows, then NST token stages of TM rows and
  // the token scales (wavefront w copies the scales of rows (64w + lane) mod
  // TM into its own 256-byte slot, so row q's scale sits at word q)
  static constexpr int W_BYTES = TN * ROW_BYTES;
  static constexpr int SCALE_OFF = TM * ROW_BYTES;      // within a token stage
  static constexpr int T_BYTES = SCALE_OFF + NW * 256;
  static constexpr int T_RING = NSW * W_BYTES;
  static constexpr int LDS_BYTES = T_RING + NST * T_BYTES;
  static constexpr uint32_t w_off(int s) { return s * W_BYTES; }
  static constexpr uint32_t t_off(int s) { return T_RING + s * T_BYTES; }
  // copy issued o-th in a stage: the copies of the shallower ring (awaited
  // one stage later) go first, since copies complete in issue order
  static constexpr int copy_of(int o) { return XW <= 0 ? o : (o < NTC ? NIW + o : o - NTC); }
  // copies still in flight when a stage's operands have landed: those of
  // the deeper ring for the stage after next, and whole stages (NS > 2)
  static constexpr int WAIT = (XW > 0 ? NIW : XW < 0 ? NTC : 0) + NI * (NS - 2);
  // MFMAs per wavefront per stage: one 16x16x128 per 16 x 16 block (WIDE), or
  // two 32x32x64 per 32 x 32 block
  static constexpr int NM = WIDE ? (FT / 16) * (TT / 16) : 2 * FB * TB;
  // MFMA of the first step after which the second step's fragments are read
  static constexpr int FRAG1_AFTER = NW >= 8 ? FB * TB - 1 : 0;
  // copy i of a stage is issued after MFMA issue_slot(i) of the stage
  // before: spread evenly over the first SP/8 of the MFMAs
  static constexpr int SP = SP_;
  static_assert(SP >= 1 && SP <= 8, "spread in eighths of the stage");
  static constexpr int issue_slot(int i) { return i * NM * SP / (NI * 8); }
  static_assert(TN == 256, "an N-tile must own exactly one 128-column h-scale block");
  static_assert(TM % 64 == 0 && TM <= 64 * NW, "token-scale copies cover the M-block");
  static_assert(TT % 32 == 0 && FT % 32 == 0 && FB % 2 == 0, "wavefront tile");
  static_assert(((TN + TM) / RPI) % NW == 0, "copies split evenly");
  static_assert(TN % (RPI * NW) == 0, "every wavefront copies weight rows in its first NIW instructions");
  static_assert(NS >= 2 && NI * (NS + 1) <= 63, "vmcnt range");
  static_assert(W_BYTES % 1024 == 0 && T_BYTES % 1024 == 0, "1 KiB copy slots");
};

constexpr int kMaxKBlocks = 128;   // H/128 and I/128 limit

// Physical 16-byte chunk of logical chunk c in 128-byte row r of an operand
// stage: c ^ ((r >> 1) & 7) ^ ((c & 2) << 1), a bijection of the row's 8
// chunks (and its own inverse up to the row term). The fragment reads take
// rows r16 = lane mod 16 at logical chunks 2g and 2g+1 for lane group
// g = lane / 16. Measured on MI355X with rocprofv3's SQ_LDS_BANK_CONFLICT,
// a 128-bit LDS read with the row term alone conflicts two ways (half of all
// LDS cycles, 1.8x the read time), because the lanes served together are not
// 16 consecutive ones; the (c & 2) << 1 term moves the odd lane groups to the
// other half of the banks and makes both reads conflict-free.
__device__ __forceinline__ int chunk_of(int r, int c) { return c ^ ((r >> 1) & 7) ^ ((c & 2) << 1); }
// logical chunk held by physical chunk p of row r (the inverse)
__device__ __forceinline__ int logical_chunk(int r, int p) {
  const int q = p ^ ((r >> 1) & 7);
  return q ^ ((q & 2) << 1);
}

// Operand and token-scale copies, shared by both fp8 tiles.
template <class C>
struct Tile8Copies {
  const char* src[C::NID];
  const char* ssrc;          // this lane's token-scale source for stage 0
  uint32_t ring;

  template <class WRow, class TRow, class SRow>
  __device__ __forceinline__ void setup(WRow wrow, TRow trow, SRow srow) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < C::NID; ++i) {
      const int j = wave + C::NW * i;
      const int r = j * C::RPI + lane / C::CPR;
      const int c = logical_chunk(r, lane % C::CPR);   // lands at physical chunk lane % 8
      const char* base = j * C::RPI < C::TN ? wrow(r) : trow(r - C::TN);
      src[i] = base + c * 16;
    }
    ssrc = srow((wave * 64 + lane) % C::TM);
  }

  // copy i: weight rows of K block ktw into the weight slot at LDS address
  // wslot (i < NIW), token rows of K block ktt (i < NID) or their scales
  // into the token slot at tslot
  template <bool COH>
  __device__ __forceinline__ void issue_one(int i, int ktw, int ktt, uint32_t wslot, uint32_t tslot) {
    const int wave = threadIdx.x >> 6;
    if (i < C::NIW) {
      dma16<MOE_WEIGHT_POLICY>(src[i] + (size_t)ktw * C::ROW_BYTES, uni(wslot + (wave + C::NW * i) * 1024));
    } else if (i < C::NID) {
      const uint32_t dst = uni(tslot + (wave + C::NW * (i - C::NIW)) * 1024);
      const char* sp = src[i] + (size_t)ktt * C::ROW_BYTES;
      if (COH) dma16<kCoherent>(sp, dst);
      else dma16<kCacheNormal>(sp, dst);
    } else {
      const uint32_t dst = uni(tslot + C::SCALE_OFF + wave * 256);
      if (COH) dma4<kCoherent>(ssrc + ktt * 4, dst);
      else dma4<kCacheNormal>(ssrc + ktt * 4, dst);
    }
  }

  // Where the copies of the stage being computed go: the K blocks and LDS
  // slots of the token and weight stages they fill.
  struct Next {
    int ktw, ktt;
    uint32_t wslot, tslot;
  };

  // the copy issued o-th in a stage
  template <bool COH>
  __device__ __forceinline__ void issue_nth(int o, const Next& nx) {
    issue_one<COH>(C::copy_of(o), nx.ktw, nx.ktt, nx.wslot, nx.tslot);
  }

  // 32 bytes of 128-byte row r of a weight or token stage at logical 16-byte
  // chunks c, c+1 (the XOR swizzle of the copy: TN is a multiple of 16, so a
  // token row's swizzle is the same whether counted from the weight rows or
  // from its own stage)
  __device__ __forceinline__ static i32x8 frag32(const char* stage, int r, int c) {
    const char* row = stage + r * C::ROW_BYTES;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + (chunk_of(r, c) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + (chunk_of(r, c + 1) << 4));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }

  // K loop over nk 128-wide blocks through the two rings: stage kt is
  // awaited (own copies, then one workgroup barrier), then multiplied (by the
  // tile's compute) while the token rows of stage kt+NST-1 and the weight
  // rows of stage kt+NSW-1 go into the slots stage kt-1 used. The copies are
  // issued unconditionally (the last stages re-copy stage nk-1 into their
  // free slots), so no branch splits the MFMA sequence they are spread over;
  // those extra copies are awaited at the end, before the epilogue reuses LDS.
  // The prologue issues what the stages before stage 0 would have, in the
  // same order, so that one wait count holds for every stage.
  template <bool COH, class Tile>
  __device__ __forceinline__ void kloop(Tile& t, char* lds, int nk, int wf, int wt, const float* sw,
                                        bool l1) {
    lds_barrier();
#pragma unroll
    for (int v = 1 - (C::NSW > C::NST ? C::NSW : C::NST); v < 0; ++v) {
      const int st = v + C::NST - 1, sw_ = v + C::NSW - 1;
#pragma unroll
      for (int o = 0; o < C::NI; ++o) {
        const int i = C::copy_of(o);
        if (i < C::NIW ? sw_ < 0 : st < 0) continue;
        issue_one<COH>(i, min(sw_, nk - 1), min(st, nk - 1), ring + C::w_off(sw_ < 0 ? 0 : sw_),
                       ring + C::t_off(st < 0 ? 0 : st));
      }
    }
    int ws = 0, ts = 0;   // slots of stage kt
    for (int kt = 0; kt < nk; ++kt) {
      vm_wait<C::WAIT>();   // stage kt has landed (later stages may not have)
      lds_barrier();
      Next nx;
      nx.ktt = min(kt + C::NST - 1, nk - 1);
      nx.ktw = min(kt + C::NSW - 1, nk - 1);
      nx.tslot = ring + C::t_off(ts == 0 ? C::NST - 1 : ts - 1);
      nx.wslot = ring + C::w_off(ws == 0 ? C::NSW - 1 : ws - 1);
      t.template compute<COH>(lds + C::w_off(ws), lds + C::t_off(ts), wf, wt, kt, sw, l1, nx);
      ws = ws + 1 == C::NSW ? 0 : ws + 1;
      ts = ts + 1 == C::NST ? 0 : ts + 1;
    }
    vm_wait<0>();
  }
};

// 32x32x64 MFMAs: lane l of an output block holds token column l%32 and
// feature rows 8*(v/4) + 4*(l/32) + v%4.
template <class C>
struct Tile8 : Tile8Copies<C> {
  f32x16 acc[C::FB][C::TB];
  f32x16 part[C::FB][C::TB];   // partial tile of the current K block
  float st_prev[C::TB];        // token scales of the previous K block (lagging wavefronts)
  bool lag;

  // fragment q (q < FB: weights, else tokens) of MFMA step mi: 32 K-elements
  // per lane
  __device__ __forceinline__ void load_frag(const char* wst, const char* tst, int mi, int q, int wf, int wt,
                                            i32x8 (&af)[C::FB], i32x8 (&bf)[C::TB]) {
    const int lane = threadIdx.x & 63;
    const int c0 = 4 * mi + 2 * (lane >> 5);
    if (q < C::FB) af[q] = this->frag32(wst, wf * C::FT + q * 32 + (lane & 31), c0);
    else bf[q - C::FB] = this->frag32(tst, wt * C::TT + (q - C::FB) * 32 + (lane & 31), c0);
  }

  // acc += part * (token scale x weight scale of K block kb), per output block
  __device__ __forceinline__ void promote(const float (&st)[C::TB], int kb, int wf, const float* sw,
                                          bool l1) {
#pragma unroll
    for (int tb = 0; tb < C::TB; ++tb)
#pragma unroll
      for (int fb = 0; fb < C::FB; ++fb) {
        const int sel = l1 ? (fb & 1) : ((wf * C::FT + fb * 32) >> 7);
        const float s = st[tb] * sw[sel * kMaxKBlocks + kb];
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fb][tb][v] += part[fb][tb][v] * s;
      }
  }

  // One 128-wide K block: two MFMAs per output block into the partial tile
  // (the copy of a later stage spread between them), and the promotion with
  // the block's token and weight scales (sw: LDS, [2][kMaxKBlocks]). `lag`
  // wavefronts promote a stage's partial at the start of the next stage
  // instead of at its end: the two wavefronts sharing a SIMD then alternate
  // between MFMAs and VALU promotion after every workgroup barrier rather
  // than promoting together.
  template <bool COH>
  __device__ __forceinline__ void compute(const char* wst, const char* tst, int wf, int wt, int kt,
                                          const float* sw, bool l1, const typename Tile8Copies<C>::Next& nx) {
    constexpr int NMF = C::FB * C::TB;
    constexpr int NL = C::FB + C::TB;
    const int r_lane = threadIdx.x & 31;
    i32x8 af[2][C::FB], bf[2][C::TB];
#pragma unroll
    for (int q = 0; q < NL; ++q) load_frag(wst, tst, 0, q, wf, wt, af[0], bf[0]);
    if (lag && kt > 0) promote(st_prev, kt - 1, wf, sw, l1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int m = 0; m < NMF; ++m) {
        const int fb = m / C::TB, tb = m % C::TB;
        const f32x16 cin = mi == 0 ? f32x16{} : part[fb][tb];
        // formats 0/0: e4m3 x e4m3; E8M0 scales 127 = 2^0
        part[fb][tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi][fb], bf[mi][tb], cin, 0, 0, 0, 127, 0, 127);
        if (mi == 0 && m == C::FRAG1_AFTER) {
          // the second step's fragments (after the last first-step MFMA with
          // eight wavefronts, so that the two fragment sets share registers)
#pragma unroll
          for (int q = 0; q < NL; ++q) load_frag(wst, tst, 1, q, wf, wt, af[1], bf[1]);
        }
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
          if (C::issue_slot(i) == mi * NMF + m) this->template issue_nth<COH>(i, nx);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // this stage's token scales; a lagging wavefront keeps them for the next
    // stage (the slot is refilled only by a copy issued during the next stage)
    const float* sx = reinterpret_cast<const float*>(tst + C::SCALE_OFF);
    float st[C::TB];
#pragma unroll
    for (int tb = 0; tb < C::TB; ++tb) st[tb] = sx[wt * C::TT + tb * 32 + r_lane];
    if (lag) {
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) st_prev[tb] = st[tb];
    } else {
      promote(st, kt, wf, sw, l1);
    }
  }

  // With eight wavefronts the second half (on the same SIMDs as the first
  // half) promotes one stage late.
  template <bool COH>
  __device__ __forceinline__ void mainloop(char* lds, int nk, int wf, int wt, const float* sw, bool l1) {
#pragma unroll
    for (int fb = 0; fb < C::FB; ++fb)
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) acc[fb][tb] = f32x16{};
    lag = C::NW >= 8 && (int)(threadIdx.x >> 6) >= C::NW / 2;
    this->template kloop<COH>(*this, lds, nk, wf, wt, sw, l1);
    if (lag && nk > 0) promote(st_prev, nk - 1, wf, sw, l1);
  }

  // Linear-1: SwiGLU, per-token amax over the N-tile's 128 h columns
  // (within the lane, across the lane pair l, l+32, then across the feature
  // wavefronts through LDS), e4m3 h and its scale
  __device__ __forceinline__ void epi_l1(const FfnArgs& a, int p, int n, int j0, float* amax, char*) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wf = wave % C::WF, wt = wave / C::WF;
    float hv[C::TB][C::FB / 2][16];
#pragma unroll
    for (int tb = 0; tb < C::TB; ++tb) {
      float mx = 0.f;
#pragma unroll
      for (int fp = 0; fp < C::FB / 2; ++fp)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float h = silu(acc[2 * fp][tb][v]) * acc[2 * fp + 1][tb][v];
          hv[tb][fp][v] = h;
          mx = fmaxf(mx, fabsf(h));
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (lane < 32) amax[wave * C::TT + tb * 32 + lane] = mx;
    }
    __syncthreads();
    char* hwb = static_cast<char*>(a.h);
    const int IB = a.I / 128;
#pragma unroll
    for (int tb = 0; tb < C::TB; ++tb) {
      float mx = 0.f;
#pragma unroll
      for (int f = 0; f < C::WF; ++f) mx = fmaxf(mx, amax[(wt * C::WF + f) * C::TT + tb * 32 + (lane & 31)]);
      const float scale = mx > 0.f ? mx / 448.f : 1.f;
      const float inv = mx > 0.f ? 448.f / mx : 1.f;
      const size_t hrow = (size_t)p * C::TM + wt * C::TT + tb * 32 + (lane & 31);
      char* hr = hwb + hrow * a.I;
#pragma unroll
      for (int fp = 0; fp < C::FB / 2; ++fp) {
        const int col0 = j0 + (wf * (C::FB / 2) + fp) * 32 + (lane >> 5) * 4;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float h4[4] = {hv[tb][fp][g4 * 4], hv[tb][fp][g4 * 4 + 1], hv[tb][fp][g4 * 4 + 2],
                               hv[tb][fp][g4 * 4 + 3]};
          __hip_atomic_store(reinterpret_cast<uint32_t*>(hr + col0 + g4 * 8), quant4(h4, inv),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (wf == 0 && lane < 32)
        __hip_atomic_store(a.hs + hrow * IB + n, scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // Linear-2: bf16(w * acc) into the combine slot of each routed row
  __device__ __forceinline__ void epi_l2(const FfnArgs& a, int n, int m, int Me, char* const* comb, char*,
                                         const int* pair_s, const float* wgt_s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wf = wave % C::WF, wt = wave / C::WF;
#pragma unroll
    for (int tb = 0; tb < C::TB; ++tb) {
      const int row = wt * C::TT + tb * 32 + (lane & 31);
      if (m * C::TM + row < Me) {
        const int f = pair_s[row];
        const float w = wgt_s[row];
        const int tok = f / a.k;
        const int j = f - tok * a.k;
        const int s = tok / a.T;
        char* dst = comb[s] + ((size_t)(tok - s * a.T) * a.k + j) * a.H * 2;
#pragma unroll
        for (int fb = 0; fb < C::FB; ++fb) {
          const int col0 = n * C::TN + wf * C::FT + fb * 32 + (lane >> 5) * 4;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x16& v = acc[fb][tb];
            const uint64_t o = (uint64_t)pack_bf16x2(w * v[g4 * 4 + 0], w * v[g4 * 4 + 1]) |
                               ((uint64_t)pack_bf16x2(w * v[g4 * 4 + 2], w * v[g4 * 4 + 3]) << 32);
            uint64_t* d = reinterpret_cast<uint64_t*>(dst + (size_t)(col0 + g4 * 8) * 2);
            if (MOE_COMBINE_NT) __builtin_nontemporal_store(o, d);
            else *d = o;
          }
        }
      }
    }
  }
};

// 16x16x128 MFMAs (the whole K block of a stage in one instruction): lane l
// of an output block holds token column l%16 and feature rows 4*(l/16) + i.
// Each wavefront keeps its four weight fragments for the stage and streams
// its token fragments; each block's product is promoted into acc two MFMAs
// after it was issued (three partial blocks in flight), so the VALU work
// runs under the matrix core instead of after the stage. With FT = 64 the
// accumulators take 128 registers, which makes 256 x 256 tiles (half the
// copy bytes per FLOP of 128 x 256) fit eight wavefronts.
template <class C>
struct Tile8W : Tile8Copies<C> {
  static constexpr int FB16 = C::FT / 16, TB16 = C::TT / 16;
  static_assert(C::FT == 64, "gate/up pairing assumes one 32-row gate and one 32-row up block per wavefront");
  static_assert(FB16 >= 2, "a token block's scale is replaced only after two promotion steps");
  f32x4 acc[FB16][TB16];

  __device__ __forceinline__ float block_scale(const float* sw, int kt, int wf, int i, bool l1) const {
    const int row = wf * C::FT + i * 16;   // first feature row of block i in the N-tile
    const int sel = l1 ? ((row >> 5) & 1) : (row >> 7);
    return sw[sel * kMaxKBlocks + kt];
  }

  // Partial products of the last two blocks of the previous stage and their
  // scales: they are promoted during the first two MFMAs of the next stage,
  // so that a wavefront reaches the stage barrier right after issuing its
  // last MFMA instead of first waiting for the matrix core to finish it.
  static constexpr int NB = FB16 * TB16;           // output blocks = MFMAs per stage
  static constexpr int NP = NB % 3 == 0 ? 3 : 4;    // rolling partial registers
  static_assert(NB % NP == 0, "block b of every stage uses partial register b mod NP");
  f32x4 part[NP];
  float s_tail[2];

  template <bool COH>
  __device__ __forceinline__ void compute(const char* wst, const char* tst, int wf, int wt, int kt,
                                          const float* sw, bool l1, const typename Tile8Copies<C>::Next& nx) {
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, c0 = 2 * (lane >> 4);
    i32x8 af[FB16], bf[2];
    // Only the first MFMA's operands are read before it: every wavefront
    // reads LDS at once after the stage barrier, and LDS reads complete in
    // order, so the remaining weight fragments are read one per MFMA, ahead
    // of the MFMA that needs them, instead of holding up the first one.
    bf[0] = this->frag32(tst, wt * C::TT + r16, c0);
    af[0] = this->frag32(wst, wf * C::FT + r16, c0);
    const float* sx = reinterpret_cast<const float*>(tst + C::SCALE_OFF);
    float swv[FB16];
#pragma unroll
    for (int i = 0; i < FB16; ++i) swv[i] = block_scale(sw, kt, wf, i, l1);
    float stj[2];
    stj[0] = sx[wt * C::TT + r16];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = b / FB16, i = b % FB16;   // token block, feature block
      if (b + 1 < FB16) af[b + 1] = this->frag32(wst, wf * C::FT + (b + 1) * 16 + r16, c0);
      // next token block: its fragment once this block's first MFMA is out,
      // its scale once the promotions of the block before it are done
      if (i == 0 && j + 1 < TB16)
        bf[(j + 1) & 1] = this->frag32(tst, wt * C::TT + (j + 1) * 16 + r16, c0);
      if (i == FB16 / 2 && j + 1 < TB16) stj[(j + 1) & 1] = sx[wt * C::TT + (j + 1) * 16 + r16];
      // formats 0/0: e4m3 x e4m3; E8M0 scales 127 = 2^0
      part[b % NP] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j & 1], f32x4{}, 0, 0, 0, 127,
                                                                     0, 127);
      // promote block b-2: of this stage, or the tail of the previous one
      const int q = b - 2;
      if (q >= 0) {
        const int qj = q / FB16, qi = q % FB16;
        const float s = stj[qj & 1] * swv[qi];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[qi][qj][v] += part[q % NP][v] * s;
      } else if (kt > 0) {
        const int qi = FB16 + q;   // last token block, feature blocks FB16-2, FB16-1
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[qi][TB16 - 1][v] += part[(q + NP) % NP][v] * s_tail[q + 2];
      }
#pragma unroll
      for (int k = 0; k < C::NI; ++k)
        if (C::issue_slot(k) == b) this->template issue_nth<COH>(k, nx);
      __builtin_amdgcn_sched_barrier(0);
    }
    s_tail[0] = stj[(TB16 - 1) & 1] * swv[FB16 - 2];
    s_tail[1] = stj[(TB16 - 1) & 1] * swv[FB16 - 1];
  }

  template <bool COH>
  __device__ __forceinline__ void mainloop(char* lds, int nk, int wf, int wt, const float* sw, bool l1) {
#pragma unroll
    for (int i = 0; i < FB16; ++i)
#pragma unroll
      for (int j = 0; j < TB16; ++j) acc[i][j] = f32x4{};
    this->template kloop<COH>(*this, lds, nk, wf, wt, sw, l1);
    // the last stage's tail blocks
    if (nk > 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[FB16 - 2][TB16 - 1][v] += part[(NB - 2) % NP][v] * s_tail[0];
        acc[FB16 - 1][TB16 - 1][v] += part[(NB - 1) % NP][v] * s_tail[1];
      }
    }
  }

  // Linear-1: blocks 0-1 of the wavefront are gate rows, 2-3 the matching up
  // rows (32-row interleave of W1's N-tile); per-token amax over the N-tile's
  // 128 h columns: within the lane (8 values), across the four lanes of a
  // token column (l, l^16, l^32, l^48), then across the feature wavefronts.
  // The e4m3 h tile is staged in the ring (free once every wavefront is past
  // the amax exchange) and written as whole 16-byte row pieces.
  __device__ __forceinline__ void epi_l1(const FfnArgs& a, int p, int n, int j0, float* amax, char* lds) {
    const int tid = opaque(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int wf = wave % C::WF, wt = wave / C::WF;
    const int r16 = lane & 15;
    constexpr int HROW = C::TN / 2;   // the N-tile's h columns, one byte each
    static_assert(C::TM * HROW <= C::LDS_BYTES, "h staging fits the ring");
    float hv[TB16][2][4];
#pragma unroll
    for (int j = 0; j < TB16; ++j) {
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float h = silu(acc[i][j][v]) * acc[i + 2][j][v];
          hv[j][i][v] = h;
          mx = fmaxf(mx, fabsf(h));
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (lane < 16) amax[wave * C::TT + j * 16 + lane] = mx;
    }
    __syncthreads();
    const int IB = a.I / 128;
#pragma unroll
    for (int j = 0; j < TB16; ++j) {
      float mx = 0.f;
#pragma unroll
      for (int f = 0; f < C::WF; ++f) mx = fmaxf(mx, amax[(wt * C::WF + f) * C::TT + j * 16 + r16]);
      const float scale = mx > 0.f ? mx / 448.f : 1.f;
      const float inv = mx > 0.f ? 448.f / mx : 1.f;
      const int tok_l = wt * C::TT + j * 16 + r16;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        *reinterpret_cast<uint32_t*>(lds + stage_off<HROW>(tok_l, wf * 32 + i * 16 + 4 * (lane >> 4))) =
            quant4(hv[j][i], inv);
      if (wf == 0 && lane < 16)
        __hip_atomic_store(a.hs + ((size_t)p * C::TM + tok_l) * IB + n, scale, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
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
  }

  // Linear-2: bf16(w * acc) into the combine slot of each routed row. The
  // tile is staged in the ring and stored as whole 16-byte row pieces, each
  // row's destination resolved once (from the routed pairs and weights that
  // fetch_rows copied to LDS before the mainloop).
  __device__ __forceinline__ void epi_l2(const FfnArgs& a, int n, int m, int Me, char* const* comb, char* lds,
                                         const int* pair_s, const float* wgt_s) {
    const int tid = opaque(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int wf = wave % C::WF, wt = wave / C::WF;
    const int r16 = lane & 15;
    constexpr int CROW = C::TN * 2;   // bf16 combine row piece of the N-tile
    static_assert(C::TM * CROW + C::TM * (int)sizeof(char*) <= C::LDS_BYTES,
                  "combine staging and row destinations fit the ring");
    char** const rowdst = reinterpret_cast<char**>(lds + C::TM * CROW);
    const int rows = min(C::TM, Me - m * C::TM);   // padding rows are never stored
    lds_barrier();   // every wavefront is past its last stage: the ring is free
    for (int row = tid; row < rows; row += C::THREADS) {
      const int f = pair_s[row];
      const int tok = f / a.k;
      const int slot = f - tok * a.k;
      const int s = tok / a.T;
      rowdst[row] = comb[s] + (((size_t)(tok - s * a.T) * a.k + slot) * a.H + (size_t)n * C::TN) * 2;
    }
#pragma unroll
    for (int j = 0; j < TB16; ++j) {
      const int tok_l = wt * C::TT + j * 16 + r16;
      const float w = wgt_s[tok_l];
#pragma unroll
      for (int i = 0; i < FB16; ++i) {
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
      char* dst = rowdst[row];
      const i32x4 v = *reinterpret_cast<const i32x4*>(lds + stage_off<CROW>(row, c * 16));
      if (MOE_COMBINE_NT) store16<kStream>(dst + c * 16, v);   // not re-read by this kernel
      else store16<kCacheNormal>(dst + c * 16, v);
    }
  }
};

template <class C, bool WIDE = C::WIDE>
struct TileOf { using type = Tile8<C>; };
template <class C>
struct TileOf<C, true> { using type = Tile8W<C>; };

struct Meta8 {
  Meta m;
  const char* xs[MOE_MAX_SLICES];
  float wsc[2 * kMaxKBlocks];
};

template <class C>
__global__ void __launch_bounds__(C::THREADS, 1) moe_ffn_fp8(const FfnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
  __shared__ Meta8 meta8;
  __shared__ float amax_s[C::NW * C::TT];   // per-token h amax of each wavefront
  __shared__ int pair_s[C::TM];             // routed pair and router weight of each row of a
  __shared__ float wgt_s[C::TM];            // Linear-2 tile (fetch_rows)
  Meta& meta = meta8.m;
  // with L2-cached h loads: drop lines an earlier launch left in this XCD's L2
  if (!MOE_H_COHERENT) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wf = wave % C::WF;
  const int wt = wave / C::WF;
  const int L = a.L, H = a.H, I = a.I, K = a.k, T = a.T;
  const int HB = H / 128, IB = I / 128;   // scale blocks along H and I

  for (int i = tid; i <= L; i += C::THREADS) meta.tile_off[i] = a.tile_offset[i];
  for (int i = tid; i < a.S; i += C::THREADS) {
    meta.x[i] = static_cast<const char*>(a.x[i]);
    meta.comb[i] = static_cast<char*>(a.comb[i]);
    meta8.xs[i] = reinterpret_cast<const char*>(a.xs[i]);
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

  typename TileOf<C>::type tile;
  tile.ring = (uint32_t)(uintptr_t)lds;
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

    // weight scales of the task's two 128-row blocks, staged in LDS
    const int nk = l1 ? HB : IB;
    __syncthreads();   // the previous task's last stage no longer reads wsc
    for (int i = tid; i < 2 * nk; i += C::THREADS) {
      const int sel = i / nk, kb = i - sel * nk;
      float v;
      if (l1) v = a.w1s[((size_t)e * (2 * IB) + (sel ? IB + n : n)) * HB + kb];
      else v = a.w2s[((size_t)e * HB + 2 * n + sel) * IB + kb];
      meta8.wsc[sel * kMaxKBlocks + kb] = v;
    }
    __syncthreads();

    const int j0 = n * (C::TN / 2);
    const char* hb = static_cast<const char*>(a.h);
    const char* hsb = reinterpret_cast<const char*>(a.hs);
    if (l1) {
      const char* w1e = static_cast<const char*>(a.w1) + (size_t)e * 2 * I * H;
      auto tok_of = [&](int q) {
        const int mm = min(m * C::TM + q, Me - 1);
        return a.row_pair[r_base + mm] / K;
      };
      tile.setup(
          [&](int q) {
            const int blk = q >> 5;
            const int wrow = ((blk & 1) ? I : 0) + j0 + (blk >> 1) * 32 + (q & 31);
            return w1e + (size_t)wrow * H;
          },
          [&](int q) {
            const int tok = tok_of(q);
            const int s = tok / T;
            return meta.x[s] + (size_t)(tok - s * T) * H;
          },
          [&](int q) {
            const int tok = tok_of(q);
            const int s = tok / T;
            return meta8.xs[s] + (size_t)(tok - s * T) * HB * 4;
          });
    } else {
      const char* w2e = static_cast<const char*>(a.w2) + (size_t)e * H * I;
      tile.setup([&](int q) { return w2e + (size_t)(n * C::TN + q) * I; },
                 [&](int q) { return hb + ((size_t)p * C::TM + q) * I; },
                 [&](int q) { return hsb + ((size_t)p * C::TM + q) * IB * 4; });
    }
    if (l1 || !MOE_H_COHERENT) tile.template mainloop<false>(lds, nk, wf, wt, meta8.wsc, l1);
    else tile.template mainloop<true>(lds, nk, wf, wt, meta8.wsc, l1);
    if (rec) {
      rec[4] = (uint32_t)wall_clock64();
      rec[7] = (uint32_t)__builtin_readcyclecounter();
    }

    if (l1) {
      tile.epi_l1(a, p, n, j0, amax_s, lds);
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

// Cfg8<tokens, features, token waves, feature waves, ring stages>
using Cfg8Main = Cfg8<128, 256, 2, 2, 3>;   // 128 features x 64 tokens per wavefront
using Cfg8W8 = Cfg8<128, 256, 2, 4, 3>;     // 64 x 64 per wavefront, two wavefronts per SIMD
using Cfg8Wide = Cfg8<192, 256, 2, 4, 2, true, 2>;   // 64 features x 96 tokens per wavefront, 16x16x128
using Cfg8Wide3 = Cfg8<128, 256, 2, 4, 3, true>;  // 64 x 64 per wavefront, 16x16x128, three stages
// as Cfg8Wide with a three-stage weight ring beside the two-stage token ring
// (a weight stage is copied two stages ahead), copies spread over the whole
// stage
using Cfg8WideS = Cfg8<192, 256, 2, 4, 2, true, 8, 1>;
// as Cfg8WideS with the tokens in the deeper ring (gathered token rows come
// back later than the weights' consecutive rows), copies over six eighths
using Cfg8WideT = Cfg8<192, 256, 2, 4, 2, true, 6, -1>;

template <class C>
hipError_t launch(const FfnArgs& a, hipStream_t s) {
  moe_ffn_fp8<C><<<a.grid, C::THREADS, 0, s>>>(a);
  return hipGetLastError();
}

template <class C>
hipError_t occupancy(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, moe_ffn_fp8<C>, C::THREADS, 0);
}

}  // namespace

extern const TileInfo kFp8Tiles[];
extern const int kNumFp8Tiles;
const TileInfo kFp8Tiles[] = {
    {26, MOE_FP8_E4M3, Cfg8WideT::TM, Cfg8WideT::TN, Cfg8WideT::THREADS},   // first fitting tile is the default
    {25, MOE_FP8_E4M3, Cfg8WideS::TM, Cfg8WideS::TN, Cfg8WideS::THREADS},
    {23, MOE_FP8_E4M3, Cfg8Wide::TM, Cfg8Wide::TN, Cfg8Wide::THREADS},
    {22, MOE_FP8_E4M3, Cfg8W8::TM, Cfg8W8::TN, Cfg8W8::THREADS},
    {24, MOE_FP8_E4M3, Cfg8Wide3::TM, Cfg8Wide3::TN, Cfg8Wide3::THREADS},
    {21, MOE_FP8_E4M3, Cfg8Main::TM, Cfg8Main::TN, Cfg8Main::THREADS},
};
const int kNumFp8Tiles = sizeof(kFp8Tiles) / sizeof(kFp8Tiles[0]);

hipError_t launch_ffn_fp8(int id, const FfnArgs& a, hipStream_t s) {
  switch (id) {
    case 21: return launch<Cfg8Main>(a, s);
    case 22: return launch<Cfg8W8>(a, s);
    case 23: return launch<Cfg8Wide>(a, s);
    case 24: return launch<Cfg8Wide3>(a, s);
    case 25: return launch<Cfg8WideS>(a, s);
    case 26: return launch<Cfg8WideT>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t occupancy_ffn_fp8(int id, int* n) {
  switch (id) {
    case 21: return occupancy<Cfg8Main>(n);
    case 22: return occupancy<Cfg8W8>(n);
    case 23: return occupancy<Cfg8Wide>(n);
    case 24: return occupancy<Cfg8Wide3>(n);
    case 25: return occupancy<Cfg8WideS>(n);
    case 26: return occupancy<Cfg8WideT>(n);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
