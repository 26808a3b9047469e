// Persistent fused MoE expert FFN for gfx950 with e4m3 (OCP fp8) operands and
// fp32 block scales: x with one scale per 1x128 block, W1/W2 with one scale
// per 128x128 block (the fp8 workload of the X-Stage paper's MegaMoE
// evaluation, section 5.1, ran W8A8). Same task structure and schedules as
// the bf16 kernel (ffn_bf16.hip); what differs:
//
//  - MFMA v_mfma_scale_f32_32x32x64_f8f6f4 with unit (2^0) MX scales: the
//    fp32 block scales are not powers of two, so they cannot ride in the MFMA.
//    Each stage covers exactly one 128-wide K block: its two MFMAs accumulate
//    into a partial tile, which the VALU then adds into the fp32 accumulator
//    times (token scale x weight scale) of that block.
//  - Token scales of the stage are copied into LDS next to the operands by
//    four-byte direct-to-LDS copies; the weight scales of the task (two
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

template <int TM_, int TN_, int WT_, int WF_, int NS_>
struct Cfg8 {
  static constexpr int TM = TM_, TN = TN_, WT = WT_, WF = WF_, NS = NS_;
  static constexpr int NW = WT * WF;
  static constexpr int THREADS = 64 * NW;
  static constexpr int TT = TM / WT, FT = TN / WF;
  static constexpr int TB = TT / 32, FB = FT / 32;
  static constexpr int ROW_BYTES = 128;                 // one 128-element K block of e4m3
  static constexpr int CPR = 8, RPI = 8;
  static constexpr int NID = (TN + TM) / RPI / NW;      // operand copies per wavefront per stage
  static constexpr int NIW = TN / RPI / NW;             // of which weight rows (the first NIW)
  static constexpr int NI = NID + 1;                    // plus one token-scale copy
  static constexpr int A_BYTES = TN * ROW_BYTES;
  // token scales: wavefront w copies the scales of rows (64w + lane) mod TM
  // into its own 256-byte slot, so row q's scale sits at word q
  static constexpr int SCALE_OFF = (TN + TM) * ROW_BYTES;
  static constexpr int STAGE_BYTES = SCALE_OFF + NW * 256;
  static constexpr int NM = 2 * FB * TB;                // MFMAs per wavefront per stage
  // MFMA of the first step after which the second step's fragments are read
  static constexpr int FRAG1_AFTER = NW >= 8 ? FB * TB - 1 : 0;
  // copy i of a stage is issued after MFMA issue_slot(i) of the stage before
  static constexpr int issue_slot(int i) { return i * NM * MOE_ISSUE_SPREAD / (NI * 8); }
  static_assert(TN == 256, "an N-tile must own exactly one 128-column h-scale block");
  static_assert(TM % 64 == 0 && TM <= 64 * NW, "token-scale copies cover the M-block");
  static_assert(TT % 32 == 0 && FT % 32 == 0 && FB % 2 == 0, "wavefront tile");
  static_assert(((TN + TM) / RPI) % NW == 0, "copies split evenly");
  static_assert(TN % (RPI * NW) == 0, "every wavefront copies weight rows in its first NIW instructions");
  static_assert(NS >= 2 && NI * (NS - 1) <= 63, "vmcnt range");
};

constexpr int kMaxKBlocks = 128;   // H/128 and I/128 limit

template <class C>
struct Tile8 {
  const char* src[C::NID];
  const char* ssrc;          // this lane's token-scale source for stage 0
  f32x16 acc[C::FB][C::TB];
  f32x16 part[C::FB][C::TB];   // partial tile of the current K block
  float st_prev[C::TB];        // token scales of the previous K block (lagging wavefronts)
  uint32_t ring;

  template <class WRow, class TRow, class SRow>
  __device__ __forceinline__ void setup(WRow wrow, TRow trow, SRow srow) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < C::NID; ++i) {
      const int j = wave + C::NW * i;
      const int r = j * C::RPI + lane / C::CPR;
      const int c = (lane % C::CPR) ^ ((r >> 1) & 7);   // see the bf16 kernel's swizzle
      const char* base = j * C::RPI < C::TN ? wrow(r) : trow(r - C::TN);
      src[i] = base + c * 16;
    }
    ssrc = srow((wave * 64 + lane) % C::TM);
  }

  // copy i of stage kt into the ring slot at LDS address `slot`: operand
  // rows (weights first), then the token scales
  template <bool COH>
  __device__ __forceinline__ void issue_one(int i, int kt, uint32_t slot) {
    const int wave = threadIdx.x >> 6;
    if (i < C::NID) {
      const uint32_t dst = uni(slot + (wave + C::NW * i) * 1024);
      const char* sp = src[i] + (size_t)kt * C::ROW_BYTES;
      if (i < C::NIW) dma16<MOE_WEIGHT_POLICY>(sp, dst);
      else if (COH) dma16<kCoherent>(sp, dst);
      else dma16<kCacheNormal>(sp, dst);
    } else {
      const uint32_t dst = uni(slot + C::SCALE_OFF + wave * 256);
      if (COH) dma4<kCoherent>(ssrc + kt * 4, dst);
      else dma4<kCacheNormal>(ssrc + kt * 4, dst);
    }
  }

  // fragment q (q < FB: weights, else tokens) of MFMA step mi: 32 K-elements
  // per lane from two swizzled 16-byte chunks
  __device__ __forceinline__ void load_frag(const char* stage, int mi, int q, int wf, int wt,
                                            i32x8 (&af)[C::FB], i32x8 (&bf)[C::TB]) {
    const int lane = threadIdx.x & 63;
    const int r_lane = lane & 31;
    const int swz = (r_lane >> 1) & 7;
    const int c0 = 4 * mi + 2 * (lane >> 5);
    const int o0 = (c0 ^ swz) << 4, o1 = ((c0 + 1) ^ swz) << 4;
    const char* row = q < C::FB ? stage + (wf * C::FT + q * 32 + r_lane) * C::ROW_BYTES
                                : stage + C::A_BYTES + (wt * C::TT + (q - C::FB) * 32 + r_lane) * C::ROW_BYTES;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + o0);
    const uint4 hi = *reinterpret_cast<const uint4*>(row + o1);
    const i32x8 v = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    if (q < C::FB) af[q] = v;
    else bf[q - C::FB] = v;
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
  // (the copy of a later stage spread between them, fragments of the second
  // step read during the first), and the promotion with the block's token
  // and weight scales (sw: LDS, [2][kMaxKBlocks]). `lag` wavefronts promote
  // a stage's partial at the start of the next stage instead of at its end:
  // the two wavefronts sharing a SIMD then alternate between MFMAs and VALU
  // promotion after every workgroup barrier rather than promoting together.
  template <bool COH>
  __device__ __forceinline__ void compute(const char* stage, int wf, int wt, int kt, const float* sw,
                                          bool l1, bool lag, bool issue, int kt_next, uint32_t slot) {
    constexpr int NMF = C::FB * C::TB;
    constexpr int NL = C::FB + C::TB;
    const int lane = threadIdx.x & 63;
    const int r_lane = lane & 31;
    i32x8 af[2][C::FB], bf[2][C::TB];
#pragma unroll
    for (int q = 0; q < NL; ++q) load_frag(stage, 0, q, wf, wt, af[0], bf[0]);
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
          for (int q = 0; q < NL; ++q) load_frag(stage, 1, q, wf, wt, af[1], bf[1]);
        }
        if (issue) {
#pragma unroll
          for (int i = 0; i < C::NI; ++i)
            if (C::issue_slot(i) == mi * NMF + m) issue_one<COH>(i, kt_next, slot);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // this stage's token scales; a lagging wavefront keeps them for the next
    // stage (the slot is refilled only by a copy issued during the next stage)
    const float* sx = reinterpret_cast<const float*>(stage + C::SCALE_OFF);
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

  // K loop over nk 128-wide blocks through the NS-stage ring: stage kt is
  // awaited (own copies, then one workgroup barrier), then multiplied while
  // the copy of stage kt+NS-1 goes into the slot stage kt-1 used. With eight
  // wavefronts the second half (on the same SIMDs as the first half) promotes
  // one stage late.
  template <bool COH>
  __device__ __forceinline__ void mainloop(char* lds, int nk, int wf, int wt, const float* sw, bool l1) {
#pragma unroll
    for (int fb = 0; fb < C::FB; ++fb)
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) acc[fb][tb] = f32x16{};
    const bool lag = C::NW >= 8 && (int)(threadIdx.x >> 6) >= C::NW / 2;
    lds_barrier();
#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s)
      if (s < nk) {
#pragma unroll
        for (int i = 0; i < C::NI; ++i) issue_one<COH>(i, s, ring + s * C::STAGE_BYTES);
      }
    int slot = 0;
    for (int kt = 0; kt < nk; ++kt) {
      vm_wait_ahead<C::NI, C::NS - 2>(min(C::NS - 2, nk - 1 - kt));
      lds_barrier();
      const int nxt = kt + C::NS - 1;
      const int nslot = slot == 0 ? C::NS - 1 : slot - 1;
      compute<COH>(lds + slot * C::STAGE_BYTES, wf, wt, kt, sw, l1, lag, nxt < nk, nxt,
                   ring + nslot * C::STAGE_BYTES);
      slot = slot + 1 == C::NS ? 0 : slot + 1;
    }
    if (lag && nk > 0) promote(st_prev, nk - 1, wf, sw, l1);
  }
};

__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

struct Meta8 {
  Meta m;
  const char* xs[MOE_MAX_SLICES];
  float wsc[2 * kMaxKBlocks];
};

template <class C>
__global__ void __launch_bounds__(C::THREADS, 1) moe_ffn_fp8(const FfnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[C::NS * C::STAGE_BYTES];
  __shared__ Meta8 meta8;
  __shared__ float amax_s[C::NW][C::TB][32];   // per-token h amax: [wavefront][token block][lane]
  Meta& meta = meta8.m;

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
    meta.nwaves = build_waves(meta.tile_off, L, a.N1, a.grid, a.experts_per_wave, meta.wave_row);
  __syncthreads();
  const int P = uni(meta.tile_off[L]);
  const int G = a.grid;
  const int g = logical_instance(G, a.xcd_group);

  InterleavedStream ist;
  ExpertWaveStream ews;
  const bool interleaved = a.schedule == MOE_SCHED_INTERLEAVED;
  if (interleaved) ist.init(g, G, P, a.N1, a.N2, a.lead_d);
  else ews.init(g, G, a.N1, a.N2, meta.wave_row, uni(meta.nwaves));

  Tile8<C> tile;
  tile.ring = (uint32_t)(uintptr_t)lds;
  int seq = 0;
  for (;;) {
    const Task t = interleaved ? ist.next() : ews.next();
    if (t.kind == 0) break;
    const int p = uni(t.p), n = uni(t.n);
    uint32_t* rec = (a.trace && tid == 0 && seq < a.trace_cap)
                        ? a.trace + ((size_t)g * a.trace_cap + seq) * kTraceWords
                        : nullptr;
    if (rec) {
      rec[0] = (uint32_t)t.kind | ((uint32_t)n << 2);
      rec[1] = (uint32_t)p;
      rec[2] = (uint32_t)wall_clock64();
      rec[6] = (uint32_t)__builtin_readcyclecounter();   // shader clock
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
      // SwiGLU, per-token amax over the tile's 128 h columns, e4m3 h + scale
      float hv[C::TB][C::FB / 2][16];
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) {
        float mx = 0.f;
#pragma unroll
        for (int fp = 0; fp < C::FB / 2; ++fp)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float h = silu(tile.acc[2 * fp][tb][v]) * tile.acc[2 * fp + 1][tb][v];
            hv[tb][fp][v] = h;
            mx = fmaxf(mx, fabsf(h));
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (lane < 32) amax_s[wave][tb][lane] = mx;
      }
      __syncthreads();
      char* hwb = static_cast<char*>(a.h);
      float* hsw = a.hs;
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) {
        float mx = 0.f;
#pragma unroll
        for (int f = 0; f < C::WF; ++f) mx = fmaxf(mx, amax_s[wt * C::WF + f][tb][lane & 31]);
        const float scale = mx > 0.f ? mx / 448.f : 1.f;
        const float inv = mx > 0.f ? 448.f / mx : 1.f;
        const int tok_l = wt * C::TT + tb * 32 + (lane & 31);
        const size_t hrow = (size_t)p * C::TM + tok_l;
        char* hr = hwb + hrow * I;
#pragma unroll
        for (int fp = 0; fp < C::FB / 2; ++fp) {
          const int col0 = j0 + (wf * (C::FB / 2) + fp) * 32 + (lane >> 5) * 4;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float q[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(hv[tb][fp][g4 * 4 + i] * inv, -448.f), 448.f);
            __hip_atomic_store(reinterpret_cast<uint32_t*>(hr + col0 + g4 * 8),
                               pack_e4m3x4(q[0], q[1], q[2], q[3]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        if (wf == 0 && lane < 32)
          __hip_atomic_store(hsw + hrow * IB + n, scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      vm_wait<0>();
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(a.l2_full + p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (rec) rec[5] = (uint32_t)wall_clock64();
    } else {
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) {
        const int mm = m * C::TM + wt * C::TT + tb * 32 + (lane & 31);
        if (mm < Me) {
          const int r = r_base + mm;
          const int f = a.row_pair[r];
          const float w = a.row_weight[r];
          const int tok = f / K;
          const int j = f - tok * K;
          const int s = tok / T;
          char* dst = meta.comb[s] + ((size_t)(tok - s * T) * K + j) * H * 2;
#pragma unroll
          for (int fb = 0; fb < C::FB; ++fb) {
            const int col0 = n * C::TN + wf * C::FT + fb * 32 + (lane >> 5) * 4;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x16& v = tile.acc[fb][tb];
              const uint64_t o = (uint64_t)pack_bf16x2(w * v[g4 * 4 + 0], w * v[g4 * 4 + 1]) |
                                 ((uint64_t)pack_bf16x2(w * v[g4 * 4 + 2], w * v[g4 * 4 + 3]) << 32);
              uint64_t* d = reinterpret_cast<uint64_t*>(dst + (size_t)(col0 + g4 * 8) * 2);
              if (MOE_COMBINE_NT) __builtin_nontemporal_store(o, d);
              else *d = o;
            }
          }
        }
      }
      if (rec) {
        vm_wait<0>();
        rec[5] = (uint32_t)wall_clock64();
      }
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
    {22, MOE_FP8_E4M3, Cfg8W8::TM, Cfg8W8::TN, Cfg8W8::THREADS},   // first fitting tile is the default
    {21, MOE_FP8_E4M3, Cfg8Main::TM, Cfg8Main::TN, Cfg8Main::THREADS},
};
const int kNumFp8Tiles = sizeof(kFp8Tiles) / sizeof(kFp8Tiles[0]);

hipError_t launch_ffn_fp8(int id, const FfnArgs& a, hipStream_t s) {
  switch (id) {
    case 21: return launch<Cfg8Main>(a, s);
    case 22: return launch<Cfg8W8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t occupancy_ffn_fp8(int id, int* n) {
  switch (id) {
    case 21: return occupancy<Cfg8Main>(n);
    case 22: return occupancy<Cfg8W8>(n);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
