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
//    16-byte chunk from LDS. LDS rows are BK*2 = 128 bytes; chunk c of row r
//    is stored at chunk c ^ (r & 7) so the eight lanes of a read phase hit
//    eight distinct bank groups.
//  - Two LDS stages: the next stage's global loads are issued before the
//    current stage's MFMAs and written to the other stage after them.
//  - Linear-1 N-tiles interleave gate and up rows in 32-row blocks, so the
//    gate and up accumulators of one output column sit in the same lane.
//  - h and l2_full cross XCDs (each XCD has its own L2): the producer
//    releases at agent scope (L2 write-back) before the counter increment,
//    the consumer acquires at agent scope (L2 invalidate) before reading h.
#include <hip/hip_runtime.h>

#include "internal.hpp"
#include "sched.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int TM_, int TN_, int WT_, int WF_>
struct Cfg {
  static constexpr int TM = TM_;          // tokens per M-block (b_m)
  static constexpr int TN = TN_;          // features per N-tile (b_n)
  static constexpr int WT = WT_;          // wavefronts along tokens
  static constexpr int WF = WF_;          // wavefronts along features
  static constexpr int BK = 64;           // K elements per stage
  static constexpr int THREADS = 64 * WT * WF;
  static constexpr int TT = TM / WT;      // tokens per wavefront
  static constexpr int FT = TN / WF;      // features per wavefront
  static constexpr int TB = TT / 32;      // 32-token MFMA blocks per wavefront
  static constexpr int FB = FT / 32;      // 32-feature MFMA blocks per wavefront
  static constexpr int ROW_BYTES = BK * 2;
  static constexpr int CPR = ROW_BYTES / 16;           // 16-byte chunks per row
  static constexpr int RPP = THREADS / CPR;            // rows per copy pass
  static constexpr int LW = TN / RPP;                  // weight rows per thread
  static constexpr int LT = TM / RPP;                  // token rows per thread
  static constexpr int A_BYTES = TN * ROW_BYTES;
  static constexpr int STAGE_BYTES = (TN + TM) * ROW_BYTES;
  static_assert(TT % 32 == 0 && FT % 32 == 0, "wavefront tile must be a multiple of 32");
  static_assert(FB % 2 == 0, "gate/up pairing needs an even number of feature blocks");
  static_assert(TN % RPP == 0 && TM % RPP == 0, "copy passes must tile the block");
};

struct Meta {
  int tile_off[MOE_MAX_LOCAL_EXPERTS + 1];
  int row_off[MOE_MAX_LOCAL_EXPERTS + 1];
  int wave_row[MOE_MAX_LOCAL_EXPERTS + 2];
  const char* x[MOE_MAX_SLICES];
  char* comb[MOE_MAX_SLICES];
  int nwaves;
  int flag;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

template <class C>
struct Tile {
  const char* pa[C::LW];   // weight row bases (bytes)
  const char* pb[C::LT];   // token row bases (bytes)
  uint4 ra[C::LW];
  uint4 rb[C::LT];
  f32x16 acc[C::FB][C::TB];

  __device__ __forceinline__ void load(int kt) {
    const int col = (threadIdx.x % C::CPR) * 16 + kt * C::ROW_BYTES;
#pragma unroll
    for (int i = 0; i < C::LW; ++i) ra[i] = *reinterpret_cast<const uint4*>(pa[i] + col);
#pragma unroll
    for (int i = 0; i < C::LT; ++i) rb[i] = *reinterpret_cast<const uint4*>(pb[i] + col);
  }

  __device__ __forceinline__ void store(char* stage) {
    const int c = threadIdx.x % C::CPR;
    const int r0 = threadIdx.x / C::CPR;
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int r = r0 + i * C::RPP;
      *reinterpret_cast<uint4*>(stage + r * C::ROW_BYTES + ((c ^ (r & 7)) << 4)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::LT; ++i) {
      const int r = r0 + i * C::RPP;
      *reinterpret_cast<uint4*>(stage + C::A_BYTES + r * C::ROW_BYTES + ((c ^ (r & 7)) << 4)) = rb[i];
    }
  }

  __device__ __forceinline__ void compute(const char* stage, int wf, int wt) {
    const int lane = threadIdx.x & 63;
    const int r_lane = lane & 31;
    const int half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      const int chunk = ((2 * ks + half) ^ (lane & 7)) << 4;
      bf16x8 af[C::FB], bf[C::TB];
#pragma unroll
      for (int fb = 0; fb < C::FB; ++fb) {
        const int r = wf * C::FT + fb * 32 + r_lane;
        af[fb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(stage + r * C::ROW_BYTES + chunk));
      }
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) {
        const int r = wt * C::TT + tb * 32 + r_lane;
        bf[tb] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(stage + C::A_BYTES + r * C::ROW_BYTES + chunk));
      }
#pragma unroll
      for (int fb = 0; fb < C::FB; ++fb)
#pragma unroll
        for (int tb = 0; tb < C::TB; ++tb)
          acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fb], bf[tb], acc[fb][tb], 0, 0, 0);
    }
  }

  // Full K loop over nk stages of BK; acc starts at zero.
  __device__ __forceinline__ void mainloop(char* lds, int nk, int wf, int wt) {
#pragma unroll
    for (int fb = 0; fb < C::FB; ++fb)
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) acc[fb][tb] = f32x16{};
    load(0);
    store(lds);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) load(kt + 1);
      compute(lds + (kt & 1) * C::STAGE_BYTES, wf, wt);
      if (kt + 1 < nk) store(lds + ((kt + 1) & 1) * C::STAGE_BYTES);
      __syncthreads();
    }
  }
};

template <class C>
__global__ void __launch_bounds__(C::THREADS, 1) moe_ffn_bf16(const FfnArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * C::STAGE_BYTES];
  __shared__ Meta meta;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wf = wave % C::WF;
  const int wt = wave / C::WF;
  const int L = a.L, H = a.H, I = a.I, K = a.k, T = a.T;

  for (int i = tid; i <= L; i += C::THREADS) {
    meta.tile_off[i] = a.tile_offset[i];
    meta.row_off[i] = a.row_offset[i];
  }
  for (int i = tid; i < a.S; i += C::THREADS) {
    meta.x[i] = static_cast<const char*>(a.x[i]);
    meta.comb[i] = static_cast<char*>(a.comb[i]);
  }
  __syncthreads();
  if (tid == 0 && a.schedule == MOE_SCHED_EXPERT_WAVE)
    meta.nwaves = build_waves(meta.tile_off, L, a.N1, a.grid, a.experts_per_wave, meta.wave_row);
  __syncthreads();
  const int P = uni(meta.tile_off[L]);

  InterleavedStream ist;
  ExpertWaveStream ews;
  const bool interleaved = a.schedule == MOE_SCHED_INTERLEAVED;
  if (interleaved) ist.init(blockIdx.x, a.grid, P, a.N1, a.N2, a.lead_d);
  else ews.init(blockIdx.x, a.grid, a.N1, a.N2, meta.wave_row, uni(meta.nwaves));

  Tile<C> tile;
  int seq = 0;
  for (;;) {
    const Task t = interleaved ? ist.next() : ews.next();
    if (t.kind == 0) break;
    const int p = uni(t.p), n = uni(t.n);
    if (a.trace && tid == 0 && seq < a.trace_cap) {
      uint32_t* rec = a.trace + ((size_t)blockIdx.x * a.trace_cap + seq) * 2;
      rec[0] = (uint32_t)t.kind | ((uint32_t)n << 2);
      rec[1] = (uint32_t)p;
    }
    ++seq;
    const int e = expert_of_row(meta.tile_off, L, p);
    const int m = p - uni(meta.tile_off[e]);
    const int r_base = uni(meta.row_off[e]);
    const int Me = uni(meta.row_off[e + 1]) - r_base;
    const int r0 = tid / C::CPR;

    if (t.kind == 1) {
      if (p == a.debug_skip_row) continue;
      // ---- Linear-1: gate/up rows of W1[e], gathered token rows of x ----
      const char* w1e = static_cast<const char*>(a.w1) + (size_t)e * 2 * I * H * 2;
      const int j0 = n * (C::TN / 2);
#pragma unroll
      for (int i = 0; i < C::LW; ++i) {
        const int q = r0 + i * C::RPP;
        const int blk = q >> 5;
        const int wrow = ((blk & 1) ? I : 0) + j0 + (blk >> 1) * 32 + (q & 31);
        tile.pa[i] = w1e + (size_t)wrow * H * 2;
      }
#pragma unroll
      for (int i = 0; i < C::LT; ++i) {
        const int q = r0 + i * C::RPP;
        const int mm = min(m * C::TM + q, Me - 1);
        const int f = a.row_pair[r_base + mm];
        const int tok = f / K;
        const int s = tok / T;
        tile.pb[i] = meta.x[s] + (size_t)(tok - s * T) * H * 2;
      }
      tile.mainloop(lds, H / C::BK, wf, wt);
      // SwiGLU epilogue: h[p*TM + token][j0 + column] in bf16
      char* hb = static_cast<char*>(a.h);
#pragma unroll
      for (int tb = 0; tb < C::TB; ++tb) {
        const int tok_l = wt * C::TT + tb * 32 + (lane & 31);
        char* hrow = hb + ((size_t)p * C::TM + tok_l) * I * 2;
#pragma unroll
        for (int fp = 0; fp < C::FB / 2; ++fp) {
          const int col0 = j0 + (wf * (C::FB / 2) + fp) * 32 + (lane >> 5) * 4;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              hv[i] = silu(tile.acc[2 * fp][tb][g4 * 4 + i]) * tile.acc[2 * fp + 1][tb][g4 * 4 + i];
            uint2 v = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            *reinterpret_cast<uint2*>(hrow + (size_t)(col0 + g4 * 8) * 2) = v;
          }
        }
      }
      // publish: h visible at agent scope, then count the tile for row p
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(a.l2_full + p, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
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
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      // ---- Linear-2: rows of W2[e], rows of h ----
      const char* w2e = static_cast<const char*>(a.w2) + (size_t)e * H * I * 2;
      const char* hb = static_cast<const char*>(a.h);
#pragma unroll
      for (int i = 0; i < C::LW; ++i) {
        const int q = r0 + i * C::RPP;
        tile.pa[i] = w2e + (size_t)(n * C::TN + q) * I * 2;
      }
#pragma unroll
      for (int i = 0; i < C::LT; ++i) {
        const int q = r0 + i * C::RPP;
        tile.pb[i] = hb + ((size_t)p * C::TM + q) * I * 2;
      }
      tile.mainloop(lds, I / C::BK, wf, wt);
      // weighted combine stores
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
              uint2 o = {pack_bf16x2(w * v[g4 * 4 + 0], w * v[g4 * 4 + 1]),
                         pack_bf16x2(w * v[g4 * 4 + 2], w * v[g4 * 4 + 3])};
              *reinterpret_cast<uint2*>(dst + (size_t)(col0 + g4 * 8) * 2) = o;
            }
          }
        }
      }
    }
  }

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
using CfgLarge = Cfg<256, 256, 2, 2>;   // 128x128 per wavefront, prefill-sized experts
using CfgMid = Cfg<128, 256, 2, 2>;     // 128 features x 64 tokens per wavefront
using CfgSmall = Cfg<32, 128, 1, 2>;    // decode-sized experts: 64 features x 32 tokens

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
const TileInfo kBf16Tiles[] = {
    {1, MOE_BF16, CfgLarge::TM, CfgLarge::TN, CfgLarge::THREADS},
    {2, MOE_BF16, CfgMid::TM, CfgMid::TN, CfgMid::THREADS},
    {3, MOE_BF16, CfgSmall::TM, CfgSmall::TN, CfgSmall::THREADS},
};

hipError_t launch_ffn_bf16(int id, const FfnArgs& a, hipStream_t s) {
  switch (id) {
    case 1: return launch<CfgLarge>(a, s);
    case 2: return launch<CfgMid>(a, s);
    case 3: return launch<CfgSmall>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t occupancy_ffn_bf16(int id, int* n) {
  switch (id) {
    case 1: return occupancy<CfgLarge>(n);
    case 2: return occupancy<CfgMid>(n);
    case 3: return occupancy<CfgSmall>(n);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
