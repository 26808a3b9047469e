// Device helpers shared by the bf16 and fp8 persistent FFN kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ffn.h"
#include "sched.hpp"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Meta {
  int tile_off[MOE_MAX_LOCAL_EXPERTS + 1];
  uint16_t wave_exp[MOE_MAX_LOCAL_EXPERTS + 2];
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

// silu(g) = g * sigmoid(g) with the hardware reciprocal (v_rcp_f32, 1 ulp)
// instead of a correctly rounded division: the division's scale/fixup
// sequence was most of the Linear-1 epilogue's VALU work, and h is rounded
// to bf16 or fp8 right after. For g -> -inf, exp(-g) overflows to inf and the
// reciprocal gives 0, as the division does.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// Cache policy of a copy: kCacheNormal (weights and x rows; measured on
// MI355X, non-temporal copies stream weights markedly slower), kStream (nt),
// kCoherent (sc1, device scope: never served from a possibly stale L2 line of
// this XCD) for h, which other XCDs produced during this launch.
enum CachePolicy { kCacheNormal = 0, kStream = 1, kCoherent = 2 };

#ifndef MOE_WEIGHT_POLICY
#define MOE_WEIGHT_POLICY kCacheNormal
#endif
#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif
#ifndef MOE_ISSUE_SPREAD
#define MOE_ISSUE_SPREAD 4   // eighths of a stage's MFMAs over which the next copy is spread
#endif
#ifndef MOE_H_COHERENT
#define MOE_H_COHERENT 1
#endif

// Logical instance id of this workgroup. Workgroups are dispatched
// round-robin over the 8 XCDs (block b runs on XCD b mod 8), each with its
// own L2. By default consecutive logical ids share an XCD, so the N-tiles of
// one row (which read the same token rows) meet in one L2.
// With N-tile grouping (xcd_group = N1/8 > 0, N1 dividing G), instance g's
// Linear-1 tiles all have N-tile g mod N1 and row slot g / N1 of each round
// of G tiles. The round's grid of G/N1 row slots x N1 N-tiles is cut into
// 8 blocks, xcd_bx blocks along the N-tiles and 8/xcd_bx along the row
// slots, one per XCD: the M-blocks that read one weight tile and the N-tiles
// that read one token block then meet in one L2, and an XCD fetches the
// sum, not the product, of its block's sides. xcd_bx = 8 gives each XCD
// N1/8 N-tiles across every row slot.
__device__ __forceinline__ int logical_instance(int G, int xcd_group, int xcd_bx) {
  const int b = (int)blockIdx.x;
  if (G % 8 != 0) return b;
  const int x = b % 8, i = b / 8;
  if (xcd_group > 0) {
    const int N1 = 8 * xcd_group;
    const int nw = N1 / xcd_bx;              // N-tiles per block
    const int rh = (G / N1) / (8 / xcd_bx);  // row slots per block
    const int r = (x / xcd_bx) * rh + i / nw;
    const int n = (x % xcd_bx) * nw + i % nw;
    return r * N1 + n;
  }
  return x * (G / 8) + i;
}

// One 1 KiB global->LDS copy for the wavefront: lane l's 16 bytes from src
// land at LDS byte address m0 + 16*l. Issued from inline assembly so the
// compiler does not serialise later LDS reads behind it; completion is
// awaited explicitly with vm_wait and published with lds_barrier.
template <int POL>
__device__ __forceinline__ void dma16(const char* src, uint32_t m0) {
  if constexpr (POL == kStream)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(m0)
                 : "memory", "m0");
  else if constexpr (POL == kCoherent)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off sc1" ::"v"(src), "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most NI*ahead of this wavefront's copies are outstanding
template <int NI, int K>
__device__ __forceinline__ void vm_wait_ahead(int ahead) {
  if constexpr (K == 0) {
    vm_wait<0>();
  } else {
    if (ahead >= K) vm_wait<NI * K>();
    else vm_wait_ahead<NI, K - 1>(ahead);
  }
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }


// 16-byte store with a cache policy (inline assembly: completion is awaited
// with vm_wait like the copies). kCoherent: device scope (sc1), written
// through this XCD's L2; kStream: non-temporal.
//
// A store of more than 8 bytes reads its data registers after it issues, so
// the next instruction must not overwrite them (one wait state on this GPU
// family). The compiler inserts that wait for its own stores but cannot see
// into inline assembly, and does reuse the data registers right away (seen
// as the loop counter landing in the first four bytes of some rows); the
// s_nop inside the statement keeps the wait.
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <int POL>
__device__ __forceinline__ void store16(void* dst, i32x4 v) {
  if constexpr (POL == kCoherent)
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
  else if constexpr (POL == kStream)
    asm volatile("global_store_dwordx4 %0, %1, off nt\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
  else
    asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
}

// Trace of an epilogue's stores (`tracing` uniform over the workgroup, `rec`
// non-null in thread 0 only): word 5 once every wavefront has issued its
// stores (the sender-visible end), word 8 once they have all completed.
__device__ __forceinline__ void trace_store_span(bool tracing, uint32_t* rec) {
  if (!tracing) return;
  __syncthreads();
  if (rec) rec[5] = (uint32_t)wall_clock64();
  vm_wait<0>();
  __syncthreads();
  if (rec) rec[8] = (uint32_t)wall_clock64();
}

// Epilogue staging in LDS: rows of ROWB bytes, 16-byte chunks XOR-swizzled
// by the row so that a column of lanes (one row each) writes distinct banks
// and a row of lanes reads whole rows back.
template <int ROWB>
__device__ __forceinline__ uint32_t stage_off(int row, int byte) {
  constexpr int NCH = ROWB / 16;
  return (uint32_t)(row * ROWB + ((((byte >> 4) ^ row) & (NCH - 1)) << 4) + (byte & 15));
}

// The value itself, opaque to the optimiser: what an epilogue derives from it
// (LDS staging addresses) is computed where it is used instead of being
// hoisted out of the task loop and held, or spilled, across the mainloop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Four-byte direct-to-LDS copy: lane l's word lands at m0 + 4*l (inactive
// lanes write nothing).
template <int POL>
__device__ __forceinline__ void dma4(const char* src, uint32_t m0) {
  if constexpr (POL == kCoherent)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off sc1" ::"v"(src), "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0)
                 : "memory", "m0");
}

// e4m3 (OCP fp8) codes of four values, round to nearest even
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// e4m3 code of clamp(h * inv, +-448) for four values, round to nearest even
__device__ __forceinline__ uint32_t quant4(const float (&h)[4], float inv) {
  float q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = fminf(fmaxf(h[i] * inv, -448.f), 448.f);
  return pack_e4m3x4(q[0], q[1], q[2], q[3]);
}

// Routed pair and router weight of each row of a Linear-2 tile, copied to
// LDS by the wavefronts before the tile's mainloop copies: older than every
// stage, they have landed by the first stage's wait, and the epilogue reads
// them from LDS instead of waiting on global loads. Padding rows repeat the
// last routed row (their combine rows are never stored).
template <class C>
__device__ __forceinline__ void fetch_rows(const int* pair, const float* wgt, int m0, int Me, int* pair_s,
                                           float* wgt_s, int wave, int lane) {
  constexpr int NQ = (C::TM + 63) / 64;
  for (int j = uni(wave); j < 2 * NQ; j += C::NW) {   // uniform over the wavefront
    const int q = j >> 1;
    const int r = q * 64 + lane;
    if (r < C::TM) {
      const int mm = min(m0 + r, Me - 1);
      if (j & 1) dma4<kCacheNormal>(reinterpret_cast<const char*>(wgt + mm), (uint32_t)(uintptr_t)(wgt_s + q * 64));
      else dma4<kCacheNormal>(reinterpret_cast<const char*>(pair + mm), (uint32_t)(uintptr_t)(pair_s + q * 64));
    }
  }
}

}  // namespace moe
