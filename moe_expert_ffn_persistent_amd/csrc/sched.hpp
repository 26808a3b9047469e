// Tile schedules of the persistent MoE FFN kernel (device side).
//
// A task is one output tile: Linear-1 (kind 1) of scheduler row p and
// N-tile n of the gate/up outputs, or Linear-2 (kind 2) of row p and N-tile
// n of the hidden outputs. Scheduler rows are the M-blocks of all local
// experts laid end to end (the X-Stage paper's rows p; expert e owns rows
// O_e .. O_{e+1}-1, Algorithm 1 legend). Each persistent workgroup g of G
// walks its own task stream; every quantity here is uniform across the
// workgroup and is kept in scalar registers.
//
// Interleaved order (X-Stage paper, section 4.2, Algorithm 1): workgroup g
// owns the Linear-1 tiles and the Linear-2 tiles whose global index (row p
// times the N-tiles per row, plus n) is g modulo G, and runs each kind in
// ascending index. The two kinds are merged on the fly by the lead rule: the
// next own Linear-2 tile, of row p2, is due once the next own Linear-1 tile
// lies at row p2 + D or beyond, or none is left. Two cursors walk the own
// indices (start g, step G). CDNA4 has no CTA pairs, so the paper's paired
// role is dropped and n = k mod N_i.
//
// Expert-Wave order (X-Stage paper, section 2.2 and Figure 4(a)): waves of
// consecutive local experts; within a wave, the Linear-1 stream, then the
// Linear-2 stream, each walked from g with stride G. A wave closes, in
// local-expert order, once it holds at least G Linear-1 tiles, unless an
// explicit experts-per-wave count is given.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

struct Task {
  int kind;   // 0 = no more tasks, 1 = Linear-1, 2 = Linear-2
  int p;      // scheduler row
  int n;      // N-tile
};

// The streams below also run on the host, in the schedule planner's model of
// the kernel (planner.cpp), so that the model walks exactly these streams.
__host__ __device__ __forceinline__ int uni(int v) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_readfirstlane(v);
#else
  return v;
#endif
}

struct InterleavedStream {
  int k1, k2, G, P, N1, N2, D;
  __host__ __device__ void init(int g, int G_, int P_, int N1_, int N2_, int D_) {
    k1 = g; k2 = g; G = G_; P = P_; N1 = N1_; N2 = N2_; D = D_;
  }
  __host__ __device__ Task next() {
    const int t1 = P * N1, t2 = P * N2;
    if (k1 >= t1 && k2 >= t2) return Task{0, 0, 0};
    // the Linear-2 tile is due when no own Linear-1 tile is left (whatever
    // the lead: a lead near INT_MAX must not turn the comparison around and
    // hand out a Linear-1 tile past the end) or the next one is D rows ahead
    const bool l1_done = k1 >= t1;
    const int p1 = l1_done ? 0 : k1 / N1;
    const int p2 = k2 / N2;
    const bool l2_due = k2 < t2 && (l1_done || (long long)p2 + D <= (long long)p1);
    if (l2_due) {
      Task t{2, p2, k2 - p2 * N2};
      k2 += G;
      return t;
    }
    Task t{1, p1, k1 - p1 * N1};
    k1 += G;
    return t;
  }
};

// Wave boundaries live in LDS as expert indices: wave w holds the scheduler
// rows tile_off[wave_exp[w]] .. tile_off[wave_exp[w + 1]].
struct ExpertWaveStream {
  int g, G, N1, N2, w, phase, c, nwaves;
  const int* tile_off;        // LDS
  const uint16_t* wave_exp;   // LDS
  __host__ __device__ void init(int g_, int G_, int N1_, int N2_, const int* tile_off_,
                                const uint16_t* wave_exp_, int nwaves_) {
    g = g_; G = G_; N1 = N1_; N2 = N2_; tile_off = tile_off_; wave_exp = wave_exp_; nwaves = nwaves_;
    w = 0; phase = 0; c = g_;
  }
  __host__ __device__ Task next() {
    while (w < nwaves) {
      const int r0 = uni(tile_off[wave_exp[w]]);
      const int rows = uni(tile_off[wave_exp[w + 1]]) - r0;
      if (phase == 0) {
        if (c < rows * N1) {
          const int q = c / N1;
          Task t{1, r0 + q, c - q * N1};
          c += G;
          return t;
        }
        phase = 1;
        c = g;
      }
      if (c < rows * N2) {
        const int q = c / N2;
        Task t{2, r0 + q, c - q * N2};
        c += G;
        return t;
      }
      phase = 0;
      c = g;
      ++w;
    }
    return Task{0, 0, 0};
  }
};

// Greedy wave grouping over local experts, written to LDS by one thread.
// Returns the number of waves; wave_exp gets nwaves + 1 boundaries (expert
// indices, at most L <= MOE_MAX_LOCAL_EXPERTS).
__host__ __device__ inline int build_waves(const int* tile_off, int L, int N1, int G, int experts_per_wave,
                                  uint16_t* wave_exp) {
  int nw = 0;
  int start = tile_off[0];
  int n_exp = 0;
  wave_exp[0] = 0;
  for (int e = 0; e < L; ++e) {
    ++n_exp;
    const int r1 = tile_off[e + 1];
    const bool full = experts_per_wave > 0 ? (n_exp >= experts_per_wave)
                                           : ((long long)(r1 - start) * N1 >= G);
    if (full || e == L - 1) {
      if (r1 > start) wave_exp[++nw] = (uint16_t)(e + 1);
      start = r1;
      n_exp = 0;
    }
  }
  return nw;
}

// e(p): the expert whose scheduler rows hold p (tile_off[e] <= p < tile_off[e+1]).
__device__ __forceinline__ int expert_of_row(const int* tile_off, int L, int p) {
  int lo = 0, hi = L;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(tile_off[mid]) <= p) lo = mid;
    else hi = mid;
  }
  return lo;
}

}  // namespace moe
