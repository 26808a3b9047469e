// Routing and dispatch layout kernels for gfx950.
//
// The fused MoE kernel of the X-Stage paper (section 2.2) starts after the
// router: Dispatch brings each token to the GPU owning its expert, and the
// grouped GEMM walks a flattened row space in which expert e owns scheduler
// rows O_e .. O_{e+1}-1 (Algorithm 1 legend). On one GPU the Dispatch stage
// becomes this layout: which (token, slot) pairs are local, how many rows
// each local expert gets, their order and their offsets. All of it is
// integer work except the router softmax, and it must be bit-exact.
//
// Kernels, all launched on the caller's stream, no host round trip:
//   route_topk16  (E <= 128, or E <= 256 with N >= 16384) one 16-lane row per token, four tokens per
//                 wavefront: k rounds of a row argmax over (z desc, index
//                 asc) by DPP row reductions of order keys, softmax over the
//                 kept z.
//   route_topk    (otherwise) the same with one wavefront per token.
//   layout_count  one wavefront per chunk of 256 flat pairs: per-expert
//                 counts of the chunk.
//   layout_scan_cols  one workgroup per local expert: the prefix scan of
//                 its chunk counts (each chunk's first row of the expert)
//                 and its count.
//   layout_place  one wavefront per chunk: the offsets over experts (row
//                 and scheduler-row offsets; the first workgroup also
//                 stores them and the totals), then stable placement
//                 (layout_offsets stores them for an empty batch). Pairs are taken
//                 64 at a time in flat order; lanes with the same expert are
//                 grouped with ballots and ranked by the popcount of the
//                 lower lanes, so rows of an expert keep ascending f.
#include <hip/hip_runtime.h>

#include <climits>

#include "internal.hpp"

namespace moe {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ bool better(float za, int ia, float zb, int ib) {
  return za > zb || (za == zb && ia < ib);
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int t = __shfl_up(v, d, kWave);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, kWave));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Order-preserving integer key of a float: keys compare like the values,
// -0 and +0 get the same key, and NaN gets a key below every number (a
// stable descending sort puts it last).
__device__ __forceinline__ int order_key(float z) {
  if (z != z) return INT_MIN + 1;
  if (z == 0.f) return 0;
  const int b = __float_as_int(z);
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}

// Wavefront maximum (kMin) or minimum of v, returned to every lane. Lane 15
// of each row gathers its row with four row shifts, row broadcasts carry
// rows 0 and 2 into rows 1 and 3 and then row 1 into rows 2 and 3, so lane 63
// ends up holding the result. Lanes whose shifted source lies outside the
// row keep the identity.
template <bool kMin>
__device__ __forceinline__ int wave_extreme(int v) {
  constexpr int id = kMin ? INT_MAX : INT_MIN;
  auto f = [](int a, int b) { return kMin ? min(a, b) : max(a, b); };
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xF, 0xF, false));   // row_shr:1
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xF, 0xF, false));   // row_shr:2
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xF, 0xF, false));   // row_shr:4
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xF, 0xF, false));   // row_shr:8
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x142, 0xA, 0xF, false));   // row_bcast:15
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// PER: logits per lane (E <= 64 * PER); instantiated for PER = 1, 2, 4, 8, 16.
// Lane l holds experts l, l+64, ... Each of the k rounds takes every lane's
// best remaining expert (largest key, then lowest index, which within a lane
// is the lowest slot), the wavefront's largest key, and, among the lanes
// holding it, the lowest expert index (a second reduction only when several
// lanes tie); the winning lane retires that expert.
template <int PER>
__global__ void __launch_bounds__(256) route_topk(LayoutArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (n >= a.N) return;
  float z[PER];
  int key[PER];
  const float* row = a.logits + (size_t)n * a.E;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + i * kWave;
    float v = -INFINITY;
    if (e < a.E) {
      v = row[e];
      if (a.bias) v = v + a.bias[e];
    }
    z[i] = v;
    key[i] = e < a.E ? order_key(v) : INT_MIN;   // below NaN: never taken while k <= E
  }
  float myz = 0.f;   // lane j < k keeps the j-th selection
  int myi = 0;
  for (int j = 0; j < a.k; ++j) {
    int hk = key[0], hs = 0;
#pragma unroll
    for (int i = 1; i < PER; ++i)
      if (key[i] > hk) {
        hk = key[i];
        hs = i;
      }
    const int best = wave_extreme<false>(hk);
    const unsigned long long tied = __ballot(hk == best);
    int e;
    if ((tied & (tied - 1)) == 0) {
      const int wl = __ffsll((long long)tied) - 1;
      e = wl + kWave * __builtin_amdgcn_readlane(hs, wl);
    } else {
      e = wave_extreme<true>(hk == best ? lane + kWave * hs : INT_MAX);
    }
    const int wl = e & (kWave - 1), ws = e / kWave;
    float wz = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i == ws) wz = z[i];
    wz = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wz), wl));
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == ws) key[i] = INT_MIN;
    }
    if (lane == j) {
      myz = wz;
      myi = e;
    }
  }
  // softmax over the kept values; the first selection is the largest
  const float zmax = __shfl(myz, 0, kWave);
  const float ex = lane < a.k ? expf(myz - zmax) : 0.f;
  float sum = ex;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, kWave);
  if (lane < a.k) {
    a.topk_idx[(size_t)n * a.k + lane] = myi;
    a.topk_w[(size_t)n * a.k + lane] = ex / sum;
  }
}

// Maximum (kMin false) or minimum of v over each 16-lane row of the
// wavefront, returned to every lane of the row: four row shifts leave the
// result in lane 15 of the row (lanes whose shifted source lies outside the
// row keep the identity), which is then read by the whole row.
template <bool kMin>
__device__ __forceinline__ int row_extreme(int v) {
  constexpr int id = kMin ? INT_MAX : INT_MIN;
  auto f = [](int a, int b) { return kMin ? min(a, b) : max(a, b); };
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xF, 0xF, false));   // row_shr:1
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xF, 0xF, false));   // row_shr:2
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xF, 0xF, false));   // row_shr:4
  v = f(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xF, 0xF, false));   // row_shr:8
  const int lane = threadIdx.x & (kWave - 1);
  return __shfl(v, (lane & ~15) | 15, kWave);
}

// As route_topk with one token per 16-lane row (four per wavefront), for
// E <= 16 * PER; PER = 4, 8, 16. Lane l of a row holds experts l, l+16, ...
// Each of the k rounds takes every lane's best remaining expert (largest
// key, then lowest index, which within a lane is the lowest slot), the row's
// largest key, and among the lanes holding it the lowest expert index; the
// winning lane retires that expert.
template <int PER>
__global__ void __launch_bounds__(256) route_topk16(LayoutArgs a) {
  constexpr int kRow = 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int rl = lane & (kRow - 1), rbase = lane & ~(kRow - 1);
  const int n = blockIdx.x * (blockDim.x / kRow) + threadIdx.x / kRow;
  if (n >= a.N) return;   // whole rows: the row count per wavefront is fixed
  float z[PER];
  int key[PER];
  const float* row = a.logits + (size_t)n * a.E;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = rl + i * kRow;
    float v = -INFINITY;
    if (e < a.E) {
      v = row[e];
      if (a.bias) v = v + a.bias[e];
    }
    z[i] = v;
    key[i] = e < a.E ? order_key(v) : INT_MIN;   // below NaN: never taken while k <= E
  }
  float myz = 0.f;   // lane j < k of the row keeps the j-th selection
  int myi = 0;
  for (int j = 0; j < a.k; ++j) {
    int hk = key[0], hs = 0;
#pragma unroll
    for (int i = 1; i < PER; ++i)
      if (key[i] > hk) {
        hk = key[i];
        hs = i;
      }
    const int best = row_extreme<false>(hk);
    const int e = row_extreme<true>(hk == best ? rl + kRow * hs : INT_MAX);
    const int wl = e & (kRow - 1), ws = e / kRow;
    float zs = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i == ws) zs = z[i];
    const float wz = __int_as_float(__shfl(__float_as_int(zs), rbase | wl, kWave));
    if (rl == wl) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == ws) key[i] = INT_MIN;
    }
    if (rl == j) {
      myz = wz;
      myi = e;
    }
  }
  // softmax over the kept values; the first selection is the largest
  const float zmax = __shfl(myz, rbase, kWave);
  const float ex = rl < a.k ? expf(myz - zmax) : 0.f;
  float sum = ex;
#pragma unroll
  for (int d = kRow / 2; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, kWave);
  if (rl < a.k) {
    a.topk_idx[(size_t)n * a.k + rl] = myi;
    a.topk_w[(size_t)n * a.k + rl] = ex / sum;
  }
}

__global__ void __launch_bounds__(kWave) layout_count(LayoutArgs a) {
  extern __shared__ int s_cnt[];   // [L]
  const int lane = threadIdx.x;
  for (int e = lane; e < a.L; e += kWave) s_cnt[e] = 0;
  __syncthreads();
  const int total = a.N * a.k;
  const int f0 = blockIdx.x * kLayoutChunk;
  const int f1 = min(total, f0 + kLayoutChunk);
  for (int f = f0 + lane; f < f1; f += kWave) {
    const int e = a.topk_idx[f] - a.e0;
    if (e >= 0 && e < a.L) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  for (int e = lane; e < a.L; e += kWave) a.block_counts[(size_t)blockIdx.x * a.L + e] = s_cnt[e];
}

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 4;   // consecutive chunks per thread per pass

// One workgroup per local expert e: the exclusive scan of column e of
// block_counts over the chunks (each chunk's first row of expert e), in
// place, and counts[e]. A thread takes kScanPer consecutive chunks (their
// loads in flight together), the workgroup scans the thread sums: wavefront
// scans, then one wavefront over the wavefront totals.
__global__ void __launch_bounds__(kScanThreads) layout_scan_cols(LayoutArgs a) {
  __shared__ int s_wsum[kScanThreads / kWave];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int carry = 0;
  for (int c0 = 0; c0 < a.nchunks; c0 += kScanThreads * kScanPer) {
    const int cb = c0 + threadIdx.x * kScanPer;
    int v[kScanPer];
#pragma unroll
    for (int u = 0; u < kScanPer; ++u)
      v[u] = cb + u < a.nchunks ? a.block_counts[(size_t)(cb + u) * a.L + e] : 0;
    int tsum = 0;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) tsum += v[u];
    const int winc = wave_inclusive_scan(tsum);
    if (lane == kWave - 1) s_wsum[wave] = winc;
    __syncthreads();
    if (wave == 0) {
      const int w = lane < kScanThreads / kWave ? s_wsum[lane] : 0;
      const int wi = wave_inclusive_scan(w);
      if (lane < kScanThreads / kWave) s_wsum[lane] = wi - w;   // exclusive over wavefronts
    }
    __syncthreads();
    int run = carry + s_wsum[wave] + winc - tsum;   // exclusive prefix of this thread's first chunk
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
      if (cb + u < a.nchunks) a.block_counts[(size_t)(cb + u) * a.L + e] = run;
      run += v[u];
    }
    // the pass total, from the last thread's inclusive sum
    const int total = __shfl(winc, kWave - 1, kWave);
    __syncthreads();
    if (wave == kScanThreads / kWave - 1 && lane == 0) s_wsum[0] = s_wsum[wave] + total;
    __syncthreads();
    carry += s_wsum[0];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.counts[e] = carry;
}

// The expert-level offsets from counts[]: one wavefront scans the experts
// (row offsets, scheduler-row offsets, the largest count, the active
// experts). Every lane < L ends with its expert's row offset in *rowoff.
// With `write`, the offsets, the totals and the end entries are stored.
__device__ __forceinline__ void expert_offsets(const LayoutArgs& a, int* s_rowoff, bool write) {
  const int lane = threadIdx.x & (kWave - 1);
  int row_carry = 0, tile_carry = 0, mx = 0, active = 0;
  for (int e0 = 0; e0 < a.L; e0 += kWave) {
    const int e = e0 + lane;
    const int cnt = e < a.L ? a.counts[e] : 0;
    const int tiles = (cnt + a.block_m - 1) / a.block_m;
    const int rinc = wave_inclusive_scan(cnt);
    const int tinc = wave_inclusive_scan(tiles);
    if (e < a.L) {
      s_rowoff[e] = row_carry + rinc - cnt;
      if (write) {
        a.row_offset[e] = row_carry + rinc - cnt;
        a.tile_offset[e] = tile_carry + tinc - tiles;
      }
    }
    row_carry += __shfl(rinc, kWave - 1, kWave);
    tile_carry += __shfl(tinc, kWave - 1, kWave);
    mx = max(mx, wave_max(cnt));
    active += wave_sum(cnt > 0 ? 1 : 0);
  }
  if (write && lane == 0) {
    a.row_offset[a.L] = row_carry;
    a.tile_offset[a.L] = tile_carry;
    a.totals[0] = row_carry;
    a.totals[1] = tile_carry;
    a.totals[2] = mx;
    a.totals[3] = active;
  }
}

// The offsets alone, for an empty batch (no chunk to place).
__global__ void __launch_bounds__(kWave) layout_offsets(LayoutArgs a) {
  extern __shared__ int s_rowoff[];   // [L]
  expert_offsets(a, s_rowoff, true);
}

__global__ void __launch_bounds__(kWave) layout_place(LayoutArgs a) {
  extern __shared__ int s_base[];   // [L] next row of each expert in this chunk
  const int lane = threadIdx.x;
  // every workgroup scans the experts itself (L values); the first one also
  // stores the offsets and totals
  expert_offsets(a, s_base, blockIdx.x == 0);
  __syncthreads();
  for (int e = lane; e < a.L; e += kWave) s_base[e] += a.block_counts[(size_t)blockIdx.x * a.L + e];
  __syncthreads();
  const int total = a.N * a.k;
  const int f0 = blockIdx.x * kLayoutChunk;
  const int f1 = min(total, f0 + kLayoutChunk);
  const unsigned long long below = (1ull << lane) - 1ull;
  constexpr int kSub = kLayoutChunk / kWave;
  int ge[kSub];     // the chunk's expert ids and weights, loaded before any placement
  float gw[kSub];
#pragma unroll
  for (int i = 0; i < kSub; ++i) {
    const int f = f0 + i * kWave + lane;
    ge[i] = f < f1 ? a.topk_idx[f] - a.e0 : -1;
    gw[i] = f < f1 ? a.topk_w[f] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kSub; ++i) {
    const int f = f0 + i * kWave + lane;
    int e = -1;
    if (f < f1) {
      const int g = ge[i];
      if (g >= 0 && g < a.L) e = g;
      else a.pair_row[f] = -1;
    }
    unsigned long long pending = __ballot(e >= 0);
    while (pending) {
      const int leader = __ffsll((long long)pending) - 1;
      const int le = __shfl(e, leader, kWave);
      const unsigned long long same = __ballot(e == le);
      const int base = s_base[le];
      if (e == le) {
        const int r = base + __popcll(same & below);
        a.row_pair[r] = f;
        a.row_weight[r] = gw[i];
        a.pair_row[f] = r;
      }
      __syncthreads();
      if (lane == 0) s_base[le] = base + __popcll(same);
      __syncthreads();
      pending &= ~same;
    }
  }
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
  if (a.logits && a.N > 0) {
    // four tokens per wavefront where it measured faster on MI355X: E <= 128
    // (20% at 8 x 8192 tokens, 128 experts), and E <= 256 with many tokens
    // (8% at 8 x 4096 tokens; 8% slower at 8 x 512, where fewer wavefronts
    // leave the routing latency-bound)
    if (a.E <= 128 || (a.E <= 256 && a.N >= 16384)) {
      const int per_block = 16;   // tokens (16-lane rows) per workgroup
      const dim3 grid((a.N + per_block - 1) / per_block), block(256);
      if (a.E <= 64) route_topk16<4><<<grid, block, 0, stream>>>(a);
      else if (a.E <= 128) route_topk16<8><<<grid, block, 0, stream>>>(a);
      else route_topk16<16><<<grid, block, 0, stream>>>(a);
    } else {
      const int per_block = 4;   // tokens (wavefronts) per workgroup
      const dim3 grid((a.N + per_block - 1) / per_block), block(per_block * kWave);
      if (a.E <= 256) route_topk<4><<<grid, block, 0, stream>>>(a);
      else if (a.E <= 512) route_topk<8><<<grid, block, 0, stream>>>(a);
      else route_topk<16><<<grid, block, 0, stream>>>(a);
    }
  }
  const size_t lds = sizeof(int) * (size_t)a.L;
  if (a.nchunks > 0) layout_count<<<a.nchunks, kWave, lds, stream>>>(a);
  layout_scan_cols<<<a.L, kScanThreads, 0, stream>>>(a);
  if (a.nchunks > 0) layout_place<<<a.nchunks, kWave, lds, stream>>>(a);
  else layout_offsets<<<1, kWave, lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
