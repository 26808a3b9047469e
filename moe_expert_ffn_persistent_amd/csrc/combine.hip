// Combine audit and source-side reduction for gfx950.
//
// After the fused kernel, each source slice holds one bf16 row per
// (token, top-k slot); the X-Stage paper's Combine then aggregates the top-k
// results of each token (section 2.2). This kernel does that aggregation for
// the slots this GPU owns (y_local[n] = sum over local j, ascending j, in
// fp32) and, optionally, audits the buffers against the 0xFFFF sentinel the
// caller filled them with: every local slot must have been written, and no
// other slot may have been touched.
//
// One workgroup per token; each thread owns chunks of 8 consecutive hidden
// elements (one 16-byte load per slot, so the reads of a slot are fully
// coalesced), up to kChunks of them at a time: a slot's loads of all of a
// thread's chunks are issued together, ahead of the arithmetic and of the
// y_local stores.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunks = 4;   // chunks per thread in flight (H <= 8192 in one pass)

__global__ void __launch_bounds__(kThreads) combine_check(CheckArgs a) {
  __shared__ int s_cnt[4];   // unwritten, clobbered, nonfinite flags; [3]: local-slot mask
  const int n = blockIdx.x;
  const int s = n / a.T;
  const int t = n - s * a.T;
  const bool audit = a.report != nullptr;
  if (threadIdx.x < 4) s_cnt[threadIdx.x] = 0;
  __syncthreads();
  if (threadIdx.x < a.k && a.pair_row[(size_t)n * a.k + threadIdx.x] >= 0)
    atomicOr(&s_cnt[3], 1 << threadIdx.x);
  __syncthreads();
  const int local_mask = s_cnt[3];
  int unwritten = 0, clobbered = 0, nonfinite = 0;
  const char* __restrict__ base = static_cast<const char*>(a.comb[s]) + (size_t)t * a.k * a.H * 2;
  float* __restrict__ yrow = a.y ? a.y + (size_t)n * a.H : nullptr;
  const int nchunk = a.H / 8;
  for (int c0 = 0; c0 < nchunk; c0 += kChunks * kThreads) {
    float y[kChunks][8];
#pragma unroll
    for (int u = 0; u < kChunks; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) y[u][i] = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const bool local = (local_mask >> j) & 1;
      if (!local && !audit) continue;
      uint4 v[kChunks];
#pragma unroll
      for (int u = 0; u < kChunks; ++u) {
        const int c = c0 + u * kThreads + (int)threadIdx.x;
        if (c < nchunk) v[u] = *reinterpret_cast<const uint4*>(base + ((size_t)j * a.H + c * 8) * 2);
      }
#pragma unroll
      for (int u = 0; u < kChunks; ++u) {
        const int c = c0 + u * kThreads + (int)threadIdx.x;
        if (c >= nchunk) continue;
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t bits = (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
          const float f = __uint_as_float(bits << 16);
          if (local) {
            y[u][i] += f;
            if (audit) {
              if (bits == 0xFFFFu) unwritten |= 1 << j;
              else if (!isfinite(f)) nonfinite |= 1 << j;
            }
          } else if (bits != 0xFFFFu) {
            clobbered |= 1 << j;
          }
        }
      }
    }
    if (yrow) {   // streamed out: not re-read here
      typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int u = 0; u < kChunks; ++u) {
        const int c = c0 + u * kThreads + (int)threadIdx.x;
        if (c >= nchunk) continue;
        f32x4* dst = reinterpret_cast<f32x4*>(yrow + c * 8);
        __builtin_nontemporal_store(f32x4{y[u][0], y[u][1], y[u][2], y[u][3]}, dst);
        __builtin_nontemporal_store(f32x4{y[u][4], y[u][5], y[u][6], y[u][7]}, dst + 1);
      }
    }
  }
  if (audit) {
    // per-slot flags (bit j), merged over the workgroup, then counted
    atomicOr(&s_cnt[0], unwritten);
    atomicOr(&s_cnt[1], clobbered);
    atomicOr(&s_cnt[2], nonfinite);
    __syncthreads();
    if (threadIdx.x == 0) {
      if (s_cnt[0]) atomicAdd(a.report + 0, __popc(s_cnt[0]));
      if (s_cnt[1]) atomicAdd(a.report + 1, __popc(s_cnt[1]));
      if (s_cnt[2]) atomicAdd(a.report + 2, __popc(s_cnt[2]));
    }
  }
}

__global__ void zero_words(uint32_t* p, size_t words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
  const int N = a.S * a.T;
  if (N > 0) combine_check<<<N, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t words = bytes / 4;
  if (words) {
    const size_t blocks = (words + 255) / 256;
    zero_words<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(static_cast<uint32_t*>(p), words);
  }
  return hipGetLastError();
}

}  // namespace moe
