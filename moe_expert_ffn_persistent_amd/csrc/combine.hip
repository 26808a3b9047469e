// Combine audit and source-side reduction for gfx950.
//
// After the fused kernel, each source slice holds one bf16 row per
// (token, top-k slot); the X-Stage paper's Combine then aggregates the top-k
// results of each token (section 2.2). This kernel does that aggregation for
// the slots this GPU owns (y_local[n] = sum over local j, ascending j, in
// fp32, stored as fp32 or rounded to bf16) and, optionally, audits the buffers against the 0xFFFF sentinel the
// caller filled them with: every local slot must have been written, and no
// other slot may have been touched.
//
// With a report, the status word the FFN calls wrote is copied into report[3]
// by the first workgroup (one workgroup runs even for an empty batch).
//
// One workgroup of eight wavefronts per token. Each wavefront reads the
// token's k row indices itself and ballots them into the local-slot mask, so
// no LDS or barrier precedes the data loads. Each thread owns quads of 4
// consecutive hidden elements (an 8-byte load per slot, a 16-byte store), so
// one load instruction of a wavefront covers 512 contiguous bytes of a slot
// row and one store 1 KiB of the y row; a thread's loads of all its quads of
// one slot are issued together, and before the arithmetic of the slot
// before it, so two slots' loads are in flight at a time.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQuads = 4;   // quads per thread in flight (H <= 8192 in one pass)

__global__ void __launch_bounds__(kThreads) combine_check(CheckArgs a) {
  __shared__ int s_flag[3];   // unwritten, clobbered, nonfinite slots (bit j)
  const int n = blockIdx.x;
  if (n == 0 && threadIdx.x == 0 && a.report && a.status)
    __hip_atomic_store(a.report + 3, __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (n >= a.S * a.T) return;
  const int s = n / a.T;
  const int t = n - s * a.T;
  const int lane = threadIdx.x & 63;
  const bool audit = a.report != nullptr;
  const int pr = lane < a.k ? a.pair_row[(size_t)n * a.k + lane] : -1;
  const uint32_t local_mask = (uint32_t)__ballot(lane < a.k && pr >= 0);
  // slots visited in ascending order: the local ones, or all k when auditing
  const uint32_t visit = audit ? (uint32_t)((1ull << a.k) - 1ull) : local_mask;
  uint32_t unwritten = 0, clobbered = 0, nonfinite = 0;
  const char* __restrict__ base = static_cast<const char*>(a.comb[s]) + (size_t)t * a.k * a.H * 2;
  char* __restrict__ yrow = a.y ? static_cast<char*>(a.y) + (size_t)n * a.H * (a.y_bf16 ? 2 : 4) : nullptr;
  const int nquad = a.H / 4;
  for (int q0 = 0; q0 < nquad; q0 += kQuads * kThreads) {
    float y[kQuads][4];
#pragma unroll
    for (int u = 0; u < kQuads; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) y[u][i] = 0.f;
    // the loads of the next slot go out before this slot's arithmetic, so
    // two slots' loads are in flight at a time
    uint2 v[kQuads], vn[kQuads];
    auto load_slot = [&](int j, uint2 (&dst)[kQuads]) {
#pragma unroll
      for (int u = 0; u < kQuads; ++u) {
        const int q = q0 + u * kThreads + (int)threadIdx.x;
        if (q < nquad) dst[u] = *reinterpret_cast<const uint2*>(base + ((size_t)j * a.H + q * 4) * 2);
      }
    };
    if (visit) load_slot(__builtin_ctz(visit), v);
    for (uint32_t m = visit; m; m &= m - 1) {
      const int j = __builtin_ctz(m);
      const bool local = (local_mask >> j) & 1;
      const uint32_t rest = m & (m - 1);
      if (rest) load_slot(__builtin_ctz(rest), vn);
#pragma unroll
      for (int u = 0; u < kQuads; ++u) {
        const int q = q0 + u * kThreads + (int)threadIdx.x;
        if (q >= nquad) continue;
        const uint32_t bits[4] = {v[u].x & 0xFFFFu, v[u].x >> 16, v[u].y & 0xFFFFu, v[u].y >> 16};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float f = __uint_as_float(bits[i] << 16);
          if (local) {
            y[u][i] += f;
            if (audit) {
              if (bits[i] == 0xFFFFu) unwritten |= 1u << j;
              else if (!isfinite(f)) nonfinite |= 1u << j;
            }
          } else if (bits[i] != 0xFFFFu) {
            clobbered |= 1u << j;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kQuads; ++u) v[u] = vn[u];
    }
    if (yrow) {   // streamed out: not re-read here
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int u = 0; u < kQuads; ++u) {
        const int q = q0 + u * kThreads + (int)threadIdx.x;
        if (q >= nquad) continue;
        if (a.y_bf16) {
          // the hardware conversion rounds to nearest even
          const bf16x2 lo = {(__bf16)y[u][0], (__bf16)y[u][1]}, hi = {(__bf16)y[u][2], (__bf16)y[u][3]};
          __builtin_nontemporal_store(u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)},
                                      reinterpret_cast<u32x2*>(yrow + (size_t)q * 8));
        } else {
          __builtin_nontemporal_store(f32x4{y[u][0], y[u][1], y[u][2], y[u][3]},
                                      reinterpret_cast<f32x4*>(yrow + (size_t)q * 16));
        }
      }
    }
  }
  if (audit) {
    // per-slot flags, merged over the workgroup, then counted
    if (threadIdx.x < 3) s_flag[threadIdx.x] = 0;
    __syncthreads();
    if (unwritten) atomicOr(&s_flag[0], (int)unwritten);
    if (clobbered) atomicOr(&s_flag[1], (int)clobbered);
    if (nonfinite) atomicOr(&s_flag[2], (int)nonfinite);
    __syncthreads();
    if (threadIdx.x == 0) {
      if (s_flag[0]) atomicAdd(a.report + 0, __popc(s_flag[0]));
      if (s_flag[1]) atomicAdd(a.report + 1, __popc(s_flag[1]));
      if (s_flag[2]) atomicAdd(a.report + 2, __popc(s_flag[2]));
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
  const int blocks = N > 0 ? N : (a.report && a.status ? 1 : 0);
  if (blocks > 0) combine_check<<<blocks, kThreads, 0, stream>>>(a);
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
