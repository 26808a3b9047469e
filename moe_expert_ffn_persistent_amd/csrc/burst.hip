// Store burst-gap probe for gfx950: the X-Stage paper's remote-store
// microbenchmark (section 3.1) carried over to one GPU, where the combine
// stores of the Linear-2 epilogue are scattered stores to local HBM.
//
// K workgroups (producers) each issue bursts of B bytes (16-byte stores,
// 256 lanes per instruction round) into destination rows of row_bytes
// contiguous bytes, the way an epilogue writes one N-tile piece of each
// routed row, then idle for a gap G, and repeat. Around every burst the
// workgroup's thread 0 stamps the wall clock: after a barrier before the
// first store and after a barrier once every wavefront has issued its last
// store, so the difference is the sender-visible issue time T_iss, and the
// start-to-start difference of consecutive bursts is T_period (Table 1 of the
// paper). Scattered mode streams the stores with the non-temporal policy of
// the combine epilogue over the whole destination buffer; the control mode
// confines them to a 256 KiB region that stays in L2 (no HBM drain behind
// the issue), separating instruction overhead from drain backpressure.
#include <hip/hip_runtime.h>

#include "ffn_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kBurstThreads = 256;
constexpr size_t kControlBytes = 256 * 1024;

__device__ __forceinline__ uint32_t burst_row(uint32_t i, uint32_t nrows) {
  // a fixed scatter of the (producer, burst, row) index over the destination
  // rows: a 32-bit multiplicative hash mapped to [0, nrows) by the high half
  // of a 32x32 product, so the address costs a few instructions per store
  return __umulhi(i * 0x9E3779B1u, nrows);
}

template <int POLICY>
__device__ __forceinline__ void burst_stores(const BurstArgs& a, int p, int b, int tid, uint32_t nrows,
                                             i32x4 v) {
  // row_bytes is a power of two of at most 4096 and bytes_per_burst a
  // multiple of 4096: each lane keeps one 16-byte column of a row and every
  // lane makes the same number of stores
  const int cpr = a.row_bytes >> 4;
  const int rstep = kBurstThreads / cpr;
  const int rows = a.bytes_per_burst / a.row_bytes;
  const uint32_t first = ((uint32_t)p * (uint32_t)a.bursts + (uint32_t)b) * (uint32_t)rows;
  char* col = a.dst + (tid & (cpr - 1)) * 16;
  for (int r = tid / cpr; r < rows; r += rstep)
    store16<POLICY>(col + (size_t)burst_row(first + r, nrows) * a.row_bytes, v);
}

__global__ void __launch_bounds__(kBurstThreads) store_burst(BurstArgs a) {
  const int p = blockIdx.x, tid = threadIdx.x;
  const uint32_t nrows = (uint32_t)((a.control ? kControlBytes : a.dst_bytes) / a.row_bytes);
  const i32x4 v = {p, tid, 0x7f7f7f7f, 0};
  uint32_t* st = a.stamps + (size_t)p * a.bursts * 2;
  for (int b = 0; b < a.bursts; ++b) {
    __syncthreads();
    const long long t0 = wall_clock64();
    if (a.control) burst_stores<kCacheNormal>(a, p, b, tid, nrows, v);
    else burst_stores<kStream>(a, p, b, tid, nrows, v);
    __syncthreads();   // every wavefront has issued its stores
    const long long t1 = wall_clock64();
    if (tid == 0) {
      st[2 * b] = (uint32_t)t0;
      st[2 * b + 1] = (uint32_t)t1;
    }
    if (a.gap_ticks > 0)
      while (wall_clock64() - t1 < a.gap_ticks) __builtin_amdgcn_s_sleep(1);
  }
  vm_wait<0>();
}

}  // namespace

hipError_t launch_burst(const BurstArgs& a, hipStream_t stream) {
  store_burst<<<a.producers, kBurstThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
