// MFMA issue-rate probe for gfx950: the matrix cores' sustained rate when
// nothing but MFMAs runs, on every CU, under the board's power limit.
//
// The roofline fractions of the FFN kernels are taken against the dense
// MFMA figures at 2.4 GHz. Under load the power limit lowers the shader
// clock, so those figures cannot be reached; this probe measures the rate
// that can. Each workgroup runs eight wavefronts (two per SIMD, as the FFN
// kernels do); each wavefront loads sixteen operand fragments from the
// caller's buffer once, then issues back-to-back MFMAs from registers into
// four or eight independent accumulator chains, every MFMA taking a
// different pair of fragments, so consecutive MFMAs never see the same
// operands. Thread 0 of each workgroup stamps the shader clock (s_memtime)
// and the wall clock (s_memrealtime) around the loop.
#include <hip/hip_runtime.h>

#include <cstring>

#include "internal.hpp"

namespace moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kProbeThreads = 512;   // eight wavefronts
constexpr int kFrags = 16;           // 16-byte fragments per lane
constexpr int kSlots = 64;           // distinct fragment sets in the operand buffer

// format 0: v_mfma_f32_32x32x16_bf16; 1: v_mfma_scale_f32_16x16x128_f8f6f4
// (e4m3 x e4m3, unit scales); 2: v_mfma_scale_f32_32x32x64_f8f6f4
template <int FMT>
__global__ void __launch_bounds__(kProbeThreads, 1) mfma_rate(const int4* ops, long long iters,
                                                               long long* stamps, float* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int4* p = ops + (size_t)((blockIdx.x * 8 + wave) % kSlots) * 64 * kFrags + lane;
  int4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = p[i * 64];
    b[i] = p[(8 + i) * 64];
  }
  long long c0 = 0, w0 = 0;
  if (threadIdx.x == 0) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  float s = 0.f;
  if constexpr (FMT == 0) {
    bf16x8 A[8], B[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      memcpy(&A[i], &a[i], 16);
      memcpy(&B[i], &b[i], 16);
    }
    f32x16 acc[4] = {};
    for (long long it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j & 7], B[(j * 3 + (j >> 3)) & 7], acc[j & 3], 0,
                                                             0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[j][v];
  } else {
    i32x8 A[4], B[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      A[i] = i32x8{a[2 * i].x, a[2 * i].y, a[2 * i].z, a[2 * i].w,
                   a[2 * i + 1].x, a[2 * i + 1].y, a[2 * i + 1].z, a[2 * i + 1].w};
      B[i] = i32x8{b[2 * i].x, b[2 * i].y, b[2 * i].z, b[2 * i].w,
                   b[2 * i + 1].x, b[2 * i + 1].y, b[2 * i + 1].z, b[2 * i + 1].w};
    }
    if constexpr (FMT == 1) {
      f32x4 acc[8] = {};
      for (long long it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          acc[j & 7] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[j & 3], B[(j * 3 + (j >> 2)) & 3],
                                                                        acc[j & 7], 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) s += acc[j][v];
    } else {
      f32x16 acc[4] = {};
      for (long long it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          acc[j & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[j & 3], B[(j * 3 + (j >> 2)) & 3],
                                                                       acc[j & 3], 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    }
  }
  if (threadIdx.x == 0) {
    stamps[blockIdx.x * 2] = clock64() - c0;
    stamps[blockIdx.x * 2 + 1] = wall_clock64() - w0;
  }
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace

size_t mfma_probe_operand_bytes() { return (size_t)kSlots * 64 * kFrags * 16; }
int mfma_probe_threads() { return kProbeThreads; }

hipError_t launch_mfma_probe(int format, int blocks, long long iters, const void* ops, long long* stamps,
                             float* sink, hipStream_t stream) {
  const int4* o = static_cast<const int4*>(ops);
  switch (format) {
    case 0: mfma_rate<0><<<blocks, kProbeThreads, 0, stream>>>(o, iters, stamps, sink); break;
    case 1: mfma_rate<1><<<blocks, kProbeThreads, 0, stream>>>(o, iters, stamps, sink); break;
    case 2: mfma_rate<2><<<blocks, kProbeThreads, 0, stream>>>(o, iters, stamps, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
