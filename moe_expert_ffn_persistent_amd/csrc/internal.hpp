// Internal declarations shared by the host API and the kernel launchers of
// the persistent MoE expert-FFN library. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_ffn.h"

namespace moe {

// Arguments of the layout kernels.
struct LayoutArgs {
  int N, E, k, e0, L, block_m;
  const float* logits;     // [N, E] or nullptr
  const float* bias;       // [E] or nullptr
  int32_t* topk_idx;       // [N, k]
  float* topk_w;           // [N, k]
  int32_t* counts;         // [L]
  int32_t* row_offset;     // [L+1]
  int32_t* tile_offset;    // [L+1]
  int32_t* row_pair;       // [N*k]
  float* row_weight;       // [N*k]
  int32_t* pair_row;       // [N*k]
  int32_t* totals;         // [4]
  int32_t* block_counts;   // [nchunks, L]
  int nchunks;
};

constexpr int kLayoutChunk = 256;    // flat pairs per layout workgroup
constexpr int kTraceWords = MOE_TRACE_WORDS;   // uint32 words per task record

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);

// Store burst-gap probe (burst.hip).
struct BurstArgs {
  char* dst;                // destination buffer
  size_t dst_bytes;
  uint32_t* stamps;         // [producers][bursts][2] wall clock: issue start, issue end
  int producers;            // K workgroups
  int bytes_per_burst;      // B per producer, multiple of 4096 and of row_bytes
  int bursts;
  int row_bytes;            // contiguous bytes per destination row, multiple of 16
  int control;              // 1: rows confined to a 256 KiB region (stays in L2)
  long long gap_ticks;      // wall-clock ticks of idling after each burst
};

hipError_t launch_burst(const BurstArgs& a, hipStream_t stream);

// MFMA issue-rate probe (mfma_probe.hip)
size_t mfma_probe_operand_bytes();
int mfma_probe_threads();
hipError_t launch_mfma_probe(int format, int blocks, long long iters, const void* ops, long long* stamps,
                             float* sink, hipStream_t stream);

// Arguments of the persistent FFN kernel. Passed by value; the slice tables
// are copied to LDS at kernel start.
struct FfnArgs {
  int S, T, k, L, H, I;
  int N1, N2;              // Linear-1 / Linear-2 N-tiles per scheduler row
  int grid;                // persistent workgroups (== gridDim.x)
  int xcd_group;           // logical-id placement: 0 = consecutive ids per XCD; R > 0 = grouped by
                           // Linear-1 N-tile (N1 == 8R, N1 | grid): see logical_instance
  int xcd_bx;              // with xcd_group: XCD blocks along the N-tiles (1, 2, 4 or 8)
  int schedule;            // moe_schedule
  int lead_d;              // Interleaved lead D (>= 1)
  int experts_per_wave;    // 0 = greedy
  int debug_skip_row;      // -1 = off
  int trace_cap;
  long long timeout_ticks; // wall-clock ticks before a wait gives up
  const void* x[MOE_MAX_SLICES];
  const float* xs[MOE_MAX_SLICES];   // fp8: fp32 1x128 scales; W4A8: E8M0 bytes per 1x32
  void* comb[MOE_MAX_SLICES];
  const void* w1;
  const float* w1s;        // fp8: fp32 128x128 scales; W4A8: E8M0 bytes per 1x32
  const void* w2;
  const float* w2s;
  const int32_t* row_offset;
  const int32_t* tile_offset;
  const int32_t* row_pair;
  const float* row_weight;
  void* h;                 // [P_cap * block_m, I] intermediate activations
  float* hs;               // fp8: [P_cap * block_m, I/128] fp32 scales; W4A8:
                           // [P_cap * block_m, I/32] E8M0 bytes
  int32_t* l2_full;        // [P_cap] finished Linear-1 tiles per row
  int32_t* done;           // [1] finished workgroups
  int32_t* status;         // device status word or nullptr
  uint32_t* trace;         // task trace or nullptr
};

// Tile configurations. Each id maps to one kernel instantiation.
struct TileInfo {
  int id;
  int dtype;       // moe_dtype
  int block_m;     // tokens per M-block
  int block_n;     // features per N-tile (both GEMMs)
  int threads;
};


struct CheckArgs {
  int S, T, k, H, L;
  void* comb[MOE_MAX_SLICES];
  const int32_t* pair_row;
  void* y;
  int y_bf16;              // y is bf16 (round to nearest even) instead of fp32
  const int32_t* status;   // FFN status word or nullptr (copied to report[3])
  int32_t* report;
};
hipError_t launch_check(const CheckArgs& a, hipStream_t stream);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

// The shape checks every entry point makes (api.cpp).
bool shape_valid(const moe_shape* s);

}  // namespace moe
