// Host side of the C ABI declared in include/moe_ffn.h: argument checks,
// tile/grid/lead resolution, workspace carving and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <climits>
#include <mutex>

#include "internal.hpp"

#ifndef MOE_XCD_BX
// XCD blocks along the Linear-1 N-tiles when grouping by N-tile: measured on
// MI355X, 4 (each XCD takes a quarter of the N-tiles over half the row slots
// of a round) is 0.6-0.9% faster than 8 on the skewed, fp8 and W4A8 workloads
#define MOE_XCD_BX 4
#endif
#ifndef MOE_XCD_BY_NTILE
#define MOE_XCD_BY_NTILE -1   // -1: automatic, 0: never, 1: whenever the grid allows
#endif

namespace moe {

extern const TileInfo kBf16Tiles[];
extern const int kNumBf16Tiles;
hipError_t launch_ffn_bf16(int id, const FfnArgs& a, hipStream_t s);
hipError_t occupancy_ffn_bf16(int id, int* n);
extern const TileInfo kFp8Tiles[];
extern const int kNumFp8Tiles;
hipError_t launch_ffn_fp8(int id, const FfnArgs& a, hipStream_t s);
hipError_t occupancy_ffn_fp8(int id, int* n);
extern const TileInfo kW4a8Tiles[];
extern const int kNumW4a8Tiles;
hipError_t launch_ffn_w4a8(int id, const FfnArgs& a, hipStream_t s);
hipError_t occupancy_ffn_w4a8(int id, int* n);

namespace {


struct DeviceProps {
  bool ready = false;
  int cus = 0;
  int wall_khz = 0;
  int occ[64] = {};
};

std::mutex g_mu;
DeviceProps g_props[64];

int device_props(DeviceProps** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceProps& p = g_props[dev];
  if (!p.ready) {
    if (hipDeviceGetAttribute(&p.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MOE_ERR_HIP;
    if (hipDeviceGetAttribute(&p.wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        p.wall_khz <= 0)
      p.wall_khz = 100000;
    for (int i = 0; i < kNumBf16Tiles; ++i) {
      int n = 0;
      const int id = kBf16Tiles[i].id;
      if (occupancy_ffn_bf16(id, &n) != hipSuccess) return MOE_ERR_HIP;
      p.occ[id] = n;
    }
    for (int i = 0; i < kNumFp8Tiles; ++i) {
      int n = 0;
      const int id = kFp8Tiles[i].id;
      if (occupancy_ffn_fp8(id, &n) != hipSuccess) return MOE_ERR_HIP;
      p.occ[id] = n;
    }
    for (int i = 0; i < kNumW4a8Tiles; ++i) {
      int n = 0;
      const int id = kW4a8Tiles[i].id;
      if (occupancy_ffn_w4a8(id, &n) != hipSuccess) return MOE_ERR_HIP;
      p.occ[id] = n;
    }
    p.ready = true;
  }
  *out = &p;
  return MOE_OK;
}

bool shape_ok(const moe_shape* s) {
  if (!s) return false;
  if (s->num_slices < 1 || s->num_slices > MOE_MAX_SLICES) return false;
  if (s->tokens_per_slice < 0) return false;
  if (s->num_experts < 1 || s->num_experts > 1024) return false;
  if (s->top_k < 1 || s->top_k > 16 || s->top_k > s->num_experts) return false;
  if (s->num_local_experts < 1 || s->num_local_experts > MOE_MAX_LOCAL_EXPERTS) return false;
  if (s->local_expert_begin < 0 || s->local_expert_begin + s->num_local_experts > s->num_experts)
    return false;
  if (s->hidden < 128 || s->hidden % 128 || s->inter < 128 || s->inter % 128) return false;
  if (s->dtype != MOE_BF16 && s->dtype != MOE_FP8_E4M3 && s->dtype != MOE_W4A8) return false;
  const long long pairs = (long long)s->num_slices * s->tokens_per_slice * s->top_k;
  if (pairs > (1ll << 30)) return false;
  return true;
}

long long num_tokens(const moe_shape* s) { return (long long)s->num_slices * s->tokens_per_slice; }

const TileInfo* find_tile(int id) {
  for (int i = 0; i < kNumBf16Tiles; ++i)
    if (kBf16Tiles[i].id == id) return &kBf16Tiles[i];
  for (int i = 0; i < kNumFp8Tiles; ++i)
    if (kFp8Tiles[i].id == id) return &kFp8Tiles[i];
  for (int i = 0; i < kNumW4a8Tiles; ++i)
    if (kW4a8Tiles[i].id == id) return &kW4a8Tiles[i];
  return nullptr;
}

// Expected rows an expert's M-blocks cover when its routed rows M are rounded
// up to a multiple of `unit`, with M normal of mean and variance avg (uniform
// routing: a binomial count), evaluated on a grid of +-6 standard deviations.
double expected_padded_rows(double avg, int unit) {
  const double sd = std::sqrt(std::max(avg, 1.0));
  double num = 0.0, den = 0.0;
  for (int i = -240; i <= 240; ++i) {
    const double m = avg + sd * i / 40.0;
    if (m <= 0.0) continue;
    const double w = std::exp(-0.5 * (i / 40.0) * (i / 40.0));
    num += w * std::ceil(m / unit) * unit;
    den += w;
  }
  return den > 0.0 ? num / den : 0.0;
}

bool tile_fits(const TileInfo* t, const moe_shape* s) {
  if (!t || t->dtype != s->dtype) return false;
  if (s->hidden % t->block_n || (2 * s->inter) % t->block_n) return false;
  // fp8: one 128-wide scale block per K stage, at most 128 blocks along H and I
  if (s->dtype == MOE_FP8_E4M3 && (s->hidden / 128 > 128 || s->inter / 128 > 128)) return false;
  return true;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct WsLayout {
  size_t h, hs, l2_full, done, total;
};

WsLayout carve(const moe_shape* s, int block_m, int max_rows) {
  WsLayout w{};
  const size_t rows = (size_t)max_rows * block_m;
  const size_t elt = s->dtype == MOE_BF16 ? 2 : 1;
  w.h = 0;
  size_t off = align_up(rows * s->inter * elt, 256);
  w.hs = off;
  // h scales: fp32 per 1x128 block (fp8), one E8M0 byte per 1x32 block (W4A8)
  if (s->dtype == MOE_FP8_E4M3) off = align_up(off + rows * (s->inter / 128) * 4, 256);
  if (s->dtype == MOE_W4A8) off = align_up(off + rows * (s->inter / 32), 256);
  w.l2_full = off;
  off = align_up(off + (size_t)max_rows * 4, 256);
  w.done = off;
  off += 256;
  w.total = off;
  return w;
}

// Workspace of the allocation-free entry point (moe_ffn_forward_noalloc):
// the row counters and the done counter sit at fixed offsets, so that these
// bytes only ever hold counters, which every launch leaves cleared, whatever
// the shape of the call before; h and its scales follow.
WsLayout carve_static(const moe_shape* s, int block_m, int max_rows) {
  WsLayout w{};
  const size_t rows = (size_t)max_rows * block_m;
  const size_t elt = s->dtype == MOE_BF16 ? 2 : 1;
  w.l2_full = 0;
  w.done = (size_t)MOE_NOALLOC_MAX_SCHED_ROWS * 4;
  w.h = align_up(w.done + 256, 256);
  size_t off = align_up(w.h + rows * s->inter * elt, 256);
  w.hs = off;
  if (s->dtype == MOE_FP8_E4M3) off = align_up(off + rows * (s->inter / 128) * 4, 256);
  if (s->dtype == MOE_W4A8) off = align_up(off + rows * (s->inter / 32), 256);
  w.total = off;
  return w;
}

}  // namespace

bool shape_valid(const moe_shape* s) { return shape_ok(s); }

}  // namespace moe

using namespace moe;

// The allocation-free entry point's workspace: one copy per GPU, held from
// the load of this library's code object until the process ends. In host
// code this name is a host-side stand-in; the device address comes from
// hipGetSymbolAddress, once per device (static_workspace below).
static __device__ __align__(256) char scratch[MOE_NOALLOC_WORKSPACE_BYTES];

namespace {

struct StaticWorkspace {
  bool ready = false;
  char* ptr = nullptr;
};
StaticWorkspace g_static_ws[64];

// Device address of `scratch` on the current device. On the first call on a
// device its counter region is cleared by a fill kernel on `stream` (no
// memset node, so a call under graph capture records a kernel).
int static_workspace(char** out, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  StaticWorkspace& w = g_static_ws[dev];
  if (!w.ready) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    if (launch_zero(p, (size_t)MOE_NOALLOC_MAX_SCHED_ROWS * 4 + 256, stream) != hipSuccess)
      return MOE_ERR_HIP;
    w.ptr = static_cast<char*>(p);
    w.ready = true;
  }
  *out = w.ptr;
  return MOE_OK;
}

// moe_ffn_forward and moe_ffn_forward_noalloc: argument checks, the
// workspace carve (given workspace, or the fixed layout in `scratch`) and
// the launch.
int32_t ffn_forward_impl(const moe_shape* s, const moe_layout* lay, const void* const* x_slices,
                         const void* const* x_scales, const void* w1, const void* w1_scales,
                         const void* w2, const void* w2_scales, void* const* comb, void* ws,
                         size_t ws_bytes, bool static_ws, const moe_sched_params* prm, void* stream) {
  if (!shape_ok(s) || !lay || !prm || !x_slices || !comb || !w1 || !w2 || (!static_ws && !ws))
    return MOE_ERR_INVALID_ARG;
  const bool scaled = s->dtype != MOE_BF16;   // fp8 and W4A8 carry block scales
  if (scaled && (!x_scales || !w1_scales || !w2_scales)) return MOE_ERR_INVALID_ARG;
  moe_plan plan{};
  int st = moe_ffn_plan(s, prm, &plan);
  if (st != MOE_OK) return st;
  if (lay->block_m != plan.block_m) return MOE_ERR_INVALID_ARG;
  const WsLayout w = static_ws ? carve_static(s, plan.block_m, plan.max_sched_rows)
                               : carve(s, plan.block_m, plan.max_sched_rows);
  if (static_ws) {
    if (plan.max_sched_rows > MOE_NOALLOC_MAX_SCHED_ROWS || w.total > MOE_NOALLOC_WORKSPACE_BYTES)
      return MOE_ERR_WORKSPACE_TOO_SMALL;
  } else if (ws_bytes < plan.workspace_bytes) {
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  if (!lay->row_offset || !lay->tile_offset || !lay->row_pair || !lay->row_weight)
    return MOE_ERR_INVALID_ARG;
  if (prm->trace && prm->trace_capacity < 1) return MOE_ERR_INVALID_ARG;
  if (num_tokens(s) == 0) return MOE_OK;
  for (int i = 0; i < s->num_slices; ++i)
    if (!x_slices[i] || !comb[i] || (scaled && !x_scales[i])) return MOE_ERR_INVALID_ARG;
  DeviceProps* dp = nullptr;
  st = device_props(&dp);
  if (st != MOE_OK) return st;
  if (static_ws) {
    char* p = nullptr;
    st = static_workspace(&p, (hipStream_t)stream);
    if (st != MOE_OK) return st;
    ws = p;
  }

  FfnArgs a{};
  a.S = s->num_slices;
  a.T = s->tokens_per_slice;
  a.k = s->top_k;
  a.L = s->num_local_experts;
  a.H = s->hidden;
  a.I = s->inter;
  a.N1 = plan.n1_tiles;
  a.N2 = plan.n2_tiles;
  a.grid = plan.grid;
  // Group logical ids by Linear-1 N-tile per XCD when the experts span
  // several M-blocks (their weight tiles are then read once per XCD instead
  // of once per M-block); otherwise keep a row's N-tiles on one XCD.
  {
    const double avg = (double)num_tokens(s) * s->top_k / s->num_experts;
    const bool fits = a.grid % 8 == 0 && a.N1 % 8 == 0 && a.grid % a.N1 == 0;
    const bool want = MOE_XCD_BY_NTILE > 0 || (MOE_XCD_BY_NTILE < 0 && avg >= 2.0 * plan.block_m);
    a.xcd_group = fits && want ? a.N1 / 8 : 0;
    // blocks of the round's row-slot x N-tile grid per XCD: MOE_XCD_BX along
    // the N-tiles when it divides both sides, else every XCD takes N1/8
    // N-tiles across all row slots
    const int bx = MOE_XCD_BX;
    a.xcd_bx = a.xcd_group > 0 && (bx == 1 || bx == 2 || bx == 4) && a.N1 % bx == 0 &&
                       (a.grid / a.N1) % (8 / bx) == 0
                   ? bx
                   : 8;
  }
  a.schedule = prm->schedule;
  a.lead_d = plan.lead_d;
  a.experts_per_wave = prm->experts_per_wave;
  a.debug_skip_row = prm->debug_skip_l1_row;
  a.trace_cap = prm->trace ? prm->trace_capacity : 0;
  a.timeout_ticks = (long long)(prm->timeout_ms > 0 ? prm->timeout_ms : 2000) * dp->wall_khz;
  for (int i = 0; i < s->num_slices; ++i) {
    a.x[i] = x_slices[i];
    a.xs[i] = x_scales ? static_cast<const float*>(x_scales[i]) : nullptr;
    a.comb[i] = comb[i];
  }
  a.w1 = w1;
  a.w1s = static_cast<const float*>(w1_scales);
  a.w2 = w2;
  a.w2s = static_cast<const float*>(w2_scales);
  a.row_offset = lay->row_offset;
  a.tile_offset = lay->tile_offset;
  a.row_pair = lay->row_pair;
  a.row_weight = lay->row_weight;
  char* base = static_cast<char*>(ws);
  a.h = base + w.h;
  a.hs = reinterpret_cast<float*>(base + w.hs);
  a.l2_full = reinterpret_cast<int32_t*>(base + w.l2_full);
  a.done = reinterpret_cast<int32_t*>(base + w.done);
  a.status = prm->status;
  a.trace = prm->trace;
  const hipError_t err = s->dtype == MOE_FP8_E4M3 ? launch_ffn_fp8(plan.tile, a, (hipStream_t)stream)
                         : s->dtype == MOE_W4A8   ? launch_ffn_w4a8(plan.tile, a, (hipStream_t)stream)
                                                  : launch_ffn_bf16(plan.tile, a, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_FFN_ABI_VERSION; }

const char* moe_status_string(int32_t st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or configuration";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_TIMEOUT: return "a Linear-2 tile timed out waiting for its Linear-1 inputs";
  }
  return "unknown status";
}

size_t moe_layout_scratch_bytes(const moe_shape* s) {
  if (!shape_ok(s)) return 0;
  const long long pairs = num_tokens(s) * s->top_k;
  const long long chunks = (pairs + kLayoutChunk - 1) / kLayoutChunk;
  return (size_t)std::max<long long>(chunks, 1) * s->num_local_experts * 4;
}

int32_t moe_ffn_plan(const moe_shape* s, const moe_sched_params* prm, moe_plan* out) {
  if (!shape_ok(s) || !prm || !out) return MOE_ERR_INVALID_ARG;
  if (prm->schedule != MOE_SCHED_EXPERT_WAVE && prm->schedule != MOE_SCHED_INTERLEAVED)
    return MOE_ERR_INVALID_ARG;
  if (prm->lead_d < 0 || prm->grid < 0 || prm->experts_per_wave < 0 || prm->timeout_ms < 0)
    return MOE_ERR_INVALID_ARG;
  DeviceProps* dp = nullptr;
  int st = device_props(&dp);
  if (st != MOE_OK) return st;

  const TileInfo* t = nullptr;
  if (prm->tile > 0) {
    t = find_tile(prm->tile);
    if (!t) return MOE_ERR_INVALID_ARG;
    if (!tile_fits(t, s)) return MOE_ERR_UNSUPPORTED;
  } else if (s->dtype == MOE_FP8_E4M3) {
    for (int i = 0; i < kNumFp8Tiles && !t; ++i)
      if (tile_fits(&kFp8Tiles[i], s)) t = &kFp8Tiles[i];
    if (!t) return MOE_ERR_UNSUPPORTED;
  } else if (s->dtype == MOE_W4A8) {
    for (int i = 0; i < kNumW4a8Tiles && !t; ++i)
      if (tile_fits(&kW4a8Tiles[i], s)) t = &kW4a8Tiles[i];
    if (!t) return MOE_ERR_UNSUPPORTED;
  } else {
    // expected rows per local expert under uniform routing; pick the
    // smallest M-block that holds a typical expert whole (so each weight
    // tile is streamed once), the large block when experts are big
    const double avg = (double)num_tokens(s) * s->top_k / s->num_experts;
    const double sd = std::sqrt(avg);
    int order[6] = {7, 1, 6, 2, 5, 3};
    if (avg <= 24.0) {
      order[0] = 3; order[1] = 5; order[2] = 2; order[3] = 7;
    } else if (avg + 2.5 * sd <= 160.0) {
      order[0] = 5; order[1] = 2; order[2] = 7; order[3] = 3;
    } else if (avg + 4.0 * sd <= 192.0) {
      order[0] = 2; order[1] = 5; order[2] = 7; order[3] = 3;
    } else if (expected_padded_rows(avg, 256) > 1.35 * expected_padded_rows(avg, 32)) {
      // Experts just past a multiple of 256 rows: the 256-row tile (two token
      // wavefronts, no padding skip) would multiply a nearly empty second
      // block; the 160-row tile skips padding-only 32-row blocks. Measured on
      // the DeepSeek-V3-shaped share at 8 x 1024 tokens (256 rows per expert):
      // 937 against 1357 us.
      order[0] = 5; order[1] = 7; order[2] = 2; order[3] = 3;
    }
    for (int i = 0; i < 6 && !t; ++i)
      if (tile_fits(find_tile(order[i]), s)) t = find_tile(order[i]);
    if (!t) return MOE_ERR_UNSUPPORTED;
  }
  const int capacity = dp->occ[t->id] * dp->cus;
  if (capacity < 1) return MOE_ERR_UNSUPPORTED;
  int grid = capacity;
  if (prm->grid > 0) {
    if (prm->grid > capacity) return MOE_ERR_INVALID_ARG;   // all workgroups must be co-resident
    grid = prm->grid;
  }
  moe_plan p{};
  p.tile = t->id;
  p.block_m = t->block_m;
  p.block_n1 = t->block_n;
  p.block_n2 = t->block_n;
  p.n1_tiles = 2 * s->inter / t->block_n;
  p.n2_tiles = s->hidden / t->block_n;
  p.grid = grid;
  // X-Stage paper, Eq. 16: rows spanned by G concurrently running Linear-1 tiles
  p.lead_d = prm->lead_d > 0 ? prm->lead_d : std::max(1, (grid + p.n1_tiles - 1) / p.n1_tiles);
  const long long pairs = num_tokens(s) * s->top_k;
  long long rows = (pairs + (long long)s->num_local_experts * (t->block_m - 1)) / t->block_m;
  p.max_sched_rows = (int)std::max<long long>(rows, 1);
  // the task streams count tiles in int: every tile index plus one grid
  // stride must stay below INT_MAX
  if (std::max<long long>(rows, 1) * std::max(p.n1_tiles, p.n2_tiles) + grid >= INT_MAX)
    return MOE_ERR_UNSUPPORTED;
  p.workspace_bytes = carve(s, p.block_m, p.max_sched_rows).total;
  p.wall_clock_khz = dp->wall_khz;
  *out = p;
  return MOE_OK;
}

int32_t moe_workspace_init(void* ws, size_t bytes, void* stream) {
  if (!ws && bytes) return MOE_ERR_INVALID_ARG;
  return launch_zero(ws, bytes, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int32_t moe_dispatch_layout(const moe_shape* s, const float* logits, const float* bias,
                            const moe_layout* lay, void* stream) {
  if (!shape_ok(s) || !lay) return MOE_ERR_INVALID_ARG;
  if (lay->block_m < 1) return MOE_ERR_INVALID_ARG;
  if (!lay->counts || !lay->row_offset || !lay->tile_offset || !lay->totals || !lay->scratch)
    return MOE_ERR_INVALID_ARG;
  if (num_tokens(s) > 0 && (!lay->topk_idx || !lay->topk_w || !lay->row_pair || !lay->row_weight ||
                            !lay->pair_row))
    return MOE_ERR_INVALID_ARG;
  LayoutArgs a{};
  a.N = (int)num_tokens(s);
  a.E = s->num_experts;
  a.k = s->top_k;
  a.e0 = s->local_expert_begin;
  a.L = s->num_local_experts;
  a.block_m = lay->block_m;
  a.logits = logits;
  a.bias = bias;
  a.topk_idx = lay->topk_idx;
  a.topk_w = lay->topk_w;
  a.counts = lay->counts;
  a.row_offset = lay->row_offset;
  a.tile_offset = lay->tile_offset;
  a.row_pair = lay->row_pair;
  a.row_weight = lay->row_weight;
  a.pair_row = lay->pair_row;
  a.totals = lay->totals;
  a.block_counts = lay->scratch;
  a.nchunks = (int)(((long long)a.N * a.k + kLayoutChunk - 1) / kLayoutChunk);
  return launch_layout(a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}


int32_t moe_ffn_forward(const moe_shape* s, const moe_layout* lay, const void* const* x_slices,
                        const void* const* x_scales, const void* w1, const void* w1_scales,
                        const void* w2, const void* w2_scales, void* const* comb, void* ws,
                        size_t ws_bytes, const moe_sched_params* prm, void* stream) {
  return ffn_forward_impl(s, lay, x_slices, x_scales, w1, w1_scales, w2, w2_scales, comb, ws, ws_bytes,
                          false, prm, stream);
}

int32_t moe_ffn_forward_noalloc(const moe_shape* s, const moe_layout* lay, const void* const* x_slices,
                                const void* const* x_scales, const void* w1, const void* w1_scales,
                                const void* w2, const void* w2_scales, void* const* comb,
                                const moe_sched_params* prm, void* stream) {
  return ffn_forward_impl(s, lay, x_slices, x_scales, w1, w1_scales, w2, w2_scales, comb, nullptr, 0, true,
                          prm, stream);
}

int32_t moe_combine_check(const moe_shape* s, const moe_layout* lay, void* const* comb, void* y,
                          int32_t y_dtype, const int32_t* status, int32_t* report, void* stream) {
  if (!shape_ok(s) || !lay || !lay->pair_row || !comb) return MOE_ERR_INVALID_ARG;
  if (y_dtype != MOE_Y_FP32 && y_dtype != MOE_Y_BF16) return MOE_ERR_INVALID_ARG;
  CheckArgs a{};
  a.S = s->num_slices;
  a.T = s->tokens_per_slice;
  a.k = s->top_k;
  a.H = s->hidden;
  a.L = s->num_local_experts;
  for (int i = 0; i < s->num_slices; ++i) {
    if (!comb[i] && a.T > 0) return MOE_ERR_INVALID_ARG;
    a.comb[i] = comb[i];
  }
  a.pair_row = lay->pair_row;
  a.y = y;
  a.y_bf16 = y_dtype == MOE_Y_BF16;
  a.status = status;
  a.report = report;
  return launch_check(a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int32_t moe_mfma_rate_probe(int32_t format, int32_t blocks, int64_t iters, const void* operands,
                            size_t operand_bytes, int64_t* stamps, float* sink, void* stream) {
  static_assert(MOE_MFMA_PROBE_THREADS == 512, "probe workgroup size");
  if (format < 0 || format > 2 || blocks < 1 || blocks > 65535 || iters < 1 || !operands || !stamps || !sink)
    return MOE_ERR_INVALID_ARG;
  if (operand_bytes < mfma_probe_operand_bytes() || mfma_probe_operand_bytes() != MOE_MFMA_PROBE_OPERAND_BYTES ||
      mfma_probe_threads() != MOE_MFMA_PROBE_THREADS)
    return MOE_ERR_INVALID_ARG;
  return launch_mfma_probe(format, blocks, (long long)iters, operands, reinterpret_cast<long long*>(stamps), sink,
                           (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

int32_t moe_store_burst_probe(const moe_burst_params* prm, void* dst, size_t dst_bytes, uint32_t* stamps,
                              void* stream) {
  if (!prm || !dst || !stamps) return MOE_ERR_INVALID_ARG;
  const int row_bytes = prm->row_bytes > 0 ? prm->row_bytes : 512;
  if (prm->producers < 1 || prm->producers > 65535 || prm->bursts < 1 || prm->gap_ns < 0)
    return MOE_ERR_INVALID_ARG;
  if (row_bytes < 16 || row_bytes > 4096 || (row_bytes & (row_bytes - 1)) || prm->bytes_per_burst <= 0 ||
      prm->bytes_per_burst % 4096)
    return MOE_ERR_INVALID_ARG;
  if (dst_bytes < (size_t)row_bytes || dst_bytes / row_bytes > 0xFFFFFFFFull ||
      (prm->control && dst_bytes < 256 * 1024))
    return MOE_ERR_INVALID_ARG;
  DeviceProps* dp = nullptr;
  const int32_t st = device_props(&dp);
  if (st != MOE_OK) return st;
  BurstArgs a{};
  a.dst = static_cast<char*>(dst);
  a.dst_bytes = dst_bytes;
  a.stamps = stamps;
  a.producers = prm->producers;
  a.bytes_per_burst = prm->bytes_per_burst;
  a.bursts = prm->bursts;
  a.row_bytes = row_bytes;
  a.control = prm->control ? 1 : 0;
  a.gap_ticks = prm->gap_ns * (long long)dp->wall_khz / 1000000;
  return launch_burst(a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
