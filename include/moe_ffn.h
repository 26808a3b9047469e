/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) persistent MoE expert-FFN library.
 *
 * One GPU's expert-parallel share of a Mixture-of-Experts FFN layer, as the
 * X-Stage paper describes DeepGEMM's MegaMoE kernel (section 2.2, "MegaMoE
 * Execution"; section 4.2, "Capacity-Aware Scheduling across Expert Waves"):
 *
 *   routing + dispatch layout  ->  moe_dispatch_layout
 *   persistent grouped GEMM    ->  moe_ffn_forward: for every local expert,
 *       Linear-1 (gate and up projections) with the SwiGLU activation fused
 *       into its epilogue, then Linear-2 (down projection) whose epilogue
 *       multiplies each row by its router weight and stores it into the
 *       combine buffer of the source slice the token came from; tiles run
 *       in the Expert-Wave order or in the paper's Interleaved order
 *       (Algorithm 1).
 *   combine audit + reduction  ->  moe_combine_check
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers owned by the caller, unless a
 *    comment says "host". The library never allocates memory in a call and
 *    keeps no state besides cached device properties.
 *  - Every call is enqueued on `stream` (a hipStream_t; NULL means the
 *    default stream) and returns without waiting for the GPU.
 *  - Return value: MOE_OK (0) or a negative moe_status. Argument errors are
 *    detected on the host, before anything is enqueued. Errors found while
 *    the kernels run (a dependency wait that exceeded its time limit) are
 *    written to the device status word given in moe_sched_params.status and
 *    are readable after the stream has been synchronised.
 *  - Token numbering: source slice s holds tokens_per_slice (T) tokens; the
 *    global token index is n = s*T + t. Flat pair index f = n*k + j names
 *    top-k slot j of token n.
 *  - Layouts are row-major; sizes are in elements unless stated.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_ABI_VERSION 5
#define MOE_MAX_SLICES 64
#define MOE_MAX_LOCAL_EXPERTS 256
#define MOE_TRACE_WORDS 10      /* uint32 words per task record */
/* Workspace held by the library for moe_ffn_forward_noalloc, per GPU. */
#define MOE_NOALLOC_WORKSPACE_BYTES (64u << 20)
#define MOE_NOALLOC_MAX_SCHED_ROWS 16384

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,        /* a size, pointer or parameter is invalid */
  MOE_ERR_UNSUPPORTED = -2,        /* valid, but no kernel handles this shape */
  MOE_ERR_WORKSPACE_TOO_SMALL = -3,
  MOE_ERR_HIP = -4,                /* a HIP runtime call failed */
  MOE_ERR_TIMEOUT = -5,            /* device status: a dependency wait timed out */
} moe_status;

/* Operand formats.
 *   MOE_BF16      bf16 x and weights.
 *   MOE_FP8_E4M3  OCP e4m3 x and weights with fp32 scales: one per 1x128
 *                 block of x, one per 128x128 block of each weight matrix.
 *   MOE_W4A8      OCP Microscaling (MX): weights e2m1 (4-bit, two per byte,
 *                 element 2i in the low nibble of byte i), x e4m3, every
 *                 block of 32 consecutive elements along K with one E8M0
 *                 scale byte (2^(byte-127)). The X-Stage paper evaluates
 *                 W4A8 and W8A8 (section 5.2.1) without naming the 4-bit
 *                 format; MX is the format gfx950's matrix cores scale
 *                 natively. */
typedef enum { MOE_BF16 = 0, MOE_FP8_E4M3 = 1, MOE_W4A8 = 2 } moe_dtype;

typedef enum { MOE_SCHED_EXPERT_WAVE = 0, MOE_SCHED_INTERLEAVED = 1 } moe_schedule;

/* Problem shape. Global experts are 0..num_experts-1; this GPU owns
 * local_expert_begin .. local_expert_begin+num_local_experts-1. */
typedef struct {
  int32_t num_slices;          /* S: source slices (one per EP rank), 1..MOE_MAX_SLICES */
  int32_t tokens_per_slice;    /* T */
  int32_t num_experts;         /* E: global experts, 1..1024 */
  int32_t top_k;               /* k: experts per token, 1..min(E, 16) */
  int32_t local_expert_begin;  /* e0 */
  int32_t num_local_experts;   /* L, 1..MOE_MAX_LOCAL_EXPERTS */
  int32_t hidden;              /* H, a multiple of 128 */
  int32_t inter;               /* I, a multiple of 128 */
  int32_t dtype;               /* moe_dtype of x and the weights */
} moe_shape;

/* Dispatch layout (device arrays, caller-allocated; sizes from the shape,
 * N = S*T tokens, L local experts, R <= N*k routed rows).
 * Rows of local expert e are rows row_offset[e] .. row_offset[e+1]-1, in
 * ascending flat pair index. Scheduler rows (the M-blocks of the grouped
 * GEMM, the X-Stage paper's rows p with first row O_e per expert in
 * Algorithm 1) of expert e are tile_offset[e] .. tile_offset[e+1]-1, with
 * ceil(M_e / block_m) blocks per expert. */
typedef struct {
  int32_t* topk_idx;     /* [N, k] global expert of each slot (input when logits == NULL) */
  float* topk_w;         /* [N, k] router weight of each slot (same)                        */
  int32_t* counts;       /* [L]    routed rows per local expert (M_e)                       */
  int32_t* row_offset;   /* [L+1]  exclusive prefix sum of counts                           */
  int32_t* tile_offset;  /* [L+1]  exclusive prefix sum of ceil(M_e / block_m)              */
  int32_t* row_pair;     /* [N*k]  flat pair f of each routed row (first R entries valid)   */
  float* row_weight;     /* [N*k]  router weight of each routed row (first R valid)         */
  int32_t* pair_row;     /* [N*k]  routed row of pair f, or -1 when its expert is not local */
  int32_t* totals;       /* [4]    R, P (scheduler rows), max M_e, experts with M_e > 0     */
  int32_t* scratch;      /* moe_layout_scratch_bytes() bytes of scratch                     */
  int32_t block_m;       /* M-block size the FFN will use: moe_ffn_plan().block_m           */
} moe_layout;

/* Scheduling parameters. Zero fields select the automatic choice; an
 * explicit value always wins. */
typedef struct {
  int32_t schedule;          /* moe_schedule                                                */
  int32_t lead_d;            /* Interleaved lead D in scheduler rows, >= 1; 0 = the
                                X-Stage paper's anti-starvation knee, Eq. 16               */
  int32_t experts_per_wave;  /* Expert-Wave group size; 0 = close a wave once it holds at
                                least one Linear-1 tile per persistent workgroup           */
  int32_t grid;              /* persistent workgroups G; 0 = all that can be co-resident   */
  int32_t tile;              /* tile configuration id (moe_ffn_plan); 0 = automatic        */
  int32_t timeout_ms;        /* dependency-wait limit; 0 = 2000 ms                         */
  int32_t* status;           /* device int32, or NULL: set to MOE_ERR_TIMEOUT by a wait
                                that gave up (never cleared by the library)                */
  uint32_t* trace;           /* device [grid][trace_capacity][MOE_TRACE_WORDS] task records
                                of each persistent workgroup (indexed by its logical
                                instance), in execution order, or NULL:
                                word 0 = kind (1 = Linear-1, 2 = Linear-2) | n << 2,
                                word 1 = scheduler row p,
                                words 2..5 = low 32 bits of the device wall clock
                                (moe_plan.wall_clock_khz) at task start, after the
                                dependency wait, after the mainloop, and when the
                                epilogue stores were issued (Linear-2: the
                                sender-visible end of the combine stores),
                                words 6..7 = low 32 bits of the shader clock counter
                                at task start and after the mainloop,
                                word 8 = wall clock when the epilogue stores have
                                completed (Linear-2) or the row counter was
                                published (Linear-1: the bf16 kernel publishes
                                during the workgroup's next task, the fp8 and W4A8
                                kernels as soon as the h stores complete, with
                                word 5 = word 8),
                                word 9 = hardware workgroup id (blockIdx.x; it runs
                                on XCD word9 mod 8).
                                Unused records stay untouched                          */
  int32_t trace_capacity;    /* records per workgroup                                      */
  int32_t debug_skip_l1_row; /* testing only: when >= 0, Linear-1 tiles of this scheduler
                                row are not run, so its Linear-2 waits time out            */
} moe_sched_params;

/* Resolved plan for a shape and parameters. */
typedef struct {
  int32_t tile;        /* tile configuration id                         */
  int32_t block_m;     /* tokens per M-block (b_m)                      */
  int32_t block_n1;    /* Linear-1 N-tile width over the 2I gate/up outputs */
  int32_t block_n2;    /* Linear-2 N-tile width over the H outputs      */
  int32_t n1_tiles;    /* N1 = 2I / block_n1                            */
  int32_t n2_tiles;    /* N2 = H / block_n2                             */
  int32_t grid;        /* persistent workgroups G                       */
  int32_t lead_d;      /* resolved D                                    */
  int32_t max_sched_rows;    /* upper bound of P for this shape          */
  size_t workspace_bytes;    /* bytes moe_ffn_forward needs              */
  int32_t wall_clock_khz;    /* frequency of the trace time stamps       */
} moe_plan;

/* Library version (MOE_FFN_ABI_VERSION). */
int32_t moe_abi_version(void);

/* Text for a moe_status value (static storage). */
const char* moe_status_string(int32_t status);

/* Bytes of layout scratch (moe_layout.scratch) for this shape. */
size_t moe_layout_scratch_bytes(const moe_shape* shape);

/* Resolve tile configuration, grid and lead for a shape on the current
 * device. Returns MOE_ERR_UNSUPPORTED when no kernel handles the shape. */
int32_t moe_ffn_plan(const moe_shape* shape, const moe_sched_params* params, moe_plan* plan);

/* Zero a workspace before its first use (moe_ffn_forward leaves it zeroed
 * again when it completes, so this is needed only once per allocation). */
int32_t moe_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Routing and dispatch layout (the MegaMoE paper's Dispatch stage run
 * locally; the X-Stage paper, section 2.2, and Algorithm 1's row space).
 *   logits      [N, E] fp32 router logits, or NULL: then layout->topk_idx
 *               and layout->topk_w are inputs and routing is skipped.
 *   expert_bias [E] fp32 added to every token's logits before selection and
 *               softmax, or NULL.
 * Routing: z = logits + bias (fp32); the k largest z in descending order,
 * equal values broken by the lower expert index; weights are the softmax of
 * the k kept z values. Layout: see moe_layout. Everything stays on the
 * device; nothing is copied to the host. */
int32_t moe_dispatch_layout(const moe_shape* shape, const float* logits,
                            const float* expert_bias, const moe_layout* layout,
                            void* stream);

/* Persistent fused expert FFN (X-Stage paper, section 2.2 and Algorithm 1).
 *   x_slices       host array [S] of device pointers, each [T, H] of bf16
 *                  (MOE_BF16) or e4m3 bytes (MOE_FP8_E4M3, MOE_W4A8).
 *   x_scales       host array [S] of device pointers, each [T, H/128] fp32
 *                  (MOE_FP8_E4M3: one scale per 1x128 block) or [T, H/32]
 *                  E8M0 bytes (MOE_W4A8); NULL for MOE_BF16.
 *   w1             [L, 2I, H]: rows 0..I-1 of expert e are the gate
 *                  projection, rows I..2I-1 the up projection (MOE_W4A8:
 *                  [L, 2I, H/2] bytes of packed e2m1).
 *   w1_scales      MOE_FP8_E4M3: [L, 2I/128, H/128] fp32 per 128x128 block;
 *                  MOE_W4A8: [L, 2I, H/32] E8M0 bytes; NULL for MOE_BF16.
 *   w2             [L, H, I] down projection (MOE_W4A8: [L, H, I/2] bytes).
 *   w2_scales      MOE_FP8_E4M3: [L, H/128, I/128] fp32; MOE_W4A8:
 *                  [L, H, I/32] E8M0 bytes.
 *   combine_slices host array [S] of device pointers, each [T, k, H] bf16.
 *                  Slot (t, j) of slice s receives
 *                     bf16( w[n, j] * FFN_e(x[n]) ),  n = s*T + t,
 *                  for every pair whose expert e is local; other slots are
 *                  not touched.
 *   workspace      moe_ffn_plan().workspace_bytes bytes, zeroed once with
 *                  moe_workspace_init.
 * The layout must come from moe_dispatch_layout with layout->block_m equal
 * to moe_ffn_plan().block_m for the same shape and parameters. */
int32_t moe_ffn_forward(const moe_shape* shape, const moe_layout* layout,
                        const void* const* x_slices, const void* const* x_scales,
                        const void* w1, const void* w1_scales,
                        const void* w2, const void* w2_scales,
                        void* const* combine_slices,
                        void* workspace, size_t workspace_bytes,
                        const moe_sched_params* params, void* stream);

/* moe_ffn_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, kernels, outputs and
 * status word as moe_ffn_forward, bit for bit; the workspace (h, its scales
 * and the per-row counters) is a library-held device array of
 * MOE_NOALLOC_WORKSPACE_BYTES on each GPU, held until the process ends.
 * Allocates nothing: no hipMalloc, hipFree or allocating library call. The
 * first call on a device clears the array's counters with a fill kernel on
 * `stream`; every launch leaves them cleared again.
 * Returns MOE_ERR_WORKSPACE_TOO_SMALL (before anything is enqueued) when the
 * plan for the shape needs more than MOE_NOALLOC_MAX_SCHED_ROWS scheduler
 * rows or more than the array holds (decode-sized batches fit: e.g. 128
 * tokens in each of 8 slices of a DeepSeek-V3-shaped share of 32 experts,
 * top-8 of 256, H = 7168, I = 2048).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams, or from several threads without ordering)
 * race and give wrong results; calls ordered on one stream are safe. */
int32_t moe_ffn_forward_noalloc(const moe_shape* shape, const moe_layout* layout,
                                const void* const* x_slices, const void* const* x_scales,
                                const void* w1, const void* w1_scales,
                                const void* w2, const void* w2_scales,
                                void* const* combine_slices,
                                const moe_sched_params* params, void* stream);

/* Element type of moe_combine_check's y_local. */
#define MOE_Y_FP32 0
#define MOE_Y_BF16 1

/* Combine audit and source-side reduction (the "aggregate the top-k
 * results" half of Combine, X-Stage paper, section 2.2).
 *   combine_slices host array [S] of device pointers, each [T, k, H] bf16.
 *   y_local        [N, H] or NULL: y_local[n] = sum over the local slots j
 *                  of token n, in ascending j, of combine[n, j], summed in
 *                  fp32 and stored as y_dtype says.
 *   y_dtype        MOE_Y_FP32 (the fp32 sum) or MOE_Y_BF16 (that sum rounded
 *                  to nearest even bf16: the model's activation format, half
 *                  the bytes written).
 *   status         device int32 or NULL: the status word the FFN calls
 *                  wrote (moe_sched_params.status), read on the stream after
 *                  them.
 *   report         device int32 [4] or NULL; slot counts are ADDED to it:
 *                  [0] local slots with an element still holding the
 *                      sentinel 0xFFFF (not fully written),
 *                  [1] non-local slots with an element that is not the
 *                      sentinel (written although not local),
 *                  [2] local slots holding a non-finite value,
 *                  [3] receives *status (MOE_OK, or MOE_ERR_TIMEOUT when a
 *                      Linear-2 tile gave up waiting and left its rows
 *                      unwritten) when status is given; unchanged otherwise.
 *                  The audit reads every slot; pass NULL to skip it.
 * Neither the status word nor the report is cleared by the library. */
int32_t moe_combine_check(const moe_shape* shape, const moe_layout* layout,
                          void* const* combine_slices, void* y_local, int32_t y_dtype,
                          const int32_t* status, int32_t* report, void* stream);

/* One schedule configuration and what the planner's model predicts for it. */
typedef struct {
  int32_t schedule;          /* moe_schedule                                             */
  int32_t lead_d;            /* Interleaved lead D (0 for Expert-Wave)                   */
  int32_t experts_per_wave;  /* Expert-Wave wave size (0 = the automatic wave rule)      */
  double makespan;           /* predicted kernel time in model units (see below)         */
  double working_set;        /* time-averaged bytes of the expert weight matrices (an
                                expert's W1 or W2) that running tasks read              */
  double hbm_bytes;          /* predicted reads that miss an LRU cache of
                                MOE_PLANNER_CACHE_BYTES (the Infinity Cache): weight
                                tiles and activation blocks, in the model's start order */
  double unique_bytes;       /* bytes of those reads read at least once (compulsory)     */
} moe_schedule_estimate;

#define MOE_PLANNER_CACHE_BYTES (256.0 * 1024 * 1024)

#define MOE_MAX_SCHEDULE_CANDIDATES 8

typedef struct {
  moe_schedule_estimate given;        /* the configuration passed in `params`            */
  moe_schedule_estimate recommended;  /* the planner's choice among the candidates       */
  moe_schedule_estimate candidates[MOE_MAX_SCHEDULE_CANDIDATES];
  int32_t num_candidates;
  int32_t sched_rows;                 /* P for these counts                              */
  double lower_bound;                 /* total task cost / G, in model units             */
} moe_schedule_prediction;

/* Schedule planner for one routing (the X-Stage paper, section 6.3,
 * "Adaptive Burst Shaping and Scope": weigh each order's predicted stall
 * against its weight locality for the current routing and working set and
 * pick the original or the interleaved order; section 4.2 on the lead D:
 * below the knee of Eq. 16 Linear-2 tiles catch up with Linear-1 and wait,
 * far above it the concurrent expert-weight working set grows).
 * Host only; touches no device and enqueues nothing.
 *
 * Model: G persistent instances walk exactly the task streams
 * moe_ffn_forward runs (the kernel's own stream code, built for the host).
 * A Linear-1 task costs H/128 + 2 units, a Linear-2 task I/128 + 2 (one unit
 * is one 128-wide K block of the mainloop; 2 stands for the epilogue). A
 * Linear-2 task of scheduler row p starts once all N1 Linear-1 tasks of p
 * have ended. An event simulation gives each configuration's makespan and
 * the time average of the weight bytes in use.
 *   counts  HOST int32 [L]: routed rows of each local expert (the layout's
 *           counts, copied to the host by the caller).
 *   plan    from moe_ffn_plan for the same shape: block_m, n1_tiles,
 *           n2_tiles, grid and lead_d (the knee) are read.
 *   params  HOST; the configuration reported as `given` (schedule, lead_d
 *           with 0 = plan->lead_d, experts_per_wave); NULL = Interleaved at
 *           plan->lead_d.
 * Candidates, in this order: Expert-Wave with the automatic wave rule,
 * Interleaved with D = knee, Expert-Wave with all local experts in one wave,
 * Interleaved with D = knee/2, 2 knee, 4 knee and P, each capped at P (a
 * lead of P or more behaves as P; duplicates dropped).
 * Locality: the reads of the tasks, in the model's start order (time, then
 * instance), go through an LRU cache of MOE_PLANNER_CACHE_BYTES, an entry
 * being what a task reads whole: its weight tile (the N-tile's rows of the
 * expert's W1 or W2) and its activation block (the M-block's token rows for
 * Linear-1, its h rows for Linear-2). Misses are hbm_bytes.
 * Recommendation, among the candidates predicted within 2% of the fastest:
 * the first of the two first candidates (the original order, then the knee
 * lead), else the first of them; replaced by the one with the fewest
 * hbm_bytes (the earlier one on a tie) when that is lower by more than 2% of
 * the chosen one's unique_bytes. (The X-Stage paper, section 6.3, weighs
 * stall against weight locality; on this GPU the locality that orders lose
 * is the Infinity Cache's, when many experts of a few M-blocks each run at
 * once.)
 * Returns MOE_ERR_INVALID_ARG for a NULL pointer, a negative count, counts
 * whose M-blocks exceed plan->max_sched_rows or plan fields that are not
 * positive. */
int32_t moe_predict_schedule(const moe_shape* shape, const moe_plan* plan, const int32_t* counts,
                             const moe_sched_params* params, moe_schedule_prediction* out);

/* Parameters of the store burst-gap probe. */
typedef struct {
  int32_t producers;        /* K: concurrent producer workgroups, 1..65535            */
  int32_t bytes_per_burst;  /* B: bytes each producer stores per burst, a positive
                               multiple of 4096 and of row_bytes                        */
  int32_t bursts;           /* bursts per producer, >= 1                                */
  int32_t row_bytes;        /* contiguous bytes per destination row, a power of two
                               from 16 to 4096; 0 = 512 (one 256-feature bf16 N-tile
                               piece of a row)                                         */
  int32_t control;          /* 0: rows scattered over the whole destination buffer with
                               the combine epilogue's non-temporal stores; 1: rows
                               confined to its first 256 KiB (L2-resident control)     */
  int64_t gap_ns;           /* G: idle time of each producer after each burst          */
} moe_burst_params;

/* Store burst-gap probe: the X-Stage paper's remote-store microbenchmark
 * (section 3.1, "Remote-Store Microbenchmarks"; notation of Table 1) applied
 * to the stores this GPU's Linear-2 epilogue makes, scattered rows of local
 * HBM. K workgroups each issue bytes_per_burst bytes of 16-byte stores into
 * destination rows at fixed scattered positions, then idle gap_ns, bursts
 * times. For producer k and burst b, stamps[(k*bursts + b)*2 + 0/1] receive
 * the low 32 bits of the device wall clock (moe_plan.wall_clock_khz ticks)
 * just before the first store and once every wavefront of the producer has
 * issued its last store: their difference is the sender-visible issue time
 * T_iss, the start-to-start difference of consecutive bursts the period
 * T_period. From zero-gap, gap-swept and isolated runs the host fits the
 * model of section 3.2 (Eq. 1-5) and the capacity of section 3.5 (Eq. 6-7).
 *   dst     device buffer of dst_bytes (>= row_bytes and < 2^32 rows of
 *           row_bytes; >= 256 KiB with control); its contents are overwritten.
 *   stamps  device uint32 [producers * bursts * 2].
 * Enqueued on `stream`; returns MOE_ERR_INVALID_ARG for inconsistent sizes. */
int32_t moe_store_burst_probe(const moe_burst_params* params, void* dst, size_t dst_bytes,
                              uint32_t* stamps, void* stream);

/* MFMA issue-rate probe: the rate the matrix cores sustain when nothing but
 * MFMAs runs, on every CU, under the board's power limit -- the ceiling
 * beside the dense MFMA figures against which the FFN kernels' roofline
 * fractions are read (the X-Stage paper's evaluation reads its kernels
 * against the Tensor Core activity of its GPU, section 5.2.2).
 *   format    0: v_mfma_f32_32x32x16_bf16 (32,768 FLOP per MFMA);
 *             1: v_mfma_scale_f32_16x16x128_f8f6f4, e4m3 x e4m3 (65,536);
 *             2: v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3 (131,072).
 *   blocks    workgroups of MOE_MFMA_PROBE_THREADS threads (two wavefronts
 *             per SIMD), 1..65535; one per CU fills the chip.
 *   iters     loop trips, >= 1; each wavefront issues 16 MFMAs per trip.
 *   operands  device buffer of MOE_MFMA_PROBE_OPERAND_BYTES random operand
 *             bytes (bf16 values for format 0, e4m3 codes otherwise; each
 *             wavefront loads 16 fragments once, from one of 64 slots).
 *   stamps    device int64 [blocks][2]: shader-clock cycles (s_memtime) and
 *             wall-clock ticks (moe_plan.wall_clock_khz) of each workgroup's
 *             MFMA loop.
 *   sink      device float [blocks * MOE_MFMA_PROBE_THREADS]: the
 *             accumulator sums, written so that the loop is not removed.
 * Enqueued on `stream`; returns MOE_ERR_INVALID_ARG for a bad format, count
 * or buffer size. */
#define MOE_MFMA_PROBE_THREADS 512
#define MOE_MFMA_PROBE_OPERAND_BYTES (64u * 64u * 16u * 16u)
int32_t moe_mfma_rate_probe(int32_t format, int32_t blocks, int64_t iters, const void* operands,
                            size_t operand_bytes, int64_t* stamps, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
