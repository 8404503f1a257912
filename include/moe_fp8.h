/*
 * moe_fp8.h — C ABI of the MI355X (gfx950) FP8 MoE expert forward.
 *
 * One GPU, all experts resident.  A forward takes FP8 (OCP e4m3) tokens with
 * 1x128 float scales, a top-k routing, FP8 expert weights with 128x128 float
 * block scales, and writes the BF16 layer output.  The steps, each a HIP
 * kernel of this library, follow the fused MoE forward described on the
 * DeepGEMM "MegaMoE" pages:
 *   1. routing planner: per-expert count, aligned prefix sum, slot
 *      assignment into per-expert contiguous pool segments
 *      ("07 · MegaMoE" §4 token pool, §7 dispatch counting);
 *   2. L1 grouped FP8 GEMM (gate+up) with per-128-K scale FMAs
 *      ("MegaMoE SM90 Implementation Design" §5.3);
 *   3. fused epilogue: silu(gate)*up*topk_w, per-128 e4m3 requantisation
 *      with sf = max(amax, 1e-10)/448 (design doc §10.1; DeepGEMM PR #440
 *      "How it works");
 *   4. L2 grouped FP8 GEMM (down), BF16 partial per (token, slot)
 *      (design doc §11.1);
 *   5. combine: per token, f32 sum of its slots' BF16 partials, cast to
 *      BF16 (design doc §11.2; "07 · MegaMoE" §9).
 * Variants a plan can select: the FP8 x MXFP4 recipe of the SM100 kernel
 * (moe_forward_mx; e2m1 weights, UE8M0 scales per 32), an activation clamp,
 * power-of-two or per-64 intermediate scales; moe_quantize_act prepares x.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major,
 *     densely packed.  The library never allocates or frees device memory;
 *     all scratch lives in a caller-provided workspace (moe_forward_noalloc:
 *     in a static device array of the library, see there).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; no entry point synchronises the host, except
 *     moe_read_status, which says so.
 *   - Every argument is validated on the host BEFORE any HIP call, so an
 *     invalid call returns an error code and enqueues nothing.
 *   - Return value: MOE_OK or a negative MOE_ERR_* code (moe_strerror).
 *   - A plan is immutable after creation and may be shared between threads;
 *     concurrent forwards need distinct workspaces.
 *
 * Shapes: T tokens, H hidden, I intermediate, E experts, K top-k.
 * Constraints: H % 128 == 0, I % 128 == 0, 1 <= K <= E <= 1024,
 * 0 <= T <= max_tokens, max_tokens * K < 2^24.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)        /* null pointer, T out of range, K > E, ... */
#define MOE_ERR_UNSUPPORTED_SHAPE (-2)  /* H or I not a multiple of 128, E > 1024, ... */
#define MOE_ERR_WORKSPACE_TOO_SMALL (-3)
#define MOE_ERR_HIP (-4)                /* a HIP launch or copy failed */
#define MOE_ERR_NOT_GFX950 (-5)         /* current device is not gfx950 */

/* Status bits written into the workspace by a forward (moe_read_status). */
#define MOE_STATUS_EXPERT_OUT_OF_RANGE 1 /* some topk_idx >= E; those slots were skipped */
#define MOE_STATUS_WAIT_TIMEOUT 2        /* single launch: a wait for other tiles gave up
                                            (bounded spin); y of that call is invalid */

/* Plan flags (moe_shape_t.flags). */
#define MOE_FLAG_SINGLE_LAUNCH 1  /* L1, L2 and combine of direct-tile calls in one
                                     launch ("07 · MegaMoE" §5-6) */
#define MOE_FLAG_SPLIT_LAUNCH 2   /* one launch per step; neither flag: the library's
                                     choice (see moe_plan_info's single_launch) */
#define MOE_FLAG_POW2_SCALE 4     /* FP8 recipe: requant scales rounded up to a power of
                                     two (DeepGEMM PR #440 "How it works", #383's choice) */
#define MOE_FLAG_DIRECT_TILES 8   /* 64-row tiles use the direct-load kernels even where
                                     the shared-A 64-row kernel fits (so that
                                     MOE_FLAG_SINGLE_LAUNCH can apply to them) */
#define MOE_FLAG_RING_POOL 16     /* FP8 recipe with per-128 intermediate scales: L1,
                                     L2 and the combine run as one launch in the lag
                                     order of DeepGEMM PR #440 "How it works", and h /
                                     h_sf become a ring of 8 (lag + 4) + 4 row blocks
                                     ("Ring sizing, recycling, and why that
                                     granularity") wherever the call's pool has more
                                     row blocks than that (moe_plan_info reports
                                     ring_blocks and l2_lag_units).  Direct-load tiles
                                     (tile_m 16, 32 or 64), no L1 split.  Invalid with
                                     MOE_FLAG_SPLIT_LAUNCH, MXFP4 or per-64 scales;
                                     tile_m 128 is unsupported.  y is bitwise that of
                                     MOE_FLAG_SINGLE_LAUNCH with the same tiles. */
#define MOE_FLAG_TEST_NO_WAIT 256 /* test-only: the single launch's waits give up at
                                     once, so MOE_STATUS_WAIT_TIMEOUT is set and y is
                                     invalid; exercises the timeout path */
#define MOE_FLAG_TEST_SMALL_GRID 512 /* test-only: the persistent LDS-tile kernels
                                        launch at most 4 workgroups, so each walks many
                                        tiles (same results as the full grid) */

/* Quantisation recipes (moe_shape_t.recipe). */
#define MOE_RECIPE_FP8_BLOCK128 0 /* e4m3 x e4m3, f32 scales: x per 1x128, weights per
                                     128x128, intermediate per 1x128 (moe_forward) */
#define MOE_RECIPE_MXFP4 1        /* e4m3 activations x e2m1 weights, UE8M0 scales per
                                     1x32 on x, weights and the intermediate
                                     (moe_forward_mx; the SM100 recipe (1,1,32) of
                                     "07 · MegaMoE" §0) */

/* Weight layouts a plan can expect for w1/w2 (scales are always row-major). */
#define MOE_WEIGHTS_ROW_MAJOR 0 /* w1 [E,2I,H], w2 [E,H,I] as documented at moe_forward */
#define MOE_WEIGHTS_PACKED 1    /* written by moe_prepare_weights (needs H % 256 == 0) */

typedef struct moe_shape {
    int32_t hidden;        /* H */
    int32_t intermediate;  /* I */
    int32_t num_experts;   /* E */
    int32_t top_k;         /* K */
    int32_t max_tokens;    /* largest T any call on this plan may pass */
    int32_t tile_m;        /* 0 = choose per call from T*K/E; else 16, 32, 64, 128
                              or 160.  Where the LDS tiles fit (H % 256 == 0, H and
                              I >= 256 (MXFP4: 384), per-128 scales) 128 runs the
                              LDS-staged kernel and 64 the shared-A kernel;
                              128 requires it, 64 otherwise (or with
                              MOE_FLAG_DIRECT_TILES) runs the direct-load kernel.
                              160 (the 160-row LDS-staged kernel) requires the FP8
                              recipe with per-128 scales, packed weights, no ring
                              pool, max_tokens * H < 2^31 and
                              (max_tokens * K + 160 E) * I < 2^31 */
    int32_t weight_layout; /* MOE_WEIGHTS_ROW_MAJOR or MOE_WEIGHTS_PACKED */
    int32_t flags;         /* MOE_FLAG_* bits, 0 = defaults */
    int32_t recipe;        /* MOE_RECIPE_*; MXFP4 plans: no single launch,
                              max_tokens * H < 2^31, tile_m 128 needs H, I >= 384 */
    int32_t act_sf_gran;   /* FP8 recipe: columns per intermediate (h) scale: 0 or 128,
                              64 (L2 then scales each 128-K block as two 64-K halves,
                              design doc §5.4), or -1 for the rule of PR #440 "How it
                              works" (128 when H % 512 == 0 and 2I % 512 == 0, else 64).
                              Per-64 plans run every tile kind as split launches (no
                              single launch, no ring pool).  MXFP4 plans: 0 (their
                              blocks are 32). */
    float activation_clamp; /* > 0: gate and up are clamped to [-c, c] before the
                               SwiGLU (design doc §10.1); <= 0: no clamp */
} moe_shape_t;

typedef struct moe_plan* moe_plan_t;

/* Tile configuration a forward with T tokens uses. */
typedef struct moe_tile_info {
    int32_t tile_m;      /* rows per GEMM tile = pool segment alignment */
    int32_t row_align;   /* == tile_m */
    int32_t pool_rows;   /* capacity R of the pool: T*K + E*(tile_m-1), rounded up to tile_m */
    int32_t l1_tile_n;   /* L1 output columns per tile (gate + up) */
    int32_t l2_tile_n;   /* L2 output columns per tile */
    int32_t kernel;      /* 0 = direct-load tile kernel, 1 = LDS-staged tile kernel,
                            2 = shared-A tile kernel (64 rows), 3 = 160-row
                            LDS-staged tile kernel */
    int32_t l1_split;    /* workgroups sharing one L1 tile's K range (1 = no split;
                            16-row tiles with fewer tiles than compute units) */
    int32_t single_launch; /* 1: L1, L2 and combine run as one launch */
    int32_t l2_group_tiles; /* L2 tiles (of l2_tile_n columns) per workgroup: 2 for
                               16-row tiles when at least 1024 workgroups remain, else 1 */
    int32_t act_sf_gran;    /* columns per intermediate (h) scale: 128 or 64 (FP8), 32 (MXFP4) */
    int32_t l2_split;       /* workgroups sharing one L2 tile's K range (1 = no split;
                               16-row tiles with fewer tiles than compute units) */
    int32_t ring_blocks;    /* MOE_FLAG_RING_POOL calls whose pool has more row blocks
                               than the ring: row blocks (of tile_m rows) that h and
                               h_sf hold, block mb at slot mb % ring_blocks; the ring
                               capacity PR #440's buffer query returns ("API, Tests,
                               Files").  0: h and h_sf hold the whole pool */
    int32_t l2_lag_units;   /* with ring_blocks > 0: units (up to 8 row blocks of one
                               expert) that L2 trails L1 by, clamp(round(0.45 units),
                               8, 64) for the call's T*K / (8 tile_m) units; a call
                               whose used blocks fit the ring runs the single-wave
                               order instead.  0 otherwise */
} moe_tile_info_t;

/* Byte offsets of the workspace sections used by a forward with T tokens.
 * Tests read the intermediate tensors through these views.
 *   counts   int32 [E]            tokens routed to each expert
 *   offsets  int32 [E+1]          first pool row of each expert's segment
 *   row_src  int32 [pool_rows]    flat slot f = t*K + j held by a pool row, -1 = padding
 *   src_row  int32 [T*K]          pool row of slot f, -1 = skipped slot
 *   h        uint8 [pool_rows, I] e4m3 SwiGLU output (valid rows only)
 *   h_sf     f32   [pool_rows, I/128]  (per-64 plans: [pool_rows, I/64];
 *                                       MXFP4 plans: uint8 UE8M0 [pool_rows, I/32])
 *            (ring-pool calls, moe_tile_info.ring_blocks > 0: ring_blocks * tile_m rows
 *            in place of pool_rows, each slot holding the last row block that used it)
 *   partial  uint16 [K, T, H]     bf16 L2 output of slot (t, j) at [j][t]
 *   status   int32 [4]            status[0] = MOE_STATUS_* bits, status[1] = #ids >= E,
 *                                  status[2] = pool rows used, status[3] = rows of the
 *                                  largest expert segment (both after alignment) */
typedef struct moe_ws_layout {
    size_t counts, offsets, row_src, src_row, h, h_sf, partial, status;
    size_t total;
} moe_ws_layout_t;

/* Validate a shape and create a plan (host only, no HIP call).  The pages
 * reject unsupported shapes on the host before anything launches: hidden and
 * intermediate multiples of 128, the architecture checked at dispatch
 * ("07 · MegaMoE" §0), intermediate size bounded when the buffer is sized
 * (DeepGEMM PR #440 "What a per-rank token count changes").  Here: the
 * constraints at the top of this file and those noted per field of
 * moe_shape_t; MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED_SHAPE otherwise,
 * *out then NULL.  The plan is host memory owned by the caller until
 * moe_plan_destroy (which accepts NULL and always returns MOE_OK). */
int moe_plan_create(const moe_shape_t* shape, moe_plan_t* out);
int moe_plan_destroy(moe_plan_t plan);

/* Tile configuration for a call with num_tokens tokens (host only).  As on
 * the pages, the row tile is chosen per call from the call's token count
 * (PR #440 "What a per-rank token count changes": block_m flips 64 -> 128
 * with the routed rows per expert, and the library reports the chosen
 * configuration); the pool segments are aligned to it ("07 · MegaMoE" §4).
 * MOE_ERR_INVALID_ARG for a null plan or info, or num_tokens outside
 * [0, max_tokens]. */
int moe_plan_info(moe_plan_t plan, int32_t num_tokens, moe_tile_info_t* info);

/* Workspace bytes a call with num_tokens tokens needs, and where its
 * sections sit: the pages' buffer-size query, which returns the byte count
 * and a slicer of the buffer into its regions (PR #440 "API, Tests, Files";
 * the input, L1-pool, L2-pool and combine regions of "07 · MegaMoE" §3).
 * Host only.  The amount is nondecreasing in num_tokens, so the value for
 * max_tokens serves every call on the plan.  No zeroing is required: every
 * call rewrites what it reads.  MOE_ERR_INVALID_ARG for a null plan or
 * output, or num_tokens outside [0, max_tokens]. */
int moe_workspace_bytes(moe_plan_t plan, int32_t num_tokens, size_t* bytes);
int moe_workspace_layout(moe_plan_t plan, int32_t num_tokens, moe_ws_layout_t* layout);

/*
 * Full forward (steps 1-5).
 *   x        uint8  [T, H]        e4m3 tokens
 *   x_sf     f32    [T, H/128]    per 1x128 block scale
 *   topk_idx int32  [T, K]        expert ids; < 0 masks the slot; >= E is
 *                                 skipped and flagged in the status word
 *   topk_w   f32    [T, K]        router weights, applied in the SwiGLU step
 *   w1       uint8  [E, 2I, H]    e4m3, rows [0,I) gate, rows [I,2I) up
 *                                 (packed plans: the moe_prepare_weights output)
 *   w1_sf    f32    [E, 2I/128, H/128]
 *   w2       uint8  [E, H, I]     e4m3 (packed plans: moe_prepare_weights output)
 *   w2_sf    f32    [E, H/128, I/128]
 *   y        uint16 [T, H]        bf16 output, written in full (a token with
 *                                 no active slot gets zeros)
 *   workspace / workspace_bytes   at least moe_workspace_bytes(plan, T)
 * x, w1, w2 and y must be 16-byte aligned and workspace 256-byte aligned
 * (MOE_ERR_INVALID_ARG otherwise; torch allocations are).
 * T == 0 is a no-op returning MOE_OK.
 */
int moe_forward(moe_plan_t plan, int32_t num_tokens,
                const uint8_t* x, const float* x_sf,
                const int32_t* topk_idx, const float* topk_w,
                const uint8_t* w1, const float* w1_sf,
                const uint8_t* w2, const float* w2_sf,
                uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward, plus five hipEvent_t recorded on `stream` for measurement:
 * step_events[0] before the planner, [1] after the planner, [2] after the
 * L1 GEMM + SwiGLU/requant epilogue, [3] after the L2 GEMM, [4] after the
 * combine.  With a single launch, [2], [3] and [4] are all recorded after
 * it.  Any entry may be NULL (not recorded).  Same validation and error
 * behaviour as moe_forward; with T == 0 nothing is recorded. */
int moe_forward_timed(moe_plan_t plan, int32_t num_tokens,
                      const uint8_t* x, const float* x_sf,
                      const int32_t* topk_idx, const float* topk_w,
                      const uint8_t* w1, const float* w1_sf,
                      const uint8_t* w2, const float* w2_sf,
                      uint16_t* y, void* workspace, size_t workspace_bytes, void* stream,
                      void* const* step_events);

/*
 * moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same steps, kernels and results as moe_forward (bit-identical y), with the
 * workspace replaced by a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * that the library owns: one per GPU, alive until the process ends.  No
 * call allocates or frees device memory.  The caller still passes inputs,
 * output and stream; operands as documented at moe_forward (FP8 plans only).
 *   - A call whose workspace (moe_workspace_bytes(plan, T)) exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE_TOO_SMALL before
 *     any HIP call (up to 404 tokens of the flash-decode shape, hidden 4096,
 *     intermediate 2048, 256 experts, top-6; 142 of the pro shape).
 *   - Every call on one GPU uses that GPU's one array, which keeps the last
 *     call's contents (each call rewrites what it reads): calls that overlap
 *     on one GPU (other streams, other threads) race and give undefined y.
 *   - MOE_ERR_INVALID_ARG for non-FP8 plans, null or misaligned operands, T
 *     out of range; MOE_ERR_HIP if the scratch address cannot be found.
 * The first call on a device also looks up the array's device address
 * (hipGetSymbolAddress, no allocation).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_forward_noalloc(moe_plan_t plan, int32_t num_tokens,
                        const uint8_t* x, const float* x_sf,
                        const int32_t* topk_idx, const float* topk_w,
                        const uint8_t* w1, const float* w1_sf,
                        const uint8_t* w2, const float* w2_sf,
                        uint16_t* y, void* stream);

/*
 * Full forward of the FP8 x MXFP4 recipe (plans with recipe =
 * MOE_RECIPE_MXFP4; MOE_ERR_INVALID_ARG for other plans, and moe_forward
 * rejects MXFP4 plans the same way).  Same steps, routing, workspace and
 * output as moe_forward; what differs is the operand encoding:
 *   x      uint8 [T, H]          e4m3 tokens
 *   x_sf   uint8 [T, H/32]       UE8M0 scale codes (2^(c-127)), one per 1x32 block
 *   w1     uint8 [E, 2I, H/2]    e2m1 pairs, element k of a row in byte k/2,
 *                                even k in the low nibble; rows [0,I) gate, [I,2I) up
 *   w1_sf  uint8 [E, 2I, H/32]   UE8M0 per row and 32 K values
 *   w2     uint8 [E, H, I/2]     e2m1 pairs
 *   w2_sf  uint8 [E, H, I/32]
 * L1 and L2 are block-scaled GEMMs with both operands' scales applied per 32
 * K values and f32 accumulation; the SwiGLU output is requantised per 1x32
 * with sf = the smallest power of two >= max(amax, 1e-10)/448 (a UE8M0
 * code), q = e4m3(h / sf) ("07 · MegaMoE" §8 per-block UE8M0 scale).
 * Scale codes of 0xFF (NaN) give NaN in the rows they touch.
 * x, w1, w2 and y must be 16-byte aligned, x_sf, w1_sf and w2_sf 4-byte
 * aligned, workspace 256-byte aligned.
 */
int moe_forward_mx(moe_plan_t plan, int32_t num_tokens,
                   const uint8_t* x, const uint8_t* x_sf,
                   const int32_t* topk_idx, const float* topk_w,
                   const uint8_t* w1, const uint8_t* w1_sf,
                   const uint8_t* w2, const uint8_t* w2_sf,
                   uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward_mx with the five step events of moe_forward_timed. */
int moe_forward_mx_timed(moe_plan_t plan, int32_t num_tokens,
                         const uint8_t* x, const uint8_t* x_sf,
                         const int32_t* topk_idx, const float* topk_w,
                         const uint8_t* w1, const uint8_t* w1_sf,
                         const uint8_t* w2, const uint8_t* w2_sf,
                         uint16_t* y, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* step_events);

/*
 * One-time weight re-layout for plans with weight_layout = MOE_WEIGHTS_PACKED
 * (the pages transform the expert weights once before any forward as well:
 * "MegaMoE SM90 Implementation Design" §15.1, "07 · MegaMoE" §8).
 *   w1 [E,2I,H], w2 [E,H,I]: row-major e4m3 input (device, read only)
 *   w1_packed, w2_packed: device outputs of the same byte sizes; must not
 *   overlap the inputs.  Scales are not touched and stay row-major.
 * Packed order: for expert e, column tile n (L1: 128 gate + 128 up rows;
 * L2: 256 rows), 128-wide K block kb, wave w (0..3), 16-row subtile s (0..3),
 * half h (bytes [0,64) or [64,128) of the block): 64 lanes x 16 bytes, lane
 * l = 16*g + r holding bytes [16g, 16g+16) of that half for subtile row r.
 * One 1 KiB run is exactly one MFMA operand load of one wave.
 * Returns MOE_ERR_INVALID_ARG if the plan is not a packed plan.
 */
int moe_prepare_weights(moe_plan_t plan, const uint8_t* w1, const uint8_t* w2,
                        uint8_t* w1_packed, uint8_t* w2_packed, void* stream);

/*
 * One-time re-layout of FP8 x MXFP4 weights for plans with recipe =
 * MOE_RECIPE_MXFP4 and weight_layout = MOE_WEIGHTS_PACKED (needs H % 256 ==
 * 0); moe_forward_mx then takes the four packed arrays in place of w1,
 * w1_sf, w2, w2_sf.
 *   w1 [E,2I,H/2], w1_sf [E,2I,H/32], w2 [E,H,I/2], w2_sf [E,H,I/32]: the
 *   row-major inputs (device, read only); the outputs have the same byte
 *   sizes and must not overlap any input or each other; w1, w2 and their
 *   packed copies 16-byte aligned.
 * Packed order: for expert e, column tile n (L1: 128 gate + 128 up rows;
 * L2: 256 rows), 128-wide K block kb, wave w (0..3), 16-row subtile s
 * (0..3): 64 lanes x 16 bytes, lane l = 16*g + r holding bytes
 * [64*kb + 16*g, 64*kb + 16*g + 16) of subtile row r (K values 128*kb + 32*g
 * .. + 31), i.e. one wave's e2m1 MFMA operand; the scales in the same order,
 * one byte per lane (code 4*kb + g of row r).
 * Returns MOE_ERR_INVALID_ARG for any other plan.
 */
int moe_prepare_weights_mx(moe_plan_t plan, const uint8_t* w1, const uint8_t* w1_sf,
                           const uint8_t* w2, const uint8_t* w2_sf, uint8_t* w1_packed,
                           uint8_t* w1_sf_packed, uint8_t* w2_packed, uint8_t* w2_sf_packed,
                           void* stream);

/*
 * Activation quantisation, the step the pages leave to the caller before each
 * call ("07 · MegaMoE" §3 copies FP8 x and its scales into the buffer):
 *   x_bf16 uint16 [T, H] bf16 (16-byte aligned), written to
 *   FP8 plans:   x uint8 [T, H] e4m3, x_sf f32 [T, H/128];
 *                per 1x128 block sf = max(amax, 1e-10)/448, q = e4m3(v / sf)
 *                (correctly rounded division; RNE, saturating)
 *   MXFP4 plans: x uint8 [T, H] e4m3, x_sf uint8 [T, H/32] UE8M0 codes;
 *                per 1x32 block sf = the smallest power of two >= that
 * x 16-byte aligned.  T == 0 is a no-op.  Same errors as moe_forward.
 */
int moe_quantize_act(moe_plan_t plan, int32_t num_tokens, const uint16_t* x_bf16, uint8_t* x,
                     void* x_sf, void* stream);

/*
 * Routing planner alone (step 1) with an explicit row alignment in [1, 1024]
 * ("07 · MegaMoE" §4: segments aligned to the row tile; §7: masked slots
 * skipped).  Rows of one expert hold its slots in ascending flat index f.
 *   counts  int32 [E], offsets int32 [E+1]
 *   row_src int32 [row_src_len]: row_src_len >= T*K + E*(row_align-1);
 *           rows past offsets[E] are set to -1
 *   src_row int32 [T*K]
 * Scratch comes from the workspace (moe_workspace_bytes of a plan covers it
 * when row_align <= the plan's tile_m; otherwise pass the bytes of
 * moe_route_workspace_bytes).
 */
int moe_route(moe_plan_t plan, int32_t num_tokens, const int32_t* topk_idx,
              int32_t row_align, int32_t* counts, int32_t* offsets,
              int32_t* row_src, int32_t row_src_len, int32_t* src_row,
              void* workspace, size_t workspace_bytes, void* stream);
/* Scratch bytes of moe_route alone (its per-chunk count table and status
 * word); same errors as moe_workspace_bytes. */
int moe_route_workspace_bytes(moe_plan_t plan, int32_t num_tokens, size_t* bytes);

/* Blocking: synchronises `stream`, then copies the 4-int status word of the
 * last call that used `workspace` into host_status[4] (MOE_STATUS_* bits,
 * the number of ids >= E, the pool rows used, the rows of the largest
 * expert segment; rows counted after alignment to the call's tile height).  The pages' kernels return
 * nothing from the device and abort on a timed-out wait (PR #440 "Register
 * inventory": the wait timeout and its handler); this library reports
 * instead: an id the pages leave undefined (>= E) is skipped and counted,
 * and a single-launch wait that gives up sets MOE_STATUS_WAIT_TIMEOUT.
 * MOE_ERR_WORKSPACE_TOO_SMALL if the workspace cannot hold the status word
 * of a call with num_tokens tokens; MOE_ERR_HIP if the copy fails. */
int moe_read_status(moe_plan_t plan, int32_t num_tokens, const void* workspace,
                    size_t workspace_bytes, int32_t* host_status, void* stream);

/* A static, human-readable name of a MOE_OK / MOE_ERR_* code ("unknown error"
 * otherwise).  The pages raise on the host (PR #440 "API, Tests, Files": a
 * token bound above capacity raises before any launch; fused-only keywords
 * on the split arm raise a ValueError); a C ABI returns codes instead. */
const char* moe_strerror(int code);

/* Library version, for the binding's sanity check. */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
