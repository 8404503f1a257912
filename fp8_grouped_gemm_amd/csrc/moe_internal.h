// Internal interface between the host entry points (moe_api.cpp) and the
// HIP kernels of the FP8 MoE forward.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Routing planner arguments ("07 · MegaMoE" §4 pool layout, §7 counting).
struct RouteArgs {
    const int32_t* idx;   // [TK] expert id per flat slot f = t*K + j
    int32_t TK;           // T*K
    int32_t E;
    int32_t row_align;
    int32_t NB;           // number of 1024-slot chunks
    int32_t* blk;         // [NB][E+1] per-chunk counts, then per-chunk bases
    int32_t* counts;      // [E]
    int32_t* offsets;     // [E+1]
    int32_t* row_src;     // [r_cap]
    int32_t r_cap;
    int32_t* src_row;     // [TK]
    int32_t* mblock_expert;  // [mb_cap] expert of each row_align block, -1 past the pool (may be null)
    int32_t mb_cap;
    int32_t* status;      // [4]
    int32_t* sync;        // [n_sync] single-launch counters, zeroed here (may be null)
    int32_t n_sync;
};

// Everything the GEMM, epilogue and combine kernels read or write.
struct FwdArgs {
    int32_t T, H, I, E, K, BM;
    int32_t packed;  // w1/w2 in moe_prepare_weights order
    const uint8_t* x;
    const float* x_sf;
    const int32_t* idx;
    const float* topk_w;
    const uint8_t* w1;
    const float* w1_sf;
    const uint8_t* w2;
    const float* w2_sf;
    const int32_t* row_src;
    const int32_t* offsets;        // [E+1] first pool row of each expert's segment
    const int32_t* mblock_expert;
    int32_t num_mblocks;   // row blocks of the pool's capacity (array sizes)
    // row blocks the launch grids cover: min(num_mblocks, T*K), since the
    // routed slots fill at most one new block each; blocks past the used
    // ones are empty and their workgroups would only read -1 and exit
    int32_t grid_mblocks;
    uint8_t* h;
    float* h_sf;
    uint16_t* partial;
    uint16_t* y;
    const int32_t* src_row;
    // Split-K across workgroups (16-row L1 tiles): K slices per tile (1 =
    // off) and their f32 partial sums, part[slice][slot][2I] for the
    // splitk_slots = T*K routed slots (slot f = t*K + j).
    int32_t split_l1;
    // L2 likewise for 16-row tiles of one or two tokens: K slices per tile
    // (1 = off), f32 sums in splitk_part[slice][slot][H]; the per-tile slice
    // counts follow the L1 ones in sync (kSyncReady + grid_mblocks * I/128)
    int32_t split_l2;
    int32_t l2_wide;  // 16-row L2 tiles: 1 = 8-wave workgroups over two 256-column tiles
    int32_t splitk_slots;
    float* splitk_part;
    // Single launch: counters sync[kSyncL2Done] (L2 items finished),
    // sync[kSyncQueue] (next item to claim) and sync[kSyncReady + mb] (L1
    // tiles of row block mb finished), zeroed by the planner; status word for
    // a wait that gave up; polls before giving up.
    int32_t* sync;
    int32_t* status;
    int32_t spin_limit;
    // Lag-ordered ring pool of the single launch (ring_blocks > 0; DeepGEMM
    // PR #440 "How it works", "Ring sizing, recycling"): h / h_sf hold
    // ring_blocks row blocks, row block mb in slot mb % ring_blocks.  The
    // planner's route_stream writes the unit table unit_mb[U + 1] (first row
    // block of each unit of up to kUnitBlocks blocks of one expert; the
    // last entry is the used row-block count) and the stream: entry p covers
    // items [stream_start[p], stream_start[p + 1]) of unit stream_desc[p] &
    // kStreamUnitMask, its L2 tiles when kStreamL2 is set, else its L1 tiles,
    // and item_tab[q] names item q: its tile (row block x column tiles + column
    // tile), with the top bit set for an L2 tile.  Where the used row blocks
    // fit the ring, the stream is the single-wave order (every L1 unit, then
    // every L2 unit) and no slot is reused.
    int32_t ring_blocks;
    int32_t lag_units;
    int32_t* unit_mb;
    int32_t* stream_start;
    int32_t* stream_desc;
    int32_t* item_tab;
    int32_t grid_cap;  // > 0: at most this many workgroups for the persistent kernels
    // FP8 x MXFP4 recipe (mx = 1): UE8M0 scale codes, one per 32 K values,
    // x_sfq [T,H/32], w1_sfq [E,2I,H/32], w2_sfq [E,H,I/32], h_sfq [R,I/32];
    // w1/w2 hold packed e2m1 pairs.  The f32 scale pointers are unused.
    // Recipe options: activation clamp of gate/up before the SwiGLU (<= 0:
    // none), power-of-two requant scales, per-64 intermediate scales (h_sf
    // [R, I/64] and the dual-half L2) -- the last two for the FP8 recipe.
    float clamp;
    int32_t pow2_scale;
    int32_t sf_gran64;
    int32_t mx;
    const uint8_t* x_sfq;
    const uint8_t* w1_sfq;
    const uint8_t* w2_sfq;
    uint8_t* h_sfq;
};

constexpr int kSyncL2Done = 0;
constexpr int kSyncQueue = 1;        // next unclaimed item
constexpr int kSyncStreamItems = 2;  // ring pool: L1 + L2 items of the stream
constexpr int kSyncUnits = 3;        // ring pool: units in the stream
constexpr int kSyncReady = 4;        // [num_mblocks]: L1 tiles finished per row block, then
                                     // [num_mblocks]: L2 tiles finished per row block
constexpr int kUnitBlocks = 8;       // row blocks per unit of the lag order
constexpr int kStreamGroup = 4;      // units per L2 group of the lag order
constexpr int32_t kStreamL2 = 1 << 30;
constexpr int32_t kStreamUnitMask = kStreamL2 - 1;
constexpr int32_t kItemL2 = INT32_MIN;  // item_tab: an L2 tile
constexpr int32_t kStatusWaitTimeout = 2;  // == MOE_STATUS_WAIT_TIMEOUT

constexpr int kRouteThreads = 1024;
constexpr int kMaxExperts = 1024;

hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_route_stream(const FwdArgs& a, hipStream_t s);  // ring pool: lag-ordered stream
hipError_t launch_l1(const FwdArgs& a, int kernel, hipStream_t s);
hipError_t launch_l2(const FwdArgs& a, int kernel, hipStream_t s);
hipError_t launch_fused(const FwdArgs& a, hipStream_t s);  // L1 + L2 + combine, direct tiles
hipError_t launch_combine(const FwdArgs& a, hipStream_t s);
hipError_t launch_l1_mx(const FwdArgs& a, hipStream_t s);  // direct tiles, tile_m 16/32/64
hipError_t launch_l2_mx(const FwdArgs& a, hipStream_t s);
hipError_t launch_l1_lds(const FwdArgs& a, hipStream_t s);
hipError_t launch_l2_lds(const FwdArgs& a, hipStream_t s);
hipError_t launch_l1_lds160(const FwdArgs& a, hipStream_t s);  // 160-row tiles
hipError_t launch_l2_lds160(const FwdArgs& a, hipStream_t s);
hipError_t launch_l1_sa(const FwdArgs& a, hipStream_t s);  // 64-row shared-A tiles
hipError_t launch_l2_sa(const FwdArgs& a, hipStream_t s);
hipError_t launch_quantize_act(const uint16_t* x, int T, int H, uint8_t* q, void* sf, bool mx,
                               hipStream_t s);
hipError_t launch_pack(const uint8_t* w1, const uint8_t* w2, uint8_t* w1p, uint8_t* w2p, int E,
                       int H, int I, hipStream_t s);
hipError_t launch_pack_mx(const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2,
                          const uint8_t* w2_sf, uint8_t* w1p, uint8_t* w1_sfp, uint8_t* w2p,
                          uint8_t* w2_sfp, int E, int H, int I, hipStream_t s);

}  // namespace moe
