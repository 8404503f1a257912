// L1 / L2 grouped FP8 GEMMs for large row tiles (prefill): 128 pool rows x
// 256 columns per tile, operands staged through LDS, one persistent
// workgroup per compute unit.
//
// Same arithmetic as the direct-load kernels ("MegaMoE SM90 Implementation
// Design" §5.3 promotion per 128-K block, §10.1 / §11.1 epilogues): for every
// K block kb, p = 16x16x128 e4m3 MFMA with C = 0, then
//   acc = fmaf(sa[row, kb] * sb[col block, kb], p, acc).
//
// gfx950 mapping.  A workgroup is 8 waves, 2 (rows) x 4 (columns); wave
// (wm, wn) owns 64 rows x 64 columns: for L1 the gate columns
// [128 n + 32 wn, +32) and the same up columns (gate and up of one element
// meet in one lane, and the workgroup owns the whole 128-wide requant
// block), for L2 the columns [256 n + 64 wn, +64).  Those are exactly the
// four 16-row weight subtiles wave wn reads in the packed layout
// (pack.hip), so each wave's B operand is 8 KiB in a row of LDS.
//
// Each 128-wide K block (A: 128 x 128 B, B: 256 x 128 B, plus the block's
// activation and weight scales) is copied global -> LDS with gfx950's
// global_load_lds_dwordx4 (each lane's 16 bytes land at base + 16 * lane, so
// one wave instruction fills 1 KiB in MFMA fragment order: [subtile][half]
// [lane][16 B], conflict-free ds_read_b128), three stages deep.
//
// Persistence.  With 150 KiB of stages only one workgroup fits a compute
// unit, so a workgroup that ended after each tile left its unit's memory
// stream idle through the tile's epilogue, its exit and the next
// workgroup's start (measured: a quarter of the L1 time at the
// flash-prefill shape).  Instead each workgroup walks tiles t = blockIdx +
// k * gridDim (tiles of unused row blocks form a suffix) and the copies run
// as one stream over (tile, K block), two blocks ahead of the multiply and
// across tile boundaries, so the next tile's first blocks arrive during the
// current tile's epilogue.  Everything the copies of a tile need from
// memory -- the tile's row sources, its expert, and (L1) the top-k weight of
// each row for the epilogue -- also travels by LDS copy, one tile ahead, so
// the loop holds no other vector memory access and the explicit vmcnt
// accounting stays exact.  The copy is issued as inline assembly: a batch
// (one K block's copies, plus on a tile's first block one metadata copy) is
// the same number of instructions in every wave, so "block j landed" is
// vmcnt <= the sizes of the batches issued after it.
//
// FP8 x MXFP4 recipe (MX = true; the SM100 recipe of the "07 · MegaMoE"
// page §0): e2m1 weights halve B to 16 KiB per K block (subtile = 16 rows x
// 32 K-values per lane group, 1 KiB, the packed MXFP4 order of pack.hip),
// and each stage carries the block's UE8M0 codes -- 4 per activation row
// and 64 per weight subtile -- which the block-scaled MFMA
// (mfma_16x16x128_e4m3_e2m1) applies itself, accumulating in f32.  With
// 34 KiB stages, four fit and three blocks stay in flight.  L1's epilogue
// requantises per 32 columns: one wave's gate columns, so no cross-wave
// amax; sf = the smallest power of two >= max(amax, 1e-10)/448.
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_lds.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 256;
constexpr int A_BYTES = BM * 128;   // 16 KiB: 8 m-subtiles x 2 halves x 1 KiB
constexpr int S_BYTES = 8 * 256;    // one 256-byte scale copy per wave
// Per-tile metadata slot: row_src of the 128 rows, top-k weight per row
// (L1), the tile's expert replicated over 64 lanes.
constexpr int META = 512 + 512 + 256;
constexpr int NMETA = 4;
constexpr int META_W = 512, META_E = 1024;
constexpr int kThreads = 512;
constexpr int kHotBlocks = 4;  // row blocks of an expert that make the walk use panels

// Stage geometry per recipe.  FP8: B = 16 n-subtiles x 2 halves x 1 KiB,
// copies per wave and block = 2 A + 4 B + 1 scale.  MXFP4: B = 16 subtiles
// x 1 KiB of e2m1, 2 A + 2 B + 1 scale.
template <bool MX>
struct LdsCfg {
    static constexpr int B_BYTES = MX ? BN * 64 : BN * 128;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int NSTAGE = MX ? 4 : 3;
    // copies each wave issues per K block: the loops of issue_next run
    // exactly these counts, and the vmcnt waits are sized by their sum
    static constexpr int A_COPIES = A_BYTES / 1024 / 8;     // 1 KiB each, 8 waves
    static constexpr int B_COPIES = B_BYTES / 1024 / 8;
    static constexpr int S_COPIES = S_BYTES / 256 / 8;      // one 256-byte scale copy
    static constexpr int COPIES = A_COPIES + B_COPIES + S_COPIES;
    static constexpr int SMEM = NSTAGE * STAGE + NMETA * META;
};
static_assert(LdsCfg<false>::COPIES == 2 + 4 + 1 && LdsCfg<true>::COPIES == 2 + 2 + 1,
              "copy counts per wave and K block");
static_assert(LdsCfg<false>::SMEM <= 160 * 1024 && LdsCfg<true>::SMEM <= 160 * 1024, "LDS");

// MXFP4: address of the 16 bytes lane `lane` copies for weight subtile
// q = 4 w + s of K block kb (packed: moe_prepare_weights_mx order).
template <bool L1, bool PK>
__device__ __forceinline__ const uint8_t* weight_src_mx(const FwdArgs& a, int e, int nt, int kb,
                                                        int q, int lane)
{
    const int H = a.H, I = a.I;
    const int K = L1 ? H : I;
    if constexpr (PK) {
        const int NT = L1 ? I / 128 : H / 256;
        const uint8_t* base = L1 ? a.w1 : a.w2;
        return base + (((size_t)e * NT + nt) * (K / 128) + kb) * 16384 + q * 1024 + lane * 16;
    } else {
        const int w4 = q >> 2, s = q & 3, lr = lane & 15, lg = lane >> 4;
        const int row = L1 ? (s >= 2 ? I : 0) + nt * 128 + w4 * 32 + (s & 1) * 16 + lr
                           : nt * 256 + w4 * 64 + s * 16 + lr;
        const size_t n = (size_t)e * (L1 ? 2 * I : H) + row;
        return (L1 ? a.w1 : a.w2) + n * (K / 2) + kb * 64 + lg * 16;
    }
}

}  // namespace

// L1 (gate + up) when L1 is true, L2 (down) otherwise.  Needs at least two
// K blocks (H >= 256 and I >= 256; the plan enforces it).
// G64 (FP8 recipe): per-64 intermediate scales ("MegaMoE SM90 Implementation
// Design" §5.4).  L1 requantises each 64-column half of its 128 gate/up
// columns on its own (waves wn = 2b, 2b + 1 hold block b); L2's scale copy
// carries both scales of each row and K block (lanes 0-15 the first, 32-47
// the second; lanes 16-17 stay the weight scales), and each 128-K block is
// multiplied as its two 64-K halves -- bytes 0-15 of every A fragment are K
// 0-63, bytes 16-31 K 64-127, so a copy with one half zeroed gives that
// half's sum -- each promoted with its own activation scale.
// HOT: the walk orders the tiles of hot experts in panels (below).
template <bool L1, bool PK, bool MX, bool G64, bool HOT>
__device__ __forceinline__ void lds_walk(const FwdArgs& a)
{
    static_assert(!(MX && G64), "per-64 scales are an FP8-recipe option");
    constexpr bool D64 = G64 && !L1;  // L2 multiplies dual halves
    using C = LdsCfg<MX>;
    constexpr int B_BYTES = C::B_BYTES, STAGE = C::STAGE, NSTAGE = C::NSTAGE;
    constexpr int kCopiesPerBlock = C::COPIES;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int H = a.H, I = a.I, K = a.K, T = a.T;
    const int NT = L1 ? I / 128 : H / 256;
    const int nkb = L1 ? H / 128 : I / 128;
    const int G = gridDim.x, b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int lr = lane & 15, lg = lane >> 4;
    const int TK = T * K;
    // Every index read from a metadata slot is range-checked before it forms
    // an address: a slot read before its copy landed (or never written)
    // then costs a wrong result, never an access outside the buffers.
    auto slot_f = [&](int f) { return (f >= 0 && f < TK) ? f : -1; };
    const uint32_t smem_base = lds_addr(smem);
    uint8_t* meta_base = smem + NSTAGE * STAGE;
    const uint32_t meta_lds = smem_base + NSTAGE * STAGE;
    auto slot = [&](int k) { return meta_base + (k % NMETA) * META; };
    auto slot_lds = [&](int k) { return meta_lds + (k % NMETA) * META; };
    // Tiles are numbered by position p = mb * NT + nt over the row blocks
    // that hold routed slots (the planner's used-row count; unused row
    // blocks are never visited).  Workgroups go to the 8 XCDs round-robin
    // (b % 8); XCD x takes the contiguous positions [x W, x W + W) of every
    // round of G, so the column tiles of a row block (shared activations)
    // and neighbouring row blocks of one expert (shared weights) meet in one
    // L2.  (Pro-prefill shape: L1 fabric reads 32.1 -> 25.8 GB, L2 14.7 ->
    // 12.5 GB against plain b + k G; grouping row blocks column tile by
    // column tile measured no better.)
    const int used_mb = min(a.num_mblocks, a.status[2] / BM);
    const int n_pos = used_mb * NT;
    const int W = G / 8;
    const int pos = (G % 8 == 0) ? (b % 8) * W + b / 8 : b;
    auto tile_of = [&](int k) { return pos + k * G; };  // position of tile k
    // Hot experts (HOT: some expert's segment spans >= kHotBlocks row
    // blocks).  Such an expert's R row blocks hold R * NT consecutive
    // positions, so each XCD's W of them would cover a few row blocks x
    // every column tile and stream the expert's whole weight matrix; its
    // positions are walked in panels of PC column tiles instead, row block
    // by row block within a panel (a chunk of 32 positions is 8 row blocks x
    // 4 columns: a quarter of the weight bytes, 4x the activation bytes).
    // The map is a bijection on the expert's own positions; only the order
    // of the tiles changes, never their arithmetic.
    const int PC = NT % 4 == 0 ? 4 : 2;  // (HOT implies NT even)
    // wave-uniform reads of the planner's tables through the scalar cache
    // (they take no part in the vmcnt accounting of the copies)
    auto sload = [&](const int32_t* q) {
        return __builtin_amdgcn_readfirstlane(*(const __attribute__((address_space(4))) int32_t*)q);
    };
    auto tile_at = [&](int p, int& mb, int& nt) {
        mb = p / NT;
        nt = p - mb * NT;
        if constexpr (HOT) {
            const int e = sload(a.mblock_expert + mb);
            if (e < 0 || e >= a.E)
                return;
            const int s0 = sload(a.offsets + e) / BM;
            const int R = sload(a.offsets + e + 1) / BM - s0;
            if (R < kHotBlocks || mb < s0 || mb >= s0 + R)
                return;
            const int q = (mb - s0) * NT + nt;  // the position within the expert's R x NT
            const int g = q / (R * PC), rem = q - g * (R * PC);
            const int r = rem / PC;
            mb = s0 + r;
            nt = g * PC + (rem - r * PC);
        }
    };

    if (tile_of(0) >= n_pos)
        return;

    // ---- metadata copy for tile k + 1 (and the weights of tile k's rows):
    // one dma4 per wave.  Waves 0/1 (and duplicates 5/6) copy row_src of
    // tile k + 1, rows [64 h, 64 h + 64); waves 2/3 gather topk_w of tile k's
    // rows (L1; L2: duplicates of 0/1); waves 4/7 copy tile k + 1's expert.
    // A tile past the end reads row block 0's (valid) rows instead: its slot
    // is never used.
    auto issue_meta = [&](int k) {
        int mbn = 0, ntn;  // (row block 0 holds routed slots)
        if (tile_of(k + 1) < n_pos)
            tile_at(tile_of(k + 1), mbn, ntn);
        const int rown = mbn * BM;
        const int role = (wave == 5) ? 0 : (wave == 6) ? 1 : (wave == 7) ? 4 : wave;
        if (role <= 1 || (!L1 && role <= 3)) {
            const int h = role & 1;
            dma4(a.row_src + rown + 64 * h + lane, slot_lds(k + 1) + 256 * h);
        } else if (role <= 3) {
            const int h = role - 2;
            const int f = slot_f(reinterpret_cast<const int32_t*>(slot(k))[64 * h + lane]);
            dma4(a.topk_w + (f >= 0 ? f : 0), slot_lds(k) + META_W + 256 * h);
        } else {
            dma4(a.mblock_expert + rown / BM, slot_lds(k + 1) + META_E);
        }
    };

    // ---- issue side: the next K block of the flattened (tile, kb) stream
    int i_k = 0, i_kb = 0;
    // LDS offset of the stage the next block is copied into, kept in a
    // scalar register (each copy's M0 is this plus a constant)
    uint32_t i_st = smem_base;
    bool i_done = false;
    int i_e = 0, i_nt = 0;
    const uint8_t* a_src[2] = {nullptr, nullptr};
    const float* s_src = nullptr;
    int s_step = 1;                     // floats between K blocks of s_src
    const uint8_t* s_src_mx = nullptr;  // MXFP4: this wave's 4 scale bytes per lane
    uint32_t s_stride = 0;              // bytes between K blocks of s_src_mx
    // Starts issuing tile k: reads its expert and row sources from its
    // metadata slot (landed and visible: copied with tile k - 1's first
    // block, at least two batches and one barrier ago).
    auto begin_tile = [&](int k) {
        if (tile_of(k) >= n_pos) {
            i_done = true;
            return;
        }
        const int e = __builtin_amdgcn_readfirstlane(
            reinterpret_cast<const int32_t*>(slot(k) + META_E)[lane]);
        if (e < 0 || e >= a.E) {
            i_done = true;
            return;
        }
        int mb, nt;
        tile_at(tile_of(k), mb, nt);
        const int row0 = mb * BM;
        i_e = e;
        i_nt = nt;
        // A: wave v copies m-subtile v, both halves: rows row0 + 16 v + lr.
        // Padding rows (f < 0) copy a valid row instead (L1: token 0; L2:
        // the block's first row, which always holds a routed slot), so their
        // lanes share cache lines with others; their products land only in
        // padding rows of the accumulator, which are never stored.
        const int f = slot_f(reinterpret_cast<const int32_t*>(slot(k))[wave * 16 + lr]);
        const int r = f >= 0 ? row0 + wave * 16 + lr : row0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (L1)
                a_src[j] = a.x + (size_t)(f >= 0 ? f / K : 0) * H + j * 64 + 16 * lg;
            else
                a_src[j] = a.h + (size_t)r * I + j * 64 + 16 * lg;
        }
        if constexpr (MX) {
            // UE8M0 codes of K block kb, 4 bytes per lane: waves 0-1 the
            // activation rows 64 wave + lane (a padding row: token 0 resp.
            // the block's first row), waves 2-5 the weight subtile rows
            // 64 (wave - 2) + lane (packed: that part of the block's 1 KiB),
            // waves 6-7 a spare copy of row 0's codes (every wave issues the
            // same copies).
            const int HS = H / 32, IS = I / 32;
            const int rr = wave < 2 ? wave * 64 + lane : lane;
            const int fr = slot_f(reinterpret_cast<const int32_t*>(slot(k))[rr]);
            if (wave < 2 || wave >= 6) {
                const bool spare = wave >= 6;
                if constexpr (L1)
                    s_src_mx = a.x_sfq + (size_t)(fr >= 0 && !spare ? fr / K : 0) * HS;
                else
                    s_src_mx = a.h_sfq + (size_t)(row0 + (fr >= 0 && !spare ? rr : 0)) * IS;
                s_stride = 4;
            } else {
                const int i = (wave - 2) * 64 + lane;
                const uint8_t* wsf = L1 ? a.w1_sfq : a.w2_sfq;
                if constexpr (PK) {
                    const int NT2 = L1 ? I / 128 : H / 256;
                    s_src_mx = wsf + ((size_t)e * NT2 + nt) * nkb * 1024 + i * 4;
                    s_stride = 1024;
                } else {
                    const int w4 = i >> 6, sq = (i >> 4) & 3, r2 = i & 15;
                    const int row = L1 ? (sq >= 2 ? I : 0) + nt * 128 + w4 * 32 + (sq & 1) * 16 + r2
                                       : nt * 256 + w4 * 64 + sq * 16 + r2;
                    s_src_mx = wsf + ((size_t)e * (L1 ? 2 * I : H) + row) * (L1 ? HS : IS);
                    s_stride = 4;
                }
            }
        } else {
            // Scales: lanes 16 and 17 the block's two weight scales (L1:
            // gate and up block of column tile nt; L2: blocks 2 nt, 2 nt + 1),
            // the other lanes the activation scale of row 16 v + (lane & 15).
            if (lane == 16 || lane == 17) {
                const int q = lane - 16;
                if constexpr (L1)
                    s_src = a.w1_sf + ((size_t)e * (2 * I / 128) + (q ? I / 128 + nt : nt)) * nkb;
                else
                    s_src = a.w2_sf + ((size_t)e * (H / 128) + 2 * nt + q) * nkb;
                s_step = 1;
            } else {
                if constexpr (L1) {
                    s_src = a.x_sf + (size_t)(f >= 0 ? f / K : 0) * (H / 128);
                } else if constexpr (D64) {  // lanes 32-47: the second half's scale
                    s_src = a.h_sf + (size_t)r * (I / 64) + (lg == 2 ? 1 : 0);
                    s_step = 2;
                } else {
                    s_src = a.h_sf + (size_t)r * (I / 128);
                }
            }
        }
    };
    // Issues the next block; returns the batch size (0 when nothing is left).
    auto issue_next = [&]() -> int {
        if (i_done)
            return 0;
        if (i_kb == nkb) {
            ++i_k;
            i_kb = 0;
        }
        if (i_kb == 0) {
            begin_tile(i_k);
            if (i_done)
                return 0;
        }
        const uint32_t st = __builtin_amdgcn_readfirstlane(i_st);
        const int kb = i_kb;
        static_assert(C::A_COPIES == 2 && C::S_COPIES == 1, "the loops below");
#pragma unroll
        for (int j = 0; j < C::A_COPIES; ++j)
            dma16(a_src[j] + (size_t)kb * 128, st + (wave * 2 + j) * 1024);
        if constexpr (MX) {
#pragma unroll
            for (int j = 0; j < C::B_COPIES; ++j) {
                const int q = wave * C::B_COPIES + j;
                dma16(weight_src_mx<L1, PK>(a, i_e, i_nt, kb, q, lane), st + A_BYTES + q * 1024);
            }
            dma4(s_src_mx + (size_t)kb * s_stride, st + A_BYTES + B_BYTES + wave * 256);
        } else {
#pragma unroll
            for (int j = 0; j < C::B_COPIES; ++j) {
                const int q = wave * C::B_COPIES + j, sub = q >> 1, half = q & 1;
                dma16(weight_src<L1, PK>(a, i_e, i_nt, kb, sub, half, lane), st + A_BYTES + q * 1024);
            }
            dma4(s_src + (size_t)kb * s_step, st + A_BYTES + B_BYTES + wave * 256);
        }
        int n = kCopiesPerBlock;
        if (kb == 0) {
            issue_meta(i_k);
            ++n;
        }
        ++i_kb;
        i_st = st + STAGE == smem_base + NSTAGE * STAGE ? smem_base : st + STAGE;
        return n;
    };

    // ---- prologue: tile 0's metadata, then blocks 0 and 1 of the stream
    {
        const int role = (wave == 5) ? 0 : (wave == 6) ? 1 : (wave == 7) ? 4 : wave;
        int mb0, nt0;
        tile_at(tile_of(0), mb0, nt0);
        const int row0 = mb0 * BM;
        if (role <= 3)
            dma4(a.row_src + row0 + 64 * (role & 1) + lane, slot_lds(0) + 256 * (role & 1));
        else
            dma4(a.mblock_expert + row0 / BM, slot_lds(0) + META_E);
        MOE_WAIT_VMCNT(0);
        __syncthreads();
    }
    // Blocks 0 .. NSTAGE - 2 in flight; pend[] = the sizes of the batches
    // issued after the block the next step multiplies, oldest first.
    (void)issue_next();
    int pend[NSTAGE - 2];
#pragma unroll
    for (int q = 0; q < NSTAGE - 2; ++q)
        pend[q] = issue_next();

    v4f acc[4][4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    // ---- multiply side
    int m_k = 0, m_kb = 0, j = 0;
    int ms_live = 4;     // this wave's m-subtiles holding routed rows in tile m_k
    bool drain = false;  // global stores since the last wait: wait for everything
    for (;;) {
        if (i_done && m_k >= i_k)
            break;  // tiles 0 .. i_k - 1 were valid and are finished
        // Block j has landed (its batch is not the newest one) and is visible
        // to all waves; the previous step's fragment reads are done, so the
        // stage issued below is free.
        if constexpr (NSTAGE == 3) {  // one newer batch: its size is one of three
            if (drain || pend[0] == 0)
                MOE_WAIT_VMCNT(0);
            else if (pend[0] == kCopiesPerBlock)
                MOE_WAIT_VMCNT(kCopiesPerBlock);
            else
                MOE_WAIT_VMCNT(kCopiesPerBlock + 1);
        } else {
            int newer = 0;
#pragma unroll
            for (int q = 0; q < NSTAGE - 2; ++q)
                newer += pend[q];
            wait_vmcnt(drain ? 0 : newer);
        }
        drain = false;
        __syncthreads();
        // Routed rows form a prefix of each tile (an expert's segment is its
        // rows, then padding up to the tile height): a wave whose 64 rows
        // are all past it (wm = 1 in a tile of <= 64 routed rows, an
        // expert's last tile mostly) skips its MFMAs and promotions --
        // nothing reads padding rows.  (Skipping single m-subtiles too needs
        // a branch per MFMA or one straight-line step per count, which
        // serialises the MFMAs or spills.)
        if (m_kb == 0) {
            const int32_t* rs = reinterpret_cast<const int32_t*>(slot(m_k));
            const int nv = __builtin_popcountll(__ballot(slot_f(rs[lane]) >= 0)) +
                           __builtin_popcountll(__ballot(slot_f(rs[64 + lane]) >= 0));
            ms_live = __builtin_amdgcn_readfirstlane(min(4, max(0, (nv - 64 * wm + 15) >> 4)));
        }

        const uint8_t* st = smem + (j % NSTAGE) * STAGE;
        // the copy of the block NSTAGE - 1 ahead, into the stage read last step
        auto issue_shift = [&]() {
#pragma unroll
            for (int q = 0; q + 1 < NSTAGE - 2; ++q)
                pend[q] = pend[q + 1];
            pend[NSTAGE - 3] = issue_next();
        };
        if constexpr (MX) {
            // A as for FP8; B: subtile wn*4 + s, 16 bytes of e2m1 per lane;
            // codes: activation row r at byte 4 r + lg, weight subtile bytes
            // after them (packed: per lane; row-major: 4 per subtile row).
            const uint8_t* s_lds = st + A_BYTES + B_BYTES;
            v8i af[4];
            uint4 bf[4];
            int sa[4], sb[4];
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                af[ms] = lds_frag(st + ((wm * 4 + ms) * 2) * 1024, lane);
                sa[ms] = s_lds[(wm * 64 + ms * 16 + lr) * 4 + lg];
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf[s] = *reinterpret_cast<const uint4*>(st + A_BYTES + (wn * 4 + s) * 1024 + lane * 16);
                sb[s] = PK ? s_lds[512 + (wn * 4 + s) * 64 + lane]
                           : s_lds[512 + ((wn * 4 + s) * 16 + lr) * 4 + lg];
            }
            issue_shift();
            if (ms_live > 0)  // (a wave whose rows are all padding has nothing to multiply)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int ms = 0; ms < 4; ++ms)
                    acc[ms][s] = mfma_16x16x128_e4m3_e2m1(af[ms], e2m1_operand(bf[s]), acc[ms][s],
                                                          sa[ms], sb[s]);
        } else {
            v8i af[4], bf[4];
            float sa[4][4], sa2[D64 ? 4 : 1][4];
            const float* s_lds = reinterpret_cast<const float*>(st + A_BYTES + B_BYTES);
            // weight scales: L1 gate / up block; L2 the wave's 128-column block
            const float sg = L1 ? s_lds[16] : s_lds[16 + (wn >> 1)];
            const float su = L1 ? s_lds[17] : sg;
            // one lane address per operand; the subtiles are constant offsets
            const uint8_t* a_rd = st + wm * 8192 + lane * 16;
            const uint8_t* b_rd = st + A_BYTES + wn * 8192 + lane * 16;
            const float* sa_rd = s_lds + wm * 256 + 4 * lg;
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                af[ms] = pack_frag(*reinterpret_cast<const uint4*>(a_rd + ms * 2048),
                                   *reinterpret_cast<const uint4*>(a_rd + ms * 2048 + 1024));
                const float4 s4 = *reinterpret_cast<const float4*>(sa_rd + ms * 64);
                sa[ms][0] = s4.x;
                sa[ms][1] = s4.y;
                sa[ms][2] = s4.z;
                sa[ms][3] = s4.w;
                if constexpr (D64) {  // the second half's scales, copied by lanes 32-47
                    const float4 t4 = *reinterpret_cast<const float4*>(sa_rd + ms * 64 + 32);
                    sa2[ms][0] = t4.x;
                    sa2[ms][1] = t4.y;
                    sa2[ms][2] = t4.z;
                    sa2[ms][3] = t4.w;
                }
                // (read in the order the MFMAs below consume them, so the
                // first ones start while the rest are in flight)
                bf[ms] = pack_frag(*reinterpret_cast<const uint4*>(b_rd + ms * 2048),
                                   *reinterpret_cast<const uint4*>(b_rd + ms * 2048 + 1024));
            }

            issue_shift();

            if (ms_live > 0)  // (a wave whose rows are all padding has nothing to multiply)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float sb = (L1 && s >= 2) ? su : sg;
                if constexpr (D64) {
#pragma unroll
                    for (int ms = 0; ms < 4; ++ms) {
                        const v8i alo = {af[ms][0], af[ms][1], af[ms][2], af[ms][3], 0, 0, 0, 0};
                        const v8i ahi = {0, 0, 0, 0, af[ms][4], af[ms][5], af[ms][6], af[ms][7]};
                        const v4f plo = mfma_16x16x128_e4m3(alo, bf[s], v4f{0.f, 0.f, 0.f, 0.f});
                        const v4f phi = mfma_16x16x128_e4m3(ahi, bf[s], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[ms][s][i] = fmaf(sa[ms][i] * sb, plo[i], acc[ms][s][i]);
                            acc[ms][s][i] = fmaf(sa2[ms][i] * sb, phi[i], acc[ms][s][i]);
                        }
                    }
                } else {
                    v4f p[4];
#pragma unroll
                    for (int ms = 0; ms < 4; ++ms)
                        p[ms] = mfma_16x16x128_e4m3(af[ms], bf[s], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[ms][s][i] = fmaf(sa[ms][i] * sb, p[ms][i], acc[ms][s][i]);
                }
            }
        }
        ++j;
        if (++m_kb < nkb)
            continue;

        // ---------------------------------------------- epilogue of tile m_k
        // It works in the stage just multiplied (the next two stages hold
        // the next tile's first blocks, in flight); the barrier orders every
        // wave's fragment reads of that stage before it is overwritten, and
        // the next step's barrier orders the epilogue before the stage is
        // refilled.
        int mb, nt;
        tile_at(tile_of(m_k), mb, nt);
        const int row0 = mb * BM;
        uint8_t* ep = smem + ((j - 1) % NSTAGE) * STAGE;
        const int32_t* m_rs = reinterpret_cast<const int32_t*>(slot(m_k));
        __syncthreads();
        if constexpr (L1 && MX) {
            // acc[ms][s] as below; wave wn's 32 gate columns are one 32-wide
            // requantisation block of each of its rows: amax over them, the
            // power-of-two scale as a UE8M0 code, codes staged in LDS.
            const float* m_w = reinterpret_cast<const float*>(slot(m_k) + META_W);
            clamp_acc<16>(&acc[0][0], a.clamp);
            uint8_t* qt = ep;  // [128][128]
            const int IS = I / 32;
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wm * 64 + ms * 16 + 4 * lg + i;
                    const bool valid = slot_f(m_rs[r]) >= 0;
                    const float w = valid ? m_w[r] : 0.f;
                    const float v0 = (silu(acc[ms][0][i]) *
                                      acc[ms][2][i]) * w;
                    const float v1 = (silu(acc[ms][1][i]) *
                                      acc[ms][3][i]) * w;
                    const float amax = max16(fmaxf(fabsf(v0), fabsf(v1)));
                    const uint32_t code = min(e8m0_ceil_code(fmaxf(amax, 1e-10f) / 448.0f), 253u);
                    const float inv = e8m0_inverse(code);
                    qt[r * 128 + wn * 32 + lr] = (uint8_t)f32_to_e4m3_hw(v0 * inv);
                    qt[r * 128 + wn * 32 + 16 + lr] = (uint8_t)f32_to_e4m3_hw(v1 * inv);
                    if (lr == 0 && valid)
                        a.h_sfq[(size_t)(row0 + r) * IS + nt * 4 + wn] = (uint8_t)code;
                }
            __syncthreads();
            for (int c = threadIdx.x; c < BM * 8; c += kThreads) {
                const int r = c >> 3, col = (c & 7) * 16;
                *reinterpret_cast<uint4*>(a.h + (size_t)(row0 + r) * I + nt * 128 + col) =
                    *reinterpret_cast<const uint4*>(qt + r * 128 + col);
            }
        } else if constexpr (L1) {
            // acc[ms][s]: rows wm*64 + 16 ms + 4 lg + i; s = 0,1 gate column
            // 32 wn + 16 s + lr of the block, s = 2,3 the matching up column.
            const float* m_w = reinterpret_cast<const float*>(slot(m_k) + META_W);
            clamp_acc<16>(&acc[0][0], a.clamp);
            float* red = reinterpret_cast<float*>(ep);  // [128][4]: row, then wave wn
            uint8_t* qt = ep + 2048;                    // [128][128]
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wm * 64 + ms * 16 + 4 * lg + i;
                    const float wr = m_w[r];  // (always a finite weight: padding rows copy slot 0's)
                    const float w = slot_f(m_rs[r]) >= 0 ? wr : 0.f;
                    float m = 0.f;
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const float g = acc[ms][s][i];
                        const float u = acc[ms][s + 2][i];
                        const float v = (silu(g) * u) * w;
                        acc[ms][s][i] = v;
                        m = fmaxf(m, fabsf(v));
                    }
                    m = max16_nonneg(m);
                    if (lr == 0)
                        red[r * 4 + wn] = m;
                }
            __syncthreads();
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wm * 64 + ms * 16 + 4 * lg + i;
                    const float4 rm = *reinterpret_cast<const float4*>(red + r * 4);
                    // per-64 scales: waves wn = 2b, 2b + 1 hold block b of the tile
                    const float amax = G64 ? (wn < 2 ? fmaxf(rm.x, rm.y) : fmaxf(rm.z, rm.w))
                                           : fmaxf(fmaxf(rm.x, rm.y), fmaxf(rm.z, rm.w));
                    float rsf;
                    const float sf = requant_sf(amax, a.pow2_scale, rsf);
                    const uint32_t c2 = requant_q2(acc[ms][0][i], acc[ms][1][i], sf, rsf, a.pow2_scale);
                    qt[r * 128 + wn * 32 + lr] = (uint8_t)c2;
                    qt[r * 128 + wn * 32 + 16 + lr] = (uint8_t)(c2 >> 8);
                    if constexpr (G64) {
                        if ((wn & 1) == 0 && lr == 0)
                            a.h_sf[(size_t)(row0 + r) * (I / 64) + nt * 2 + (wn >> 1)] = sf;
                    } else if (wn == 0 && lr == 0) {
                        a.h_sf[(size_t)(row0 + r) * (I / 128) + nt] = sf;
                    }
                }
            __syncthreads();
            // BM rows x 128 bytes, 16 bytes per thread, two per thread (rows
            // without a slot are written too: nothing reads them).
            for (int c = threadIdx.x; c < BM * 8; c += kThreads) {
                const int r = c >> 3, col = (c & 7) * 16;
                *reinterpret_cast<uint4*>(a.h + (size_t)(row0 + r) * I + nt * 128 + col) =
                    *reinterpret_cast<const uint4*>(qt + r * 128 + col);
            }
        } else {
            // acc[ms][s]: rows wm*64 + 16 ms + 4 lg + i, column 64 wn + 16 s
            // + lr.  Every wave rounds its values to bf16 at once; the rows
            // are then staged one 64-row half at a time (33 KiB: rows padded
            // to 264 columns, so the four row groups of a wave's write fall
            // on different LDS banks).
            constexpr int OT = 256 + 8;
            static_assert(64 * OT * 2 <= STAGE, "a staged half fits one stage");
            uint16_t* ot = reinterpret_cast<uint16_t*>(ep);  // [64][OT]
            uint16_t hb[4][4][4];
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        hb[ms][s][i] = f32_to_bf16(acc[ms][s][i]);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if (wm == hf) {
#pragma unroll
                    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                        for (int s = 0; s < 4; ++s)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                ot[(ms * 16 + 4 * lg + i) * OT + wn * 64 + s * 16 + lr] =
                                    hb[ms][s][i];
                }
                __syncthreads();
                for (int c = threadIdx.x; c < 64 * 32; c += kThreads) {
                    const int r = c >> 5, col = (c & 31) * 8;
                    const int f = slot_f(m_rs[hf * 64 + r]);
                    if (f >= 0) {
                        const int tt = f / K, jslot = f - tt * K;
                        *reinterpret_cast<uint4*>(a.partial + ((size_t)jslot * T + tt) * H +
                                                  nt * 256 + col) =
                            *reinterpret_cast<const uint4*>(ot + r * OT + col);
                    }
                }
                __syncthreads();
            }
        }
        drain = true;
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};
        ++m_k;
        m_kb = 0;
    }
}

// Hot experts ("MegaMoE SM90 Implementation Design" §12.2 switches its L2
// walk to N-major where experts hold many rows; PR #360 "TODO / future
// work" names the tile order as the lever for large-M cells): the planner's
// status[3], the largest segment, selects the panel walk for calls with an
// expert of >= kHotBlocks row blocks.  Each walk is its own kernel (one
// kernel holding both spilled 21 scalar registers where the plain walk
// spills 2); both are launched, and the one that does not apply exits at
// once (~3 us).  (Skewed shape: layer ~2005 -> ~1965 us; remapping 2-block
// experts too, as on the pro-prefill shape, measured 8 % slower.)
template <bool L1, bool PK, bool MX, bool G64, bool HOT>
__global__ __launch_bounds__(kThreads) void gemm_lds(FwdArgs a)
{
    const int NT = L1 ? a.I / 128 : a.H / 256;
    const bool hot = NT % 2 == 0 && a.status[3] / BM >= kHotBlocks;
    if (hot != HOT)
        return;
    lds_walk<L1, PK, MX, G64, HOT>(a);
}

template <bool L1, bool MX>
static hipError_t launch_lds(const FwdArgs& a, hipStream_t s)
{
    if (a.BM != BM)  // (64-row tiles run the shared-A kernels of gemm_sa.hip)
        return hipErrorInvalidValue;
    const int NT = L1 ? a.I / 128 : a.H / 256;
    const long long n_tiles = (long long)a.grid_mblocks * NT;
    const int nkb = L1 ? a.H / 128 : a.I / 128;
    if (n_tiles <= 0)
        return hipSuccess;
    // a tile's metadata copy must land before that tile's first block is
    // issued, NSTAGE - 1 blocks ahead of the multiply
    if (nkb < LdsCfg<MX>::NSTAGE - 1)
        return hipErrorInvalidValue;
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess)
        return err;
    long long g = n_tiles < cus ? n_tiles : cus;
    if (a.grid_cap > 0 && g > a.grid_cap)
        g = a.grid_cap;
    const dim3 grid((unsigned)g);
    const size_t smem = (size_t)LdsCfg<MX>::SMEM;
    // the plain walk, then (even column-tile counts) the hot-expert walk:
    // each kernel runs only if the planner's largest segment selects it
    const bool can_hot = NT % 2 == 0;
    for (int hot = 0; hot <= (can_hot ? 1 : 0); ++hot) {
        auto kern = a.packed ? (hot ? gemm_lds<L1, true, MX, false, true> : gemm_lds<L1, true, MX, false, false>)
                             : (hot ? gemm_lds<L1, false, MX, false, true> : gemm_lds<L1, false, MX, false, false>);
        if constexpr (!MX) {
            if (a.sf_gran64)
                kern = a.packed ? (hot ? gemm_lds<L1, true, false, true, true> : gemm_lds<L1, true, false, true, false>)
                                : (hot ? gemm_lds<L1, false, false, true, true> : gemm_lds<L1, false, false, true, false>);
        }
        err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (err != hipSuccess)
            return err;
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, s, a);
        err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

hipError_t launch_l1_lds(const FwdArgs& a, hipStream_t s)
{
    return a.mx ? launch_lds<true, true>(a, s) : launch_lds<true, false>(a, s);
}
hipError_t launch_l2_lds(const FwdArgs& a, hipStream_t s)
{
    return a.mx ? launch_lds<false, true>(a, s) : launch_lds<false, false>(a, s);
}

}  // namespace moe
