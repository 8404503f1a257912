// L1 / L2 grouped FP8 GEMMs on 160-row tiles (FP8 recipe, per-128 scales):
// 160 pool rows x 256 columns per tile, operands staged through LDS, one
// persistent workgroup per compute unit.
//
// Arithmetic as in every other tile ("MegaMoE SM90 Implementation Design"
// §5.3 promotion per 128-K block, §10.1 / §11.1 epilogues): for every K block
// kb, p = 16x16x128 e4m3 MFMA with C = 0, then
//   acc = fmaf(sa[row, kb] * sb[col block, kb], p, acc),
// so a 160-row tile's results are bitwise those of the 128-row tile.
//
// Why 160 rows.  Where experts receive about 128 routed rows (the pro-prefill
// layer: 8192 tokens x top-6 over 384 experts), half the experts overflow a
// 128-row tile by a few rows, and each such second tile streams the expert's
// whole weight matrix again for those rows (1.5x the unique weight bytes).  A
// 160-row tile holds nearly every such expert in one tile: the weights are
// streamed once, and the MFMA work (the second tile's padding row halves were
// already skipped) stays the same.  160 rows is the tallest tile whose three
// copy stages fit the 160 KiB of LDS.
//
// gfx950 mapping.  8 waves, 2 (row halves of 80 rows) x 4 (column quarters);
// wave (wm, wn) owns 5 m-subtiles x 4 n-subtiles: for L1 the gate columns
// [128 n + 32 wn, +32) and the same up columns (gate and up of one element in
// one lane, the whole 128-wide requant block in one workgroup), for L2 the
// columns [256 n + 64 wn, +64).  Each K block (A: 160 x 128 B, B: 256 x 128 B,
// the rows' activation scales and the block's two weight scales) is copied
// global -> LDS by global_load_lds_dwordx4 / _dword, three stages deep, two
// blocks ahead of the multiply and across tile boundaries (the next tile's
// first blocks arrive during the current tile's epilogue).
//
// LDS budget (163,840 bytes): three stages of 20,480 (A) + 32,768 (B) + 656
// (160 activation scales, 2 weight scales) bytes, and three 640-byte slots
// holding a tile's row sources.  To fit, the tile's expert is read through
// the scalar cache (it takes no part in the vmcnt accounting), and the L1
// epilogue gathers the rows' top-k weights with ordinary loads once per tile
// (the epilogue ends with global stores, after which the next step waits for
// every outstanding access anyway).
//
// Copies per wave and K block (every count the waits use follows from
// these): A: 20 copies of 1 KiB, wave w takes w, w + 8 and (w < 4) w + 16;
// B: 4 each; scales: waves 0-2 one 4-byte copy each (wave 2: rows 128-159
// in lanes 0-31, the weight scales in lanes 32-33); on a tile's first block
// waves 5-7 also copy the next tile's row sources.  Only the batch of the
// block after j may be outstanding when block j is multiplied, and every
// batch holds at least kMinBatch copies, so "block j landed" is
// vmcnt <= kMinBatch in every wave.
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_lds.h"

namespace moe {

namespace {

constexpr int BM = 160;             // pool rows per tile
constexpr int MS = 5;               // m-subtiles per wave (80 rows)
constexpr int BN = 256;
constexpr int A_BYTES = BM * 128;   // [subtile][half][lane][16 B]
constexpr int B_BYTES = BN * 128;
constexpr int S_FLOATS = BM + 2;    // row scales, then the two weight scales
constexpr int S_BYTES = 656;        // S_FLOATS * 4 rounded to 16
constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
constexpr int NSTAGE = 3;
constexpr int META = BM * 4;        // row_src of a tile's 160 rows
constexpr int NMETA = 3;
constexpr int SMEM = NSTAGE * STAGE + NMETA * META;
constexpr int kThreads = 512;
constexpr int kHotBlocks = 4;       // row blocks of an expert that make the walk use panels
static_assert(S_FLOATS * 4 <= S_BYTES && S_BYTES % 16 == 0 && STAGE % 16 == 0, "stage layout");
static_assert(SMEM <= 160 * 1024, "LDS");
static_assert(MS * 16 * 2 == BM, "two row halves of MS m-subtiles");

// copies wave w issues per K block (A, B, scales) and, on a tile's first
// block, for the next tile's row sources
__device__ __forceinline__ int a_copies(int w) { return w < 4 ? 3 : 2; }
constexpr int B_COPIES = B_BYTES / 1024 / 8;
__device__ __forceinline__ int s_copies(int w) { return w < 3 ? 1 : 0; }
__device__ __forceinline__ int m_copies(int w) { return w >= 5 ? 1 : 0; }
static_assert(4 * 3 + 4 * 2 == A_BYTES / 1024, "A copies: 20 of 1 KiB");
constexpr int kMinBatch = 2 + B_COPIES;  // the smallest batch any wave issues
static_assert(2 * 64 + 32 == BM, "scale and row-source copies: 64 + 64 + 32 rows");

}  // namespace

template <bool L1, bool PK, bool HOT>
__device__ __forceinline__ void lds160_walk(const FwdArgs& a)
{
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
    const int nA = a_copies(wave), nS = s_copies(wave), nM = m_copies(wave);
    // Every index read from a row-source slot is range-checked before it
    // forms an address: a slot read before its copy landed costs a wrong
    // result, never an access outside the buffers.
    auto slot_f = [&](int f) { return (f >= 0 && f < TK) ? f : -1; };
    const uint32_t smem_base = lds_addr(smem);
    uint8_t* meta_base = smem + NSTAGE * STAGE;
    const uint32_t meta_lds = smem_base + NSTAGE * STAGE;
    auto slot = [&](int k) { return reinterpret_cast<const int32_t*>(meta_base + (k % NMETA) * META); };
    auto slot_lds = [&](int k) { return meta_lds + (k % NMETA) * META; };
    auto sload = [&](const int32_t* q) {
        return __builtin_amdgcn_readfirstlane(*(const __attribute__((address_space(4))) int32_t*)q);
    };
    // Tile positions p = mb * NT + nt over the used row blocks, XCD-grouped
    // (workgroup b runs on XCD b % 8 and takes the contiguous positions
    // [x W, x W + W) of each round), as in the 128-row walk.
    const int used_mb = min(a.num_mblocks, a.status[2] / BM);
    const int n_pos = used_mb * NT;
    const int W = G / 8;
    const int pos = (G % 8 == 0) ? (b % 8) * W + b / 8 : b;
    auto tile_of = [&](int k) { return pos + k * G; };
    // Hot experts (>= kHotBlocks row blocks): their R x NT positions are
    // walked in panels of PC column tiles, row block by row block inside a
    // panel (a bijection on the expert's positions; only the order changes).
    const int PC = NT % 4 == 0 ? 4 : 2;
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
            const int q = (mb - s0) * NT + nt;
            const int g = q / (R * PC), rem = q - g * (R * PC);
            const int r = rem / PC;
            mb = s0 + r;
            nt = g * PC + (rem - r * PC);
        }
    };

    if (tile_of(0) >= n_pos)
        return;

    // ---- row sources of tile k + 1 into its slot: waves 5-7, rows
    // [64 h, 64 h + 64) (h = 2: lanes 0-31).  A tile past the end copies row
    // block 0's (valid) rows; its slot is never used.
    auto issue_meta = [&](int k) {
        if (!nM)
            return;
        int mbn = 0, ntn;
        if (tile_of(k + 1) < n_pos)
            tile_at(tile_of(k + 1), mbn, ntn);
        const int h = wave - 5;
        if (h < 2 || lane < 32)
            dma4(a.row_src + mbn * BM + 64 * h + lane, slot_lds(k + 1) + 256 * h);
    };

    // ---- issue side: the next K block of the flattened (tile, kb) stream
    int i_k = 0, i_kb = 0;
    uint32_t i_st = smem_base;  // LDS offset of the stage the next block goes to
    bool i_done = false;
    // Copy sources as a wave-uniform base plus a 32-bit per-lane offset
    // (the plan admits this tile only where every offset stays below 2^31):
    // A rows from x (L1) or h (L2) + kb * 128, B from the tile's expert and
    // column tile (packed: the lane's 16 bytes of a 1 KiB subtile).
    const uint8_t* i_wbase = nullptr;  // expert e, column tile nt, K block 0
    uint32_t a_off[3] = {0, 0, 0};
    uint32_t b_off[B_COPIES] = {};
    const float* s_src = nullptr;
    // Starts issuing tile k: its expert through the scalar cache, its row
    // sources from its slot (landed and visible: copied with tile k - 1's
    // first block, at least two batches and one barrier ago).
    auto begin_tile = [&](int k) {
        if (tile_of(k) >= n_pos) {
            i_done = true;
            return;
        }
        int mb, nt;
        tile_at(tile_of(k), mb, nt);
        const int e = sload(a.mblock_expert + mb);
        if (e < 0 || e >= a.E) {
            i_done = true;
            return;
        }
        const int row0 = mb * BM;
        const int KD = L1 ? H : I;  // bytes per weight row
        if constexpr (PK) {
            i_wbase = (L1 ? a.w1 + (size_t)e * 2 * I * H : a.w2 + (size_t)e * H * I) +
                      (size_t)nt * nkb * 32768;
            b_off[0] = (uint32_t)(lane * 16);  // (copy j adds j KiB as an immediate)
        } else {
            i_wbase = L1 ? a.w1 + (size_t)e * 2 * I * H : a.w2 + (size_t)e * H * I;
#pragma unroll
            for (int j = 0; j < B_COPIES; ++j) {
                const int q = wave * B_COPIES + j, sub = q >> 1, half = q & 1;
                const int w4 = sub >> 2, sq = sub & 3;
                const int row = L1 ? (sq >= 2 ? I : 0) + nt * 128 + w4 * 32 + (sq & 1) * 16 + lr
                                   : nt * 256 + w4 * 64 + sq * 16 + lr;
                b_off[j] = (uint32_t)row * (uint32_t)KD + (uint32_t)(half * 64 + 16 * lg);
            }
        }
        const int32_t* rs = slot(k);
        // A: copy q = wave + 8 j is m-subtile q >> 1, K half q & 1; its lane
        // copies row 16 (q >> 1) + lr.  Padding rows (f < 0) copy a valid row
        // (L1: token 0; L2: the block's first row, always routed); their
        // products land only in padding rows, which are never stored.
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int q = wave + 8 * j;
            if (j == 2 && nA < 3)
                break;
            const int ri = 16 * (q >> 1) + lr;
            const int f = slot_f(rs[ri]);
            const int koff = (q & 1) * 64 + 16 * lg;
            if constexpr (L1)
                a_off[j] = (uint32_t)(f >= 0 ? f / K : 0) * (uint32_t)H + koff;
            else
                a_off[j] = (uint32_t)(f >= 0 ? row0 + ri : row0) * (uint32_t)I + koff;
        }
        // Scales (waves 0-2): lane l of wave c the activation scale of row
        // 64 c + l (c = 2: lanes 0-31), lanes 32 and 33 of wave 2 the block's
        // two weight scales (L1: gate and up block of column tile nt; L2:
        // 128-column blocks 2 nt and 2 nt + 1).
        if (nS) {
            if (wave == 2 && lane >= 32) {
                const int q = lane & 1;
                if constexpr (L1)
                    s_src = a.w1_sf + ((size_t)e * (2 * I / 128) + (q ? I / 128 + nt : nt)) * nkb;
                else
                    s_src = a.w2_sf + ((size_t)e * (H / 128) + 2 * nt + q) * nkb;
            } else {
                const int ri = 64 * wave + lane;
                const int f = slot_f(rs[ri]);
                if constexpr (L1)
                    s_src = a.x_sf + (size_t)(f >= 0 ? f / K : 0) * (H / 128);
                else
                    s_src = a.h_sf + (size_t)(f >= 0 ? row0 + ri : row0) * (I / 128);
            }
        }
    };
    // Issues the next block; returns this wave's batch size (0: nothing left).
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
        const uint8_t* abase = (L1 ? a.x : a.h) + (size_t)kb * 128;
        dma16_off(abase, a_off[0], st + wave * 1024);
        dma16_off(abase, a_off[1], st + (wave + 8) * 1024);
        if (nA == 3)
            dma16_off(abase, a_off[2], st + (wave + 16) * 1024);
        const uint8_t* wbase = i_wbase + (size_t)kb * (PK ? 32768 : 128);
        if constexpr (PK) {  // this wave's 4 KiB of the block: one offset register
            // (the instruction's constant offset moves the global and the
            // LDS address alike, so all four copies take the same M0)
            static_assert(B_COPIES == 4, "the copies below");
            const uint8_t* wb = wbase + wave * B_COPIES * 1024;
            const uint32_t sb = st + A_BYTES + wave * B_COPIES * 1024;
            dma16_off_imm<0>(wb, b_off[0], sb);
            dma16_off_imm<1024>(wb, b_off[0], sb);
            dma16_off_imm<2048>(wb, b_off[0], sb);
            dma16_off_imm<3072>(wb, b_off[0], sb);
        } else {
#pragma unroll
            for (int j = 0; j < B_COPIES; ++j)
                dma16_off(wbase, b_off[j], st + A_BYTES + (wave * B_COPIES + j) * 1024);
        }
        if (nS && (wave < 2 || lane < 34))
            dma4(s_src + kb, st + A_BYTES + B_BYTES + wave * 256);
        int n = nA + B_COPIES + nS;
        if (kb == 0) {
            issue_meta(i_k);
            n += nM;
        }
        ++i_kb;
        i_st = st + STAGE == smem_base + NSTAGE * STAGE ? smem_base : st + STAGE;
        return n;
    };

    // ---- prologue: tile 0's row sources, then blocks 0 and 1 of the stream
    {
        int mb0, nt0;
        tile_at(tile_of(0), mb0, nt0);
        if (wave < 3 && (wave < 2 || lane < 32))
            dma4(a.row_src + mb0 * BM + 64 * wave + lane, slot_lds(0) + 256 * wave);
        MOE_WAIT_VMCNT(0);
        __syncthreads();
    }
    (void)issue_next();
    int pend = issue_next();  // size of the batch issued after the block multiplied next

    v4f acc[MS][4];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    // ---- multiply side
    int m_k = 0, m_kb = 0, j = 0;
    bool live = true;    // this wave's 80 rows hold routed rows in tile m_k
    bool drain = false;  // global accesses since the last wait: wait for everything
    for (;;) {
        if (i_done && m_k >= i_k)
            break;  // tiles 0 .. i_k - 1 were valid and are finished
        // Block j has landed (only the one newer batch may be outstanding)
        // and is visible to all waves; the previous step's fragment reads
        // are done, so the stage issued below is free.
        // Every wave's batches hold at least kMinBatch copies (2 A + 4 B), so
        // vmcnt <= kMinBatch also leaves block j landed; a wave whose newer
        // batch is larger waits for its first copies too (issued a step
        // ago), for one wait instead of a branch per batch size.
        if (drain || pend == 0)
            MOE_WAIT_VMCNT(0);
        else
            MOE_WAIT_VMCNT(kMinBatch);
        drain = false;
        __syncthreads();
        // Routed rows form a prefix of each tile: a wave whose 80 rows are
        // all padding skips its MFMAs and promotions.
        if (m_kb == 0) {
            const int32_t* rs = slot(m_k);
            const int nv = __builtin_popcountll(__ballot(slot_f(rs[lane]) >= 0)) +
                           __builtin_popcountll(__ballot(slot_f(rs[64 + lane]) >= 0)) +
                           __builtin_popcountll(__ballot(lane < 32 && slot_f(rs[128 + (lane & 31)]) >= 0));
            live = __builtin_amdgcn_readfirstlane(nv > 80 * wm ? 1 : 0) != 0;
        }

        const uint8_t* st = smem + (j % NSTAGE) * STAGE;
        v8i af[MS], bf[4];
        float sa[MS][4];
        const float* s_lds = reinterpret_cast<const float*>(st + A_BYTES + B_BYTES);
        // weight scales: L1 gate / up block; L2 the wave's 128-column block
        const float sg = L1 ? s_lds[BM] : s_lds[BM + (wn >> 1)];
        const float su = L1 ? s_lds[BM + 1] : sg;
        const uint8_t* a_rd = st + wm * (MS * 2048) + lane * 16;
        const uint8_t* b_rd = st + A_BYTES + wn * 8192 + lane * 16;
        const float* sa_rd = s_lds + wm * (MS * 16) + 4 * lg;
        auto read_a = [&](int ms) {
            af[ms] = pack_frag(*reinterpret_cast<const uint4*>(a_rd + ms * 2048),
                               *reinterpret_cast<const uint4*>(a_rd + ms * 2048 + 1024));
            const float4 s4 = *reinterpret_cast<const float4*>(sa_rd + ms * 16);
            sa[ms][0] = s4.x;
            sa[ms][1] = s4.y;
            sa[ms][2] = s4.z;
            sa[ms][3] = s4.w;
        };
        // m-subtile by m-subtile: a subtile's scale products (one per row and
        // weight scale) live only for its four MFMAs
        auto multiply = [&](int ms) {
            v4f p[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                p[s] = mfma_16x16x128_e4m3(af[ms], bf[s], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float sb = (L1 && s >= 2) ? su : sg;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[ms][s][i] = fmaf(sa[ms][i] * sb, p[s][i], acc[ms][s][i]);
            }
        };
#pragma unroll
        for (int s = 0; s < 4; ++s)
            bf[s] = pack_frag(*reinterpret_cast<const uint4*>(b_rd + s * 2048),
                              *reinterpret_cast<const uint4*>(b_rd + s * 2048 + 1024));
#pragma unroll
        for (int ms = 0; ms < 3; ++ms)
            read_a(ms);

        // the copy of the block two ahead, into the stage read last step
        pend = issue_next();

        // Two phases, so that only three subtiles' A fragments are held at
        // once (the register file holds 256 per lane at two waves per SIMD):
        // the last two subtiles' fragments are read after the first two
        // subtiles' MFMAs are issued.
        if (live) {
            multiply(0);
            multiply(1);
        }
        __builtin_amdgcn_sched_barrier(0);
        read_a(3);
        read_a(4);
        if (live) {
            multiply(2);
            multiply(3);
            multiply(4);
        }
        ++j;
        if (++m_kb < nkb)
            continue;

        // ---------------------------------------------- epilogue of tile m_k
        // It works in the stage just multiplied (the next two stages hold the
        // next tile's first blocks, in flight); the barrier orders every
        // wave's fragment reads of that stage before it is overwritten, and
        // the next step's barrier orders the epilogue before the refill.
        int mb, nt;
        tile_at(tile_of(m_k), mb, nt);
        const int row0 = mb * BM;
        uint8_t* ep = smem + ((j - 1) % NSTAGE) * STAGE;
        const int32_t* m_rs = slot(m_k);
        if constexpr (L1) {
            // acc[ms][s]: rows wm*80 + 16 ms + 4 lg + i; s = 0,1 gate column
            // 32 wn + 16 s + lr of the block, s = 2,3 the matching up column.
            float* red = reinterpret_cast<float*>(ep);              // [160][4]: row, then wave wn
            float* wts = reinterpret_cast<float*>(ep + BM * 16);    // [160]: top-k weight per row
            uint8_t* qt = ep + 4096;                                // [160][128]
            // top-k weight of each row (0 for padding rows), gathered once
            float wt = 0.f;
            if (threadIdx.x < BM) {
                const int f = slot_f(m_rs[threadIdx.x]);
                wt = f >= 0 ? a.topk_w[f] : 0.f;
            }
            __syncthreads();
            if (threadIdx.x < BM)
                wts[threadIdx.x] = wt;
            __syncthreads();
            clamp_acc<MS * 4>(&acc[0][0], a.clamp);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wm * 80 + ms * 16 + 4 * lg + i;
                    const float w = wts[r];
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
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wm * 80 + ms * 16 + 4 * lg + i;
                    const float4 rm = *reinterpret_cast<const float4*>(red + r * 4);
                    const float amax = fmaxf(fmaxf(rm.x, rm.y), fmaxf(rm.z, rm.w));
                    float rsf;
                    const float sf = requant_sf(amax, a.pow2_scale, rsf);
                    const uint32_t c2 = requant_q2(acc[ms][0][i], acc[ms][1][i], sf, rsf, a.pow2_scale);
                    qt[r * 128 + wn * 32 + lr] = (uint8_t)c2;
                    qt[r * 128 + wn * 32 + 16 + lr] = (uint8_t)(c2 >> 8);
                    if (wn == 0 && lr == 0)
                        a.h_sf[(size_t)(row0 + r) * (I / 128) + nt] = sf;
                }
            __syncthreads();
            // BM rows x 128 bytes, 16 bytes per thread (rows without a slot
            // are written too: nothing reads them)
            for (int c = threadIdx.x; c < BM * 8; c += kThreads) {
                const int r = c >> 3, col = (c & 7) * 16;
                *reinterpret_cast<uint4*>(a.h + (size_t)(row0 + r) * I + nt * 128 + col) =
                    *reinterpret_cast<const uint4*>(qt + r * 128 + col);
            }
        } else {
            // acc[ms][s]: rows wm*80 + 16 ms + 4 lg + i, column 64 wn + 16 s
            // + lr.  Every wave rounds its values to bf16 at once; the rows
            // are then staged one 80-row half at a time (rows padded to 264
            // columns, so a wave's four row groups fall on different banks).
            constexpr int OT = 256 + 8;
            constexpr int HR = MS * 16;  // rows per half
            static_assert(HR * OT * 2 <= STAGE, "a staged half fits one stage");
            uint16_t* ot = reinterpret_cast<uint16_t*>(ep);  // [80][OT]
            __syncthreads();
            uint16_t hb[MS][4][4];
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        hb[ms][s][i] = f32_to_bf16(acc[ms][s][i]);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if (wm == hf) {
#pragma unroll
                    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                        for (int s = 0; s < 4; ++s)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                ot[(ms * 16 + 4 * lg + i) * OT + wn * 64 + s * 16 + lr] =
                                    hb[ms][s][i];
                }
                __syncthreads();
                for (int c = threadIdx.x; c < HR * 32; c += kThreads) {
                    const int r = c >> 5, col = (c & 31) * 8;
                    const int f = slot_f(m_rs[hf * HR + r]);
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
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};
        ++m_k;
        m_kb = 0;
    }
}

// The plain and the hot-expert walk are separate kernels, both launched; the
// planner's largest segment (status[3]) selects the one that runs.
template <bool L1, bool PK, bool HOT>
__global__ __launch_bounds__(kThreads) void gemm_lds160(FwdArgs a)
{
    const int NT = L1 ? a.I / 128 : a.H / 256;
    const bool hot = NT % 2 == 0 && a.status[3] / BM >= kHotBlocks;
    if (hot != HOT)
        return;
    lds160_walk<L1, PK, HOT>(a);
}

template <bool L1>
static hipError_t launch_lds160(const FwdArgs& a, hipStream_t s)
{
    // packed weights only (the row-major addressing needs registers this
    // kernel does not have); FP8 recipe, per-128 intermediate scales
    if (a.BM != BM || a.mx || a.sf_gran64 || !a.packed)
        return hipErrorInvalidValue;
    const int NT = L1 ? a.I / 128 : a.H / 256;
    const long long n_tiles = (long long)a.grid_mblocks * NT;
    const int nkb = L1 ? a.H / 128 : a.I / 128;
    if (n_tiles <= 0)
        return hipSuccess;
    // a tile's row sources must land before its first block is issued,
    // NSTAGE - 1 blocks ahead of the multiply
    if (nkb < NSTAGE - 1)
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
    const bool can_hot = NT % 2 == 0;
    for (int hot = 0; hot <= (can_hot ? 1 : 0); ++hot) {
        auto kern = hot ? gemm_lds160<L1, true, true> : gemm_lds160<L1, true, false>;
        err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, SMEM);
        if (err != hipSuccess)
            return err;
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), (size_t)SMEM, s, a);
        err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

hipError_t launch_l1_lds160(const FwdArgs& a, hipStream_t s) { return launch_lds160<true>(a, s); }
hipError_t launch_l2_lds160(const FwdArgs& a, hipStream_t s) { return launch_lds160<false>(a, s); }

}  // namespace moe
