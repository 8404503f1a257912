// L1 (gate+up, fused SwiGLU x topk_w + per-128 e4m3 requant) and L2 (down,
// BF16 scatter) grouped FP8 GEMMs, direct-load form for small row tiles.
//
// Math ("MegaMoE SM90 Implementation Design" §5.3): for every 128-wide K
// block the MFMA forms the block's dot product p in f32, then
//   acc = fmaf(sa[row, kb] * sb[nblk, kb], p, acc)
// with sa the 1x128 activation scale and sb the 128x128 weight scale.
// L1 epilogue (§10.1; DeepGEMM PR #440 "How it works" for the raw scale):
//   h = silu(g) * u * topk_w,  sf = max(amax_128, 1e-10) / 448,  q = e4m3(h / sf)
// with the plan's options: gate/up clamped to [-c, c] first (§10.1), sf
// rounded up to a power of two (PR #440 on #383), or one scale per 64
// columns (§5.4, then L2 multiplies each 128-K block as two 64-K halves).
// L2 epilogue (§11.1): bf16(acc) stored at partial[j][t] for the slot
// (t, j) the pool row holds.
//
// Work split (gfx950, 64-lane waves, 4 waves per 256-thread workgroup):
//   L1 tile = BM pool rows x (128 gate + 128 up) columns of one expert, so
//   the tile owns every column of one 128-wide requantisation block.  Wave w
//   owns gate columns [32w, 32w+32) and the matching up columns, so gate and
//   up of one element meet in the same lane and register.
//   L2 tile = BM pool rows x 256 output columns; wave w owns 64 columns.
// Both operands stream straight from global memory into MFMA registers:
// each weight byte is read once per row tile (decode has ~3 rows per
// expert, so the weight stream is the whole cost), the next K block is
// loaded while the current one is multiplied, and the few activation rows
// stay in L2.  The K assignment per lane group g = lane/16 is bytes
// [16g, 16g+16) and [64+16g, 64+16g+16) of the 128-byte block for both
// operands, so one load instruction covers 64 contiguous bytes of 16 rows.
#include "moe_device.h"
#include "moe_direct.h"
#include "moe_internal.h"

namespace moe {

namespace {

// Split-K partial store: each of the S K-slices of a tile writes its f32
// sums to part[slice][slot][col] for the rows that hold a routed slot
// (slot = row_src of the row); the slice counted last adds the slices in
// slice order (splitk_finish).  Lane (lg, lr) holds rows 4*lg + i of column
// lr of each 16-column subtile.
template <int MT>
__device__ __forceinline__ void store_partial(const v4f (&acc)[MT][4], float* part, size_t ld,
                                              const int32_t* row_src, int row0, const int (&col)[4],
                                              int lg)
{
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int f = row_src[row0 + 16 * ms + 4 * lg + i];
            if (f < 0)
                continue;
#pragma unroll
            for (int s = 0; s < 4; ++s)  // written through (sc1): another workgroup adds them
                __hip_atomic_store(part + (size_t)f * ld + col[s], acc[ms][s][i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
}

// ---- single-launch hand-off between tiles
//
// In the single-launch forward, L2 tiles read the h rows that L1 tiles of
// the same row block wrote moments earlier, possibly on another XCD (each
// XCD has its own L2 cache), and the combine reads L2's partials.  A
// device-scope release fence would write back the producer XCD's whole L2
// per tile (measured: ruinous), so producers write the hand-off data with
// agent-scope relaxed atomic stores (sc1: written through to memory) and
// count a tile as done only after those stores have completed (vmcnt(0))
// and the workgroup has synchronised.  Consumers touch no hand-off data
// before the count they wait for is reached.  A cache line of h or of the
// partials has exactly one producer tile and is read by nobody earlier in
// the launch (caches start clean of it at kernel start), so ordinary loads
// see it; a line of h_sf holds scales from several producer tiles, so a
// copy cached on the reader's XCD could be partly stale, and h_sf is read
// with agent-scope loads (sc1).

__device__ __forceinline__ void st_co64(void* p, uint64_t v)
{
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_co32f(const float* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_co32f(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_co128(void* p, uint4 v)
{
    st_co64(p, (uint64_t)v.x | ((uint64_t)v.y << 32));
    st_co64(reinterpret_cast<uint8_t*>(p) + 8, (uint64_t)v.z | ((uint64_t)v.w << 32));
}
// 16 bytes of h read coherently (agent scope, two 8-byte loads): with a ring
// pool the same h lines are written again later in the launch, so a copy
// another XCD's L2 kept from the previous occupant of a slot may be stale.
__device__ __forceinline__ uint4 ld_co128(const uint8_t* p)
{
    const uint64_t lo = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p + 8),
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
}

// Counts one finished tile: every thread's hand-off stores have completed
// before the workgroup barrier, then one lane bumps the counter.
__device__ __forceinline__ void count_done(int32_t* ctr)
{
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this lane's stores are done
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until *ctr >= target.  `hint` is a value of *ctr read earlier (the
// counts only grow): when it already reaches the target the workgroup goes
// on at once.  The wait is bounded: past spin_limit polls it gives up, flags
// MOE_STATUS_WAIT_TIMEOUT in the status word and lets the workgroup go on
// (the output is then invalid, but every wave exits).
__device__ __forceinline__ void wait_count(const int32_t* ctr, int target, const FwdArgs& a,
                                           int hint)
{
    if (hint >= target && a.spin_limit >= 0)
        return;
    if (threadIdx.x == 0) {
        int spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++spins > a.spin_limit) {
                __hip_atomic_fetch_or(a.status, kStatusWaitTimeout, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
    }
    __syncthreads();
}

}  // namespace

// ------------------------------------------------- L1 split-K finish

// Finishes 16-row L1 tile `tile` whose K range ran as S workgroups: adds
// the S f32 partials in slice order, then the same SwiGLU x topk_w, per-128
// (or 64) amax and e4m3 requant as the unsplit epilogue.  Run by the
// workgroup whose slice was counted last: the other slices were written
// through (sc1) and completed before they were counted, and each of their
// cache lines has that one producer, so ordinary loads see them.  Thread t:
// row t/16, gate columns 8*(t%16) .. +8 of the tile's 128-column block and
// the matching up columns; the 16 threads of a row share one wave quarter.
template <int S>
__device__ __forceinline__ void splitk_finish(const FwdArgs& a, int tile)
{
    const int I = a.I, NT = I / 128;
    const int mb = tile / NT;
    const int nt = tile - mb * NT;
    const int r = mb * 16 + (threadIdx.x >> 4);
    const int c0 = nt * 128 + (threadIdx.x & 15) * 8;
    const int f = a.row_src[r];
    float g[8], u[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        g[q] = u[q] = 0.f;
    if (f >= 0 && f < a.splitk_slots) {
#pragma unroll
        for (int k = 0; k < S; ++k) {  // all S slices' loads in flight together
            const float* row = a.splitk_part + ((size_t)k * a.splitk_slots + f) * 2 * I;
            const float4 g0 = *reinterpret_cast<const float4*>(row + c0);
            const float4 g1 = *reinterpret_cast<const float4*>(row + c0 + 4);
            const float4 u0 = *reinterpret_cast<const float4*>(row + I + c0);
            const float4 u1 = *reinterpret_cast<const float4*>(row + I + c0 + 4);
            g[0] += g0.x; g[1] += g0.y; g[2] += g0.z; g[3] += g0.w;
            g[4] += g1.x; g[5] += g1.y; g[6] += g1.z; g[7] += g1.w;
            u[0] += u0.x; u[1] += u0.y; u[2] += u0.z; u[3] += u0.w;
            u[4] += u1.x; u[5] += u1.y; u[6] += u1.z; u[7] += u1.w;
        }
    }
    const bool valid = f >= 0 && f < a.splitk_slots;
    const float w = valid ? a.topk_w[f] : 0.f;
    float hv[8], m = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        hv[q] = (silu(clamp_act(g[q], a.clamp)) * clamp_act(u[q], a.clamp)) * w;
        m = fmaxf(m, fabsf(hv[q]));
    }
    // the row's 16 threads cover 128 columns; per-64 scales: 8 threads each
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    if (!a.sf_gran64)
        m = fmaxf(m, __shfl_xor(m, 8));
    if (!valid)
        return;
    float rsf;
    const float sf = requant_sf(m, a.pow2_scale, rsf);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t c2 = requant_q2(hv[q], hv[q + 4], sf, rsf, a.pow2_scale);
        lo |= (c2 & 0xFFu) << (8 * q);
        hi |= (c2 >> 8) << (8 * q);
    }
    *reinterpret_cast<uint2*>(a.h + (size_t)r * I + c0) = make_uint2(lo, hi);
    if (a.sf_gran64) {
        if ((threadIdx.x & 7) == 0)
            a.h_sf[(size_t)r * (I / 64) + nt * 2 + ((threadIdx.x >> 3) & 1)] = sf;
    } else if ((threadIdx.x & 15) == 0) {
        a.h_sf[(size_t)r * NT + nt] = sf;
    }
}

// ------------------------------------------------------------------- L1

// L1 tile `item` (with S > 1: K slice item % S of tile item / S).  CO: the
// single-launch form (h and h_sf handed to L2 through coherent stores and
// the row block's ready count).
template <int MT, int S, bool PK, bool CO>
__device__ __forceinline__ void l1_tile(const FwdArgs& a, int item)
{
    static_assert(!CO || S == 1, "the single-launch form does not split K");
    constexpr int BM = 16 * MT;
    const int NT = a.I / 128;
    const int tile = item / S;  // S consecutive items share a tile
    const int ks = item - tile * S;
    const int mb = tile / NT;
    const int nt = tile - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0 || e >= a.E)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int H = a.H, HB = H / 128, I = a.I, K = a.K;
    const int row0 = mb * BM;
    // h / h_sf rows of this block: its pool rows, or its ring slot's
    const int hrow0 = (CO && a.ring_blocks > 0) ? (mb % a.ring_blocks) * BM : row0;
    const int kb0 = ks * HB / S, kb1 = (ks + 1) * HB / S;

    // A operand rows: row0 + 16*ms + lr.  Padding rows (row_src < 0) read
    // token 0 and are masked out of the MFMA.
    const uint8_t* aptr[MT];
    bool avalid[MT];
    // Output rows of this lane: row0 + 16*ms + 4*lg + i (four consecutive
    // row_src entries, one 16-byte load).
    const float* asf[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
        const int f = a.row_src[row0 + 16 * ms + lr];
        const int4 fo = *reinterpret_cast<const int4*>(a.row_src + row0 + 16 * ms + 4 * lg);
        avalid[ms] = f >= 0;
        aptr[ms] = a.x + (size_t)(max(f, 0) / K) * H + lg * 16;
        asf[ms][0] = a.x_sf + (size_t)(max(fo.x, 0) / K) * HB;
        asf[ms][1] = a.x_sf + (size_t)(max(fo.y, 0) / K) * HB;
        asf[ms][2] = a.x_sf + (size_t)(max(fo.z, 0) / K) * HB;
        asf[ms][3] = a.x_sf + (size_t)(max(fo.w, 0) / K) * HB;
    }
    // B operand: subtile s = 0,1 gate, 2,3 up.  kstride: bytes between K blocks.
    const uint8_t* bptr[4];
    constexpr size_t kstride = PK ? 32768 : 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if constexpr (PK) {
            bptr[s] = a.w1 + (size_t)e * 2 * I * H + (size_t)nt * HB * 32768 + (wave * 4 + s) * 2048 +
                      lane * 16;
        } else {
            const int n = (s >= 2 ? I : 0) + nt * 128 + wave * 32 + (s & 1) * 16 + lr;
            bptr[s] = a.w1 + ((size_t)e * 2 * I + n) * H + lg * 16;
        }
    }
    const float* sfg = a.w1_sf + ((size_t)e * (2 * I / 128) + nt) * HB;
    const float* sfu = a.w1_sf + ((size_t)e * (2 * I / 128) + I / 128 + nt) * HB;

    v4f acc[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    // Everything K block kb needs (fragments and both sides' scales) is
    // fetched one block ahead, so the wait before a block's MFMAs leaves
    // the next block's loads in flight (vector loads retire in order).
    struct Blk {
        Frag2 fa[MT], fb[4];
        float sa[MT][4];
        float sg, su;
    };
    auto fetch = [&](Blk& b, int kb) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b.sa[ms][i] = asf[ms][i][kb];
        b.sg = sfg[kb];
        b.su = sfu[kb];
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            b.fa[ms] = avalid[ms] ? load_frag(aptr[ms] + kb * 128) : zero_frag();
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.fb[s] = load_wfrag<PK>(bptr[s] + kb * kstride);
    };
    auto mul = [&](const Blk& b) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            const v8i av = pack_frag(b.fa[ms].lo, b.fa[ms].hi);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const v4f p = mfma_16x16x128_e4m3(av, pack_frag(b.fb[s].lo, b.fb[s].hi),
                                                  v4f{0.f, 0.f, 0.f, 0.f});
                const float sb = s >= 2 ? b.su : b.sg;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[ms][s][i] = fmaf(b.sa[ms][i] * sb, p[i], acc[ms][s][i]);
            }
        }
    };
    // Two register sets used in turn: no copy between them, so nothing
    // waits on a load before its block is multiplied.
    kloop<Blk>(kb0, kb1, fetch, mul);

    if constexpr (S > 1) {
        // gate and up columns of this lane's four subtiles in the [R, 2I] partials
        const int col[4] = {nt * 128 + wave * 32 + lr, nt * 128 + wave * 32 + 16 + lr,
                            I + nt * 128 + wave * 32 + lr, I + nt * 128 + wave * 32 + 16 + lr};
        store_partial<MT>(acc, a.splitk_part + (size_t)ks * a.splitk_slots * 2 * I, 2 * (size_t)I,
                          a.row_src, row0, col, lg);
        // Count the slice once its stores have completed; the tile's last
        // slice to be counted finishes the tile (one counter per tile,
        // zeroed by the planner).
        static_assert(MT == 1, "split-K runs on 16-row tiles");
        __shared__ int s_last;
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this lane's stores are done
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(a.sync + kSyncReady + tile, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        if (s_last)
            splitk_finish<S>(a, tile);
        return;
    }
    const bool epi = true;

    // ---- epilogue: SwiGLU x topk_w, per-row amax over the 128 columns,
    // e4m3 requant, coalesced store through LDS.
    __shared__ float red[4][BM];
    __shared__ uint8_t qt[BM][128];
    float hv[MT][2][4];
    float wrow[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int f = a.row_src[row0 + 16 * ms + 4 * lg + i];
            wrow[ms][i] = f >= 0 ? a.topk_w[f] : 0.f;
        }
    clamp_acc<MT * 4>(&acc[0][0], a.clamp);
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const float g = acc[ms][s][i];
                const float u = acc[ms][s + 2][i];
                const float v = (silu(g) * u) * wrow[ms][i];
                hv[ms][s][i] = v;
                m = fmaxf(m, fabsf(v));
            }
            m = max16_nonneg(m);
            if (epi && lr == 0)
                red[wave][16 * ms + 4 * lg + i] = m;
        }
    }
    __syncthreads();
    if (epi) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * ms + 4 * lg + i;
                // per-64 scales: waves 2b, 2b+1 share block b of the tile
                const float amax = a.sf_gran64 ? fmaxf(red[wave & 2][r], red[(wave & 2) + 1][r])
                                               : fmaxf(fmaxf(red[0][r], red[1][r]),
                                                       fmaxf(red[2][r], red[3][r]));
                float rsf;
                const float sf = requant_sf(amax, a.pow2_scale, rsf);
                const uint32_t c2 = requant_q2(hv[ms][0][i], hv[ms][1][i], sf, rsf, a.pow2_scale);
                qt[r][wave * 32 + lr] = (uint8_t)c2;
                qt[r][wave * 32 + 16 + lr] = (uint8_t)(c2 >> 8);
                if ((a.sf_gran64 ? (wave & 1) == 0 : wave == 0) && lr == 0) {
                    float* dst = a.sf_gran64 ? a.h_sf + (size_t)(hrow0 + r) * (I / 64) + nt * 2 + (wave >> 1)
                                             : a.h_sf + (size_t)(hrow0 + r) * (I / 128) + nt;
                    if constexpr (CO)
                        st_co32f(dst, sf);
                    else
                        *dst = sf;
                }
            }
        }
    }
    __syncthreads();
    // BM rows x 128 bytes, 16 bytes per thread.
    for (int c = threadIdx.x; c < BM * 8; c += 256) {
        const int r = c >> 3, col = (c & 7) * 16;
        if (a.row_src[row0 + r] >= 0) {
            uint8_t* dst = a.h + (size_t)(hrow0 + r) * I + nt * 128 + col;
            const uint4 v = *reinterpret_cast<const uint4*>(&qt[r][col]);
            if constexpr (CO)
                st_co128(dst, v);
            else
                *reinterpret_cast<uint4*>(dst) = v;
        }
    }
    if constexpr (CO)
        count_done(a.sync + kSyncReady + mb);
}

// 32-row tiles: bounded to two waves per SIMD (<= 256 VGPRs, no spills; 260
// unbounded, i.e. one wave per SIMD).
template <int MT, int S, bool PK>
__global__ __launch_bounds__(256, MT == 2 ? 2 : 1) void l1_direct(FwdArgs a)
{
    l1_tile<MT, S, PK, false>(a, blockIdx.x);
}

// 16-row tiles (decode), under a register request that the compiler meets
// with 149-154 VGPRs and no AGPRs.  Left to itself it takes 152 VGPRs + 16
// AGPRs, and workgroup timestamps then show two workgroups resident per CU.
// Measured: L1 at one token 26.7 -> 25.4 us, equal within noise at 16-256.
template <int S, bool PK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_num_vgpr(128))) void l1_direct16(FwdArgs a)
{
    l1_tile<1, S, PK, false>(a, blockIdx.x);
}

// Finishes 16-row L2 tile `tile` (row block x 256-column tile) whose K
// range ran as S workgroups: adds the S f32 slices in slice order and
// stores the bf16 partial rows, as the unsplit epilogue does.  Run by the
// workgroup whose slice was counted last (the slices were written through
// and completed before they were counted; each cache line has one
// producer).  Thread t: row t/16, columns 16 (t%16) .. +16 of the tile.
template <int S>
__device__ __forceinline__ void l2_splitk_finish(const FwdArgs& a, int tile)
{
    const int H = a.H, NT = (H + 255) / 256;
    const int mb = tile / NT;
    const int nt = tile - mb * NT;
    const int f = a.row_src[mb * 16 + (threadIdx.x >> 4)];
    const int c0 = nt * 256 + (threadIdx.x & 15) * 16;
    if (f < 0 || f >= a.splitk_slots || c0 >= H)
        return;
    float p[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
        p[q] = 0.f;
#pragma unroll
    for (int k = 0; k < S; ++k) {  // all S slices' loads in flight together
        const float* row = a.splitk_part + ((size_t)k * a.splitk_slots + f) * H + c0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 x = *reinterpret_cast<const float4*>(row + 4 * v);
            p[4 * v] += x.x;
            p[4 * v + 1] += x.y;
            p[4 * v + 2] += x.z;
            p[4 * v + 3] += x.w;
        }
    }
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        w[q] = f32x2_to_bf16x2(p[2 * q], p[2 * q + 1]);
    const int t = f / a.K, j = f - t * a.K;
    uint4* dst = reinterpret_cast<uint4*>(a.partial + ((size_t)j * a.T + t) * H + c0);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// ------------------------------------------------------------------- L2

// L2 tile `tile`.  CO: the single-launch form (waits for the row block's
// L1 tiles, reads h coherently, hands the partials to the combine through
// coherent stores and the L2 done count).
// WV waves per workgroup: the workgroup covers WV / 4 consecutive 256-column
// tiles (a wave with no columns left re-reads column block 0 of the
// expert and stores nothing).
// G64: per-64 intermediate scales ("MegaMoE SM90 Implementation Design"
// §5.4): each 128-K block is multiplied as its two 64-K halves -- the A
// fragment's bytes 0..15 are K 0..63 of every lane group, bytes 16..31 are
// K 64..127, so zeroing one half leaves the other -- and each half is
// promoted with its own activation scale.
// S > 1 (16-row 4-wave tiles of one or two tokens, never CO): item = tile
// * S + K slice; each slice writes its f32 sums through to
// splitk_part[slice][slot][H], and the slice counted last adds them in
// slice order and stores the bf16 partials (l2_splitk_finish).
template <int MT, bool PK, bool CO, int WV = 4, bool G64 = false, int S = 1>
__device__ __forceinline__ void l2_tile_body(const FwdArgs& a, int item, int hint)
{
    static_assert(!CO || S == 1, "the single launch does not split K");
    static_assert(S == 1 || (MT == 1 && WV == 4), "split-K runs on 16-row 4-wave tiles");
    constexpr int BM = 16 * MT;
    constexpr int NTG = WV / 4;
    const int H = a.H, I = a.I, IB = I / 128, K = a.K, T = a.T;
    const int NT = (H + 255) / 256;  // H % 256 == 128: the last tile has 2 idle waves
    const int NG = (NT + NTG - 1) / NTG;
    const int tile = item / S;  // S consecutive items share a tile
    const int ks = item - tile * S;
    const int mb = tile / NG;
    const int g = tile - mb * NG;
    const int e = a.mblock_expert[mb];
    if (e < 0 || e >= a.E)
        return;
    if constexpr (CO)
        wait_count(a.sync + kSyncReady + mb, a.I / 128, a, hint);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = mb * BM;
    // h / h_sf rows of this block: its pool rows, or its ring slot's
    const bool ring = CO && a.ring_blocks > 0;
    const int hrow0 = ring ? (mb % a.ring_blocks) * BM : row0;
    const int kb0 = ks * IB / S, kb1 = (ks + 1) * IB / S;
    const int nt_w = g * NTG + (wave >> 2);               // this wave's 256-column tile
    const bool busy = nt_w < NT && nt_w * 256 + (wave & 3) * 64 < H;
    const int nt = busy ? nt_w : 0;                       // idle waves read tile 0
    const int w4 = wave & 3;

    const uint8_t* aptr[MT];
    bool avalid[MT];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
        const int r = 16 * ms + lr;
        avalid[ms] = a.row_src[row0 + r] >= 0;
        aptr[ms] = a.h + (size_t)(hrow0 + r) * I + lg * 16;
    }
    const float* asf[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            asf[ms][i] = a.h_sf + (size_t)(hrow0 + 16 * ms + 4 * lg + i) * (G64 ? 2 * IB : IB);
    // A wave's 64 columns are either all inside H or all past it; an idle
    // wave re-reads column block 0 and stores nothing.
    const int ncol0 = busy ? nt * 256 + w4 * 64 : 0;
    const uint8_t* bptr[4];
    constexpr size_t kstride = PK ? 32768 : 128;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if constexpr (PK)
            bptr[s] = a.w2 + (size_t)e * H * I + (size_t)nt * IB * 32768 +
                      ((busy ? w4 : 0) * 4 + s) * 2048 + lane * 16;
        else
            bptr[s] = a.w2 + ((size_t)e * H + ncol0 + s * 16 + lr) * I + lg * 16;
    }
    const float* sfb = a.w2_sf + ((size_t)e * (H / 128) + ncol0 / 128) * IB;

    v4f acc[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    // One K block ahead, as in l1_direct.
    struct Blk {
        Frag2 fa[MT], fb[4];
        float sa[MT][4];
        float sa2[G64 ? MT : 1][4];  // G64: the second half's scales
        float sb;
    };
    auto fetch = [&](Blk& b, int kb) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (G64) {
                    b.sa[ms][i] = asf[ms][i][2 * kb];
                    b.sa2[ms][i] = asf[ms][i][2 * kb + 1];
                } else if constexpr (CO) {
                    b.sa[ms][i] = ld_co32f(asf[ms][i] + kb);
                } else {
                    b.sa[ms][i] = asf[ms][i][kb];
                }
            }
        b.sb = sfb[kb];
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            if (!avalid[ms]) {
                b.fa[ms] = zero_frag();
            } else if (ring) {
                b.fa[ms].lo = ld_co128(aptr[ms] + kb * 128);
                b.fa[ms].hi = ld_co128(aptr[ms] + kb * 128 + 64);
            } else {
                b.fa[ms] = load_frag(aptr[ms] + kb * 128);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.fb[s] = load_wfrag<PK>(bptr[s] + kb * kstride);
    };
    auto mul = [&](const Blk& b) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            if constexpr (G64) {
                const uint4 z = make_uint4(0, 0, 0, 0);
                const v8i alo = pack_frag(b.fa[ms].lo, z), ahi = pack_frag(z, b.fa[ms].hi);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const v8i bv = pack_frag(b.fb[s].lo, b.fb[s].hi);
                    const v4f plo = mfma_16x16x128_e4m3(alo, bv, v4f{0.f, 0.f, 0.f, 0.f});
                    const v4f phi = mfma_16x16x128_e4m3(ahi, bv, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[ms][s][i] = fmaf(b.sa[ms][i] * b.sb, plo[i], acc[ms][s][i]);
                        acc[ms][s][i] = fmaf(b.sa2[ms][i] * b.sb, phi[i], acc[ms][s][i]);
                    }
                }
            } else {
                const v8i av = pack_frag(b.fa[ms].lo, b.fa[ms].hi);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const v4f p = mfma_16x16x128_e4m3(av, pack_frag(b.fb[s].lo, b.fb[s].hi),
                                                      v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[ms][s][i] = fmaf(b.sa[ms][i] * b.sb, p[i], acc[ms][s][i]);
                }
            }
        }
    };
    kloop<Blk>(kb0, kb1, fetch, mul);

    if constexpr (S > 1) {
        // ---- K slice: its f32 sums written through, row by row (16 lanes =
        // 64 bytes); counted once stored; the last slice finishes the tile
        if (busy) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = a.row_src[row0 + 4 * lg + i];
                if (f < 0 || f >= a.splitk_slots)
                    continue;
                float* dst = a.splitk_part + ((size_t)ks * a.splitk_slots + f) * H + ncol0 + lr;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    __hip_atomic_store(dst + s * 16, acc[0][s][i], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __shared__ int s_last;
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this lane's stores are done
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(a.sync + kSyncReady + a.grid_mblocks * (I / 128) + tile,
                                            1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        if (s_last)
            l2_splitk_finish<S>(a, tile);
        return;
    }

    // ---- epilogue: bf16, stage BM x 256 in LDS, 16-byte stores to the
    // (slot, token) row of the partial buffer.
    __shared__ uint16_t ot[BM][WV * 64 + 8];
    {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ot[16 * ms + 4 * lg + i][wave * 64 + s * 16 + lr] = f32_to_bf16(acc[ms][s][i]);
    }
    __syncthreads();
    const int gcol0 = g * NTG * 256;  // first column of the workgroup
    for (int c = threadIdx.x; c < BM * WV * 8; c += WV * 64) {
        const int r = c / (WV * 8), col = (c - r * WV * 8) * 8;
        const int f = a.row_src[row0 + r];
        if (f >= 0 && gcol0 + col < H) {
            const int t = f / K, j = f - t * K;
            uint4 v;
            v.x = (uint32_t)ot[r][col + 0] | ((uint32_t)ot[r][col + 1] << 16);
            v.y = (uint32_t)ot[r][col + 2] | ((uint32_t)ot[r][col + 3] << 16);
            v.z = (uint32_t)ot[r][col + 4] | ((uint32_t)ot[r][col + 5] << 16);
            v.w = (uint32_t)ot[r][col + 6] | ((uint32_t)ot[r][col + 7] << 16);
            uint16_t* dst = a.partial + ((size_t)j * T + t) * H + gcol0 + col;
            if constexpr (CO)
                st_co128(dst, v);
            else
                *reinterpret_cast<uint4*>(dst) = v;
        }
    }
}

template <int MT, bool PK, bool CO>
__device__ __forceinline__ void l2_tile(const FwdArgs& a, int tile, int hint = 0)
{
    l2_tile_body<MT, PK, CO>(a, tile, hint);
    if constexpr (CO) {
        count_done(a.sync + kSyncL2Done);  // every L2 item counts, idle ones too
        // ring pool: and per row block, for the L1 tiles that reuse its slot
        if (a.ring_blocks > 0 && threadIdx.x == 0)
            __hip_atomic_fetch_add(a.sync + kSyncReady + a.num_mblocks + tile / ((a.H + 255) / 256), 1,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int MT, bool PK, int WV = 4, bool G64 = false, int S = 1>
__global__ __launch_bounds__(WV * 64, MT == 2 && PK && !G64 ? 2 : 1) void l2_direct(FwdArgs a)
{
    l2_tile_body<MT, PK, false, WV, G64, S>(a, blockIdx.x, 0);
}

// -------------------------------------------------------------- combine

// y[t, n] = bf16( sum over active slots j ascending of f32(partial[j][t][n]) )
// ("MegaMoE SM90 Implementation Design" §11.2).  8 columns per thread.
// Combine chunk `blk` (256 threads x 8 columns).  CO: the single-launch
// form (waits until all n_l2 L2 items are counted, reads the partials
// coherently).
template <bool CO>
__device__ __forceinline__ void combine_chunk(const FwdArgs& a, int blk, int n_l2, int hint = 0)
{
    if constexpr (CO)
        wait_count(a.sync + kSyncL2Done, n_l2, a, hint);
    const int H8 = a.H / 8;
    const long long g = (long long)blk * 256 + threadIdx.x;
    if (g >= (long long)a.T * H8)
        return;
    const int t = (int)(g / H8);
    const int c = (int)(g - (long long)t * H8) * 8;
    float s[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        s[q] = 0.f;
    auto add = [&](const uint4& v) {
        s[0] += bf16_to_f32(v.x & 0xFFFFu);
        s[1] += bf16_to_f32(v.x >> 16);
        s[2] += bf16_to_f32(v.y & 0xFFFFu);
        s[3] += bf16_to_f32(v.y >> 16);
        s[4] += bf16_to_f32(v.z & 0xFFFFu);
        s[5] += bf16_to_f32(v.z >> 16);
        s[6] += bf16_to_f32(v.w & 0xFFFFu);
        s[7] += bf16_to_f32(v.w >> 16);
    };
    const uint16_t* prow = a.partial + (size_t)t * a.H + c;  // slot j: + j * T * H
    const size_t jstride = (size_t)a.T * a.H;
    if (a.K <= 8) {
        // the rows of all valid slots are loaded before any is added, so
        // their loads are in flight together (a masked slot's row is neither
        // read nor added); the sum runs over the valid slots in ascending j
        bool ok[8];
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < a.K) {
                const int e = a.idx[t * a.K + j];
                ok[j] = e >= 0 && e < a.E;
                if (ok[j])
                    v[j] = *reinterpret_cast<const uint4*>(prow + j * jstride);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < a.K && ok[j])
                add(v[j]);
    } else {
        for (int j = 0; j < a.K; ++j) {
            const int e = a.idx[t * a.K + j];
            if (e >= 0 && e < a.E)
                add(*reinterpret_cast<const uint4*>(prow + j * jstride));
        }
    }
    uint4 o;
    o.x = f32x2_to_bf16x2(s[0], s[1]);
    o.y = f32x2_to_bf16x2(s[2], s[3]);
    o.z = f32x2_to_bf16x2(s[4], s[5]);
    o.w = f32x2_to_bf16x2(s[6], s[7]);
    *reinterpret_cast<uint4*>(a.y + (size_t)t * a.H + c) = o;
}

__global__ __launch_bounds__(256) void combine_kernel(FwdArgs a)
{
    combine_chunk<false>(a, blockIdx.x, 0);
}

// ------------------------------------------------- single launch (a6)

// L1 tiles, L2 tiles and combine chunks of one forward in one launch
// ("07 · MegaMoE" §5-6: L2 tiles of a row block start once all of its L1
// tiles are in).  Items are numbered L1 tiles first, then L2 tiles, then
// combine chunks, and workgroups claim them in that order from a counter
// (two claims ahead, so the claim's latency hides behind the current item).
// An item only ever waits for items with smaller numbers, which were
// claimed earlier by running workgroups; a workgroup that holds an
// unstarted claim is busy with an earlier item, and L1 items never wait, so
// every wait ends (no co-residency is assumed).  While an item runs, the
// workgroup also reads the count the next claimed item will wait for, so a
// row block that is long finished costs no round trip.
template <int MT, bool PK>
__global__ __launch_bounds__(256) void fused_direct(FwdArgs a)
{
    // Items of the row blocks that hold routed slots only (the planner's
    // used-row count): the pool's capacity T*K + E*(BM - 1) rows is mostly
    // empty at small T, and every item costs a claim on the shared queue.
    const int used_mb = min(a.num_mblocks, a.status[2] / (16 * MT));
    const int n1 = used_mb * (a.I / 128);
    const int NT2 = (a.H + 255) / 256;
    const int n2 = used_mb * NT2;
    const int n3 = (int)(((long long)a.T * (a.H / 8) + 255) / 256);
    const int total = n1 + n2 + n3;
    int32_t* queue = a.sync + kSyncQueue;
    // counter an item waits for (null: none)
    auto wait_ctr = [&](int it) -> const int32_t* {
        if (it < n1 || it >= total)
            return nullptr;
        if (it < n1 + n2)
            return a.sync + kSyncReady + (it - n1) / NT2;
        return a.sync + kSyncL2Done;
    };
    __shared__ int s_cur[2], s_nxt[2], s_hint[2];
    if (threadIdx.x == 0) {
        s_cur[0] = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_nxt[0] = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_hint[0] = 0;
    }
    __syncthreads();
    int slot = 0;
    for (;;) {
        const int cur = s_cur[slot], nxt = s_nxt[slot], hint = s_hint[slot];
        if (cur >= total)
            break;
        int claim = total, nhint = 0;
        if (threadIdx.x == 0) {
            if (nxt < total)
                claim = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (const int32_t* c = wait_ctr(nxt))
                nhint = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (cur < n1)
            l1_tile<MT, 1, PK, true>(a, cur);
        else if (cur < n1 + n2)
            l2_tile<MT, PK, true>(a, cur - n1, hint);
        else
            combine_chunk<true>(a, cur - n1 - n2, n2, hint);
        slot ^= 1;
        if (threadIdx.x == 0) {
            s_cur[slot] = nxt;
            s_nxt[slot] = claim;
            s_hint[slot] = nhint;
        }
        __syncthreads();
    }
}

// The single launch over a ring pool (DeepGEMM PR #440 "How it works",
// "Ring sizing, recycling"): items are the route_stream's lag-ordered
// stream, then the combine chunks.  Row block mb writes h / h_sf slot
// mb % ring_blocks, so its L1 tiles first wait until the L2 tiles of the
// slot's previous occupant, block mb - ring_blocks, are all finished (a
// per-block count, bumped after the tile's loads have returned).  The
// stream puts those L2 tiles before these L1 tiles whenever the ring holds
// 8 (lag + group) + 1 blocks (the host sizes it 8 (lag + group) + 4), and
// an L2 tile only waits for its own block's L1 tiles, earlier in the stream:
// every wait is for smaller item numbers, as in fused_direct, and ends.
// Claims run three deep: while an item runs, thread 0 claims the item after
// next, reads the next item's table entry, and reads the count that the
// item after this one will wait for.
template <int MT, bool PK>
__global__ __launch_bounds__(256) void fused_ring(FwdArgs a)
{
    const int used_mb = min(a.num_mblocks, a.status[2] / (16 * MT));
    const int NT1 = a.I / 128, NT2 = (a.H + 255) / 256;
    const int S = min(a.sync[kSyncStreamItems], used_mb * (NT1 + NT2));
    const int n2 = used_mb * NT2;
    const int n3 = (int)(((long long)a.T * (a.H / 8) + 255) / 256);
    const int total = S + n3;
    const int RB = a.ring_blocks;
    int32_t* queue = a.sync + kSyncQueue;
    const int32_t* l2_done = a.sync + kSyncReady + a.num_mblocks;
    auto code_of = [&](int q) { return q < S ? a.item_tab[q] : -1; };
    // counter item q (table entry code) waits for, and its target
    auto wait_of = [&](int q, int code, int& target) -> const int32_t* {
        if (q >= total)
            return nullptr;
        if (q >= S) {
            target = n2;
            return a.sync + kSyncL2Done;
        }
        const int tile = code & ~kItemL2;
        if (code & kItemL2) {
            target = NT1;
            return a.sync + kSyncReady + tile / NT2;
        }
        const int mb = tile / NT1;
        target = NT2;
        return mb >= RB ? l2_done + (mb - RB) : nullptr;
    };
    __shared__ int s_cur[2], s_code[2], s_hint[2], s_nxt[2], s_ncode[2], s_nxt2[2];
    if (threadIdx.x == 0) {
        const int c0 = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int c1 = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int c2 = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_cur[0] = c0;
        s_code[0] = code_of(c0);
        s_hint[0] = 0;
        s_nxt[0] = c1;
        s_ncode[0] = code_of(c1);
        s_nxt2[0] = c2;
    }
    __syncthreads();
    int slot = 0;
    for (;;) {
        const int cur = s_cur[slot];
        if (cur >= total)
            break;
        const int code = s_code[slot], hint = s_hint[slot];
        const int nxt = s_nxt[slot], ncode = s_ncode[slot], nxt2 = s_nxt2[slot];
        int claim = total, code2 = -1, nhint = 0;
        if (threadIdx.x == 0) {
            if (nxt2 < total)
                claim = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            code2 = code_of(nxt2);
            int tgt = 0;
            if (const int32_t* c = wait_of(nxt, ncode, tgt))
                nhint = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (cur < S) {
            const int tile = code & ~kItemL2;
            if (code & kItemL2) {
                l2_tile<MT, PK, true>(a, tile, hint);
            } else {
                const int mb = tile / NT1;
                if (mb >= RB)
                    wait_count(l2_done + (mb - RB), NT2, a, hint);
                l1_tile<MT, 1, PK, true>(a, tile);
            }
        } else {
            combine_chunk<true>(a, cur - S, n2, hint);
        }
        slot ^= 1;
        if (threadIdx.x == 0) {
            s_cur[slot] = nxt;
            s_code[slot] = ncode;
            s_hint[slot] = nhint;
            s_nxt[slot] = nxt2;
            s_ncode[slot] = code2;
            s_nxt2[slot] = claim;
        }
        __syncthreads();
    }
}

template <bool PK>
static hipError_t launch_l1_t(const FwdArgs& a, hipStream_t s)
{
    const unsigned tiles = a.grid_mblocks * (a.I / 128);
    switch (a.BM) {
    case 16:
        if (a.split_l1 > 1) {
            if (!a.sync)  // the slice counts
                return hipErrorInvalidValue;
            switch (a.split_l1) {
            case 2:  // (the last slice of each tile finishes it)
                hipLaunchKernelGGL((l1_direct16<2, PK>), dim3(tiles * 2), dim3(256), 0, s, a);
                break;
            case 4:
                hipLaunchKernelGGL((l1_direct16<4, PK>), dim3(tiles * 4), dim3(256), 0, s, a);
                break;
            default: return hipErrorInvalidValue;
            }
        } else {
            hipLaunchKernelGGL((l1_direct16<1, PK>), dim3(tiles), dim3(256), 0, s, a);
        }
        break;
    case 32: hipLaunchKernelGGL((l1_direct<2, 1, PK>), dim3(tiles), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((l1_direct<4, 1, PK>), dim3(tiles), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool PK>
static hipError_t launch_l2_t(const FwdArgs& a, hipStream_t s)
{
    const unsigned tiles = a.grid_mblocks * ((a.H + 255) / 256);
    if (a.sf_gran64) {  // per-64 intermediate scales: dual-half L2, 4-wave tiles
        switch (a.BM) {
        case 16: hipLaunchKernelGGL((l2_direct<1, PK, 4, true>), dim3(tiles), dim3(256), 0, s, a); break;
        case 32: hipLaunchKernelGGL((l2_direct<2, PK, 4, true>), dim3(tiles), dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL((l2_direct<4, PK, 4, true>), dim3(tiles), dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (a.split_l2 > 1) {  // 16-row 4-wave tiles, K over split_l2 workgroups
        if (a.BM != 16 || a.l2_wide || !a.sync)
            return hipErrorInvalidValue;
        switch (a.split_l2 * (a.sf_gran64 ? -1 : 1)) {
        case 2: hipLaunchKernelGGL((l2_direct<1, PK, 4, false, 2>), dim3(tiles * 2), dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((l2_direct<1, PK, 4, false, 4>), dim3(tiles * 4), dim3(256), 0, s, a); break;
        case -2: hipLaunchKernelGGL((l2_direct<1, PK, 4, true, 2>), dim3(tiles * 2), dim3(256), 0, s, a); break;
        case -4: hipLaunchKernelGGL((l2_direct<1, PK, 4, true, 4>), dim3(tiles * 4), dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (a.BM) {
    case 16:
        if (a.l2_wide) {  // two 256-column tiles per workgroup, 8 waves
            const unsigned groups = a.grid_mblocks * (((a.H + 255) / 256 + 1) / 2);
            hipLaunchKernelGGL((l2_direct<1, PK, 8>), dim3(groups), dim3(512), 0, s, a);
        } else {
            hipLaunchKernelGGL((l2_direct<1, PK, 4>), dim3(tiles), dim3(256), 0, s, a);
        }
        break;
    case 32: hipLaunchKernelGGL((l2_direct<2, PK>), dim3(tiles), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((l2_direct<4, PK>), dim3(tiles), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int MT, bool PK>
static hipError_t launch_fused_t(const FwdArgs& a, hipStream_t s)
{
    auto kern = a.ring_blocks > 0 ? fused_ring<MT, PK> : fused_direct<MT, PK>;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess)
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess)
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0);
    if (err != hipSuccess)
        return err;
    if (cus <= 0 || per_cu <= 0)
        return hipErrorInvalidConfiguration;
    const long long n = (long long)a.grid_mblocks * (a.I / 128 + (a.H + 255) / 256) +
                        ((long long)a.T * (a.H / 8) + 255) / 256;
    long long cap = (long long)cus * per_cu;  // resident workgroups
    if (a.grid_cap > 0 && cap > a.grid_cap)
        cap = a.grid_cap;
    const unsigned grid = (unsigned)(n < cap ? n : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fused(const FwdArgs& a, hipStream_t s)
{
    if (a.split_l1 != 1 || !a.sync || !a.status)
        return hipErrorInvalidValue;
    // ring pool: the stream tables, and a ring that holds the live set
    if (a.ring_blocks > 0 &&
        (!a.item_tab || a.lag_units < 1 ||
         a.ring_blocks < kUnitBlocks * (a.lag_units + kStreamGroup) + 1))
        return hipErrorInvalidValue;
    switch (a.BM) {
    case 16: return a.packed ? launch_fused_t<1, true>(a, s) : launch_fused_t<1, false>(a, s);
    case 32: return a.packed ? launch_fused_t<2, true>(a, s) : launch_fused_t<2, false>(a, s);
    case 64: return a.packed ? launch_fused_t<4, true>(a, s) : launch_fused_t<4, false>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_l1(const FwdArgs& a, int kernel, hipStream_t s)
{
    if (kernel == 1)
        return launch_l1_lds(a, s);
    if (kernel == 2)
        return launch_l1_sa(a, s);
    if (kernel == 3)
        return launch_l1_lds160(a, s);
    return a.packed ? launch_l1_t<true>(a, s) : launch_l1_t<false>(a, s);
}

hipError_t launch_l2(const FwdArgs& a, int kernel, hipStream_t s)
{
    if (kernel == 1)
        return launch_l2_lds(a, s);
    if (kernel == 2)
        return launch_l2_sa(a, s);
    if (kernel == 3)
        return launch_l2_lds160(a, s);
    return a.packed ? launch_l2_t<true>(a, s) : launch_l2_t<false>(a, s);
}

hipError_t launch_combine(const FwdArgs& a, hipStream_t s)
{
    const long long n = (long long)a.T * (a.H / 8);
    const dim3 grid((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
