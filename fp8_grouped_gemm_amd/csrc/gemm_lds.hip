// L1 / L2 grouped FP8 GEMMs for large row tiles (prefill): 128 pool rows x
// 256 columns per workgroup, operands staged through LDS.
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
// 128 activation scales) is copied global -> LDS with gfx950's
// global_load_lds_dwordx4 (each lane's 16 bytes land at base + 16 * lane, so
// one wave instruction fills 1 KiB in MFMA fragment order: [subtile][half]
// [lane][16 B], conflict-free ds_read_b128).  Three LDS stages keep two K
// blocks in flight while the third is multiplied.  The copy is issued as
// inline assembly and its completion tracked by explicit vmcnt waits: every
// wave issues exactly kCopiesPerStage copies per stage, so "all but the
// newest stage landed" is vmcnt <= kCopiesPerStage.  Each step reads all its
// fragments into registers before issuing the next copy, and the barrier at
// the top of a step orders the previous step's reads before a stage is
// overwritten.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 256;
constexpr int A_BYTES = BM * 128;   // 16 KiB: 8 m-subtiles x 2 halves x 1 KiB
constexpr int B_BYTES = BN * 128;   // 32 KiB: 16 n-subtiles x 2 halves x 1 KiB
constexpr int S_BYTES = 8 * 256;    // one 64-scale copy per wave; rows 0..127 are the first 512 B
constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
constexpr int NSTAGE = 3;
constexpr int kThreads = 512;
constexpr int kCopiesPerStage = 2 + 4 + 1;  // A halves, B halves, scales (per wave)

// s_waitcnt with vmcnt = n (n < 16) and no wait on expcnt / lgkmcnt
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
#define MOE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0xF70 | (n))
static_assert(kCopiesPerStage < 16, "vmcnt immediate");

// Asynchronous copy global -> LDS of 16 (or 4) bytes per lane to
// lds_base + 16 * lane (4 * lane).  lds_base must be wave-uniform.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base)
                 : "memory", "m0");
}

__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_base)
                 : "memory", "m0");
}

// 32-bit LDS offset of a __shared__ object (what M0 expects).
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p)
{
    const __attribute__((address_space(3))) uint8_t* lp =
        (const __attribute__((address_space(3))) uint8_t*)p;
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lp);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* sub_base, int lane)
{
    const uint4 lo = *reinterpret_cast<const uint4*>(sub_base + lane * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(sub_base + 1024 + lane * 16);
    return pack_frag(lo, hi);
}

// Address of the 16 bytes lane `lane` copies for weight subtile `sub`
// (packed order w4 * 4 + s, see pack.hip), half `half`, K block kb.
template <bool L1, bool PK>
__device__ __forceinline__ const uint8_t* weight_src(const FwdArgs& a, int e, int nt, int kb,
                                                     int sub, int half, int lane)
{
    const int H = a.H, I = a.I;
    if constexpr (PK) {
        const size_t nkb = L1 ? H / 128 : I / 128;
        const uint8_t* base = L1 ? a.w1 + (size_t)e * 2 * I * H : a.w2 + (size_t)e * H * I;
        return base + ((size_t)nt * nkb + kb) * 32768 + (sub * 2 + half) * 1024 + lane * 16;
    } else {
        const int w4 = sub >> 2, s = sub & 3, lr = lane & 15, lg = lane >> 4;
        const int col = kb * 128 + half * 64 + 16 * lg;
        if constexpr (L1) {
            const int row = (s >= 2 ? I : 0) + nt * 128 + w4 * 32 + (s & 1) * 16 + lr;
            return a.w1 + ((size_t)e * 2 * I + row) * H + col;
        } else {
            const int row = nt * 256 + w4 * 64 + s * 16 + lr;
            return a.w2 + ((size_t)e * H + row) * I + col;
        }
    }
}

}  // namespace

// L1 (gate + up) when L1 is true, L2 (down) otherwise.
template <bool L1, bool PK>
__global__ __launch_bounds__(kThreads) void gemm_lds(FwdArgs a)
{
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int H = a.H, I = a.I, K = a.K, T = a.T;
    const int NT = L1 ? I / 128 : H / 256;
    const int nkb = L1 ? H / 128 : I / 128;
    const int mb = blockIdx.x / NT;
    const int nt = blockIdx.x - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0)
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = mb * BM;

    // ---- copy sources for K block 0 (later blocks add 128 bytes per block
    // for activations and scales' kb index).
    // A: wave v copies m-subtile halves q = 2v, 2v+1 (subtile q>>1, half q&1).
    const uint8_t* a_src[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = wave * 2 + j, ms = q >> 1, half = q & 1;
        const int r = row0 + ms * 16 + lr;
        if constexpr (L1) {
            const int f = a.row_src[r];
            a_src[j] = a.x + (size_t)(f >= 0 ? f / K : 0) * H + half * 64 + 16 * lg;
        } else {
            a_src[j] = a.h + (size_t)r * I + half * 64 + 16 * lg;
        }
    }
    // Scales ride in the stage too (one 4-byte-per-lane copy per wave):
    // waves 0 and 1 copy the activation scales of rows [0, 64) and
    // [64, 128) into the first 512 bytes of the scale area, wave 2 copies
    // the block's two weight scales (L1: gate and up block; L2: the two
    // 128-column blocks of the tile) into lanes 0 and 1 of its slot, and the
    // other waves copy duplicates, so that every wave issues the same number
    // of copies and the K loop holds no other vector memory access.
    const float* s_src;
    if (wave == 2) {
        if constexpr (L1)
            s_src = a.w1_sf + ((size_t)e * (2 * I / 128) + ((lane & 1) ? I / 128 + nt : nt)) * nkb;
        else
            s_src = a.w2_sf + ((size_t)e * (H / 128) + 2 * nt + (lane & 1)) * nkb;
    } else {
        const int r = row0 + (wave & 1) * 64 + lane;
        if constexpr (L1) {
            const int f = a.row_src[r];
            s_src = a.x_sf + (size_t)(f >= 0 ? f / K : 0) * (H / 128);
        } else {
            s_src = a.h_sf + (size_t)r * (I / 128);
        }
    }
    const uint32_t smem_base = lds_addr(smem);

    auto issue = [&](int kb, int stage) {
        const uint32_t st = smem_base + stage * STAGE;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dma16(a_src[j] + (size_t)kb * 128, st + (wave * 2 + j) * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = wave * 4 + j, sub = q >> 1, half = q & 1;
            dma16(weight_src<L1, PK>(a, e, nt, kb, sub, half, lane), st + A_BYTES + q * 1024);
        }
        dma4(s_src + kb, st + A_BYTES + B_BYTES + wave * 256);
    };

    v4f acc[4][4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    if (nkb > 1)
        issue(1, 1);

    int stage = 0;
    for (int kb = 0; kb < nkb; ++kb) {
        // This wave's copies for block kb have landed (block kb + 1's may be
        // in flight); the barrier makes every wave's copies visible and
        // orders the previous step's reads before the refill below.
        if (kb + 1 < nkb)
            MOE_WAIT_VMCNT(kCopiesPerStage);
        else
            MOE_WAIT_VMCNT(0);
        __syncthreads();

        const uint8_t* st = smem + stage * STAGE;
        v8i af[4], bf[4];
        float sa[4][4];
        const float* sa_lds = reinterpret_cast<const float*>(st + A_BYTES + B_BYTES);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
            af[ms] = lds_frag(st + ((wm * 4 + ms) * 2) * 1024, lane);
            const float4 s4 = *reinterpret_cast<const float4*>(sa_lds + wm * 64 + ms * 16 + 4 * lg);
            sa[ms][0] = s4.x;
            sa[ms][1] = s4.y;
            sa[ms][2] = s4.z;
            sa[ms][3] = s4.w;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
            bf[s] = lds_frag(st + A_BYTES + (wn * 4 + s) * 2048, lane);
        // weight scales (copied by wave 2): L1 gate / up block; L2 the
        // wave's 128-column block (256 n + 64 wn) / 128
        const float* sb_lds = sa_lds + 2 * 64;
        const float sg = L1 ? sb_lds[0] : sb_lds[wn >> 1];
        const float su = L1 ? sb_lds[1] : sg;

        if (kb + 2 < nkb)
            issue(kb + 2, stage == 0 ? 2 : stage - 1);

#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float sb = (L1 && s >= 2) ? su : sg;
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
        stage = stage == NSTAGE - 1 ? 0 : stage + 1;
    }
    __syncthreads();  // all fragment reads done before the epilogue reuses LDS

    // ------------------------------------------------------------ epilogues
    if constexpr (L1) {
        // acc[ms][s]: rows wm*64 + 16 ms + 4 lg + i; s = 0,1 gate column
        // 32 wn + 16 s + lr of the block, s = 2,3 the matching up column.
        float* red = reinterpret_cast<float*>(smem + A_BYTES);  // [4][128]
        uint8_t* qt = smem;                                     // [128][128]
        float wrow[4][4];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = a.row_src[row0 + wm * 64 + ms * 16 + 4 * lg + i];
                wrow[ms][i] = f >= 0 ? a.topk_w[f] : 0.f;
            }
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m = 0.f;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const float g = acc[ms][s][i], u = acc[ms][s + 2][i];
                    const float silu = g / (1.0f + expf(-g));
                    const float v = (silu * u) * wrow[ms][i];
                    acc[ms][s][i] = v;
                    m = fmaxf(m, fabsf(v));
                }
                m = max16(m);
                if (lr == 0)
                    red[wn * 128 + wm * 64 + ms * 16 + 4 * lg + i] = m;
            }
        __syncthreads();
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + ms * 16 + 4 * lg + i;
                const float amax =
                    fmaxf(fmaxf(red[r], red[128 + r]), fmaxf(red[256 + r], red[384 + r]));
                const float sf = fmaxf(amax, 1e-10f) / 448.0f;
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    qt[r * 128 + wn * 32 + s * 16 + lr] = (uint8_t)f32_to_e4m3(acc[ms][s][i] / sf);
                if (wn == 0 && lr == 0)
                    a.h_sf[(size_t)(row0 + r) * (I / 128) + nt] = sf;
            }
        __syncthreads();
        for (int c = threadIdx.x; c < BM * 8; c += kThreads) {
            const int r = c >> 3, col = (c & 7) * 16;
            if (a.row_src[row0 + r] >= 0)
                *reinterpret_cast<uint4*>(a.h + (size_t)(row0 + r) * I + nt * 128 + col) =
                    *reinterpret_cast<const uint4*>(qt + r * 128 + col);
        }
    } else {
        // acc[ms][s]: rows wm*64 + 16 ms + 4 lg + i, column 64 wn + 16 s + lr.
        uint16_t* ot = reinterpret_cast<uint16_t*>(smem);  // [128][256] bf16 = 64 KiB
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ot[(wm * 64 + ms * 16 + 4 * lg + i) * 256 + wn * 64 + s * 16 + lr] =
                        f32_to_bf16(acc[ms][s][i]);
        __syncthreads();
        for (int c = threadIdx.x; c < BM * 32; c += kThreads) {
            const int r = c >> 5, col = (c & 31) * 8;
            const int f = a.row_src[row0 + r];
            if (f >= 0) {
                const int t = f / K, jslot = f - t * K;
                *reinterpret_cast<uint4*>(a.partial + ((size_t)jslot * T + t) * H + nt * 256 + col) =
                    *reinterpret_cast<const uint4*>(ot + r * 256 + col);
            }
        }
    }
}

size_t gemm_lds_smem_bytes() { return (size_t)NSTAGE * STAGE; }

template <bool L1>
static hipError_t launch_lds(const FwdArgs& a, hipStream_t s)
{
    const unsigned NT = L1 ? a.I / 128 : a.H / 256;
    const dim3 grid(a.num_mblocks * NT);
    const size_t smem = gemm_lds_smem_bytes();
    if (a.packed) {
        hipFuncSetAttribute((const void*)gemm_lds<L1, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        hipLaunchKernelGGL((gemm_lds<L1, true>), grid, dim3(kThreads), smem, s, a);
    } else {
        hipFuncSetAttribute((const void*)gemm_lds<L1, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        hipLaunchKernelGGL((gemm_lds<L1, false>), grid, dim3(kThreads), smem, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_l1_lds(const FwdArgs& a, hipStream_t s) { return launch_lds<true>(a, s); }
hipError_t launch_l2_lds(const FwdArgs& a, hipStream_t s) { return launch_lds<false>(a, s); }

}  // namespace moe
