// L1 (gate+up, fused SwiGLU x topk_w + per-32 power-of-two e4m3 requant)
// and L2 (down, BF16 scatter) grouped GEMMs of the FP8 x MXFP4 recipe,
// direct-load tiles.
//
// Recipe (the SM100 MegaMoE kernel on the "07 · MegaMoE" page §0: e4m3
// activations, e2m1 weights, one UE8M0 scale per 32 K values, recipe
// (1,1,32); "MegaMoE SM90 Implementation Design" §2.1 and §15.2 on the
// UE8M0 scale format; §8 of the former page on the L1 epilogue's per-block
// UE8M0 scale):
//   acc[r, n] = sum_k (x[t,k] 2^(sx[t,k/32]-127)) (W[e,n,k] 2^(sw[e,n,k/32]-127))
// Each MFMA applies both operands' block scales to its 128 K values and
// accumulates in f32, so there is no per-block promotion step.  L1 epilogue:
//   h = silu(g) u topk_w;  per 32 columns s = max(amax, 1e-10)/448,
//   sf = the smallest power of two >= s (a UE8M0 code),  q = e4m3(h / sf)
// L2 epilogue: bf16(acc) stored at partial[j][t] for the row's slot (t, j).
//
// Layout: x [T,H] e4m3 + x_sf [T,H/32] UE8M0; w1 [E,2I,H/2] packed e2m1
// (gate rows, then up rows; even K in the low nibble) + w1_sf [E,2I,H/32];
// w2 [E,H,I/2] + w2_sf [E,H,I/32]; h [R,I] e4m3 + h_sf [R,I/32] UE8M0.
//
// Work split as in the FP8 direct tiles (gemm_direct.hip): 4 waves of 64
// lanes; L1 tile = BM pool rows x (128 gate + 128 up) columns of one expert,
// wave w owning gate columns [32w, 32w+32) and the matching up columns --
// exactly one 32-column requantisation block, so the epilogue's amax needs
// no exchange between waves; L2 tile = BM rows x 256 output columns, 64 per
// wave.  Per 128-K block a lane loads 32 activation bytes (two 16-byte
// loads 64 bytes apart: the MFMA's e4m3 K order), 16 weight bytes per
// 16-column subtile (32 contiguous K values: the e2m1 K order), and one
// scale byte per operand row (its K block lane / 16).
#include "moe_device.h"
#include "moe_direct.h"
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ v8i e2m1_operand(const uint4& v)
{
    v8i r;
    r[0] = (int)v.x; r[1] = (int)v.y; r[2] = (int)v.z; r[3] = (int)v.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

}  // namespace

// ------------------------------------------------------------------- L1

template <int MT>
__global__ __launch_bounds__(256) void l1_mx(FwdArgs a)
{
    constexpr int BM = 16 * MT;
    const int NT = a.I / 128;
    const int mb = blockIdx.x / NT;
    const int nt = blockIdx.x - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int H = a.H, HS = H / 32, I = a.I, IS = I / 32, K = a.K;
    const int row0 = mb * BM;

    // A rows row0 + 16 ms + lr; padding rows (row_src < 0) read token 0
    // and are masked out of the MFMA.
    const uint8_t* aptr[MT];
    const uint8_t* asp[MT];
    bool avalid[MT];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
        const int f = a.row_src[row0 + 16 * ms + lr];
        const int t = max(f, 0) / K;
        avalid[ms] = f >= 0;
        aptr[ms] = a.x + (size_t)t * H + lg * 16;
        asp[ms] = a.x_sfq + (size_t)t * HS + lg;
    }
    // B subtile s = 0,1 gate, 2,3 up: weight row n, this lane's 16 bytes of
    // each 64-byte K block, and its K block's scale byte.
    const uint8_t* bptr[4];
    const uint8_t* bsp[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const size_t n = (size_t)e * 2 * I + (s >= 2 ? I : 0) + nt * 128 + wave * 32 + (s & 1) * 16 + lr;
        bptr[s] = a.w1 + n * (H / 2) + lg * 16;
        bsp[s] = a.w1_sfq + n * HS + lg;
    }

    v4f acc[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    struct Blk {
        Frag2 fa[MT];
        uint4 fb[4];
        int sa[MT], sb[4];
    };
    auto fetch = [&](Blk& b, int kb) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            b.sa[ms] = asp[ms][kb * 4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.sb[s] = bsp[s][kb * 4];
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            b.fa[ms] = avalid[ms] ? load_frag(aptr[ms] + kb * 128) : zero_frag();
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.fb[s] = *reinterpret_cast<const uint4*>(bptr[s] + kb * 64);
    };
    auto mul = [&](const Blk& b) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            const v8i av = pack_frag(b.fa[ms].lo, b.fa[ms].hi);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[ms][s] = mfma_16x16x128_e4m3_e2m1(av, e2m1_operand(b.fb[s]), acc[ms][s],
                                                      b.sa[ms], b.sb[s]);
        }
    };
    kloop<Blk>(0, H / 128, fetch, mul);

    // ---- epilogue: SwiGLU x topk_w, per-row amax over this wave's 32
    // columns (one requantisation block), power-of-two scale, e4m3 codes
    // staged in LDS for 16-byte row stores.
    __shared__ uint8_t qt[BM][128];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ms + 4 * lg + i;
            const int f = a.row_src[row0 + r];
            const float w = f >= 0 ? a.topk_w[f] : 0.f;
            const float v0 = (silu(acc[ms][0][i]) * acc[ms][2][i]) * w;
            const float v1 = (silu(acc[ms][1][i]) * acc[ms][3][i]) * w;
            const float amax = max16(fmaxf(fabsf(v0), fabsf(v1)));
            const uint32_t code = min(e8m0_ceil_code(fmaxf(amax, 1e-10f) / 448.0f), 253u);
            const float inv = e8m0_inverse(code);
            qt[r][wave * 32 + lr] = (uint8_t)f32_to_e4m3_hw(v0 * inv);
            qt[r][wave * 32 + 16 + lr] = (uint8_t)f32_to_e4m3_hw(v1 * inv);
            if (lr == 0 && f >= 0)
                a.h_sfq[(size_t)(row0 + r) * IS + nt * 4 + wave] = (uint8_t)code;
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < BM * 8; c += 256) {
        const int r = c >> 3, col = (c & 7) * 16;
        if (a.row_src[row0 + r] >= 0)
            *reinterpret_cast<uint4*>(a.h + (size_t)(row0 + r) * I + nt * 128 + col) =
                *reinterpret_cast<const uint4*>(&qt[r][col]);
    }
}

// ------------------------------------------------------------------- L2

template <int MT>
__global__ __launch_bounds__(256) void l2_mx(FwdArgs a)
{
    constexpr int BM = 16 * MT;
    const int H = a.H, I = a.I, IS = I / 32, K = a.K, T = a.T;
    const int NT = (H + 255) / 256;  // H % 256 == 128: the last tile has 2 idle waves
    const int mb = blockIdx.x / NT;
    const int nt = blockIdx.x - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = mb * BM;
    const bool busy = nt * 256 + wave * 64 < H;
    const int ncol0 = busy ? nt * 256 + wave * 64 : 0;  // an idle wave re-reads columns 0..63

    const uint8_t* aptr[MT];
    const uint8_t* asp[MT];
    bool avalid[MT];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
        const int r = row0 + 16 * ms + lr;
        avalid[ms] = a.row_src[r] >= 0;
        aptr[ms] = a.h + (size_t)r * I + lg * 16;
        asp[ms] = a.h_sfq + (size_t)r * IS + lg;
    }
    const uint8_t* bptr[4];
    const uint8_t* bsp[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const size_t n = (size_t)e * H + ncol0 + s * 16 + lr;
        bptr[s] = a.w2 + n * (I / 2) + lg * 16;
        bsp[s] = a.w2_sfq + n * IS + lg;
    }

    v4f acc[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    struct Blk {
        Frag2 fa[MT];
        uint4 fb[4];
        int sa[MT], sb[4];
    };
    auto fetch = [&](Blk& b, int kb) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            b.sa[ms] = asp[ms][kb * 4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.sb[s] = bsp[s][kb * 4];
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            b.fa[ms] = avalid[ms] ? load_frag(aptr[ms] + kb * 128) : zero_frag();
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.fb[s] = *reinterpret_cast<const uint4*>(bptr[s] + kb * 64);
    };
    auto mul = [&](const Blk& b) {
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            const v8i av = pack_frag(b.fa[ms].lo, b.fa[ms].hi);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[ms][s] = mfma_16x16x128_e4m3_e2m1(av, e2m1_operand(b.fb[s]), acc[ms][s],
                                                      b.sa[ms], b.sb[s]);
        }
    };
    kloop<Blk>(0, I / 128, fetch, mul);

    // ---- epilogue: bf16, stage BM x 256 in LDS, 16-byte stores to the
    // (slot, token) row of the partial buffer.
    __shared__ uint16_t ot[BM][256 + 8];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ot[16 * ms + 4 * lg + i][wave * 64 + s * 16 + lr] = f32_to_bf16(acc[ms][s][i]);
    __syncthreads();
    const int gcol0 = nt * 256;
    for (int c = threadIdx.x; c < BM * 32; c += 256) {
        const int r = c >> 5, col = (c & 31) * 8;
        const int f = a.row_src[row0 + r];
        if (f >= 0 && gcol0 + col < H) {
            const int t = f / K, j = f - t * K;
            uint4 v;
            v.x = (uint32_t)ot[r][col + 0] | ((uint32_t)ot[r][col + 1] << 16);
            v.y = (uint32_t)ot[r][col + 2] | ((uint32_t)ot[r][col + 3] << 16);
            v.z = (uint32_t)ot[r][col + 4] | ((uint32_t)ot[r][col + 5] << 16);
            v.w = (uint32_t)ot[r][col + 6] | ((uint32_t)ot[r][col + 7] << 16);
            *reinterpret_cast<uint4*>(a.partial + ((size_t)j * T + t) * H + gcol0 + col) = v;
        }
    }
}

// ------------------------------------------------------------ launchers

hipError_t launch_l1_mx(const FwdArgs& a, hipStream_t s)
{
    const unsigned grid = a.num_mblocks * (a.I / 128);
    switch (a.BM) {
    case 16: hipLaunchKernelGGL((l1_mx<1>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((l1_mx<2>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((l1_mx<4>), dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_l2_mx(const FwdArgs& a, hipStream_t s)
{
    const unsigned grid = a.num_mblocks * ((a.H + 255) / 256);
    switch (a.BM) {
    case 16: hipLaunchKernelGGL((l2_mx<1>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((l2_mx<2>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((l2_mx<4>), dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
