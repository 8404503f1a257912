// L1 (gate+up, fused SwiGLU x topk_w + per-128 e4m3 requant) and L2 (down,
// BF16 scatter) grouped FP8 GEMMs, direct-load form for small row tiles.
//
// Math ("MegaMoE SM90 Implementation Design" §5.3): for every 128-wide K
// block the MFMA forms the block's dot product p in f32, then
//   acc = fmaf(sa[row, kb] * sb[nblk, kb], p, acc)
// with sa the 1x128 activation scale and sb the 128x128 weight scale.
// L1 epilogue (§10.1; DeepGEMM PR #440 "How it works" for the raw scale):
//   h = silu(g) * u * topk_w,  sf = max(amax_128, 1e-10) / 448,  q = e4m3(h / sf)
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
#include "moe_internal.h"

namespace moe {

namespace {

struct Frag2 {
    uint4 lo, hi;
};

__device__ __forceinline__ Frag2 load_frag(const uint8_t* p)
{
    Frag2 f;
    f.lo = *reinterpret_cast<const uint4*>(p);
    f.hi = *reinterpret_cast<const uint4*>(p + 64);
    return f;
}

__device__ __forceinline__ Frag2 zero_frag()
{
    Frag2 f;
    f.lo = make_uint4(0, 0, 0, 0);
    f.hi = f.lo;
    return f;
}

}  // namespace

// ------------------------------------------------------------------- L1

template <int MT>
__global__ __launch_bounds__(256) void l1_direct(FwdArgs a)
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
    const int H = a.H, HB = H / 128, I = a.I, K = a.K;
    const int row0 = mb * BM;

    // A operand rows: row0 + 16*ms + lr.
    const uint8_t* aptr[MT];
    bool avalid[MT];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
        const int f = a.row_src[row0 + 16 * ms + lr];
        avalid[ms] = f >= 0;
        aptr[ms] = a.x + (size_t)(f >= 0 ? f / K : 0) * H + lg * 16;
    }
    // Output rows of this lane: row0 + 16*ms + 4*lg + i.
    const float* asf[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int f = a.row_src[row0 + 16 * ms + 4 * lg + i];
            asf[ms][i] = a.x_sf + (size_t)(f >= 0 ? f / K : 0) * HB;
        }
    // B operand: subtile s = 0,1 gate, 2,3 up.
    const uint8_t* bptr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int n = (s >= 2 ? I : 0) + nt * 128 + wave * 32 + (s & 1) * 16 + lr;
        bptr[s] = a.w1 + ((size_t)e * 2 * I + n) * H + lg * 16;
    }
    const float* sfg = a.w1_sf + ((size_t)e * (2 * I / 128) + nt) * HB;
    const float* sfu = a.w1_sf + ((size_t)e * (2 * I / 128) + I / 128 + nt) * HB;

    v4f acc[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    Frag2 fa[MT], fb[4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
        fa[ms] = avalid[ms] ? load_frag(aptr[ms]) : zero_frag();
#pragma unroll
    for (int s = 0; s < 4; ++s)
        fb[s] = load_frag(bptr[s]);

    for (int kb = 0; kb < HB; ++kb) {
        Frag2 na[MT], nb[4];
        const int kn = kb + 1 < HB ? kb + 1 : kb;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            nb[s] = load_frag(bptr[s] + kn * 128);
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            na[ms] = avalid[ms] ? load_frag(aptr[ms] + kn * 128) : zero_frag();
        const float sg = sfg[kb], su = sfu[kb];
        float sa[MT][4];
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sa[ms][i] = asf[ms][i][kb];
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            const v8i av = pack_frag(fa[ms].lo, fa[ms].hi);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const v4f p = mfma_16x16x128_e4m3(av, pack_frag(fb[s].lo, fb[s].hi),
                                                  v4f{0.f, 0.f, 0.f, 0.f});
                const float sb = s >= 2 ? su : sg;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[ms][s][i] = fmaf(sa[ms][i] * sb, p[i], acc[ms][s][i]);
            }
        }
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            fa[ms] = na[ms];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            fb[s] = nb[s];
    }

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
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const float g = acc[ms][s][i], u = acc[ms][s + 2][i];
                const float silu = g / (1.0f + expf(-g));
                const float v = (silu * u) * wrow[ms][i];
                hv[ms][s][i] = v;
                m = fmaxf(m, fabsf(v));
            }
            m = max16(m);
            if (lr == 0)
                red[wave][16 * ms + 4 * lg + i] = m;
        }
    }
    __syncthreads();
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ms + 4 * lg + i;
            const float amax = fmaxf(fmaxf(red[0][r], red[1][r]), fmaxf(red[2][r], red[3][r]));
            const float sf = fmaxf(amax, 1e-10f) / 448.0f;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                qt[r][wave * 32 + s * 16 + lr] = (uint8_t)f32_to_e4m3(hv[ms][s][i] / sf);
            if (wave == 0 && lr == 0)
                a.h_sf[(size_t)(row0 + r) * (I / 128) + nt] = sf;
        }
    }
    __syncthreads();
    // BM rows x 128 bytes, 16 bytes per thread.
    for (int c = threadIdx.x; c < BM * 8; c += 256) {
        const int r = c >> 3, col = (c & 7) * 16;
        if (a.row_src[row0 + r] >= 0)
            *reinterpret_cast<uint4*>(a.h + (size_t)(row0 + r) * I + nt * 128 + col) =
                *reinterpret_cast<const uint4*>(&qt[r][col]);
    }
}

// ------------------------------------------------------------------- L2

template <int MT>
__global__ __launch_bounds__(256) void l2_direct(FwdArgs a)
{
    constexpr int BM = 16 * MT;
    const int H = a.H, I = a.I, IB = I / 128, K = a.K, T = a.T;
    const int NT = (H + 255) / 256;  // H % 256 == 128: the last tile has 2 idle waves
    const int mb = blockIdx.x / NT;
    const int nt = blockIdx.x - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = mb * BM;

    const uint8_t* aptr[MT];
    bool avalid[MT];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
        const int r = row0 + 16 * ms + lr;
        avalid[ms] = a.row_src[r] >= 0;
        aptr[ms] = a.h + (size_t)r * I + lg * 16;
    }
    const float* asf[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            asf[ms][i] = a.h_sf + (size_t)(row0 + 16 * ms + 4 * lg + i) * IB;
    // A wave's 64 columns are either all inside H or all past it; an idle
    // wave re-reads column block 0 and stores nothing.
    const int ncol0 = (nt * 256 + wave * 64 < H) ? nt * 256 + wave * 64 : 0;
    const uint8_t* bptr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        bptr[s] = a.w2 + ((size_t)e * H + ncol0 + s * 16 + lr) * I + lg * 16;
    const float* sfb = a.w2_sf + ((size_t)e * (H / 128) + ncol0 / 128) * IB;

    v4f acc[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    Frag2 fa[MT], fb[4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
        fa[ms] = avalid[ms] ? load_frag(aptr[ms]) : zero_frag();
#pragma unroll
    for (int s = 0; s < 4; ++s)
        fb[s] = load_frag(bptr[s]);

    for (int kb = 0; kb < IB; ++kb) {
        Frag2 na[MT], nb[4];
        const int kn = kb + 1 < IB ? kb + 1 : kb;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            nb[s] = load_frag(bptr[s] + kn * 128);
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            na[ms] = avalid[ms] ? load_frag(aptr[ms] + kn * 128) : zero_frag();
        const float sb = sfb[kb];
        float sa[MT][4];
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sa[ms][i] = asf[ms][i][kb];
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            const v8i av = pack_frag(fa[ms].lo, fa[ms].hi);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const v4f p = mfma_16x16x128_e4m3(av, pack_frag(fb[s].lo, fb[s].hi),
                                                  v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[ms][s][i] = fmaf(sa[ms][i] * sb, p[i], acc[ms][s][i]);
            }
        }
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            fa[ms] = na[ms];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            fb[s] = nb[s];
    }

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
    for (int c = threadIdx.x; c < BM * 32; c += 256) {
        const int r = c >> 5, col = (c & 31) * 8;
        const int f = a.row_src[row0 + r];
        if (f >= 0 && nt * 256 + col < H) {
            const int t = f / K, j = f - t * K;
            uint4 v;
            v.x = (uint32_t)ot[r][col + 0] | ((uint32_t)ot[r][col + 1] << 16);
            v.y = (uint32_t)ot[r][col + 2] | ((uint32_t)ot[r][col + 3] << 16);
            v.z = (uint32_t)ot[r][col + 4] | ((uint32_t)ot[r][col + 5] << 16);
            v.w = (uint32_t)ot[r][col + 6] | ((uint32_t)ot[r][col + 7] << 16);
            *reinterpret_cast<uint4*>(a.partial + ((size_t)j * T + t) * H + nt * 256 + col) = v;
        }
    }
}

// -------------------------------------------------------------- combine

// y[t, n] = bf16( sum over active slots j ascending of f32(partial[j][t][n]) )
// ("MegaMoE SM90 Implementation Design" §11.2).  8 columns per thread.
__global__ __launch_bounds__(256) void combine_kernel(FwdArgs a)
{
    const int H8 = a.H / 8;
    const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
    if (g >= (long long)a.T * H8)
        return;
    const int t = (int)(g / H8);
    const int c = (int)(g - (long long)t * H8) * 8;
    float s[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        s[q] = 0.f;
    for (int j = 0; j < a.K; ++j) {
        const int e = a.idx[t * a.K + j];
        if (e < 0 || e >= a.E)
            continue;
        const uint4 v = *reinterpret_cast<const uint4*>(a.partial + ((size_t)j * a.T + t) * a.H + c);
        s[0] += bf16_to_f32(v.x & 0xFFFFu);
        s[1] += bf16_to_f32(v.x >> 16);
        s[2] += bf16_to_f32(v.y & 0xFFFFu);
        s[3] += bf16_to_f32(v.y >> 16);
        s[4] += bf16_to_f32(v.z & 0xFFFFu);
        s[5] += bf16_to_f32(v.z >> 16);
        s[6] += bf16_to_f32(v.w & 0xFFFFu);
        s[7] += bf16_to_f32(v.w >> 16);
    }
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(s[0]) | ((uint32_t)f32_to_bf16(s[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(s[2]) | ((uint32_t)f32_to_bf16(s[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(s[4]) | ((uint32_t)f32_to_bf16(s[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(s[6]) | ((uint32_t)f32_to_bf16(s[7]) << 16);
    *reinterpret_cast<uint4*>(a.y + (size_t)t * a.H + c) = o;
}

hipError_t launch_l1(const FwdArgs& a, int kernel, hipStream_t s)
{
    (void)kernel;
    const dim3 grid(a.num_mblocks * (a.I / 128));
    switch (a.BM) {
    case 16: hipLaunchKernelGGL(l1_direct<1>, grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL(l1_direct<2>, grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(l1_direct<4>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_l2(const FwdArgs& a, int kernel, hipStream_t s)
{
    (void)kernel;
    const dim3 grid(a.num_mblocks * ((a.H + 255) / 256));
    switch (a.BM) {
    case 16: hipLaunchKernelGGL(l2_direct<1>, grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL(l2_direct<2>, grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(l2_direct<4>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const FwdArgs& a, hipStream_t s)
{
    const long long n = (long long)a.T * (a.H / 8);
    const dim3 grid((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
