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
// wave.  The K loop steps two 128-K blocks at a time: a lane loads, per
// block, 32 activation bytes (two 16-byte loads 64 bytes apart: the MFMA's
// e4m3 K order) and one scale byte per operand row (its K block lane / 16),
// and per 16-column weight subtile 16 bytes of each block (32 contiguous K
// values: the e2m1 K order) -- two 16-byte loads 64 bytes apart, so the
// four lane groups read one whole 128-byte line of each weight row per step
// and every weight load keeps as many bytes in flight as the FP8 kernels'.
// An odd number of K blocks ends with a half step.
#include "moe_device.h"
#include "moe_direct.h"
#include "moe_internal.h"

namespace moe {

namespace {

// Operands of two consecutive 128-K blocks (a final half step repeats the
// first block's loads and multiplies it once).
template <int MT>
struct MxStep {
    Frag2 fa[2][MT];
    Frag2 fb[4];  // lo: block 0, hi: block 1 (64 bytes further in the row)
    int sa[2][MT], sb[2][4];
};

// Where a tile's operands sit, as buffer resources (wave-uniform, in
// SGPRs) plus 32-bit per-lane offsets, so each load costs one VGPR of
// address.  Activation row ms of the lane at ra + aoff[ms] (its scale bytes
// at ras + asoff[ms]); weight subtile s at rb + bsub[s] + boff (scales
// rbs + bssub[s] + bsoff); the K block's position goes in the uniform
// offset.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// (A nontemporal cache policy on the weight loads measured 7 % slower.)
__device__ __forceinline__ uint4 buf16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int buf1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return (int)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

template <int MT>
struct MxAddr {
    __amdgpu_buffer_rsrc_t ra, ras, rb, rbs;
    uint32_t aoff[MT], asoff[MT];
    uint32_t bsub[4], bssub[4];
    uint32_t boff, bsoff;
    uint32_t bk, bsk;  // bytes between K blocks: weights, scales
};

template <int MT>
__device__ __forceinline__ void mx_fetch(MxStep<MT>& b, int kk, int nkb, const MxAddr<MT>& p)
{
    const int kb = 2 * kk;
    const bool two = kb + 1 < nkb;  // uniform: false only in a final half step
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t k = two ? kb + h : kb;
#pragma unroll
        for (int ms = 0; ms < MT; ++ms)
            b.sa[h][ms] = buf1(p.ras, p.asoff[ms], k * 4);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b.sb[h][s] = buf1(p.rbs, p.bsoff, p.bssub[s] + k * p.bsk);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t k = two ? kb + h : kb;
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            b.fa[h][ms].lo = buf16(p.ra, p.aoff[ms], k * 128);
            b.fa[h][ms].hi = buf16(p.ra, p.aoff[ms], k * 128 + 64);
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t q = p.bsub[s] + kb * p.bk;
        b.fb[s].lo = buf16(p.rb, p.boff, q);
        b.fb[s].hi = two ? buf16(p.rb, p.boff, q + p.bk) : b.fb[s].lo;
    }
}

template <int MT>
__device__ __forceinline__ void mx_mul(const MxStep<MT>& b, bool two, v4f (&acc)[MT][4])
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h == 1 && !two)
            break;
#pragma unroll
        for (int ms = 0; ms < MT; ++ms) {
            const v8i av = pack_frag(b.fa[h][ms].lo, b.fa[h][ms].hi);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[ms][s] = mfma_16x16x128_e4m3_e2m1(av, e2m1_operand(h ? b.fb[s].hi : b.fb[s].lo),
                                                      acc[ms][s], b.sa[h][ms], b.sb[h][s]);
        }
    }
}

}  // namespace

// ------------------------------------------------------------------- L1

template <int MT, bool PK>
__global__ __launch_bounds__(256) void l1_mx(FwdArgs a)
{
    constexpr int BM = 16 * MT;
    const int NT = a.I / 128;
    const int mb = blockIdx.x / NT;
    const int nt = blockIdx.x - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0 || e >= a.E)
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int H = a.H, HS = H / 32, I = a.I, IS = I / 32, K = a.K;
    const int row0 = mb * BM;

    // A rows row0 + 16 ms + lr.  A padding row (row_src < 0) reads the
    // block's first row (which always holds a slot): its products reach only
    // that padding row of the accumulator, which is never stored.  B
    // subtile s = 0,1 gate, 2,3 up: weight row n0 + sub(s) + lr, this lane's
    // 16 bytes of each 64-byte K block, and its K block's scale byte.
    MxAddr<MT> p;
    p.ra = rsrc(a.x, (uint32_t)a.T * H);
    p.ras = rsrc(a.x_sfq, (uint32_t)a.T * HS);
    const int f0 = a.row_src[row0];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
        const int f = a.row_src[row0 + 16 * ms + lr];
        const uint32_t t = (uint32_t)((f >= 0 ? f : f0) / K);
        p.aoff[ms] = t * (uint32_t)H + lg * 16;
        p.asoff[ms] = t * (uint32_t)HS + lg;
    }
    if constexpr (PK) {
        // packed (moe_prepare_weights_mx): this wave's 4 KiB of each K block
        // of the tile, then 16 KiB to the next block
        const size_t t0 = ((size_t)e * (I / 128) + nt) * (H / 128);
        p.rb = rsrc(a.w1 + t0 * 16384 + wave * 4096, (uint32_t)(H / 128 - 1) * 16384 + 4096);
        p.rbs = rsrc(a.w1_sfq + t0 * 1024 + wave * 256, (uint32_t)(H / 128 - 1) * 1024 + 256);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            p.bsub[s] = s * 1024;
            p.bssub[s] = s * 64;
        }
        p.boff = lane * 16;
        p.bsoff = lane;
        p.bk = 16384;
        p.bsk = 1024;
    } else {
        const size_t n0 = (size_t)e * 2 * I + nt * 128 + wave * 32;  // subtile rows span I + 32
        p.rb = rsrc(a.w1 + n0 * (H / 2), (uint32_t)(I + 32) * (H / 2));
        p.rbs = rsrc(a.w1_sfq + n0 * HS, (uint32_t)(I + 32) * HS);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t sub = (s >= 2 ? I : 0) + (s & 1) * 16;
            p.bsub[s] = sub * (uint32_t)(H / 2);
            p.bssub[s] = sub * (uint32_t)HS;
        }
        p.boff = lr * (uint32_t)(H / 2) + lg * 16;
        p.bsoff = lr * (uint32_t)HS + lg;
        p.bk = 64;
        p.bsk = 4;
    }

    v4f acc[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nkb = H / 128;
    auto fetch = [&](MxStep<MT>& b, int kk) { mx_fetch<MT>(b, kk, nkb, p); };
    int kk_mul = 0;
    auto mul = [&](const MxStep<MT>& b) {
        mx_mul<MT>(b, 2 * kk_mul + 1 < nkb, acc);
        ++kk_mul;
    };
    kloop<MxStep<MT>>(0, (nkb + 1) / 2, fetch, mul);

    // ---- epilogue: SwiGLU x topk_w, per-row amax over this wave's 32
    // columns (one requantisation block), power-of-two scale, e4m3 codes
    // staged in LDS for 16-byte row stores.
    clamp_acc<MT * 4>(&acc[0][0], a.clamp);
    __shared__ uint8_t qt[BM][128];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * ms + 4 * lg + i;
            const int f = a.row_src[row0 + r];
            const float w = f >= 0 ? a.topk_w[f] : 0.f;
            const float v0 = (silu(acc[ms][0][i]) *
                              acc[ms][2][i]) * w;
            const float v1 = (silu(acc[ms][1][i]) *
                              acc[ms][3][i]) * w;
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

template <int MT, bool PK>
__global__ __launch_bounds__(256) void l2_mx(FwdArgs a)
{
    constexpr int BM = 16 * MT;
    const int H = a.H, I = a.I, IS = I / 32, K = a.K, T = a.T;
    const int NT = (H + 255) / 256;  // H % 256 == 128: the last tile has 2 idle waves
    const int mb = blockIdx.x / NT;
    const int nt = blockIdx.x - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0 || e >= a.E)
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = mb * BM;
    const bool busy = nt * 256 + wave * 64 < H;
    const int ncol0 = busy ? nt * 256 + wave * 64 : 0;  // an idle wave re-reads columns 0..63

    // A rows: pool rows row0 + 16 ms + lr of h; a padding row reads row0
    // (always a routed slot's row) instead of its own unwritten bytes.
    MxAddr<MT> p;
    p.ra = rsrc(a.h + (size_t)row0 * I, (uint32_t)BM * I);
    p.ras = rsrc(a.h_sfq + (size_t)row0 * IS, (uint32_t)BM * IS);
#pragma unroll
    for (int ms = 0; ms < MT; ++ms) {
        const uint32_t r = a.row_src[row0 + 16 * ms + lr] >= 0 ? 16 * ms + lr : 0;
        p.aoff[ms] = r * (uint32_t)I + lg * 16;
        p.asoff[ms] = r * (uint32_t)IS + lg;
    }
    if constexpr (PK) {  // packed: H % 256 == 0, every wave busy
        const size_t t0 = ((size_t)e * (H / 256) + nt) * (I / 128);
        p.rb = rsrc(a.w2 + t0 * 16384 + wave * 4096, (uint32_t)(I / 128 - 1) * 16384 + 4096);
        p.rbs = rsrc(a.w2_sfq + t0 * 1024 + wave * 256, (uint32_t)(I / 128 - 1) * 1024 + 256);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            p.bsub[s] = s * 1024;
            p.bssub[s] = s * 64;
        }
        p.boff = lane * 16;
        p.bsoff = lane;
        p.bk = 16384;
        p.bsk = 1024;
    } else {
        const size_t n0 = (size_t)e * H + ncol0;  // subtile rows span 64
        p.rb = rsrc(a.w2 + n0 * (I / 2), 64u * (I / 2));
        p.rbs = rsrc(a.w2_sfq + n0 * IS, 64u * IS);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            p.bsub[s] = s * 16 * (uint32_t)(I / 2);
            p.bssub[s] = s * 16 * (uint32_t)IS;
        }
        p.boff = lr * (uint32_t)(I / 2) + lg * 16;
        p.bsoff = lr * (uint32_t)IS + lg;
        p.bk = 64;
        p.bsk = 4;
    }

    v4f acc[MT][4];
#pragma unroll
    for (int ms = 0; ms < MT; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nkb = I / 128;
    auto fetch = [&](MxStep<MT>& b, int kk) { mx_fetch<MT>(b, kk, nkb, p); };
    int kk_mul = 0;
    auto mul = [&](const MxStep<MT>& b) {
        mx_mul<MT>(b, 2 * kk_mul + 1 < nkb, acc);
        ++kk_mul;
    };
    kloop<MxStep<MT>>(0, (nkb + 1) / 2, fetch, mul);

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

template <bool PK>
static hipError_t launch_l1_mx_t(const FwdArgs& a, hipStream_t s)
{
    const unsigned grid = a.grid_mblocks * (a.I / 128);
    switch (a.BM) {
    case 16: hipLaunchKernelGGL((l1_mx<1, PK>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((l1_mx<2, PK>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((l1_mx<4, PK>), dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool PK>
static hipError_t launch_l2_mx_t(const FwdArgs& a, hipStream_t s)
{
    const unsigned grid = a.grid_mblocks * ((a.H + 255) / 256);
    switch (a.BM) {
    case 16: hipLaunchKernelGGL((l2_mx<1, PK>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((l2_mx<2, PK>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((l2_mx<4, PK>), dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_l1_mx(const FwdArgs& a, hipStream_t s)
{
    return a.packed ? launch_l1_mx_t<true>(a, s) : launch_l1_mx_t<false>(a, s);
}

hipError_t launch_l2_mx(const FwdArgs& a, hipStream_t s)
{
    return a.packed ? launch_l2_mx_t<true>(a, s) : launch_l2_mx_t<false>(a, s);
}

}  // namespace moe
