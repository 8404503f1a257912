// Activation quantisation (moe_quantize_act): bf16 tokens -> e4m3 codes
// with one scale per block, the step the pages leave to the caller before
// each call ("07 · MegaMoE" §3).  FP8 recipe: 1x128 blocks, sf =
// max(amax, 1e-10)/448 (f32 division), q = e4m3(v / sf) -- the same rule as
// the L1 epilogue's requantisation; MXFP4: 1x32 blocks, sf the smallest
// power of two at or above that, stored as its UE8M0 code.
//
// HBM-bound: each thread reads 16 bytes (8 bf16 of one block), the block's
// amax is a shuffle max over the 16 (resp. 4) threads sharing the block,
// and each thread writes its 8 codes as one 8-byte store.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <bool MX>
__global__ __launch_bounds__(256) void quantize_act(const uint16_t* __restrict__ x, int T, int H,
                                                    uint8_t* __restrict__ q, void* __restrict__ sf)
{
    const size_t n = (size_t)T * H / 8;
    const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
    // every lane of a block's group is present: the groups tile the row and
    // the grid covers n exactly up to whole groups (H % 128 == 0)
    const bool live = c < n;
    const uint4 raw = live ? *reinterpret_cast<const uint4*>(x + c * 8) : make_uint4(0, 0, 0, 0);
    float v[8];
    v[0] = bf16_to_f32(raw.x & 0xFFFFu); v[1] = bf16_to_f32(raw.x >> 16);
    v[2] = bf16_to_f32(raw.y & 0xFFFFu); v[3] = bf16_to_f32(raw.y >> 16);
    v[4] = bf16_to_f32(raw.z & 0xFFFFu); v[5] = bf16_to_f32(raw.z >> 16);
    v[6] = bf16_to_f32(raw.w & 0xFFFFu); v[7] = bf16_to_f32(raw.w >> 16);
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        m = fmaxf(m, fabsf(v[k]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    if constexpr (!MX) {
        m = fmaxf(m, __shfl_xor(m, 4));
        m = fmaxf(m, __shfl_xor(m, 8));
    }
    if (!live)
        return;
    float rsf;
    const float s = requant_sf(m, MX, rsf);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        lo |= requant_q(v[k], s, rsf, MX) << (8 * k);
        hi |= requant_q(v[k + 4], s, rsf, MX) << (8 * k);
    }
    *reinterpret_cast<uint2*>(q + c * 8) = make_uint2(lo, hi);
    const int group = MX ? 4 : 16;  // threads per scale block
    if ((c & (group - 1)) == 0) {
        const size_t blk = c / group;  // = t * (H / block) + block index
        if constexpr (MX)
            static_cast<uint8_t*>(sf)[blk] = (uint8_t)(__float_as_uint(s) >> 23);
        else
            static_cast<float*>(sf)[blk] = s;
    }
}

hipError_t launch_quantize_act(const uint16_t* x, int T, int H, uint8_t* q, void* sf, bool mx,
                               hipStream_t s)
{
    const size_t n = (size_t)T * H / 8;
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (mx)
        hipLaunchKernelGGL((quantize_act<true>), dim3(grid), dim3(256), 0, s, x, T, H, q, sf);
    else
        hipLaunchKernelGGL((quantize_act<false>), dim3(grid), dim3(256), 0, s, x, T, H, q, sf);
    return hipGetLastError();
}

}  // namespace moe
