// Ceiling measurements for MI355X (gfx950): a streaming HBM read and a dense
// FP8 MFMA loop.  The MoE kernels are bound by one or the other, so their
// rates are reported against these measured ceilings beside the published
// ones.  C ABI in include/moe_peaks.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <cstring>

#include "moe_peaks.h"
#include "moe_device.h"
#include "moe_direct.h"

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Each lane keeps U 16-byte loads in flight: one round of a workgroup covers
// U * 256 consecutive 16-byte words, lane l taking words l, l + 256, ...;
// workgroups take rounds b, b + G, ....  Full rounds load unconditionally;
// the one partial round at the end checks each word.
template <int U, bool NT>
__global__ void __launch_bounds__(256) stream_read(const v4u* __restrict__ p, size_t n,
                                                   uint32_t* __restrict__ out)
{
    const size_t round = (size_t)256 * U;
    const size_t stride = (size_t)gridDim.x * round;
    const size_t full = n / round * round;  // words covered by full rounds
    uint32_t acc = 0;
    size_t base = (size_t)blockIdx.x * round;
    for (; base < full; base += stride) {
        v4u v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const v4u* q = p + base + (size_t)u * 256 + threadIdx.x;
            v[u] = NT ? __builtin_nontemporal_load(q) : *q;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (base < n) {  // the partial round, if any, falls to exactly one workgroup
        for (int u = 0; u < U; ++u) {
            const size_t j = base + (size_t)u * 256 + threadIdx.x;
            if (j < n) {
                const v4u v = p[j];
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            }
        }
    }
    for (int o = 32; o > 0; o >>= 1)
        acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0)
        out[blockIdx.x * 4 + threadIdx.x / 64] = acc;
}

// 8 independent accumulators per wave, so consecutive MFMAs never wait on
// each other's results.
__global__ void __launch_bounds__(256) mfma_fp8_loop(int iters, float* __restrict__ out)
{
    using moe::v4f;
    using moe::v8i;
    const int ones = 0x38383838;    // e4m3 1.0 in every byte
    const int halves = 0x30303030;  // e4m3 0.5
    // The operands come from a lane-dependent expression so the compiler
    // cannot treat the loop as constant.
    const int lane_zero = (int)(threadIdx.x >> 8);  // 0 for every lane of a 256-lane block
    const v8i a = {ones + lane_zero, ones, ones, ones, ones, ones, ones, ones};
    const v8i b = {halves + lane_zero, halves, halves, halves, halves, halves, halves, halves};
    // eight named accumulators: an array here made the register allocator
    // shuffle accumulator registers inside the loop
    v4f c0{}, c1{}, c2{}, c3{}, c4{}, c5{}, c6{}, c7{};
    for (int i = 0; i < iters; ++i) {
        c0 = moe::mfma_16x16x128_e4m3(a, b, c0);
        c1 = moe::mfma_16x16x128_e4m3(a, b, c1);
        c2 = moe::mfma_16x16x128_e4m3(a, b, c2);
        c3 = moe::mfma_16x16x128_e4m3(a, b, c3);
        c4 = moe::mfma_16x16x128_e4m3(a, b, c4);
        c5 = moe::mfma_16x16x128_e4m3(a, b, c5);
        c6 = moe::mfma_16x16x128_e4m3(a, b, c6);
        c7 = moe::mfma_16x16x128_e4m3(a, b, c7);
    }
    const v4f t = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
    out[blockIdx.x * 256 + threadIdx.x] = (t.x + t.y) + (t.z + t.w);
}

// One 16 x 16 x 128 product per wave, with the operands loaded exactly as
// the GEMM kernels load them: lane l = 16 g + r reads bytes [16 g, 16 g + 16)
// and [64 + 16 g, 64 + 16 g + 16) of A row r; for e4m3 B the same bytes of
// B row (output column) r; for e2m1 B the 16 bytes [16 g, 16 g + 16) of its
// packed row (K values 32 g .. 32 g + 31), with the UE8M0 code of K block g
// of the row / column as each operand's scale.  Lane l writes column r,
// rows 4 g + i of its tile.  Waves past the last tile do nothing.
template <bool MX>
__global__ void __launch_bounds__(256) mfma_block_probe(const uint8_t* __restrict__ A,
                                                        const uint8_t* __restrict__ B,
                                                        const uint8_t* __restrict__ SA,
                                                        const uint8_t* __restrict__ SB,
                                                        int n_tiles, float* __restrict__ out)
{
    const int tile = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (tile >= n_tiles)
        return;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const size_t row = (size_t)tile * 16 + r;
    const moe::Frag2 fa = moe::load_frag(A + row * 128 + 16 * g);
    const moe::v8i av = moe::pack_frag(fa.lo, fa.hi);
    moe::v4f d;
    if constexpr (MX) {
        const uint4 fb = *reinterpret_cast<const uint4*>(B + row * 64 + 16 * g);
        d = moe::mfma_16x16x128_e4m3_e2m1(av, moe::e2m1_operand(fb), moe::v4f{0.f, 0.f, 0.f, 0.f},
                                          SA[row * 4 + g], SB[row * 4 + g]);
    } else {
        const moe::Frag2 fb = moe::load_frag(B + row * 128 + 16 * g);
        d = moe::mfma_16x16x128_e4m3(av, moe::pack_frag(fb.lo, fb.hi), moe::v4f{0.f, 0.f, 0.f, 0.f});
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        out[((size_t)tile * 16 + 4 * g + i) * 16 + r] = d[i];
}

// Every f32 bit pattern through the two conversions the epilogues rely on:
// the library's f32 -> bf16 (the hardware conversion) against round to
// nearest even written out on the integer bits (a NaN quieted, payload
// kept), and the hardware f32 -> e4m3 (f32_to_e4m3_hw) against the integer
// encoder f32_to_e4m3.  Lane t of the grid takes patterns t, t + N, ...
// (N lanes) and writes its two mismatch counts to counts[t], counts[N + t].
__global__ void __launch_bounds__(256) conversion_probe(uint32_t* __restrict__ counts)
{
    const uint32_t n = gridDim.x * 256u;
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    uint32_t c_bf = 0, c_e4 = 0;
    for (uint64_t i = t; i < (1ull << 32); i += n) {
        const uint32_t u = (uint32_t)i;
        const float f = __uint_as_float(u);
        const uint32_t ref = (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) & 0xFFFFu
                                                             : (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
        c_bf += moe::f32_to_bf16(f) != (uint16_t)ref ? 1u : 0u;
        c_e4 += moe::f32_to_e4m3_hw(f) != moe::f32_to_e4m3(f) ? 1u : 0u;
    }
    counts[t] = c_bf;
    counts[n + t] = c_e4;
}

int device_is_gfx950()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOE_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return MOE_ERR_HIP;
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? MOE_OK : MOE_ERR_NOT_GFX950;
}

}  // namespace

extern "C" int moe_peak_stream_read(const void* buf, size_t bytes, int32_t blocks, int32_t unroll,
                                    int32_t mode, uint32_t* out, void* stream)
{
    if (!buf || !out || (reinterpret_cast<uintptr_t>(buf) & 15) || bytes == 0 || (bytes & 15) ||
        blocks < 1 || blocks > 65536 || (unroll != 4 && unroll != 8) ||
        (mode != MOE_PEAK_READ_PLAIN && mode != MOE_PEAK_READ_NONTEMPORAL))
        return MOE_ERR_INVALID_ARG;
    const int dev = device_is_gfx950();
    if (dev != MOE_OK)
        return dev;
    const v4u* p = static_cast<const v4u*>(buf);
    const size_t n = bytes / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool nt = mode == MOE_PEAK_READ_NONTEMPORAL;
    if (unroll == 4) {
        if (nt)
            hipLaunchKernelGGL((stream_read<4, true>), dim3(blocks), dim3(256), 0, s, p, n, out);
        else
            hipLaunchKernelGGL((stream_read<4, false>), dim3(blocks), dim3(256), 0, s, p, n, out);
    } else {
        if (nt)
            hipLaunchKernelGGL((stream_read<8, true>), dim3(blocks), dim3(256), 0, s, p, n, out);
        else
            hipLaunchKernelGGL((stream_read<8, false>), dim3(blocks), dim3(256), 0, s, p, n, out);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int moe_peak_mfma_fp8(int32_t blocks, int32_t iters, float* out, void* stream)
{
    if (!out || blocks < 1 || blocks > 65536 || iters < 1 || iters > 2048)
        return MOE_ERR_INVALID_ARG;
    const int dev = device_is_gfx950();
    if (dev != MOE_OK)
        return dev;
    hipLaunchKernelGGL(mfma_fp8_loop, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       iters, out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int moe_probe_mfma_block(int32_t mode, int32_t n_tiles, const uint8_t* a,
                                    const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                    float* out, void* stream)
{
    if (!a || !b || !out || n_tiles < 1 || n_tiles > (1 << 20) ||
        (mode != MOE_PROBE_E4M3 && mode != MOE_PROBE_E4M3_E2M1) ||
        (reinterpret_cast<uintptr_t>(a) & 15) || (reinterpret_cast<uintptr_t>(b) & 15))
        return MOE_ERR_INVALID_ARG;
    if (mode == MOE_PROBE_E4M3_E2M1 && (!sa || !sb))
        return MOE_ERR_INVALID_ARG;
    const int dev = device_is_gfx950();
    if (dev != MOE_OK)
        return dev;
    const dim3 grid((unsigned)((n_tiles + 3) / 4));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mode == MOE_PROBE_E4M3_E2M1)
        hipLaunchKernelGGL(mfma_block_probe<true>, grid, dim3(256), 0, s, a, b, sa, sb, n_tiles, out);
    else
        hipLaunchKernelGGL(mfma_block_probe<false>, grid, dim3(256), 0, s, a, b, sa, sb, n_tiles, out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" int moe_probe_conversions(int32_t blocks, uint32_t* counts, void* stream)
{
    if (!counts || blocks < 1 || blocks > 65536)
        return MOE_ERR_INVALID_ARG;
    const int dev = device_is_gfx950();
    if (dev != MOE_OK)
        return dev;
    hipLaunchKernelGGL(conversion_probe, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       counts);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
