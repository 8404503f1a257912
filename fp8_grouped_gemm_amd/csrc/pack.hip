// One-time re-layout of the expert weights into MFMA operand order
// (moe_prepare_weights).  Each 1 KiB run of the packed buffer is what one
// wave loads for one 16-row x 64-byte half of a 16x16x128 MFMA operand, so
// the forward's weight stream is contiguous: a tile's 128-wide K block is
// 32 KiB in a row, and a tile's K slice of 8 blocks is 256 KiB in a row.
//
// W1 (per expert, [2I, H]):  [n-tile I/128][kb H/128][wave 4][subtile 4][half 2][lane 64][16 B]
//   subtile s of wave w holds rows (s >= 2 ? I : 0) + 128 n + 32 w + 16 (s & 1) + r
// W2 (per expert, [H, I]):   [n-tile H/256][kb I/128][wave 4][subtile 4][half 2][lane 64][16 B]
//   subtile s of wave w holds rows 256 n + 64 w + 16 s + r
// lane l = 16 g + r carries bytes [64 h + 16 g, 64 h + 16 g + 16) of K block kb of row r.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void pack_w1(const uint8_t* __restrict__ src,
                                               uint8_t* __restrict__ dst, int E, int H, int I)
{
    const int HB = H / 128;
    const size_t per_e = (size_t)2 * I * H / 16;
    const size_t total = per_e * E;
    for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (size_t)gridDim.x * 256) {
        const size_t e = c / per_e;
        size_t rest = c - e * per_e;
        const int lane = (int)(rest & 63);
        rest >>= 6;
        const int half = (int)(rest & 1);
        rest >>= 1;
        const int s = (int)(rest & 3);
        rest >>= 2;
        const int w = (int)(rest & 3);
        rest >>= 2;
        const int kb = (int)(rest % HB);
        const int nt = (int)(rest / HB);
        const int row = (s >= 2 ? I : 0) + nt * 128 + w * 32 + (s & 1) * 16 + (lane & 15);
        const int col = kb * 128 + half * 64 + 16 * (lane >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(src + (e * 2 * I + row) * (size_t)H + col);
        *reinterpret_cast<uint4*>(dst + c * 16) = v;
    }
}

__global__ __launch_bounds__(256) void pack_w2(const uint8_t* __restrict__ src,
                                               uint8_t* __restrict__ dst, int E, int H, int I)
{
    const int IB = I / 128;
    const size_t per_e = (size_t)H * I / 16;
    const size_t total = per_e * E;
    for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (size_t)gridDim.x * 256) {
        const size_t e = c / per_e;
        size_t rest = c - e * per_e;
        const int lane = (int)(rest & 63);
        rest >>= 6;
        const int half = (int)(rest & 1);
        rest >>= 1;
        const int s = (int)(rest & 3);
        rest >>= 2;
        const int w = (int)(rest & 3);
        rest >>= 2;
        const int kb = (int)(rest % IB);
        const int nt = (int)(rest / IB);
        const int row = nt * 256 + w * 64 + s * 16 + (lane & 15);
        const int col = kb * 128 + half * 64 + 16 * (lane >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(src + (e * H + row) * (size_t)I + col);
        *reinterpret_cast<uint4*>(dst + c * 16) = v;
    }
}

// FP8 x MXFP4 weights (moe_prepare_weights_mx): one 16-row x 32-K-value
// subtile of one 128-K block is 64 lanes x 16 bytes of e2m1 pairs -- one
// wave's MFMA operand load, 1 KiB -- and its scales 64 lanes x 1 byte.
// W1 (per expert, [2I, H/2]):  [n-tile I/128][kb H/128][wave 4][subtile 4][lane 64][16 B]
//   subtile rows as for the FP8 W1 above
// W2 (per expert, [H, I/2]):   [n-tile H/256][kb I/128][wave 4][subtile 4][lane 64][16 B]
// lane l = 16 g + r carries bytes [64 kb + 16 g, 64 kb + 16 g + 16) of row r
// (K values 128 kb + 32 g .. + 31); the scales, same order with one byte per
// lane: byte 4 kb + g of row r's scale codes.
template <bool L1>
__global__ __launch_bounds__(256) void pack_mx(const uint8_t* __restrict__ src,
                                               const uint8_t* __restrict__ src_sf,
                                               uint8_t* __restrict__ dst,
                                               uint8_t* __restrict__ dst_sf, int E, int H, int I)
{
    const int N = L1 ? 2 * I : H;        // rows per expert
    const int Kv = L1 ? H : I;           // K values per row
    const int nkb = Kv / 128;
    const size_t per_e = (size_t)N * Kv / 32;  // 16-byte pieces per expert
    const size_t total = per_e * E;
    for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (size_t)gridDim.x * 256) {
        const size_t e = c / per_e;
        size_t rest = c - e * per_e;
        const int lane = (int)(rest & 63);
        rest >>= 6;
        const int s = (int)(rest & 3);
        rest >>= 2;
        const int w = (int)(rest & 3);
        rest >>= 2;
        const int kb = (int)(rest % nkb);
        const int nt = (int)(rest / nkb);
        const int r = lane & 15, g = lane >> 4;
        const int row = L1 ? (s >= 2 ? I : 0) + nt * 128 + w * 32 + (s & 1) * 16 + r
                           : nt * 256 + w * 64 + s * 16 + r;
        const size_t srow = e * N + row;
        *reinterpret_cast<uint4*>(dst + c * 16) =
            *reinterpret_cast<const uint4*>(src + srow * (Kv / 2) + kb * 64 + g * 16);
        dst_sf[c] = src_sf[srow * (Kv / 32) + kb * 4 + g];
    }
}

hipError_t launch_pack_mx(const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2,
                          const uint8_t* w2_sf, uint8_t* w1p, uint8_t* w1_sfp, uint8_t* w2p,
                          uint8_t* w2_sfp, int E, int H, int I, hipStream_t s)
{
    const dim3 grid(8192), block(256);
    hipLaunchKernelGGL((pack_mx<true>), grid, block, 0, s, w1, w1_sf, w1p, w1_sfp, E, H, I);
    hipLaunchKernelGGL((pack_mx<false>), grid, block, 0, s, w2, w2_sf, w2p, w2_sfp, E, H, I);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* w1, const uint8_t* w2, uint8_t* w1p, uint8_t* w2p, int E,
                       int H, int I, hipStream_t s)
{
    const dim3 grid(8192), block(256);
    hipLaunchKernelGGL(pack_w1, grid, block, 0, s, w1, w1p, E, H, I);
    hipLaunchKernelGGL(pack_w2, grid, block, 0, s, w2, w2p, E, H, I);
    return hipGetLastError();
}

}  // namespace moe
