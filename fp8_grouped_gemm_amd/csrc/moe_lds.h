// Helpers of the kernels that stage operands through LDS with gfx950's
// asynchronous global -> LDS copies (global_load_lds_dword[x4]) and count
// their completion by hand: the copies are inline assembly, invisible to the
// compiler's own wait insertion, so each kernel waits on vmcnt itself.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// s_waitcnt with vmcnt = n (n < 64) and no wait on expcnt / lgkmcnt
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in
// bits [15:14]).
#define MOE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0xF70 | ((n) & 15) | (((n) >> 4) << 14))

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 15] (the immediate must
// be a constant).
__device__ __forceinline__ void wait_vmcnt(int n)
{
    switch (n) {
    case 0: MOE_WAIT_VMCNT(0); break;
    case 1: MOE_WAIT_VMCNT(1); break;
    case 2: MOE_WAIT_VMCNT(2); break;
    case 3: MOE_WAIT_VMCNT(3); break;
    case 4: MOE_WAIT_VMCNT(4); break;
    case 5: MOE_WAIT_VMCNT(5); break;
    case 6: MOE_WAIT_VMCNT(6); break;
    case 7: MOE_WAIT_VMCNT(7); break;
    case 8: MOE_WAIT_VMCNT(8); break;
    case 9: MOE_WAIT_VMCNT(9); break;
    case 10: MOE_WAIT_VMCNT(10); break;
    case 11: MOE_WAIT_VMCNT(11); break;
    case 12: MOE_WAIT_VMCNT(12); break;
    case 13: MOE_WAIT_VMCNT(13); break;
    case 14: MOE_WAIT_VMCNT(14); break;
    default: MOE_WAIT_VMCNT(0); break;  // (never larger here; waiting for all is safe)
    }
}

// Asynchronous copy global -> LDS of 16 (or 4) bytes per lane to
// lds_base + 16 * lane (4 * lane).  lds_base is wave-uniform (read from the
// first lane into the scalar register M0 takes).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

// The same copy with a wave-uniform 64-bit base in scalar registers and a
// 32-bit unsigned per-lane byte offset (the global SADDR form): one vector
// register per lane address instead of two.
__device__ __forceinline__ void dma16_off(const void* base, uint32_t off, uint32_t lds_base)
{
    // (the base is wave-uniform; reading it from the first lane keeps it in
    // scalar registers whatever the compiler concluded about it)
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off),
                 "s"(reinterpret_cast<const void*>(ub)),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}

// dma16_off with a constant byte offset IMM (0 <= IMM < 4096) that the
// instruction adds to both the global and the LDS address (the LDS copy
// lands at lds_base + IMM + 16 * lane), so copies that differ by a constant
// share one offset register and one M0.
template <int IMM>
__device__ __forceinline__ void dma16_off_imm(const void* base, uint32_t off, uint32_t lds_base)
{
    static_assert(IMM >= 0 && IMM < 4096, "the instruction's offset field");
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(off),
                 "s"(reinterpret_cast<const void*>(ub)),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base)), "n"(IMM)
                 : "memory", "m0");
}

__device__ __forceinline__ void dma4_off(const void* base, uint32_t off, uint32_t lds_base)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off),
                 "s"(reinterpret_cast<const void*>(ub)),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
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

// FP8 weights of the LDS-staged tiles (256 columns per tile): address of
// the 16 bytes lane `lane` copies for weight subtile `sub` (packed order
// w4 * 4 + s, see pack.hip), half `half`, K block kb of column tile nt.
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

}  // namespace moe
