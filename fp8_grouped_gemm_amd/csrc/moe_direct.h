// Direct-load helpers shared by the gfx950 tile kernels that stream their
// MFMA operands from global memory straight into registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A weight fragment.  Row-major weights: the two 16-byte halves sit 64 bytes
// apart in the row.  Packed weights (moe_prepare_weights order): each half is
// one lane's slice of a contiguous 1 KiB run and the other half follows 1 KiB
// later; the stream is read once, so it is loaded nontemporally.
template <bool PK>
__device__ __forceinline__ Frag2 load_wfrag(const uint8_t* p)
{
    if constexpr (PK) {
        const u32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const u32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 1024));
        Frag2 f;
        f.lo = make_uint4(lo.x, lo.y, lo.z, lo.w);
        f.hi = make_uint4(hi.x, hi.y, hi.z, hi.w);
        return f;
    } else {
        return load_frag(p);
    }
}

__device__ __forceinline__ Frag2 zero_frag()
{
    Frag2 f;
    f.lo = make_uint4(0, 0, 0, 0);
    f.hi = f.lo;
    return f;
}

// K loop over blocks [kb0, kb1): the fetch of block kb + 1 is issued before
// block kb is multiplied, into two register sets used in turn (a copy from
// one set to the other would wait on its loads).  Every fetch inside the
// steady-state loop is unconditional, so the wait before a multiply leaves
// exactly the next block's loads outstanding (vector loads retire in
// order); the last one or two blocks run in a straight-line tail.  (A third
// set, two blocks ahead, needs over 256 VGPRs and halves the waves per SIMD;
// it measured slower.)
template <class B, class F, class M>
__device__ __forceinline__ void kloop(int kb0, int kb1, F& fetch, M& mul)
{
    B b0, b1;
    int kb = kb0;
    if (kb >= kb1)
        return;
    fetch(b0, kb);
    for (; kb + 2 < kb1; kb += 2) {
        fetch(b1, kb + 1);
        __builtin_amdgcn_sched_barrier(0);  // issue every load before the wait
        mul(b0);
        fetch(b0, kb + 2);
        __builtin_amdgcn_sched_barrier(0);
        mul(b1);
    }
    if (kb + 1 < kb1) {
        fetch(b1, kb + 1);
        __builtin_amdgcn_sched_barrier(0);
        mul(b0);
        mul(b1);
    } else {
        mul(b0);
    }
}

}  // namespace moe
