// Device helpers shared by the gfx950 GEMM, epilogue and combine kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// One gfx950 MFMA: D(16x16, f32) = A(16x128, e4m3) * B(128x16, e4m3) + C.
// Operand format codes 0/0 select OCP e4m3 for both sides; zero scale
// operands make the compiler emit the unscaled v_mfma_f32_16x16x128_f8f6f4.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, 32 K-values
// each; the K values a lane group (l / 16) supplies are the same set for A
// and B, so any fixed assignment of K positions to bytes that both operands
// share yields the full 128-term dot product.  Result: lane l holds column
// (l % 16), rows 4*(l/16) + i for i = 0..3.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(const v8i& a, const v8i& b, const v4f& c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// One gfx950 block-scaled MFMA: D(16x16, f32) = A(16x128, e4m3) * B(128x16,
// e2m1) + C, each operand with one UE8M0 scale per 32 K values applied in
// the instruction (A format 0 = e4m3, B format 4 = e2m1).  Operand layout
// (checked on the GPU against exact arithmetic), g = lane / 16:
//   A lane l: row l % 16; bytes 0..15 hold K 16g .. 16g+15 and bytes 16..31
//     hold K 64+16g .. 64+16g+15 (the same bytes mfma_16x16x128_e4m3 uses);
//   B lane l: column l % 16; the low 16 bytes hold K 32g .. 32g+31, two per
//     byte, the even K in the low nibble (the upper 16 bytes are unused);
//   scale operands: the low byte of lane l's value is the UE8M0 exponent
//     of K block g (K 32g .. 32g+31) of row (A) / column (B) l % 16.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3_e2m1(const v8i& a, const v8i& b,
                                                        const v4f& c, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

// The e2m1 operand of mfma_16x16x128_e4m3_e2m1: a lane's 16 bytes in the
// low half (the upper half is not read).
__device__ __forceinline__ v8i e2m1_operand(const uint4& v)
{
    v8i r;
    r[0] = (int)v.x; r[1] = (int)v.y; r[2] = (int)v.z; r[3] = (int)v.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

// UE8M0 code of the smallest power of two >= s, for a positive normal f32 s
// (the f32 exponent field has the same bias, 127, as UE8M0).
__device__ __forceinline__ uint32_t e8m0_ceil_code(float s)
{
    const uint32_t u = __float_as_uint(s);
    return (u >> 23) + ((u & 0x7FFFFFu) != 0u);
}

// 2^(127 - code) as an f32, for 1 <= code <= 253: the reciprocal of the
// scale a UE8M0 code stands for, exact.
__device__ __forceinline__ float e8m0_inverse(uint32_t code)
{
    return __uint_as_float((254u - code) << 23);
}

// f32 -> OCP e4m3 (E4M3FN) code, round to nearest even, magnitudes >= 448
// saturate to 448, sign of zero kept, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return 0x7Fu;
    if (a >= 0x43E00000u)  // 448.0f
        return sign | 0x7Eu;
    if (a >= 0x3C800000u) {  // 2^-6: normal e4m3 range
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;  // RNE to 3 mantissa bits
        return sign | (r - (120u << 3));
    }
    // Subnormal e4m3: multiples of 2^-9; 8 * 2^-9 is the smallest normal.
    const float s = __uint_as_float(a) * 512.0f;
    return sign | (uint32_t)__builtin_rintf(s);
}

// The same code from the gfx950 converter: v_cvt_pk_fp8_f32 rounds to
// nearest even; clamping to +-448 first gives the saturation, and NaN is
// mapped explicitly.  Equal to f32_to_e4m3 for every one of the 2^32 f32
// bit patterns (checked exhaustively on the GPU).
__device__ __forceinline__ uint32_t f32_to_e4m3_hw(float v)
{
    if (v != v)
        return 0x7Fu;
    const float c = __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// e4m3 code of the correctly rounded quotient v / sf, given rsf = 1 / sf
// from the hardware reciprocal (<= 1 ulp): y = v * rsf lies within 2^-22
// (relative) of the rounded quotient, so the quotient lies between
// y (1 - 2^-20) and y (1 + 2^-20); the encoder is monotone, so when both ends
// give the same code, so does the quotient.  Only otherwise (y within ~2^-20
// of a rounding boundary of the e4m3 grid) is the division done.
// (f32_to_e4m3_hw's NaN test is made once, on y: for a NaN y both bracket
// ends clamp to -448, agree, and the code is 0x7F.)
__device__ __forceinline__ uint32_t requant_e4m3(float v, float sf, float rsf)
{
    const float y = v * rsf;
    auto sat = [](float x) {
        const float c = __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
    };
    const uint32_t lo = sat(y * (1.0f - 0x1p-20f));
    const uint32_t hi = sat(y * (1.0f + 0x1p-20f));
    if (lo == hi)
        return y != y ? 0x7Fu : lo;
    return f32_to_e4m3_hw(v / sf);
}

// x / 448 correctly rounded without the division sequence: q0 = x * c with
// c = RN(1/448), the residual x - 448 q0 (exact in f32, one fma), and one
// correction q0 + r c (one fma).  Equal to the IEEE quotient for every
// f32 significand (checked exhaustively on the CPU; the quotient of a
// normal x depends on its significand only); x = inf gives q0 = inf.
__device__ __forceinline__ float div448(float x)
{
    constexpr float c = 1.0f / 448.0f;
    const float q0 = x * c;
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, 448.0f, x), c, q0);
    return q == q ? q : q0;
}

// Requant scale of a block with the given amax: the raw max(amax, 1e-10)/448
// or, with pow2, the smallest power of two at or above it (PR #383's choice).
// rsf: the hardware reciprocal of the raw scale (requant_q brackets it) or
// the exact inverse of the power of two.
__device__ __forceinline__ float requant_sf(float amax, bool pow2, float& rsf)
{
    const float s = div448(fmaxf(amax, 1e-10f));
    if (pow2) {
        const uint32_t c = min(e8m0_ceil_code(s), 253u);
        rsf = e8m0_inverse(c);
        return __uint_as_float(c << 23);
    }
    rsf = __builtin_amdgcn_rcpf(s);
    return s;
}

// e4m3 code of v / sf for a scale from requant_sf (a power-of-two scale
// divides exactly by multiplying with its inverse).
__device__ __forceinline__ uint32_t requant_q(float v, float sf, float rsf, bool pow2)
{
    return pow2 ? f32_to_e4m3_hw(v * rsf) : requant_e4m3(v, sf, rsf);
}

// requant_q of two values of one block (v0's code in bits 0-7, v1's in bits
// 8-15) with one v_cvt_pk_fp8_f32 per bracket end for both.  The pair
// leaves the fast path (each value then takes requant_q) where either
// value's bracket ends disagree or its quotient is NaN -- exactly where
// requant_q would divide or return 0x7F -- so the codes are requant_q's.
__device__ __forceinline__ uint32_t requant_q2(float v0, float v1, float sf, float rsf, bool pow2)
{
    auto sat = [](float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f); };
    const float y0 = v0 * rsf, y1 = v1 * rsf;
    if (pow2) {  // y is the exact quotient
        const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(y0), sat(y1), 0, false);
        return (y0 != y0 ? 0x7Fu : c & 0xFFu) | ((y1 != y1 ? 0x7Fu : (c >> 8) & 0xFFu) << 8);
    }
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                            sat(y0 * (1.0f - 0x1p-20f)), sat(y1 * (1.0f - 0x1p-20f)), 0, false) & 0xFFFFu;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                            sat(y0 * (1.0f + 0x1p-20f)), sat(y1 * (1.0f + 0x1p-20f)), 0, false) & 0xFFFFu;
    if (lo == hi && y0 == y0 && y1 == y1)
        return lo;
    return requant_e4m3(v0, sf, rsf) | (requant_e4m3(v1, sf, rsf) << 8);
}

// Activation clamp of gate / up before the SwiGLU ("MegaMoE SM90
// Implementation Design" §10.1); c <= 0: none.
__device__ __forceinline__ float clamp_act(float v, float c)
{
    return c > 0.f ? fminf(fmaxf(v, -c), c) : v;
}

// clamp_act applied in place to N accumulator vectors: one branch on the
// (workgroup-uniform) bound instead of a select per value.
template <int N>
__device__ __forceinline__ void clamp_acc(v4f* acc, float c)
{
    if (c > 0.f) {
#pragma unroll
        for (int q = 0; q < N; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[q][i] = fminf(fmaxf(acc[q][i], -c), c);
    }
}

// SiLU with the hardware exp2 and reciprocal (a few ulp from
// g / (1 + expf(-g)); g -> -inf gives -0, g -> +inf gives g).
__device__ __forceinline__ float silu(float g)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f));
}

// f32 -> bf16 bits, round to nearest even, a NaN quieted with its payload
// kept: gfx950's v_cvt_pk_bf16_f32 (the compiler's conversion), which
// equals that rounding done on the integer bits for every one of the 2^32
// f32 patterns (denormals preserved; moe_probe_conversions checks it).
__device__ __forceinline__ uint16_t f32_to_bf16(float v)
{
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Two values in one conversion: a in bits 0-15, b in bits 16-31.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b)
{
    return __uint_as_float(b << 16);
}

// v from another lane of the same 16-lane row, by a DPP row permutation.
template <int CTRL>
__device__ __forceinline__ float row_perm(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                      0xF, 0xF, false));
}

// Max over the 16 lanes that share (lane / 16), all of them active: swap
// neighbours, swap pairs, mirror each 8-lane half, mirror the row (DPP, no
// LDS round trip; max is exact, so the pairing does not change the value).
__device__ __forceinline__ float max16(float v)
{
    v = fmaxf(v, row_perm<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, row_perm<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, row_perm<0x141>(v));  // row_half_mirror
    v = fmaxf(v, row_perm<0x140>(v));  // row_mirror
    return v;
}

// max16 for values that are >= 0 and never NaN (a running fmaxf(m, |v|)
// from m = 0 ignores NaN): on such floats the order of the bit patterns is
// the order of the values, so the max runs on the integer bits and needs
// no NaN handling (each step one DPP max instead of a move, a canonicalise
// and a max).
template <int CTRL>
__device__ __forceinline__ uint32_t row_perm_u(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float max16_nonneg(float x)
{
    uint32_t v = __float_as_uint(x);
    v = max(v, row_perm_u<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max(v, row_perm_u<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max(v, row_perm_u<0x141>(v));  // row_half_mirror
    v = max(v, row_perm_u<0x140>(v));  // row_mirror
    return __uint_as_float(v);
}

__device__ __forceinline__ v8i pack_frag(const uint4& lo, const uint4& hi)
{
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

}  // namespace moe
