// L1 / L2 grouped GEMMs on 64-row tiles with the activation rows shared
// through LDS ("shared-A" tiles, prefill shapes with ~24-64 routed rows per
// expert), for the FP8 recipe (gemm_sa) and the FP8 x MXFP4 recipe
// (gemm_sa_mx, further below).
//
// Same arithmetic as the direct-load and LDS-staged kernels ("MegaMoE SM90
// Implementation Design" §5.3 promotion per 128-K block, §10.1 / §11.1
// epilogues): for every K block kb, p = 16x16x128 e4m3 MFMA with C = 0, then
//   acc = fmaf(sa[row, kb] * sb[col block, kb], p, acc).
//
// gfx950 mapping.  A workgroup is 4 waves over one tile of 64 pool rows:
// L1 128 gate + 128 up columns (wave w: gate columns [32w, 32w+32) and the
// same up columns), L2 256 output columns (wave w: [64w, 64w+64)).  Each
// wave streams its own weight subtiles straight into registers, one K block
// ahead, as the decode tiles do (each weight byte is read by exactly one
// wave).  The tile's 64 activation rows (and their scales) are the operand
// every wave needs: instead of four register copies per workgroup they are
// copied once per K block global -> LDS (gfx950's global_load_lds, in MFMA
// fragment order) into a three-stage ring, and each wave reads its fragments
// from there after one barrier.  That keeps a wave within 256 VGPRs, so two
// workgroups share a compute unit and one's epilogue runs under the other's
// weight stream.  (A third register set, two blocks ahead, spills.)
//
// Waits.  The copies are inline assembly the compiler does not count, so the
// wait for K block kb's activation copies is explicit: vector-memory
// operations retire in order, and after kb's copies each wave has issued
// kb's 8 weight loads and, when block kb + 1 has been fetched, that block's
// 3 copies and 8 weight loads.  The weight-scale loads are left out of the
// count (the compiler may make them scalar loads, which vmcnt does not
// count): a count that omits operations issued after the copies only makes
// the wait longer, which is always safe.  The compiler's own wait before
// the MFMAs covers the weight registers.
#include "moe_device.h"
#include "moe_direct.h"
#include "moe_internal.h"
#include "moe_lds.h"

namespace moe {

namespace {

constexpr int SA_BM = 64;
constexpr int SA_NS = 3;                    // activation stages
constexpr int SA_A = SA_BM * 128;           // 8 KiB: 4 m-subtiles x 2 halves x 1 KiB
constexpr int SA_STAGE = SA_A + 4 * 256;    // + one 256-byte scale copy per wave
constexpr int SA_SUBTILES = 4;              // weight subtiles per wave
constexpr int SA_WLOADS = SA_SUBTILES * 2;  // weight loads per wave and K block (load_wfrag: 2)
constexpr int SA_ACOPIES = 2;               // activation copies per wave and K block (2 halves)
constexpr int SA_SCOPIES = 1;               //   + the activation scales
constexpr int SA_COPIES = SA_ACOPIES + SA_SCOPIES;
static_assert(SA_A == 4 * SA_ACOPIES * 1024, "four waves copy the A stage");

}  // namespace

// G64: per-64 intermediate scales ("MegaMoE SM90 Implementation Design"
// §5.4).  L1 requantises each 64-column half of its 128 gate/up columns on
// its own (waves 2b and 2b + 1 hold block b); L2 copies both scales of each
// row and K block (lanes 0-15 the first, 16-31 the second) and multiplies
// each 128-K block as its two 64-K halves -- bytes 0-15 of every A fragment
// are K 0-63, bytes 16-31 K 64-127, so a copy with one half zeroed gives
// that half's sum -- each promoted with its own activation scale.  The
// dual-half L2 needs more registers than two workgroups per compute unit
// leave (18-32 VGPRs spill); one workgroup per unit fits without spills but
// measured slower (flash-prefill L2 478 -> 589 us), so the spills stay.
template <bool L1, bool PK, bool G64>
__global__ __launch_bounds__(256, 2) void gemm_sa(FwdArgs a)
{
    __shared__ __attribute__((aligned(1024))) uint8_t stage_mem[SA_NS * SA_STAGE];
    constexpr bool D64 = G64 && !L1;  // L2 multiplies dual halves
    const int H = a.H, I = a.I, K = a.K, T = a.T;
    const int NT = L1 ? I / 128 : H / 256;
    const int nkb = L1 ? H / 128 : I / 128;
    const int mb = blockIdx.x / NT;
    const int nt = blockIdx.x - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0 || e >= a.E)
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = mb * SA_BM;
    const uint32_t stage_lds = lds_addr(stage_mem);
    // slot indices are range-checked before they form addresses
    const int TK = T * K;
    auto slot_f = [&](int f) { return (f >= 0 && f < TK) ? f : -1; };

    // Activation copies: wave w copies m-subtile w (rows row0 + 16 w + lr),
    // both 64-byte halves, and the scale of row 16 w + (lane & 15).  A
    // padding row (row_src < 0) copies a valid row (L1: token 0; L2: the
    // block's first row, which always holds a slot): its products reach
    // only that padding row of the accumulator, which is never stored.
    const int fr = slot_f(a.row_src[row0 + 16 * wave + lr]);
    const uint8_t* asrc;
    const float* ssrc;
    if constexpr (L1) {
        const size_t tok = fr >= 0 ? (size_t)(fr / K) : 0;
        asrc = a.x + tok * H + 16 * lg;
        ssrc = a.x_sf + tok * (H / 128);
    } else {
        const size_t r = fr >= 0 ? (size_t)(row0 + 16 * wave + lr) : (size_t)row0;
        asrc = a.h + r * I + 16 * lg;
        ssrc = D64 ? a.h_sf + r * (I / 64) + (lg & 1) : a.h_sf + r * (I / 128);
    }

    // Weights: subtile s of this wave (L1: s = 0,1 gate, 2,3 up).
    const uint8_t* bptr[4];
    constexpr size_t kstride = PK ? 32768 : 128;
    const float* sfg;
    const float* sfu;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if constexpr (L1) {
            if constexpr (PK) {
                bptr[s] = a.w1 + (size_t)e * 2 * I * H + (size_t)nt * nkb * 32768 +
                          (wave * 4 + s) * 2048 + lane * 16;
            } else {
                const int n = (s >= 2 ? I : 0) + nt * 128 + wave * 32 + (s & 1) * 16 + lr;
                bptr[s] = a.w1 + ((size_t)e * 2 * I + n) * H + lg * 16;
            }
        } else {
            if constexpr (PK) {
                bptr[s] = a.w2 + (size_t)e * H * I + (size_t)nt * nkb * 32768 +
                          (wave * 4 + s) * 2048 + lane * 16;
            } else {
                const int n = nt * 256 + wave * 64 + s * 16 + lr;
                bptr[s] = a.w2 + ((size_t)e * H + n) * I + lg * 16;
            }
        }
    }
    if constexpr (L1) {
        sfg = a.w1_sf + ((size_t)e * (2 * I / 128) + nt) * nkb;
        sfu = a.w1_sf + ((size_t)e * (2 * I / 128) + I / 128 + nt) * nkb;
    } else {
        sfg = a.w2_sf + ((size_t)e * (H / 128) + (nt * 256 + wave * 64) / 128) * nkb;
        sfu = sfg;
    }

    v4f acc[4][4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    struct Blk {
        Frag2 fb[4];
        float sg, su;
    };
    int fetched = -1;  // last K block fetched
    auto fetch = [&](Blk& b, int kb) {
        const uint32_t st = stage_lds + (kb % SA_NS) * SA_STAGE;
#pragma unroll
        for (int j = 0; j < SA_ACOPIES; ++j)
            dma16(asrc + (size_t)kb * 128 + 64 * j, st + (wave * 2 + j) * 1024);
        static_assert(SA_SCOPIES == 1, "one scale copy below");
        dma4(ssrc + (D64 ? 2 * kb : kb), st + SA_A + wave * 256);
        b.sg = sfg[kb];
        b.su = L1 ? sfu[kb] : b.sg;
#pragma unroll
        for (int s = 0; s < SA_SUBTILES; ++s)
            b.fb[s] = load_wfrag<PK>(bptr[s] + kb * kstride);
        fetched = kb;
    };
    int kb_m = 0;  // K block the next multiply takes
    auto mul = [&](const Blk& b) {
        // block kb_m's activation copies have landed (every wave's), and
        // every wave is done reading the stage the next fetch overwrites
        if (fetched > kb_m)
            MOE_WAIT_VMCNT(SA_WLOADS + SA_COPIES + SA_WLOADS);
        else
            MOE_WAIT_VMCNT(SA_WLOADS);
        __syncthreads();
        const uint8_t* st = stage_mem + (kb_m % SA_NS) * SA_STAGE;
        const float* s_lds = reinterpret_cast<const float*>(st + SA_A);
        if constexpr (D64) {
            // one m-subtile at a time (its fragment, both halves' scales),
            // which keeps the dual-half multiply within the register budget
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                const v8i af = lds_frag(st + ms * 2048, lane);
                const float4 s4 = *reinterpret_cast<const float4*>(s_lds + ms * 64 + 4 * lg);
                // the second half's scales, copied by lanes 16-31
                const float4 t4 = *reinterpret_cast<const float4*>(s_lds + ms * 64 + 16 + 4 * lg);
                const float sa[4] = {s4.x, s4.y, s4.z, s4.w}, sa2[4] = {t4.x, t4.y, t4.z, t4.w};
                const v8i alo = {af[0], af[1], af[2], af[3], 0, 0, 0, 0};
                const v8i ahi = {0, 0, 0, 0, af[4], af[5], af[6], af[7]};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const v8i bv = pack_frag(b.fb[s].lo, b.fb[s].hi);
                    const float sb = b.sg;
                    const v4f plo = mfma_16x16x128_e4m3(alo, bv, v4f{0.f, 0.f, 0.f, 0.f});
                    const v4f phi = mfma_16x16x128_e4m3(ahi, bv, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[ms][s][i] = fmaf(sa[i] * sb, plo[i], acc[ms][s][i]);
                        acc[ms][s][i] = fmaf(sa2[i] * sb, phi[i], acc[ms][s][i]);
                    }
                }
            }
        } else {
            v8i af[4];
            float sa[4][4];
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                af[ms] = lds_frag(st + ms * 2048, lane);
                const float4 s4 = *reinterpret_cast<const float4*>(s_lds + ms * 64 + 4 * lg);
                sa[ms][0] = s4.x;
                sa[ms][1] = s4.y;
                sa[ms][2] = s4.z;
                sa[ms][3] = s4.w;
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const v8i bv = pack_frag(b.fb[s].lo, b.fb[s].hi);
                const float sb = (L1 && s >= 2) ? b.su : b.sg;
#pragma unroll
                for (int ms = 0; ms < 4; ++ms) {
                    const v4f p = mfma_16x16x128_e4m3(af[ms], bv, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[ms][s][i] = fmaf(sa[ms][i] * sb, p[i], acc[ms][s][i]);
                }
            }
        }
        ++kb_m;
    };
    // The ring has three stages and a fetch runs one block ahead of the
    // multiply, so the stage a fetch writes was last read two multiplies
    // ago, before the barrier of the one in between.
    kloop<Blk>(0, nkb, fetch, mul);

    if constexpr (L1) {
        // ---- SwiGLU x topk_w, per-row amax over the 128 columns, e4m3
        // requant, coalesced store through LDS (as the direct tiles).
        __shared__ __align__(16) float red[SA_BM][4];  // row, then wave
        __shared__ uint8_t qt[SA_BM][128];
        float hv[4][2][4];
        clamp_acc<16>(&acc[0][0], a.clamp);
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = slot_f(a.row_src[row0 + 16 * ms + 4 * lg + i]);
                const float w = f >= 0 ? a.topk_w[f] : 0.f;
                float m = 0.f;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const float g = acc[ms][s][i];
                    const float u = acc[ms][s + 2][i];
                    const float v = (silu(g) * u) * w;
                    hv[ms][s][i] = v;
                    m = fmaxf(m, fabsf(v));
                }
                m = max16(m);
                if (lr == 0)
                    red[16 * ms + 4 * lg + i][wave] = m;
            }
        }
        __syncthreads();
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * ms + 4 * lg + i;
                const float4 rm = *reinterpret_cast<const float4*>(red[r]);
                // per-64 scales: waves 2b, 2b + 1 hold block b of the tile
                const float amax = G64 ? (wave < 2 ? fmaxf(rm.x, rm.y) : fmaxf(rm.z, rm.w))
                                       : fmaxf(fmaxf(rm.x, rm.y), fmaxf(rm.z, rm.w));
                float rsf;
                const float sf = requant_sf(amax, a.pow2_scale, rsf);
                const uint32_t c2 = requant_q2(hv[ms][0][i], hv[ms][1][i], sf, rsf, a.pow2_scale);
                qt[r][wave * 32 + lr] = (uint8_t)c2;
                qt[r][wave * 32 + 16 + lr] = (uint8_t)(c2 >> 8);
                if constexpr (G64) {
                    if ((wave & 1) == 0 && lr == 0)
                        a.h_sf[(size_t)(row0 + r) * (I / 64) + nt * 2 + (wave >> 1)] = sf;
                } else if (wave == 0 && lr == 0) {
                    a.h_sf[(size_t)(row0 + r) * (I / 128) + nt] = sf;
                }
            }
        }
        __syncthreads();
        for (int c = threadIdx.x; c < SA_BM * 8; c += 256) {
            const int r = c >> 3, col = (c & 7) * 16;
            if (slot_f(a.row_src[row0 + r]) >= 0)
                *reinterpret_cast<uint4*>(a.h + (size_t)(row0 + r) * I + nt * 128 + col) =
                    *reinterpret_cast<const uint4*>(&qt[r][col]);
        }
    } else {
        // ---- bf16, staged in LDS one 32-row half at a time, 16-byte stores
        // to the (slot, token) row of the partial buffer.
        __shared__ __align__(16) uint16_t ot[SA_BM / 2][256 + 8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int mh = 0; mh < 2; ++mh)
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        ot[16 * mh + 4 * lg + i][wave * 64 + s * 16 + lr] =
                            f32_to_bf16(acc[2 * hf + mh][s][i]);
            __syncthreads();
            for (int c = threadIdx.x; c < (SA_BM / 2) * 32; c += 256) {
                const int r = c >> 5, col = (c & 31) * 8;
                const int f = slot_f(a.row_src[row0 + 32 * hf + r]);
                if (f >= 0) {
                    const int t = f / K, j = f - t * K;
                    const uint4 v = *reinterpret_cast<const uint4*>(&ot[r][col]);  // 8 bf16
                    *reinterpret_cast<uint4*>(a.partial + ((size_t)j * T + t) * H + nt * 256 + col) = v;
                }
            }
            __syncthreads();
        }
    }
}

// FP8 x MXFP4 recipe (e4m3 activations, e2m1 weights, UE8M0 scales per 32
// K values; "07 · MegaMoE" §0): the same tile with the block-scaled MFMA
// (mfma_16x16x128_e4m3_e2m1), which applies both operands' codes and
// accumulates in f32.  A wave's weight fragments of one K block are 4 x 16
// bytes of e2m1 plus 4 scale bytes per lane (~170 VGPRs in all: three
// workgroups fit a compute unit).  Each stage holds the 64 rows' e4m3
// fragments and each row's 4 UE8M0 codes of the block.  L1's epilogue
// requantises per 32 columns, one wave's gate columns.
namespace {
constexpr int SX_NS = 3;
constexpr int SX_A = 64 * 128;
constexpr int SX_STAGE = SX_A + 4 * 256;
constexpr int SX_WLOADS = 2 * SA_SUBTILES;  // per subtile a fragment and a scale byte
}  // namespace

template <bool L1, bool PK>
__global__ __launch_bounds__(256, 2) void gemm_sa_mx(FwdArgs a)
{
    __shared__ __attribute__((aligned(1024))) uint8_t stage_mem[SX_NS * SX_STAGE];
    const int H = a.H, I = a.I, K = a.K, T = a.T;
    const int HS = H / 32, IS = I / 32;
    const int NT = L1 ? I / 128 : H / 256;
    const int nkb = L1 ? H / 128 : I / 128;
    const int mb = blockIdx.x / NT;
    const int nt = blockIdx.x - mb * NT;
    const int e = a.mblock_expert[mb];
    if (e < 0 || e >= a.E)
        return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int row0 = mb * 64;
    const uint32_t stage_lds = lds_addr(stage_mem);
    const int TK = T * K;
    auto slot_f = [&](int f) { return (f >= 0 && f < TK) ? f : -1; };

    // Activation copies as in gemm_sa; the scale copy moves the row's 4
    // codes of the block (one 4-byte word).
    const int fr = slot_f(a.row_src[row0 + 16 * wave + lr]);
    const uint8_t* asrc;
    const uint8_t* ssrc;
    if constexpr (L1) {
        const size_t tok = fr >= 0 ? (size_t)(fr / K) : 0;
        asrc = a.x + tok * H + 16 * lg;
        ssrc = a.x_sfq + tok * HS;
    } else {
        const size_t r = fr >= 0 ? (size_t)(row0 + 16 * wave + lr) : (size_t)row0;
        asrc = a.h + r * I + 16 * lg;
        ssrc = a.h_sfq + r * IS;
    }

    // Weight subtile s of this wave (L1: 0,1 gate, 2,3 up): this lane's 16
    // bytes of K block kb at wl + woff[s] + kb * wk, its scale byte at
    // sl + soff[s] + kb * sk (one per-lane base, wave-uniform offsets).
    const uint8_t* wl;
    const uint8_t* sl;
    uint32_t woff[4], soff[4];
    uint32_t wk, sk;
    const uint8_t* wbase = L1 ? a.w1 : a.w2;
    const uint8_t* sbase = L1 ? a.w1_sfq : a.w2_sfq;
    if constexpr (PK) {
        const size_t t0 = ((size_t)e * NT + nt) * nkb;
        wl = wbase + t0 * 16384 + wave * 4096 + lane * 16;
        sl = sbase + t0 * 1024 + wave * 256 + lane;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            woff[s] = s * 1024;
            soff[s] = s * 64;
        }
        wk = 16384;
        sk = 1024;
    } else {
        const uint32_t KB = (L1 ? H : I) / 2, KS = L1 ? HS : IS;  // row bytes
        const size_t row0w = L1 ? (size_t)e * 2 * I + nt * 128 + wave * 32 + lr
                                : (size_t)e * H + nt * 256 + wave * 64 + lr;
        wl = wbase + row0w * KB + lg * 16;
        sl = sbase + row0w * KS + lg;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t dr = L1 ? (s >= 2 ? I : 0) + (s & 1) * 16 : s * 16;
            woff[s] = dr * KB;
            soff[s] = dr * KS;
        }
        wk = 64;
        sk = 4;
    }

    v4f acc[4][4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc[ms][s] = v4f{0.f, 0.f, 0.f, 0.f};

    struct Blk {
        uint4 fb[4];
        int sb[4];
    };
    int fetched = -1;
    auto fetch = [&](Blk& b, int kb) {
        const uint32_t st = stage_lds + (kb % SX_NS) * SX_STAGE;
#pragma unroll
        for (int j = 0; j < SA_ACOPIES; ++j)
            dma16(asrc + (size_t)kb * 128 + 64 * j, st + (wave * 2 + j) * 1024);
        dma4(ssrc + (size_t)kb * 4, st + SX_A + wave * 256);
#pragma unroll
        for (int s = 0; s < SA_SUBTILES; ++s) {
            b.fb[s] = *reinterpret_cast<const uint4*>(wl + woff[s] + (size_t)kb * wk);
            b.sb[s] = sl[soff[s] + (size_t)kb * sk];
        }
        fetched = kb;
    };
    int kb_m = 0;
    auto mul = [&](const Blk& b) {
        if (fetched > kb_m)
            MOE_WAIT_VMCNT(SX_WLOADS + SA_COPIES + SX_WLOADS);
        else
            MOE_WAIT_VMCNT(SX_WLOADS);
        __syncthreads();
        const uint8_t* st = stage_mem + (kb_m % SX_NS) * SX_STAGE;
        const uint8_t* s_lds = st + SX_A;  // row 16 ms + r: bytes 256 ms + 4 r + [0, 4)
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
            const v8i av = lds_frag(st + ms * 2048, lane);
            const int sa = s_lds[ms * 256 + 4 * lr + lg];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[ms][s] = mfma_16x16x128_e4m3_e2m1(av, e2m1_operand(b.fb[s]), acc[ms][s], sa,
                                                      b.sb[s]);
        }
        ++kb_m;
    };
    // One block ahead, two register sets (a third, two blocks ahead, made
    // the kernel spill and measured no faster); the ring's three stages
    // suffice as in gemm_sa.
    kloop<Blk>(0, nkb, fetch, mul);

    if constexpr (L1) {
        // ---- SwiGLU x topk_w; wave w's 32 gate columns are one
        // requantisation block of each row: its amax, the power-of-two
        // scale as a UE8M0 code, codes staged in LDS for row stores.
        clamp_acc<16>(&acc[0][0], a.clamp);
        __shared__ uint8_t qt[64][128];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * ms + 4 * lg + i;
                const int f = slot_f(a.row_src[row0 + r]);
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
        __syncthreads();
        for (int c = threadIdx.x; c < 64 * 8; c += 256) {
            const int r = c >> 3, col = (c & 7) * 16;
            if (slot_f(a.row_src[row0 + r]) >= 0)
                *reinterpret_cast<uint4*>(a.h + (size_t)(row0 + r) * I + nt * 128 + col) =
                    *reinterpret_cast<const uint4*>(&qt[r][col]);
        }
    } else {
        __shared__ __align__(16) uint16_t ot[32][256 + 8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int mh = 0; mh < 2; ++mh)
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        ot[16 * mh + 4 * lg + i][wave * 64 + s * 16 + lr] =
                            f32_to_bf16(acc[2 * hf + mh][s][i]);
            __syncthreads();
            for (int c = threadIdx.x; c < 32 * 32; c += 256) {
                const int r = c >> 5, col = (c & 31) * 8;
                const int f = slot_f(a.row_src[row0 + 32 * hf + r]);
                if (f >= 0) {
                    const int t = f / K, j = f - t * K;
                    const uint4 v = *reinterpret_cast<const uint4*>(&ot[r][col]);  // 8 bf16
                    *reinterpret_cast<uint4*>(a.partial + ((size_t)j * T + t) * H + nt * 256 + col) = v;
                }
            }
            __syncthreads();
        }
    }
}

template <bool L1>
static hipError_t launch_sa(const FwdArgs& a, hipStream_t s)
{
    const int NT = L1 ? a.I / 128 : a.H / 256;
    const long long grid = (long long)a.grid_mblocks * NT;
    // FP8 needs two K blocks per layer, MXFP4 three
    if (a.BM != SA_BM || (!L1 && a.H % 256) || (L1 ? a.H : a.I) < (a.mx ? 384 : 256))
        return hipErrorInvalidValue;
    if (grid <= 0)
        return hipSuccess;
    if (a.mx) {
        auto kern = a.packed ? gemm_sa_mx<L1, true> : gemm_sa_mx<L1, false>;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, a);
    } else if (a.sf_gran64) {
        auto kern = a.packed ? gemm_sa<L1, true, true> : gemm_sa<L1, false, true>;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, a);
    } else {
        auto kern = a.packed ? gemm_sa<L1, true, false> : gemm_sa<L1, false, false>;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_l1_sa(const FwdArgs& a, hipStream_t s) { return launch_sa<true>(a, s); }
hipError_t launch_l2_sa(const FwdArgs& a, hipStream_t s) { return launch_sa<false>(a, s); }

}  // namespace moe
