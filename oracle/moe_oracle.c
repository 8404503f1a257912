/*
 * CPU oracle for the FP8 MoE expert forward.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke entry and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or helper with
 * the HIP path under fp8_grouped_gemm_amd/, and the HIP path never calls it.
 *
 * What it computes, step by step, and the passage each step follows
 * (pages cited by title and section; the reading taken where a page is
 * silent is stated at the step):
 *
 *   route      "07 · MegaMoE" §7 (count tokens per expert, skip masked
 *              slots) and §4 (per-expert pool segments aligned to the row
 *              tile, pool offset = prefix sum of aligned segment sizes).
 *              Reading: rows inside a segment are in ascending flat slot
 *              index f = t*K + j; §7 says the order inside a segment does
 *              not affect correctness, so a fixed order is a free choice.
 *   L1         "MegaMoE SM90 Implementation Design" §5.3: block-scaled FP8
 *              GEMM, fp32 accumulation, one activation scale per 1x128 and
 *              one weight scale per 128x128 block (§15.2 scale layout
 *              [E, N/128, K/128]).  Reading: the sum inside one 128-wide K
 *              block is taken exactly and rounded once to f32, then
 *              acc = fmaf(sa*sb, p, acc) over K blocks in ascending order.
 *   SwiGLU     same doc §10.1 and "07 · MegaMoE" §8: silu(g)*u*w with
 *              silu(g) = g / (1 + exp(-g)), the router weight applied here
 *              once.  Gate = rows [0, I) of W1, up = rows [I, 2I).
 *   requant    DeepGEMM PR #440 "How it works"/"Ring sizing" text on the
 *              raw scale: sf = max(amax, 1e-10) / 448, q = e4m3(h / sf), one
 *              scale per 128 consecutive intermediate columns (PR #360 on
 *              per-128 quantisation of the L1 output).  Division correctly
 *              rounded; e4m3 is OCP E4M3FN with round-to-nearest-even and
 *              saturation to +-448.
 *   L2         design doc §3.3 / §11.1: same block-scaled GEMM over the
 *              intermediate dimension, fp32 result cast to BF16 (RNE) per
 *              (token, slot) partial.
 *   combine    design doc §11.2 and "07 · MegaMoE" §9: per token, fp32 sum
 *              of its active slots' BF16 partials (slot order ascending,
 *              starting from 0), cast to BF16.  Slots with an expert id < 0
 *              (masked) or >= E (out of range) contribute nothing; a token
 *              with no active slot gets y = 0.
 *
 * Second recipe, FP8 activations x MXFP4 weights ("07 · MegaMoE" §0 and the
 * "MegaMoE SM90 Implementation Design" §2.1/§15.2 contrast of the SM100
 * kernel: e4m3 activations, e2m1 weights, one UE8M0 scale per 32 K values,
 * recipe (1,1,32), and the L1 epilogue's per-block UE8M0 scale for the
 * requantised intermediate).  Readings where the pages are silent:
 *   - scales apply per element inside the sum (they are the MX block
 *     scales of both operands); the GEMM value is the sum over all of K,
 *     each 32-block's sum exact, the blocks added in ascending order in
 *     binary64, rounded once to f32 -- the exact sum whenever a row's block
 *     sums span fewer than 53 bits, as for every input drawn here (checked
 *     against exact rationals);
 *   - the intermediate uses the same 1x32 blocks as the activations, with
 *     sf = the smallest power of two >= max(amax, 1e-10)/448 (PR #440 "How
 *     it works" names rounding the scale up to a power of two as #383's
 *     choice; a power of two is what a UE8M0 code can hold), q = e4m3(h/sf);
 *   - e2m1 pairs are packed two per byte, element k in byte k/2, the even
 *     element in the low nibble; UE8M0 code c means 2^(c-127), 0xFF is NaN.
 *
 * Recipe options (both recipes unless noted):
 *   clamp      "MegaMoE SM90 Implementation Design" §10.1: with an activation
 *              clamp c, gate = clamp(gate, -c, c) and up = clamp(up, -c, c)
 *              before the SwiGLU (c <= 0 here means no clamp, the default).
 *   pow2 scale (FP8 recipe) DeepGEMM PR #440 "How it works": #383 rounds the
 *              requant scale up to the next power of two; sf = the smallest
 *              power of two >= max(amax, 1e-10)/448, q = e4m3(h / sf).
 *   per-64     (FP8 recipe) design doc §5.4: one scale per 64 intermediate
 *              columns, and L2 splits each 128-K block into two 64-K halves,
 *              each scaled by its own activation scale and the block's weight
 *              scale.  Reading: within block kb, acc = fmaf(sa[2kb] sb, p_lo,
 *              acc) then acc = fmaf(sa[2kb+1] sb, p_hi, acc), p_lo / p_hi the
 *              exact 64-term sums rounded once to f32.
 *
 * Steps 5-6 alone: orc_moe_l2_combine (and its MXFP4 form) start L2 from a
 * given intermediate h / h_sf, so a test can feed it the GPU's own h and
 * compare each later step with the GPU's; fed the forward's own h it
 * returns the forward's partials and y bit for bit.  The forward can also
 * return the L1 accumulator, its magnitude sum |a||b| scale per column (the
 * scale of a bound on rounding inside a block), and the SwiGLU value before
 * requantisation, for the same step-by-step comparison.
 *
 * Pins: every function here is checked against something other than itself
 * (tests/test_oracle_pins*.py): closed forms, library codecs, an fp64
 * unquantised MoE, a dense SwiGLU FFN written separately, brute-force
 * routing, exact rational arithmetic, and the forward itself for the
 * L2 + combine entries.  No function here is unpinned.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- codecs */

/* OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, 0x7F / 0xFF are NaN, largest finite magnitude 448. */
float orc_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int exp = (code >> 3) & 0xF;
    int man = code & 0x7;
    float mag;
    if (exp == 0xF && man == 0x7)
        return NAN;
    if (exp == 0)
        mag = ldexpf((float)man, -9);                 /* man/8 * 2^-6 */
    else
        mag = ldexpf(1.0f + (float)man / 8.0f, exp - 7);
    return sign ? -mag : mag;
}

/* Nearest finite E4M3FN value; ties go to the even code (even mantissa
 * LSB); magnitudes at or above 448 saturate to 448; the sign of zero is
 * kept; NaN maps to 0x7F.  Written as a search over the 127 non-negative
 * finite codes so that it is the definition, not a bit trick. */
uint8_t orc_e4m3_encode(float v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;
    int best = 0;
    double best_err = a;                               /* distance to code 0 */
    for (int c = 1; c <= 0x7E; ++c) {
        double err = fabs((double)orc_e4m3_decode((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return sign | (uint8_t)best;
}

/* BF16 is the top half of an IEEE binary32; round to nearest even. */
uint16_t orc_bf16_rne(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    if (isnan(v))
        return (uint16_t)((u >> 16) | 0x40);
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1;
    return (uint16_t)upper;
}

float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* --------------------------------------------------------------- routing */

/* Plan of the per-expert pool ("07 · MegaMoE" §4, §7).
 *   counts[e]   number of slots f with idx[f] == e (ids < 0 or >= E skipped)
 *   offsets[e]  start row of expert e's segment; offsets[E] = pool rows used;
 *               offsets[e+1] = offsets[e] + ceil(counts[e]/row_align)*row_align
 *   row_src[r]  flat slot f stored in pool row r, -1 on padding rows,
 *               for r < r_cap (rows past offsets[E] are -1)
 *   src_row[f]  pool row of slot f, -1 for skipped slots
 * Returns the number of slots with an id >= E (flagged, skipped). */
int orc_route(int T, int K, int E, int row_align, const int32_t* idx,
              int32_t* counts, int32_t* offsets, int32_t* row_src, int r_cap,
              int32_t* src_row)
{
    int bad = 0;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int f = 0; f < T * K; ++f) {
        if (idx[f] >= E)
            ++bad;
        else if (idx[f] >= 0)
            ++counts[idx[f]];
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + (counts[e] + row_align - 1) / row_align * row_align;
    for (int r = 0; r < r_cap; ++r)
        row_src[r] = -1;
    for (int f = 0; f < T * K; ++f)
        src_row[f] = -1;
    for (int e = 0; e < E; ++e) {
        int r = offsets[e];
        for (int f = 0; f < T * K; ++f) {
            if (idx[f] == e) {
                if (r < r_cap)
                    row_src[r] = f;
                src_row[f] = r;
                ++r;
            }
        }
    }
    return bad;
}

/* ----------------------------------------------------- block-scaled GEMM */

/* Decoded values of every e4m3 code and every e2m1 nibble, filled once from
 * orc_e4m3_decode / orc_e2m1_decode (a table of the decoder's own values, so
 * the sums below read exactly what the decoder defines, only faster). */
float orc_e2m1_decode(uint8_t code);
static double g_e4m3[256];
static double g_e2m1[16];
static int g_tables_ready;

static void init_tables(void)
{
    if (g_tables_ready)
        return;
    for (int c = 0; c < 256; ++c)
        g_e4m3[c] = (double)orc_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 16; ++c)
        g_e2m1[c] = (double)orc_e2m1_decode((uint8_t)c);
    g_tables_ready = 1;
}

/* Exact sum over one 128-wide K block of decoded e4m3 products.  Every
 * e4m3 value is an integer multiple of 2^-9 below 2^9, so each product is
 * a multiple of 2^-18 below 2^18 and 128 of them sum exactly in binary64
 * (in any order). */
double orc_block_dot_e4m3(const uint8_t* a, const uint8_t* b, int n)
{
    init_tables();
    double s = 0.0;
    for (int c = 0; c < n; ++c)
        s += g_e4m3[a[c]] * g_e4m3[b[c]];
    return s;
}

/* The same block's sum of |products| (exact for the same reason): the
 * magnitude an error bound on a rounded accumulation of the block scales
 * with. */
static double block_abs_dot_e4m3(const uint8_t* a, const uint8_t* b, int n)
{
    double s = 0.0;
    for (int c = 0; c < n; ++c)
        s += fabs(g_e4m3[a[c]] * g_e4m3[b[c]]);
    return s;
}

/* Same for an f32 activation row against e4m3 weights (test-only path
 * with the requantisation switched off; not exact, binary64 sum). */
static double block_dot_f32_e4m3(const float* a, const uint8_t* b, int n)
{
    double s = 0.0;
    for (int c = 0; c < n; ++c)
        s += (double)a[c] * g_e4m3[b[c]];
    return s;
}

/* One output element of a block-scaled FP8 GEMM (design doc §5.3):
 *   acc = sum over K blocks kb, ascending, of fmaf(sa[kb]*sb[kb], p_kb, acc)
 * with p_kb the exact block dot product rounded once to f32. */
static float scaled_row_dot(const uint8_t* a, const float* sa, const uint8_t* b,
                            const float* sb, int kblocks)
{
    float acc = 0.0f;
    for (int kb = 0; kb < kblocks; ++kb) {
        float p = (float)orc_block_dot_e4m3(a + 128 * kb, b + 128 * kb, 128);
        float s = sa[kb] * sb[kb];
        acc = fmaf(s, p, acc);
    }
    return acc;
}

/* The same element together with its magnitude: *mag = the sum over K
 * blocks of |sa*sb| * (sum of |products| of the block), in binary64 (not
 * part of the forward; tests scale the error bound of an accumulation that
 * rounds inside a block by it).  The returned value is scaled_row_dot's:
 * the same block sums, promoted in the same order. */
static float scaled_row_dot_mag(const uint8_t* a, const float* sa, const uint8_t* b,
                                const float* sb, int kblocks, double* mag)
{
    float acc = 0.0f;
    double m = 0.0;
    for (int kb = 0; kb < kblocks; ++kb) {
        const uint8_t* ak = a + 128 * kb;
        const uint8_t* bk = b + 128 * kb;
        double ps = 0.0, pm = 0.0;
        for (int c = 0; c < 128; ++c) {
            const double pr = g_e4m3[ak[c]] * g_e4m3[bk[c]];
            ps += pr;
            pm += fabs(pr);
        }
        float s = sa[kb] * sb[kb];
        acc = fmaf(s, (float)ps, acc);
        m += fabs((double)sa[kb] * (double)sb[kb]) * pm;
    }
    *mag = m;
    return acc;
}

/* ------------------------------------------------- SwiGLU and requantise */

float orc_swiglu(float g, float u, float w)
{
    float silu = g / (1.0f + expf(-g));
    return (silu * u) * w;
}

/* Per-block requantisation of n values: sf = max(amax, 1e-10)/448 and
 * q[i] = e4m3(v[i] / sf) with a correctly rounded f32 division. */
void orc_requant_block(const float* v, int n, uint8_t* q, float* sf_out)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    float sf = fmaxf(amax, 1e-10f) / 448.0f;
    for (int i = 0; i < n; ++i)
        q[i] = orc_e4m3_encode(v[i] / sf);
    *sf_out = sf;
}

/* Forward declaration (defined with the MX codecs below). */
uint8_t orc_e8m0_ceil(float s);
double orc_e8m0_decode(uint8_t code);

/* The same with the scale rounded up to a power of two (PR #383's choice):
 * sf = the smallest power of two >= max(amax, 1e-10)/448. */
void orc_requant_block_pow2(const float* v, int n, uint8_t* q, float* sf_out)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    float sf = (float)orc_e8m0_decode(orc_e8m0_ceil(fmaxf(amax, 1e-10f) / 448.0f));
    for (int i = 0; i < n; ++i)
        q[i] = orc_e4m3_encode(v[i] / sf);
    *sf_out = sf;
}

/* Activation clamp before the SwiGLU (design doc §10.1); c <= 0: none. */
static float clamp_act(float v, float c)
{
    return c > 0.0f ? fminf(fmaxf(v, -c), c) : v;
}

/* Per-1x128 quantisation of an activation matrix, the step the pages leave
 * to the caller before each call ("07 · MegaMoE" §3 copies FP8 x and its
 * scales into the buffer): x [T,H] f32 (bf16 inputs are exact in f32) ->
 * q [T,H] e4m3, sf [T,H/128] with the requant rule above. */
void orc_quantize_rows(const float* x, int T, int H, uint8_t* q, float* sf)
{
    for (int t = 0; t < T; ++t)
        for (int kb = 0; kb < H / 128; ++kb)
            orc_requant_block(x + (size_t)t * H + 128 * kb, 128, q + (size_t)t * H + 128 * kb,
                              sf + (size_t)t * (H / 128) + kb);
}

/* ------------------------------------------ MX codecs and block scaling */

/* OCP E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0, no
 * infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Only the low
 * nibble of `code` is read. */
float orc_e2m1_decode(uint8_t code)
{
    int sign = (code >> 3) & 1;
    int exp = (code >> 1) & 3;
    int man = code & 1;
    float mag = exp == 0 ? 0.5f * (float)man : ldexpf(1.0f + 0.5f * (float)man, exp - 1);
    return sign ? -mag : mag;
}

/* Element k of a row of packed e2m1 pairs. */
static double e2m1_at(const uint8_t* row, int k)
{
    uint8_t b = row[k >> 1];
    return g_e2m1[(k & 1) ? (b >> 4) : (b & 0xF)];
}

/* UE8M0: value 2^(code - 127); code 0xFF is NaN. */
double orc_e8m0_decode(uint8_t code)
{
    if (code == 0xFF)
        return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* The smallest power of two >= s (s > 0), as a UE8M0 code; found by search
 * over the codes so that it is the definition. */
uint8_t orc_e8m0_ceil(float s)
{
    for (int c = 0; c < 0xFF; ++c)
        if (orc_e8m0_decode((uint8_t)c) >= (double)s)
            return (uint8_t)c;
    return 0xFE;
}

/* One output element of an MX GEMM:
 *   sum over k of (e4m3(a[k]) * 2^(sa[k/32]-127)) * (e2m1(b[k]) * 2^(sb[k/32]-127))
 * Each 32-term block sum is exact in binary64 (products are multiples of
 * 2^-10 of magnitude below 2688), scaling it by a power of two is exact,
 * and the blocks are added in ascending order in binary64.  NaN if a scale
 * code is 0xFF. */
double orc_mx_dot(const uint8_t* a, const uint8_t* sa, const uint8_t* b_packed,
                  const uint8_t* sb, int n)
{
    init_tables();
    double s = 0.0;
    for (int blk = 0; blk < n / 32; ++blk) {
        if (sa[blk] == 0xFF || sb[blk] == 0xFF)
            return NAN;
        double p = 0.0;
        for (int c = 32 * blk; c < 32 * blk + 32; ++c)
            p += g_e4m3[a[c]] * e2m1_at(b_packed, c);
        s += ldexp(p, (int)sa[blk] + (int)sb[blk] - 254);
    }
    return s;
}

/* Its magnitude: sum over 32-blocks of 2^(scales) * (sum of |products|). */
static double mx_mag(const uint8_t* a, const uint8_t* sa, const uint8_t* b_packed,
                     const uint8_t* sb, int n)
{
    double s = 0.0;
    for (int blk = 0; blk < n / 32; ++blk) {
        double p = 0.0;
        for (int c = 32 * blk; c < 32 * blk + 32; ++c)
            p += fabs(g_e4m3[a[c]] * e2m1_at(b_packed, c));
        s += ldexp(p, (int)sa[blk] + (int)sb[blk] - 254);
    }
    return s;
}

/* Test-only: the same sum for an f32 activation row (requantisation off). */
static double mx_dot_f32(const float* a, const uint8_t* b_packed, const uint8_t* sb, int n)
{
    double s = 0.0;
    for (int blk = 0; blk < n / 32; ++blk) {
        double p = 0.0;
        for (int c = 32 * blk; c < 32 * blk + 32; ++c)
            p += (double)a[c] * (double)e2m1_at(b_packed, c);
        s += ldexp(p, (int)sb[blk] - 127);
    }
    return s;
}

/* Requantisation of n values to e4m3 with one power-of-two scale:
 * s = max(amax, 1e-10)/448 (f32 division), sf = the smallest power of two
 * >= s, q[i] = e4m3(v[i] / sf) (an exact scaling, then the e4m3 rounding). */
void orc_requant_block_mx(const float* v, int n, uint8_t* q, uint8_t* sf_code)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    float s = fmaxf(amax, 1e-10f) / 448.0f;
    uint8_t c = orc_e8m0_ceil(s);
    float sf = (float)orc_e8m0_decode(c);
    for (int i = 0; i < n; ++i)
        q[i] = orc_e4m3_encode(v[i] / sf);
    *sf_code = c;
}

/* --------------------------------------------------------------- forward */

/* Combine (design doc §11.2; "07 · MegaMoE" §9): per token, slot order
 * ascending, f32 sum of the active slots' (bf16-rounded) partials, one
 * rounding to bf16. */
static void combine(int T, int H, int E, int K, const int32_t* idx, int n_tok,
                    const int32_t* toks, const float* part_f32, uint16_t* y, float* y_f32)
{
    (void)T;
#pragma omp parallel for schedule(static)
    for (int p = 0; p < n_tok; ++p) {
        int t = toks ? toks[p] : p;
        for (int n = 0; n < H; ++n) {
            float a = 0.0f;
            for (int j = 0; j < K; ++j) {
                int e = idx[t * K + j];
                if (e < 0 || e >= E)
                    continue;
                a += part_f32[((size_t)p * K + j) * H + n];
            }
            if (y)
                y[(size_t)p * H + n] = orc_bf16_rne(a);
            if (y_f32)
                y_f32[(size_t)p * H + n] = a;
        }
    }
}

/* Token-list validation shared by both recipes: -1 on a bad token id or a
 * missing expert array, else the number of slots with an id >= E. */
static int check_tokens(int T, int E, int K, const int32_t* idx, int n_tok, const int32_t* toks,
                        const void* const* w1, const void* const* w1_sf,
                        const void* const* w2, const void* const* w2_sf)
{
    int bad = 0;
    for (int p = 0; p < n_tok; ++p) {
        int t = toks ? toks[p] : p;
        if (t < 0 || t >= T)
            return -1;
        for (int j = 0; j < K; ++j) {
            int e = idx[t * K + j];
            if (e >= E)
                ++bad;
            else if (e >= 0 && (!w1[e] || !w1_sf[e] || !w2[e] || !w2_sf[e]))
                return -1;
        }
    }
    return bad;
}

enum {
    ORC_NO_REQUANT = 1, /* test-only: feed f32 SwiGLU output to L2 unquantised */
    ORC_NO_BF16 = 2,    /* test-only: keep partials and y in f32 */
    ORC_POW2_SCALE = 4, /* FP8 recipe: power-of-two requant scales */
    ORC_SF_GRAN64 = 8   /* FP8 recipe: per-64 intermediate scales, dual-half L2 */
};

/* L2 of one routed slot (design doc §11.1; per-64 halves: §5.4): for each
 * output column n, acc = the block-scaled dot product of the requantised row
 * (q, per-G scales qs) with W2[e] row n, then one bf16 rounding.
 *   part_f32[n] = the bf16-rounded value as f32 (the combine's input), or the
 *                 f32 value itself with ORC_NO_BF16
 *   partial[n]  = bf16 bits (optional), mag[n] = scaled_row_mag (optional)
 * With ORC_NO_REQUANT the unquantised f32 row hv is used instead of q/qs. */
static void l2_slot(int H, int I, int G, const uint8_t* q, const float* qs, const float* hv,
                    const uint8_t* w2e, const float* w2se, int flags, float* part_f32,
                    uint16_t* partial, float* mag)
{
    const int IB = I / 128;
    for (int n = 0; n < H; ++n) {
        const uint8_t* wr = w2e + (size_t)n * I;
        const float* ws = w2se + (size_t)(n / 128) * IB;
        float acc = 0.0f;
        if (flags & ORC_NO_REQUANT) {
            for (int ib = 0; ib < IB; ++ib) {
                float pdot = (float)block_dot_f32_e4m3(hv + 128 * ib, wr + 128 * ib, 128);
                acc = fmaf(ws[ib], pdot, acc);
            }
        } else if (G == 64) {
            /* design doc §5.4: each 128-K block as two 64-K halves */
            double m = 0.0;
            for (int kb = 0; kb < IB; ++kb) {
                float p_lo = (float)orc_block_dot_e4m3(q + 128 * kb, wr + 128 * kb, 64);
                float p_hi = (float)orc_block_dot_e4m3(q + 128 * kb + 64, wr + 128 * kb + 64, 64);
                acc = fmaf(qs[2 * kb] * ws[kb], p_lo, acc);
                acc = fmaf(qs[2 * kb + 1] * ws[kb], p_hi, acc);
                if (mag)
                    m += fabs((double)qs[2 * kb] * ws[kb]) * block_abs_dot_e4m3(q + 128 * kb, wr + 128 * kb, 64) +
                         fabs((double)qs[2 * kb + 1] * ws[kb]) *
                             block_abs_dot_e4m3(q + 128 * kb + 64, wr + 128 * kb + 64, 64);
            }
            if (mag)
                mag[n] = (float)m;
        } else if (mag) {
            double m;
            acc = scaled_row_dot_mag(q, qs, wr, ws, IB, &m);
            mag[n] = (float)m;
        } else {
            acc = scaled_row_dot(q, qs, wr, ws, IB);
        }
        part_f32[n] = (flags & ORC_NO_BF16) ? acc : orc_bf16_to_f32(orc_bf16_rne(acc));
        if (partial)
            partial[n] = orc_bf16_rne(acc);
    }
}

/* Forward for a list of tokens.
 *   x [T,H] e4m3, x_sf [T,H/128] f32, idx/w [T,K]
 *   w1[e] -> [2I,H] e4m3 (gate rows then up rows), w1_sf[e] -> [2I/128,H/128]
 *   w2[e] -> [H,I] e4m3, w2_sf[e] -> [H/128,I/128]
 *   (per-expert pointers; an expert no listed token uses may be NULL)
 *   toks [n_tok] token ids to compute (NULL: all T tokens, n_tok = T)
 * Outputs, indexed by position p in the token list (all optional but y):
 *   y [n_tok,H] bf16 (or y_f32 [n_tok,H] when ORC_NO_BF16)
 *   acc1 [n_tok*K, 2I] f32 L1 accumulator before SwiGLU
 *   acc1_mag [n_tok*K, 2I] its magnitude (scaled_row_mag; not part of the
 *            forward: the scale of a bound on rounding inside the blocks)
 *   hval [n_tok*K, I] f32 SwiGLU x top-k weight, before requantisation
 *   h [n_tok*K, I] e4m3, h_sf [n_tok*K, I/G]
 *   partial [n_tok*K, H] bf16 (skipped slots left untouched)
 * Returns the number of slots with an id >= E, or -1 when a needed expert
 * pointer is NULL or a shape is invalid. */
int orc_moe_forward(int T, int H, int I, int E, int K,
                    const uint8_t* x, const float* x_sf,
                    const int32_t* idx, const float* w,
                    const uint8_t* const* w1, const float* const* w1_sf,
                    const uint8_t* const* w2, const float* const* w2_sf,
                    int n_tok, const int32_t* toks,
                    uint16_t* y, float* y_f32,
                    float* acc1, float* acc1_mag, float* hval,
                    uint8_t* h, float* h_sf, uint16_t* partial,
                    int flags, float clamp, int nthreads)
{
    if (H % 128 || I % 128 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || T < 0)
        return -1;
    if (!toks)
        n_tok = T;
    init_tables();
    const int HB = H / 128;
    const int G = (flags & ORC_SF_GRAN64) ? 64 : 128;  /* intermediate scale block */
    const int NG = I / G;
    int bad = check_tokens(T, E, K, idx, n_tok, toks, (const void* const*)w1,
                           (const void* const*)w1_sf, (const void* const*)w2,
                           (const void* const*)w2_sf);
    if (bad < 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif

    /* L1 -> SwiGLU -> requant -> L2, one (token, slot) per iteration. */
    float* part_f32 = (float*)calloc((size_t)n_tok * K * H, sizeof(float));
    if (!part_f32)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ps = 0; ps < n_tok * K; ++ps) {
        int p = ps / K, j = ps % K;
        int t = toks ? toks[p] : p;
        int e = idx[t * K + j];
        if (e < 0 || e >= E)
            continue;
        float* a1 = (float*)malloc(sizeof(float) * 2 * I);
        float* hv = (float*)malloc(sizeof(float) * I);
        uint8_t* q = (uint8_t*)malloc(I);
        float* qs = (float*)malloc(sizeof(float) * NG);
        const uint8_t* xr = x + (size_t)t * H;
        const float* xs = x_sf + (size_t)t * HB;
        for (int n = 0; n < 2 * I; ++n) {
            const float* ws = w1_sf[e] + (size_t)(n / 128) * HB;
            if (acc1_mag) {
                double m;
                a1[n] = scaled_row_dot_mag(xr, xs, w1[e] + (size_t)n * H, ws, HB, &m);
                acc1_mag[(size_t)ps * 2 * I + n] = (float)m;
            } else {
                a1[n] = scaled_row_dot(xr, xs, w1[e] + (size_t)n * H, ws, HB);
            }
        }
        if (acc1)
            memcpy(acc1 + (size_t)ps * 2 * I, a1, sizeof(float) * 2 * I);
        for (int i = 0; i < I; ++i)
            hv[i] = orc_swiglu(clamp_act(a1[i], clamp), clamp_act(a1[I + i], clamp), w[t * K + j]);
        if (hval)
            memcpy(hval + (size_t)ps * I, hv, sizeof(float) * I);
        if (!(flags & ORC_NO_REQUANT)) {
            for (int ib = 0; ib < NG; ++ib) {
                if (flags & ORC_POW2_SCALE)
                    orc_requant_block_pow2(hv + G * ib, G, q + G * ib, qs + ib);
                else
                    orc_requant_block(hv + G * ib, G, q + G * ib, qs + ib);
            }
            if (h)
                memcpy(h + (size_t)ps * I, q, I);
            if (h_sf)
                memcpy(h_sf + (size_t)ps * NG, qs, sizeof(float) * NG);
        }
        l2_slot(H, I, G, q, qs, hv, w2[e], w2_sf[e], flags, part_f32 + (size_t)ps * H,
                partial ? partial + (size_t)ps * H : NULL, NULL);
        free(a1);
        free(hv);
        free(q);
        free(qs);
    }

    combine(T, H, E, K, idx, n_tok, toks, part_f32, y, y_f32);
    free(part_f32);
    return bad;
}

/* Steps 5-6 alone (L2 + combine), started from a given requantised
 * intermediate instead of the one step 4 computes: h [n_tok*K, I] e4m3 and
 * h_sf [n_tok*K, I/G] (G = 64 with ORC_SF_GRAN64, else 128), indexed like
 * the forward's outputs (slot j of the p-th listed token at row p*K + j;
 * rows of skipped slots are not read).  Fed the forward's own h and h_sf it
 * returns the forward's y and partials bit for bit.  Outputs: y [n_tok,H]
 * bf16, partial [n_tok*K,H] bf16 and o_mag [n_tok*K,H] (the L2 magnitude,
 * as acc1_mag), the last two optional.  Same return values as the forward. */
int orc_moe_l2_combine(int T, int H, int I, int E, int K,
                       const int32_t* idx,
                       const uint8_t* const* w2, const float* const* w2_sf,
                       int n_tok, const int32_t* toks,
                       const uint8_t* h, const float* h_sf,
                       uint16_t* y, uint16_t* partial, float* o_mag,
                       int flags, int nthreads)
{
    if (H % 128 || I % 128 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || T < 0 ||
        (flags & (ORC_NO_REQUANT | ORC_NO_BF16)))
        return -1;
    if (!toks)
        n_tok = T;
    init_tables();
    const int G = (flags & ORC_SF_GRAN64) ? 64 : 128;
    const int NG = I / G;
    int bad = check_tokens(T, E, K, idx, n_tok, toks, (const void* const*)w2,
                           (const void* const*)w2_sf, (const void* const*)w2,
                           (const void* const*)w2_sf);
    if (bad < 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
    float* part_f32 = (float*)calloc((size_t)n_tok * K * H, sizeof(float));
    if (!part_f32)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ps = 0; ps < n_tok * K; ++ps) {
        int p = ps / K, j = ps % K;
        int t = toks ? toks[p] : p;
        int e = idx[t * K + j];
        if (e < 0 || e >= E)
            continue;
        l2_slot(H, I, G, h + (size_t)ps * I, h_sf + (size_t)ps * NG, NULL, w2[e], w2_sf[e],
                flags, part_f32 + (size_t)ps * H, partial ? partial + (size_t)ps * H : NULL,
                o_mag ? o_mag + (size_t)ps * H : NULL);
    }
    combine(T, H, E, K, idx, n_tok, toks, part_f32, y, NULL);
    free(part_f32);
    return bad;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* L2 of one routed slot of the MXFP4 recipe: per output column the MX dot
 * product of the requantised row (q, UE8M0 codes qs per 32) with W2[e] row
 * n, rounded once to f32, then to bf16 (outputs as l2_slot). */
static void l2_slot_mx(int H, int I, const uint8_t* q, const uint8_t* qs, const float* hv,
                       const uint8_t* w2e, const uint8_t* w2se, int flags, float* part_f32,
                       uint16_t* partial, float* mag)
{
    const int IS = I / 32;
    for (int n = 0; n < H; ++n) {
        const uint8_t* wr = w2e + (size_t)n * (I / 2);
        const uint8_t* ws = w2se + (size_t)n * IS;
        float acc = (flags & ORC_NO_REQUANT) ? (float)mx_dot_f32(hv, wr, ws, I)
                                             : (float)orc_mx_dot(q, qs, wr, ws, I);
        if (mag)
            mag[n] = (float)mx_mag(q, qs, wr, ws, I);
        part_f32[n] = (flags & ORC_NO_BF16) ? acc : orc_bf16_to_f32(orc_bf16_rne(acc));
        if (partial)
            partial[n] = orc_bf16_rne(acc);
    }
}

/* Forward of the FP8 x MXFP4 recipe, same structure and outputs as
 * orc_moe_forward:
 *   x [T,H] e4m3, x_sf [T,H/32] UE8M0, idx/w [T,K]
 *   w1[e] -> [2I,H/2] packed e2m1 (gate rows then up rows), w1_sf[e] -> [2I,H/32]
 *   w2[e] -> [H,I/2] packed e2m1, w2_sf[e] -> [H,I/32]
 *   acc1 [n*K,2I] f32, acc1_mag [n*K,2I] (mx_mag), hval [n*K,I] f32,
 *   h [n*K,I] e4m3, h_sf [n*K,I/32] UE8M0, partial [n*K,H]
 * ORC_NO_REQUANT feeds the f32 SwiGLU output to L2 unquantised; ORC_NO_BF16
 * keeps partials and y in f32. */
int orc_moe_forward_mx(int T, int H, int I, int E, int K,
                       const uint8_t* x, const uint8_t* x_sf,
                       const int32_t* idx, const float* w,
                       const uint8_t* const* w1, const uint8_t* const* w1_sf,
                       const uint8_t* const* w2, const uint8_t* const* w2_sf,
                       int n_tok, const int32_t* toks,
                       uint16_t* y, float* y_f32,
                       float* acc1, float* acc1_mag, float* hval,
                       uint8_t* h, uint8_t* h_sf, uint16_t* partial,
                       int flags, float clamp, int nthreads)
{
    if (H % 32 || I % 32 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || T < 0)
        return -1;
    if (!toks)
        n_tok = T;
    init_tables();
    const int HS = H / 32, IS = I / 32;
    int bad = check_tokens(T, E, K, idx, n_tok, toks, (const void* const*)w1,
                           (const void* const*)w1_sf, (const void* const*)w2,
                           (const void* const*)w2_sf);
    if (bad < 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
    float* part_f32 = (float*)calloc((size_t)n_tok * K * H, sizeof(float));
    if (!part_f32)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ps = 0; ps < n_tok * K; ++ps) {
        int p = ps / K, j = ps % K;
        int t = toks ? toks[p] : p;
        int e = idx[t * K + j];
        if (e < 0 || e >= E)
            continue;
        float* a1 = (float*)malloc(sizeof(float) * 2 * I);
        float* hv = (float*)malloc(sizeof(float) * I);
        uint8_t* q = (uint8_t*)malloc(I);
        uint8_t* qs = (uint8_t*)malloc(IS);
        const uint8_t* xr = x + (size_t)t * H;
        const uint8_t* xs = x_sf + (size_t)t * HS;
        for (int n = 0; n < 2 * I; ++n) {
            a1[n] = (float)orc_mx_dot(xr, xs, w1[e] + (size_t)n * (H / 2),
                                      w1_sf[e] + (size_t)n * HS, H);
            if (acc1_mag)
                acc1_mag[(size_t)ps * 2 * I + n] =
                    (float)mx_mag(xr, xs, w1[e] + (size_t)n * (H / 2), w1_sf[e] + (size_t)n * HS, H);
        }
        if (acc1)
            memcpy(acc1 + (size_t)ps * 2 * I, a1, sizeof(float) * 2 * I);
        for (int i = 0; i < I; ++i)
            hv[i] = orc_swiglu(clamp_act(a1[i], clamp), clamp_act(a1[I + i], clamp), w[t * K + j]);
        if (hval)
            memcpy(hval + (size_t)ps * I, hv, sizeof(float) * I);
        if (!(flags & ORC_NO_REQUANT)) {
            for (int ib = 0; ib < IS; ++ib)
                orc_requant_block_mx(hv + 32 * ib, 32, q + 32 * ib, qs + ib);
            if (h)
                memcpy(h + (size_t)ps * I, q, I);
            if (h_sf)
                memcpy(h_sf + (size_t)ps * IS, qs, IS);
        }
        l2_slot_mx(H, I, q, qs, hv, w2[e], w2_sf[e], flags, part_f32 + (size_t)ps * H,
                   partial ? partial + (size_t)ps * H : NULL, NULL);
        free(a1);
        free(hv);
        free(q);
        free(qs);
    }
    combine(T, H, E, K, idx, n_tok, toks, part_f32, y, y_f32);
    free(part_f32);
    return bad;
}

/* Steps 5-6 of the MXFP4 recipe from a given intermediate: h [n_tok*K, I]
 * e4m3, h_sf [n_tok*K, I/32] UE8M0 codes; outputs and returns as
 * orc_moe_l2_combine. */
int orc_moe_l2_combine_mx(int T, int H, int I, int E, int K,
                          const int32_t* idx,
                          const uint8_t* const* w2, const uint8_t* const* w2_sf,
                          int n_tok, const int32_t* toks,
                          const uint8_t* h, const uint8_t* h_sf,
                          uint16_t* y, uint16_t* partial, float* o_mag,
                          int flags, int nthreads)
{
    if (H % 32 || I % 32 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || T < 0 ||
        (flags & (ORC_NO_REQUANT | ORC_NO_BF16)))
        return -1;
    if (!toks)
        n_tok = T;
    init_tables();
    const int IS = I / 32;
    int bad = check_tokens(T, E, K, idx, n_tok, toks, (const void* const*)w2,
                           (const void* const*)w2_sf, (const void* const*)w2,
                           (const void* const*)w2_sf);
    if (bad < 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
    float* part_f32 = (float*)calloc((size_t)n_tok * K * H, sizeof(float));
    if (!part_f32)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ps = 0; ps < n_tok * K; ++ps) {
        int p = ps / K, j = ps % K;
        int t = toks ? toks[p] : p;
        int e = idx[t * K + j];
        if (e < 0 || e >= E)
            continue;
        l2_slot_mx(H, I, h + (size_t)ps * I, h_sf + (size_t)ps * IS, NULL, w2[e], w2_sf[e],
                   flags, part_f32 + (size_t)ps * H, partial ? partial + (size_t)ps * H : NULL,
                   o_mag ? o_mag + (size_t)ps * H : NULL);
    }
    combine(T, H, E, K, idx, n_tok, toks, part_f32, y, NULL);
    free(part_f32);
    return bad;
}
