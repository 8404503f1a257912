// Host side of the C ABI declared in include/moe_fp8.h: validation, tile
// configuration, workspace layout and kernel launches.  Every check runs
// before the first HIP call, so invalid calls enqueue nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/moe_fp8.h"
#include "moe_internal.h"

struct moe_plan {
    moe_shape_t shape;
};

namespace {

constexpr size_t kAlign = 256;
constexpr int kVersion = 1;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Config {
    int tile_m;
    int kernel;
};

// Rows per tile from the expected rows per expert T*K/E: the smallest tile
// that holds an average expert's rows reads each expert's weights once
// while padding as few MFMA rows as possible (decode: 16).
// Beyond kRows32 rows per expert the LDS-using MFMA tiles take over: the
// 64-row shared-A tile of gemm_sa.hip up to kRowsLds64 rows per expert and
// the 128 x 256 LDS-staged tile above (they need H % 256 == 0 for their
// 256-column L2 tiles and enough K blocks, lds_tile_fits; otherwise 64-row
// direct-load tiles).  kRows32: at ~24 rows a tenth of the experts already
// overflow 32 rows, and the extra row blocks start a second, mostly idle
// round of 32-row workgroups (measured on the EP8 share, 32 experts: 145 us
// at 21 rows, 183 us at 24, against 152-155 us for the shared-A tile; on the
// flash shape the two cross between 20 and 22.5 rows).
// Columns per intermediate scale of an FP8 plan (MXFP4: 32).
int sf_gran(const moe_shape_t& s)
{
    if (s.recipe == MOE_RECIPE_MXFP4)
        return 32;
    if (s.act_sf_gran < 0)  // PR #440 "How it works": 128 where the decode tile fits, else 64
        return (s.hidden % 512 == 0 && (2 * s.intermediate) % 512 == 0) ? 128 : 64;
    return s.act_sf_gran == 64 ? 64 : 128;
}

// The LDS tile keeps NSTAGE - 1 K blocks in flight and needs that many per
// layer: 2 for the FP8 recipe, 3 for FP8 x MXFP4.
bool lds_tile_fits(const moe_shape_t& s)
{
    const int min_kb = s.recipe == MOE_RECIPE_MXFP4 ? 3 : 2;
    return s.hidden % 256 == 0 && s.hidden / 128 >= min_kb && s.intermediate / 128 >= min_kb;
}

// The 160-row LDS tile (gemm_lds160.hip): FP8 recipe with per-128 scales
// and packed weights, and copy offsets that fit 31 bits (x rows, pool rows of
// h; the kernel addresses them as 32-bit offsets from one base).
bool lds160_fits(const moe_shape_t& s)
{
    if (!lds_tile_fits(s) || s.recipe != MOE_RECIPE_FP8_BLOCK128 || sf_gran(s) != 128 ||
        s.weight_layout != MOE_WEIGHTS_PACKED || (s.flags & MOE_FLAG_RING_POOL))
        return false;
    const long long rows = (long long)s.max_tokens * s.top_k + (long long)s.num_experts * 160;
    return (long long)s.max_tokens * s.hidden < (1LL << 31) && rows * s.intermediate < (1LL << 31);
}

// 160- or 128-row LDS tiles at a mean of m routed rows per expert: the
// expected number of row tiles per expert, E[ceil(n / B)] = sum over k >= 0
// of P(n > k B), with n ~ Normal(m, sqrt(m)) (uniform routing: a Poisson
// count), each 160-row tile priced at 1.1 times a 128-row one (its stage
// copies 52 KiB where the 128-row tile copies 48).  Measured on the pro and
// flash prefill shapes from 72 to 256 rows per expert, this picks the faster
// tile at every point (160 wins from ~120 to ~170 rows and again at 256;
// pro prefill at 128 rows: 6680 against 7920 us per layer).  Skewed routing
// at the same mean (the skewed workload) runs ~3 % slower on 160-row tiles;
// the plan sees only the mean.
double expected_tiles(double m, int B)
{
    const double sd = std::sqrt(std::max(m, 1.0));
    double e = 1.0;
    for (int k = 1; k < 64; ++k) {
        const double p = 0.5 * std::erfc((k * B + 0.5 - m) / (sd * std::sqrt(2.0)));
        e += p;
        if (p < 1e-12)
            break;
    }
    return e;
}
bool prefers160(double m) { return 1.1 * expected_tiles(m, 160) < expected_tiles(m, 128); }

constexpr double kRows16 = 10.0;     // FP8: 16-row tiles up to here (12 rows: 32-row 6 % faster)
constexpr double kRows16Mx = 12.0;   // MXFP4: 16-row tiles up to here, then shared-A
constexpr double kRows32 = 21.0;
constexpr double kRowsLds64 = 64.0;
// MXFP4: the 128-row LDS tile leads only between kRowsLds64 and this many
// rows per expert; beyond it the shared-A tile is 4-20 % faster (flash shape
// at 96 / 120 / 192 rows: 1222 vs 1317, 1516 vs 1463, 2462 vs 2103 us;
// pro shape at 96 / 128 / 256 rows: 4165 vs 4441, 6034 vs 5330, 10002 vs
// 8936 us; FP8 keeps the LDS tile: pro 8342 vs 10619 us).
constexpr double kRowsLds128Mx = 108.0;

Config choose_config(const moe_shape_t& s, int T)
{
    // ring-pool plans run the single launch, which has direct-load tiles only
    const bool ring = (s.flags & MOE_FLAG_RING_POOL) != 0;
    const bool lds = lds_tile_fits(s) && !ring;
    const bool lds64 = lds && !(s.flags & MOE_FLAG_DIRECT_TILES);
    // 64-row tiles where the LDS tiles fit: the shared-A tile (kernel 2)
    const int k64 = lds64 ? 2 : 0;
    if (s.tile_m > 0)
        return Config{s.tile_m, s.tile_m == 160 ? 3 : s.tile_m == 128 ? 1 : s.tile_m == 64 ? k64 : 0};
    const double rows = (double)T * s.top_k / s.num_experts;
    const bool mx = s.recipe == MOE_RECIPE_MXFP4;
    if (rows <= (mx ? kRows16Mx : kRows16))
        return Config{16, 0};
    // MXFP4: the shared-A tile beats the 32-row tile from 12 rows on
    // (flash shape at 15 rows per expert: 693 vs 706 us; EP8 share: 104 vs 108)
    if (rows <= kRows32 && !(mx && lds64))
        return Config{32, 0};
    if (!lds)
        return Config{64, 0};
    if (rows <= kRowsLds64 || (mx && lds64 && rows > kRowsLds128Mx))
        return Config{64, k64};
    if (lds160_fits(s) && prefers160(rows))
        return Config{160, 3};
    return Config{128, 1};
}

struct Layout {
    int tile_m, kernel, r_cap, mb_cap, NB;
    int split_l1, split_l2;
    bool l2_wide;
    bool single;  // L1 + L2 + combine in one launch
    int ring_blocks, lag_units;  // ring pool: row blocks of h / h_sf, lag (0: full pool)
    int n_sync;
    size_t sync;
    size_t status, counts, offsets, blk, mbe, row_src, src_row, h_sf, h, partial;
    size_t part, unit_mb, stream_start, stream_desc, item_tab, total;
};

// Ring pool sizing (DeepGEMM PR #440 "How it works", "Ring sizing,
// recycling, and why that granularity"): a unit is up to kUnitBlocks row
// blocks of one expert; the call's unit count is estimated from its token
// count (T*K rows in blocks of tile_m), L2 trails L1 by lag = clamp(round(0.45
// units), 8, 64) units in groups of kStreamGroup, so at most kUnitBlocks
// (lag + group) blocks are live and the ring holds that plus kRingMargin.
constexpr int kRingMargin = 4;

struct RingSize {
    int blocks, lag;
};

RingSize ring_size(long long TK, int tile_m)
{
    const long long per_unit = (long long)moe::kUnitBlocks * tile_m;
    const long long units = std::max<long long>(1, (TK + per_unit - 1) / per_unit);
    const int lag = (int)std::min<long long>(64, std::max<long long>(8, std::llround(0.45 * units)));
    return RingSize{moe::kUnitBlocks * (lag + moe::kStreamGroup) + kRingMargin, lag};
}

// The live set of the lag order: blocks whose h a ring slot must still hold.
bool ring_holds_live_set(int blocks, int lag)
{
    return blocks >= moe::kUnitBlocks * (lag + moe::kStreamGroup) + 1;
}

// Split-K across workgroups for the 16-row L1 tiles.  One workgroup per
// (row block, column tile) streams that tile's whole weight block (~1 MiB at
// H = 4096), which sustains the HBM stream best (measured at 1 to 256 tokens
// of the flash-decode shape) as long as there are at least as many tiles as
// compute units.  With fewer (a single token: 6 row blocks x 16 tiles) each
// tile's K range is split over S workgroups, S the smallest power of two
// (<= 4, <= the K blocks) that reaches kMinItems.  The 16-row L2 tiles
// split by the same rule; in both steps the slice counted last adds the
// slices (adding them in the combine instead cost as much as the split
// saved, measured).
constexpr long long kMinItems = 256;  // MI355X compute units

// Whether direct-tile calls run L1, L2 and the combine as one launch when
// the plan sets neither MOE_FLAG_SINGLE_LAUNCH nor MOE_FLAG_SPLIT_LAUNCH: no
// (the single launch measured 12-18 % slower than the split launches at
// decode shapes), so it is opt-in.
constexpr bool kSingleLaunchDefault = false;

// Polls of a single-launch wait before it gives up (~1 s at 8 s_sleep units
// per poll); a legitimate wait is at most one L1 phase.
constexpr int kSpinLimit = 1 << 22;

long long mblocks_expected(const moe_shape_t& s, long long T)
{
    const long long tk = T * s.top_k;
    return std::max<long long>((tk + 15) / 16, std::min<long long>(tk, s.num_experts));
}

// 16-row L2 tiles: one 8-wave workgroup per two 256-column tiles (1 MiB of
// weights at the flash shape, like an L1 tile) streams better than one
// 4-wave workgroup per tile when there are enough of them; with few routed
// rows it halves an already small workgroup count (measured at the flash
// shape: T = 128 and 32 gain ~1.7 % in L2, T = 8 loses 7 %).
bool choose_l2_wide(const moe_shape_t& s, int T, const Config& c)
{
    if (c.tile_m != 16 || T <= 0 || s.recipe != MOE_RECIPE_FP8_BLOCK128 || sf_gran(s) == 64)
        return false;
    const long long groups = mblocks_expected(s, T) * (((s.hidden + 255) / 256 + 1) / 2);
    return groups >= 4 * kMinItems;
}

// K split factor of the L1 (l2 = false) or L2 step of a call with T tokens
// and tile configuration c.
int choose_split(const moe_shape_t& s, int T, const Config& c, bool l2 = false)
{
    if (c.tile_m != 16 || T <= 0 || s.recipe != MOE_RECIPE_FP8_BLOCK128 ||
        (s.flags & MOE_FLAG_RING_POOL))
        return 1;
    const long long tiles = l2 ? (s.hidden + 255) / 256 : s.intermediate / 128;
    const long long items = mblocks_expected(s, T) * tiles;
    const int kblocks = (l2 ? s.intermediate : s.hidden) / 128;
    // L2 splits only below half a grid's worth of tiles: at the flash shape
    // one token (96 tiles) gains 2.7 us, two tokens (192 tiles, split 2)
    // lose 0.7 us (measured)
    if (l2 && 2 * items >= kMinItems)
        return 1;
    int S = 1;
    while (S < 4 && 2 * S <= kblocks && items * S < kMinItems)
        S *= 2;
    return S;
}

// Pool capacity (rows) for T tokens with row alignment ra.
long long pool_rows(const moe_shape_t& s, long long T, int ra)
{
    long long r = T * s.top_k + (long long)s.num_experts * (ra - 1);
    r = (r + ra - 1) / ra * ra;
    return std::max<long long>(r, ra);
}

// Floats of split-K scratch a call with T tokens needs, maximised over all
// token counts <= T so the workspace size never shrinks as T grows (a
// workspace sized for max_tokens serves every smaller call).  S(t) is a
// nonincreasing step function of t with values 4, 2, 1, so the maximum of
// S(t) * t sits at T or at the last t of one of the steps, found by
// bisection.
size_t splitk_floats(const moe_shape_t& s, int T)
{
    // L1 slices hold 2I floats per slot, L2 slices H; the two steps use the
    // buffer one after the other
    size_t best = 0;
    for (int l2 = 0; l2 < 2; ++l2) {
        const size_t width = (l2 ? (size_t)s.hidden : 2 * (size_t)s.intermediate) *
                             (size_t)s.top_k;
        auto S = [&](int t) { return choose_split(s, t, choose_config(s, t), l2 != 0); };
        auto need = [&](int t) -> size_t {
            const int v = S(t);
            return v > 1 ? (size_t)v * (size_t)t * width : 0;
        };
        best = std::max(best, need(T));
        for (int v = 2; v <= 4; v *= 2) {
            // last t in [1, T] with S(t) >= v (S is nonincreasing in t while
            // the tiles are 16 rows; once they are not, S is 1)
            if (T < 1 || S(1) < v)
                continue;
            int lo = 1, hi = T;
            while (lo < hi) {
                const int mid = lo + (hi - lo + 1) / 2;
                if (S(mid) >= v)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            best = std::max(best, need(lo));
        }
    }
    return best;
}

// Largest tile height the choice takes at any token count <= T.  The
// MXFP4 choice is not monotone in T (the 128-row tile between 64 and 108
// rows per expert, the 64-row tile beyond), and a workspace sized for T must
// serve every smaller call, so the pool sections are sized for this height.
int max_tile_upto(const moe_shape_t& s, int T)
{
    int m = choose_config(s, T).tile_m;
    // 160-row tiles: taken at some token count <= T once the mean reaches the
    // first mean the rule above prefers them at (scanned in quarter rows)
    if (lds160_fits(s) && s.tile_m == 0) {
        const double rows = (double)T * s.top_k / s.num_experts;
        for (double x = kRowsLds64; x <= rows; x += 0.25)
            if (prefers160(x)) {
                m = std::max(m, 160);
                break;
            }
    }
    for (double x : {kRows16, kRows16Mx, kRows32, kRowsLds64, kRowsLds128Mx}) {
        // last token count with at most x rows per expert, and the next
        const long long t = (long long)std::floor(x * s.num_experts / s.top_k);
        for (long long u = t; u <= t + 1; ++u)
            if (u >= 1 && u <= T)
                m = std::max(m, choose_config(s, (int)u).tile_m);
    }
    return m;
}

Layout make_layout(const moe_shape_t& s, int T, int row_align_override = 0)
{
    Layout L{};
    const Config c = choose_config(s, T);
    L.tile_m = c.tile_m;
    L.kernel = c.kernel;
    const int ra = row_align_override > 0 ? row_align_override : c.tile_m;
    const long long TK = (long long)T * s.top_k;
    L.r_cap = (int)pool_rows(s, T, ra);
    L.mb_cap = L.r_cap / ra;
    // the pool sections' size (>= r_cap: see max_tile_upto)
    const size_t r_alloc = row_align_override > 0
                               ? (size_t)L.r_cap
                               : (size_t)std::max<long long>(L.r_cap,
                                                             pool_rows(s, T, max_tile_upto(s, T)));
    L.NB = (int)std::max<long long>((TK + moe::kRouteThreads - 1) / moe::kRouteThreads, 1);
    const int E = s.num_experts, H = s.hidden, I = s.intermediate, K = s.top_k;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes, kAlign);
        return at;
    };
    L.status = take(4 * sizeof(int32_t));
    L.counts = take(sizeof(int32_t) * E);
    L.offsets = take(sizeof(int32_t) * (E + 1));
    L.blk = take(sizeof(int32_t) * (size_t)L.NB * (E + 1));
    L.mbe = take(sizeof(int32_t) * (size_t)L.mb_cap);
    L.row_src = take(sizeof(int32_t) * r_alloc);
    L.src_row = take(sizeof(int32_t) * (size_t)std::max<long long>(TK, 1));
    L.split_l1 = choose_split(s, T, c);
    L.split_l2 = choose_split(s, T, c, true);
    L.single = c.kernel == 0 && L.split_l1 == 1 && L.split_l2 == 1 && sf_gran(s) != 64 &&
               ((s.flags & (MOE_FLAG_SINGLE_LAUNCH | MOE_FLAG_RING_POOL)) ||
                (kSingleLaunchDefault && !(s.flags & MOE_FLAG_SPLIT_LAUNCH)));
    // the single launch's and the split L2's tiles are one 256-column tile
    // per workgroup
    L.l2_wide = choose_l2_wide(s, T, c) && !L.single && L.split_l2 == 1;
    // Ring pool: where the call's pool holds more row blocks than the ring,
    // h / h_sf hold ring_blocks blocks (block mb at slot mb % ring_blocks);
    // elsewhere the ring would be the whole pool and never wrap.
    const bool ring_plan = L.single && (s.flags & MOE_FLAG_RING_POOL);
    L.ring_blocks = L.lag_units = 0;
    if (ring_plan) {
        const RingSize rs = ring_size(TK, ra);
        if (rs.blocks < L.mb_cap) {
            L.ring_blocks = rs.blocks;
            L.lag_units = rs.lag;
        }
    }
    const size_t h_rows = L.ring_blocks > 0 ? (size_t)L.ring_blocks * ra : r_alloc;
    // f32 [R, I/128] or [R, I/64] (FP8 recipe) or UE8M0 bytes [R, I/32]
    // (MXFP4, the size of the per-128 f32 section)
    L.h_sf = take(sizeof(float) * h_rows * (I / (sf_gran(s) == 64 ? 64 : 128)));
    L.h = take(h_rows * I);
    L.partial = take(sizeof(uint16_t) * (size_t)K * T * H);
    // Split-K scratch: L1's f32 partials part[slice][slot][2I], slot
    // f = t*K + j.
    L.part = take(sizeof(float) * splitk_floats(s, T));
    // Single-launch counters: L2 done, queue, 2 for the ring's stream, one
    // L1-ready count per row block, and (ring plans) one L2-done count per
    // row block.  Ring plans size the per-block sections for mbb >= mb_cap
    // blocks, a bound that grows with T whatever the tile height.
    const size_t mbb = (size_t)((TK + 15) / 16 + E);
    L.n_sync = moe::kSyncReady + (ring_plan ? (int)(2 * mbb) : L.mb_cap);
    // split-K: one slice count per tile of the launch grid's row blocks, L1
    // tiles then L2 tiles
    if (L.split_l1 > 1 || L.split_l2 > 1)
        L.n_sync = std::max<int>(L.n_sync, moe::kSyncReady + (int)std::min<long long>(L.mb_cap, std::max<long long>(TK, 1)) * (I / 128 + (H + 255) / 256));
    L.sync = take(sizeof(int32_t) * (size_t)L.n_sync);
    L.unit_mb = L.stream_start = L.stream_desc = L.item_tab = 0;
    if (ring_plan) {
        const size_t NT1 = I / 128, NT2 = (H + 255) / 256;
        L.unit_mb = take(sizeof(int32_t) * (mbb + 1));
        L.stream_start = take(sizeof(int32_t) * (2 * mbb + 1));
        L.stream_desc = take(sizeof(int32_t) * 2 * mbb);
        L.item_tab = take(sizeof(int32_t) * mbb * (NT1 + NT2));
    }
    L.total = o;
    return L;
}

int validate_shape(const moe_shape_t* s)
{
    if (!s)
        return MOE_ERR_INVALID_ARG;
    if (s->hidden <= 0 || s->intermediate <= 0 || s->num_experts <= 0 || s->top_k <= 0 ||
        s->max_tokens < 0)
        return MOE_ERR_INVALID_ARG;
    if (s->top_k > s->num_experts)
        return MOE_ERR_INVALID_ARG;
    if (s->hidden % 128 || s->intermediate % 128)
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if (s->num_experts > moe::kMaxExperts)
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if ((long long)s->max_tokens * s->top_k >= (1LL << 24))
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if (s->hidden > (1 << 16) || s->intermediate > (1 << 16))
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if (s->tile_m != 0 && s->tile_m != 16 && s->tile_m != 32 && s->tile_m != 64 &&
        s->tile_m != 128 && s->tile_m != 160)
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if (s->tile_m == 160 && !lds160_fits(*s))
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if (s->recipe != MOE_RECIPE_FP8_BLOCK128 && s->recipe != MOE_RECIPE_MXFP4)
        return MOE_ERR_INVALID_ARG;
    if (s->tile_m == 128 && !lds_tile_fits(*s))
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if (s->weight_layout != MOE_WEIGHTS_ROW_MAJOR && s->weight_layout != MOE_WEIGHTS_PACKED)
        return MOE_ERR_INVALID_ARG;
    if (s->weight_layout == MOE_WEIGHTS_PACKED && s->hidden % 256)
        return MOE_ERR_UNSUPPORTED_SHAPE;
    if (s->flags & ~(MOE_FLAG_SINGLE_LAUNCH | MOE_FLAG_SPLIT_LAUNCH | MOE_FLAG_POW2_SCALE |
                     MOE_FLAG_DIRECT_TILES | MOE_FLAG_RING_POOL | MOE_FLAG_TEST_NO_WAIT |
                     MOE_FLAG_TEST_SMALL_GRID))
        return MOE_ERR_INVALID_ARG;
    if (s->act_sf_gran != 0 && s->act_sf_gran != 64 && s->act_sf_gran != 128 && s->act_sf_gran != -1)
        return MOE_ERR_INVALID_ARG;
    if (!(s->activation_clamp == s->activation_clamp))  // NaN
        return MOE_ERR_INVALID_ARG;
    if (sf_gran(*s) == 64) {  // per-64 plans: split launches
        if (s->flags & MOE_FLAG_SINGLE_LAUNCH)
            return MOE_ERR_INVALID_ARG;
    }
    if (s->recipe == MOE_RECIPE_MXFP4) {
        if (s->act_sf_gran != 0 || (s->flags & MOE_FLAG_POW2_SCALE))
            return MOE_ERR_INVALID_ARG;
        // the MXFP4 kernels address x with 32-bit buffer offsets
        if ((long long)s->max_tokens * s->hidden > 0x7FFFFFFFLL)
            return MOE_ERR_UNSUPPORTED_SHAPE;
        if (s->flags & MOE_FLAG_SINGLE_LAUNCH)
            return MOE_ERR_INVALID_ARG;
    }
    if ((s->flags & MOE_FLAG_SINGLE_LAUNCH) && (s->flags & MOE_FLAG_SPLIT_LAUNCH))
        return MOE_ERR_INVALID_ARG;
    if (s->flags & MOE_FLAG_RING_POOL) {  // the single launch with direct-load tiles
        if (s->flags & MOE_FLAG_SPLIT_LAUNCH)
            return MOE_ERR_INVALID_ARG;
        if (s->recipe != MOE_RECIPE_FP8_BLOCK128 || sf_gran(*s) == 64)
            return MOE_ERR_INVALID_ARG;
        if (s->tile_m == 128)
            return MOE_ERR_UNSUPPORTED_SHAPE;
    }
    return MOE_OK;
}

template <typename T>
T* at(void* base, size_t off)
{
    return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOE_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return MOE_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return MOE_ERR_NOT_GFX950;
    return MOE_OK;
}

// Checked once per process per device ordinal.
int device_ok()
{
    static int cached[64];
    static bool init[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOE_ERR_HIP;
    if (dev < 0 || dev >= 64)
        return check_device();
    if (!init[dev]) {
        cached[dev] = check_device();
        init[dev] = true;
    }
    return cached[dev];
}

// Scratch of moe_forward_noalloc: every section a forward keeps in its
// workspace (plan, pool maps, h, h_sf, partials, counters), in a static
// device array of fixed size instead of a caller's allocation.  Each GPU the
// library runs on holds its own copy until the process ends.  Host code uses
// the array only through the device address hipGetSymbolAddress returns
// (the array's name is a host-side stand-in, not a device address); that
// address is looked up once per device, with the device current, and kept.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

int noalloc_scratch(void** out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOE_ERR_HIP;
        addr[dev] = p;
    }
    *out = addr[dev];
    return MOE_OK;
}

moe::RouteArgs route_args(const moe_shape_t& s, int T, const Layout& L, void* ws,
                          const int32_t* idx, int row_align, int32_t* counts,
                          int32_t* offsets, int32_t* row_src, int r_cap, int32_t* src_row,
                          bool with_mblocks)
{
    moe::RouteArgs a{};
    a.idx = idx;
    a.TK = T * s.top_k;
    a.E = s.num_experts;
    a.row_align = row_align;
    a.NB = L.NB;
    a.blk = at<int32_t>(ws, L.blk);
    a.counts = counts;
    a.offsets = offsets;
    a.row_src = row_src;
    a.r_cap = r_cap;
    a.src_row = src_row;
    a.mblock_expert = with_mblocks ? at<int32_t>(ws, L.mbe) : nullptr;
    a.mb_cap = L.mb_cap;
    a.status = at<int32_t>(ws, L.status);
    a.sync = with_mblocks ? at<int32_t>(ws, L.sync) : nullptr;
    a.n_sync = with_mblocks ? L.n_sync : 0;
    return a;
}

}  // namespace

extern "C" {

int moe_version(void) { return kVersion; }

const char* moe_strerror(int code)
{
    switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_NOT_GFX950: return "current device is not gfx950";
    default: return "unknown error";
    }
}

int moe_plan_create(const moe_shape_t* shape, moe_plan_t* out)
{
    if (!out)
        return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    const int rc = validate_shape(shape);
    if (rc != MOE_OK)
        return rc;
    moe_plan* p = new (std::nothrow) moe_plan;
    if (!p)
        return MOE_ERR_INVALID_ARG;
    p->shape = *shape;
    *out = p;
    return MOE_OK;
}

int moe_plan_destroy(moe_plan_t plan)
{
    delete plan;
    return MOE_OK;
}

int moe_plan_info(moe_plan_t plan, int32_t T, moe_tile_info_t* info)
{
    if (!plan || !info || T < 0 || T > plan->shape.max_tokens)
        return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(plan->shape, T);
    info->tile_m = L.tile_m;
    info->row_align = L.tile_m;
    info->pool_rows = L.r_cap;
    info->l1_tile_n = 256;  // 128 gate + 128 up columns
    info->l2_tile_n = 256;
    info->kernel = L.kernel;
    info->l1_split = L.split_l1;
    info->l2_split = L.split_l2;
    info->single_launch = L.single ? 1 : 0;
    info->l2_group_tiles = L.l2_wide ? 2 : 1;
    info->act_sf_gran = sf_gran(plan->shape);
    info->ring_blocks = L.ring_blocks;
    info->l2_lag_units = L.lag_units;
    return MOE_OK;
}

int moe_workspace_bytes(moe_plan_t plan, int32_t T, size_t* bytes)
{
    if (!plan || !bytes || T < 0 || T > plan->shape.max_tokens)
        return MOE_ERR_INVALID_ARG;
    *bytes = make_layout(plan->shape, T).total;
    return MOE_OK;
}

int moe_workspace_layout(moe_plan_t plan, int32_t T, moe_ws_layout_t* out)
{
    if (!plan || !out || T < 0 || T > plan->shape.max_tokens)
        return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(plan->shape, T);
    out->counts = L.counts;
    out->offsets = L.offsets;
    out->row_src = L.row_src;
    out->src_row = L.src_row;
    out->h = L.h;
    out->h_sf = L.h_sf;
    out->partial = L.partial;
    out->status = L.status;
    out->total = L.total;
    return MOE_OK;
}

}  // extern "C"

namespace {

// Operands of one forward; the scale pointers are f32 (FP8 recipe) or
// UE8M0 bytes (MXFP4), as the plan's recipe says.
struct FwdOperands {
    const uint8_t* x;
    const void* x_sf;
    const int32_t* topk_idx;
    const float* topk_w;
    const uint8_t* w1;
    const void* w1_sf;
    const uint8_t* w2;
    const void* w2_sf;
    uint16_t* y;
};

bool misaligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) != 0; }

// Host-side checks of a forward's operands (no HIP call).
int check_operands(const FwdOperands& op)
{
    if (!op.x || !op.x_sf || !op.topk_idx || !op.topk_w || !op.w1 || !op.w1_sf || !op.w2 ||
        !op.w2_sf || !op.y)
        return MOE_ERR_INVALID_ARG;
    // The kernels move 16-byte vectors of x, the weights and y.
    if (misaligned(op.x, 16) || misaligned(op.w1, 16) || misaligned(op.w2, 16) ||
        misaligned(op.y, 16))
        return MOE_ERR_INVALID_ARG;
    // MXFP4 scale codes are copied 4 bytes at a time by the LDS tiles (f32
    // scales are naturally aligned)
    if (misaligned(op.x_sf, 4) || misaligned(op.w1_sf, 4) || misaligned(op.w2_sf, 4))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int forward_impl(moe_plan_t plan, int recipe, int32_t T, const FwdOperands& op, void* workspace,
                 size_t workspace_bytes, void* stream, void* const* step_events)
{
    if (!plan)
        return MOE_ERR_INVALID_ARG;
    const moe_shape_t& s = plan->shape;
    if (s.recipe != recipe)
        return MOE_ERR_INVALID_ARG;
    if (T < 0 || T > s.max_tokens)
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (check_operands(op) != MOE_OK || !workspace)
        return MOE_ERR_INVALID_ARG;
    // the workspace sections sit at 256-byte offsets and move as 16-byte vectors
    if (misaligned(workspace, 256))
        return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(s, T);
    if (workspace_bytes < L.total)
        return MOE_ERR_WORKSPACE_TOO_SMALL;
    // the ring must hold the lag order's live set (asserted before any launch)
    if (L.ring_blocks > 0 && !ring_holds_live_set(L.ring_blocks, L.lag_units))
        return MOE_ERR_UNSUPPORTED_SHAPE;
    int rc = device_ok();
    if (rc != MOE_OK)
        return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
        if (step_events && step_events[i])
            return hipEventRecord(static_cast<hipEvent_t>(step_events[i]), st) == hipSuccess;
        return true;
    };
    if (!mark(0))
        return MOE_ERR_HIP;

    moe::RouteArgs ra = route_args(s, T, L, workspace, op.topk_idx, L.tile_m,
                                   at<int32_t>(workspace, L.counts),
                                   at<int32_t>(workspace, L.offsets),
                                   at<int32_t>(workspace, L.row_src), L.r_cap,
                                   at<int32_t>(workspace, L.src_row), true);
    if (moe::launch_route(ra, st) != hipSuccess || !mark(1))
        return MOE_ERR_HIP;

    const bool mx = recipe == MOE_RECIPE_MXFP4;
    moe::FwdArgs a{};
    a.T = T;
    a.H = s.hidden;
    a.I = s.intermediate;
    a.E = s.num_experts;
    a.K = s.top_k;
    a.BM = L.tile_m;
    a.packed = s.weight_layout == MOE_WEIGHTS_PACKED;
    a.x = op.x;
    a.idx = op.topk_idx;
    a.topk_w = op.topk_w;
    a.w1 = op.w1;
    a.w2 = op.w2;
    a.mx = mx ? 1 : 0;
    if (mx) {
        a.x_sfq = static_cast<const uint8_t*>(op.x_sf);
        a.w1_sfq = static_cast<const uint8_t*>(op.w1_sf);
        a.w2_sfq = static_cast<const uint8_t*>(op.w2_sf);
        a.h_sfq = at<uint8_t>(workspace, L.h_sf);
    } else {
        a.x_sf = static_cast<const float*>(op.x_sf);
        a.w1_sf = static_cast<const float*>(op.w1_sf);
        a.w2_sf = static_cast<const float*>(op.w2_sf);
        a.h_sf = at<float>(workspace, L.h_sf);
    }
    a.row_src = at<int32_t>(workspace, L.row_src);
    a.offsets = at<int32_t>(workspace, L.offsets);
    a.mblock_expert = at<int32_t>(workspace, L.mbe);
    a.num_mblocks = L.mb_cap;
    a.grid_mblocks = (int)std::min<long long>(L.mb_cap, std::max<long long>(1, (long long)T * s.top_k));
    a.h = at<uint8_t>(workspace, L.h);
    a.partial = at<uint16_t>(workspace, L.partial);
    a.y = op.y;
    a.src_row = at<int32_t>(workspace, L.src_row);
    a.split_l1 = L.split_l1;
    a.split_l2 = L.split_l2;
    a.l2_wide = L.l2_wide ? 1 : 0;
    a.splitk_slots = T * s.top_k;
    a.splitk_part = at<float>(workspace, L.part);
    a.sync = at<int32_t>(workspace, L.sync);
    a.status = at<int32_t>(workspace, L.status);
    a.spin_limit = (s.flags & MOE_FLAG_TEST_NO_WAIT) ? -1 : kSpinLimit;
    a.clamp = s.activation_clamp > 0.f ? s.activation_clamp : 0.f;
    a.pow2_scale = (s.flags & MOE_FLAG_POW2_SCALE) ? 1 : 0;
    a.sf_gran64 = sf_gran(s) == 64 ? 1 : 0;
    a.grid_cap = (s.flags & MOE_FLAG_TEST_SMALL_GRID) ? 4 : 0;
    if (L.ring_blocks > 0) {
        a.ring_blocks = L.ring_blocks;
        a.lag_units = L.lag_units;
        a.unit_mb = at<int32_t>(workspace, L.unit_mb);
        a.stream_start = at<int32_t>(workspace, L.stream_start);
        a.stream_desc = at<int32_t>(workspace, L.stream_desc);
        a.item_tab = at<int32_t>(workspace, L.item_tab);
        if (moe::launch_route_stream(a, st) != hipSuccess)
            return MOE_ERR_HIP;
    }
    if (L.single) {
        if (moe::launch_fused(a, st) != hipSuccess || !mark(2) || !mark(3) || !mark(4))
            return MOE_ERR_HIP;
        return MOE_OK;
    }
    if (mx && L.kernel == 0) {
        if (moe::launch_l1_mx(a, st) != hipSuccess || !mark(2))
            return MOE_ERR_HIP;
        if (moe::launch_l2_mx(a, st) != hipSuccess || !mark(3))
            return MOE_ERR_HIP;
    } else {  // the LDS tiles serve both recipes
        if (moe::launch_l1(a, L.kernel, st) != hipSuccess || !mark(2))
            return MOE_ERR_HIP;
        if (moe::launch_l2(a, L.kernel, st) != hipSuccess || !mark(3))
            return MOE_ERR_HIP;
    }
    if (moe::launch_combine(a, st) != hipSuccess || !mark(4))
        return MOE_ERR_HIP;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_timed(moe_plan_t plan, int32_t T, const uint8_t* x, const float* x_sf,
                      const int32_t* topk_idx, const float* topk_w, const uint8_t* w1,
                      const float* w1_sf, const uint8_t* w2, const float* w2_sf, uint16_t* y,
                      void* workspace, size_t workspace_bytes, void* stream,
                      void* const* step_events)
{
    const FwdOperands op{x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y};
    return forward_impl(plan, MOE_RECIPE_FP8_BLOCK128, T, op, workspace, workspace_bytes, stream,
                        step_events);
}

int moe_forward(moe_plan_t plan, int32_t T, const uint8_t* x, const float* x_sf,
                const int32_t* topk_idx, const float* topk_w, const uint8_t* w1,
                const float* w1_sf, const uint8_t* w2, const float* w2_sf, uint16_t* y,
                void* workspace, size_t workspace_bytes, void* stream)
{
    return moe_forward_timed(plan, T, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y,
                             workspace, workspace_bytes, stream, nullptr);
}

int moe_forward_noalloc(moe_plan_t plan, int32_t T, const uint8_t* x, const float* x_sf,
                        const int32_t* topk_idx, const float* topk_w, const uint8_t* w1,
                        const float* w1_sf, const uint8_t* w2, const float* w2_sf, uint16_t* y,
                        void* stream)
{
    // every check before the first HIP call
    if (!plan)
        return MOE_ERR_INVALID_ARG;
    const moe_shape_t& s = plan->shape;
    if (s.recipe != MOE_RECIPE_FP8_BLOCK128 || T < 0 || T > s.max_tokens)
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    const FwdOperands op{x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y};
    if (check_operands(op) != MOE_OK)
        return MOE_ERR_INVALID_ARG;
    if (make_layout(s, T).total > kNoAllocScratchBytes)
        return MOE_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    const int rc = noalloc_scratch(&ws);
    if (rc != MOE_OK)
        return rc;
    return forward_impl(plan, MOE_RECIPE_FP8_BLOCK128, T, op, ws, kNoAllocScratchBytes, stream,
                        nullptr);
}

int moe_forward_mx_timed(moe_plan_t plan, int32_t T, const uint8_t* x, const uint8_t* x_sf,
                         const int32_t* topk_idx, const float* topk_w, const uint8_t* w1,
                         const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf,
                         uint16_t* y, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* step_events)
{
    const FwdOperands op{x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y};
    return forward_impl(plan, MOE_RECIPE_MXFP4, T, op, workspace, workspace_bytes, stream,
                        step_events);
}

int moe_forward_mx(moe_plan_t plan, int32_t T, const uint8_t* x, const uint8_t* x_sf,
                   const int32_t* topk_idx, const float* topk_w, const uint8_t* w1,
                   const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf, uint16_t* y,
                   void* workspace, size_t workspace_bytes, void* stream)
{
    return moe_forward_mx_timed(plan, T, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y,
                                workspace, workspace_bytes, stream, nullptr);
}

int moe_prepare_weights(moe_plan_t plan, const uint8_t* w1, const uint8_t* w2,
                        uint8_t* w1_packed, uint8_t* w2_packed, void* stream)
{
    if (!plan || !w1 || !w2 || !w1_packed || !w2_packed)
        return MOE_ERR_INVALID_ARG;
    const moe_shape_t& s = plan->shape;
    if (s.weight_layout != MOE_WEIGHTS_PACKED || s.recipe != MOE_RECIPE_FP8_BLOCK128)
        return MOE_ERR_INVALID_ARG;
    const size_t b1 = (size_t)s.num_experts * 2 * s.intermediate * s.hidden;
    const size_t b2 = (size_t)s.num_experts * s.hidden * s.intermediate;
    auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
        const char* pa = static_cast<const char*>(a);
        const char* pb = static_cast<const char*>(b);
        return pa < pb + nb && pb < pa + na;
    };
    if (overlap(w1, b1, w1_packed, b1) || overlap(w1, b1, w2_packed, b2) ||
        overlap(w2, b2, w1_packed, b1) || overlap(w2, b2, w2_packed, b2) ||
        overlap(w1_packed, b1, w2_packed, b2))
        return MOE_ERR_INVALID_ARG;
    int rc = device_ok();
    if (rc != MOE_OK)
        return rc;
    if (moe::launch_pack(w1, w2, w1_packed, w2_packed, s.num_experts, s.hidden, s.intermediate,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_prepare_weights_mx(moe_plan_t plan, const uint8_t* w1, const uint8_t* w1_sf,
                           const uint8_t* w2, const uint8_t* w2_sf, uint8_t* w1_packed,
                           uint8_t* w1_sf_packed, uint8_t* w2_packed, uint8_t* w2_sf_packed,
                           void* stream)
{
    if (!plan || !w1 || !w1_sf || !w2 || !w2_sf || !w1_packed || !w1_sf_packed || !w2_packed ||
        !w2_sf_packed)
        return MOE_ERR_INVALID_ARG;
    const moe_shape_t& s = plan->shape;
    if (s.weight_layout != MOE_WEIGHTS_PACKED || s.recipe != MOE_RECIPE_MXFP4)
        return MOE_ERR_INVALID_ARG;
    const size_t E = s.num_experts, H = s.hidden, I = s.intermediate;
    const void* in[4] = {w1, w1_sf, w2, w2_sf};
    const void* out[4] = {w1_packed, w1_sf_packed, w2_packed, w2_sf_packed};
    const size_t nb[4] = {E * 2 * I * H / 2, E * 2 * I * H / 32, E * H * I / 2, E * H * I / 32};
    auto overlap = [](const void* a, size_t na, const void* b, size_t nb2) {
        const char* pa = static_cast<const char*>(a);
        const char* pb = static_cast<const char*>(b);
        return pa < pb + nb2 && pb < pa + na;
    };
    // the weights move 16 bytes at a time; the scales byte by byte
    for (int i = 0; i < 4; i += 2)
        if (reinterpret_cast<uintptr_t>(in[i]) % 16 || reinterpret_cast<uintptr_t>(out[i]) % 16)
            return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j)
            if (overlap(out[i], nb[i], in[j], nb[j]) || (j != i && overlap(out[i], nb[i], out[j], nb[j])))
                return MOE_ERR_INVALID_ARG;
    int rc = device_ok();
    if (rc != MOE_OK)
        return rc;
    if (moe::launch_pack_mx(w1, w1_sf, w2, w2_sf, w1_packed, w1_sf_packed, w2_packed, w2_sf_packed,
                            s.num_experts, s.hidden, s.intermediate,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_quantize_act(moe_plan_t plan, int32_t T, const uint16_t* x_bf16, uint8_t* x, void* x_sf,
                     void* stream)
{
    if (!plan)
        return MOE_ERR_INVALID_ARG;
    const moe_shape_t& s = plan->shape;
    if (T < 0 || T > s.max_tokens)
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (!x_bf16 || !x || !x_sf || reinterpret_cast<uintptr_t>(x_bf16) % 16 ||
        reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(x_sf) % 4)
        return MOE_ERR_INVALID_ARG;
    int rc = device_ok();
    if (rc != MOE_OK)
        return rc;
    if (moe::launch_quantize_act(x_bf16, T, s.hidden, x, x_sf, s.recipe == MOE_RECIPE_MXFP4,
                                 static_cast<hipStream_t>(stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_route_workspace_bytes(moe_plan_t plan, int32_t T, size_t* bytes)
{
    if (!plan || !bytes || T < 0 || T > plan->shape.max_tokens)
        return MOE_ERR_INVALID_ARG;
    // The planner alone uses the status word and the per-chunk table only.
    const Layout L = make_layout(plan->shape, T);
    *bytes = L.blk + align_up(sizeof(int32_t) * (size_t)L.NB * (plan->shape.num_experts + 1), kAlign);
    return MOE_OK;
}

int moe_route(moe_plan_t plan, int32_t T, const int32_t* topk_idx, int32_t row_align,
              int32_t* counts, int32_t* offsets, int32_t* row_src, int32_t row_src_len,
              int32_t* src_row, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!plan)
        return MOE_ERR_INVALID_ARG;
    const moe_shape_t& s = plan->shape;
    if (T < 0 || T > s.max_tokens || row_align < 1 || row_align > 1024)
        return MOE_ERR_INVALID_ARG;
    if (!counts || !offsets || !workspace)
        return MOE_ERR_INVALID_ARG;
    const long long need_rows = (long long)T * s.top_k + (long long)s.num_experts * (row_align - 1);
    if (row_src_len < 0 || (long long)row_src_len < need_rows)
        return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_idx || !src_row))
        return MOE_ERR_INVALID_ARG;
    if (need_rows > 0 && !row_src)
        return MOE_ERR_INVALID_ARG;
    size_t need = 0;
    moe_route_workspace_bytes(plan, T, &need);
    if (workspace_bytes < need)
        return MOE_ERR_WORKSPACE_TOO_SMALL;
    int rc = device_ok();
    if (rc != MOE_OK)
        return rc;
    const Layout L = make_layout(s, T);
    moe::RouteArgs ra = route_args(s, T, L, workspace, topk_idx, row_align, counts, offsets,
                                   row_src, row_src_len, src_row, false);
    if (T == 0) {
        // Still defines counts = 0, offsets = 0 and every row as padding.
        ra.NB = 0;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (moe::launch_route(ra, st) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_read_status(moe_plan_t plan, int32_t T, const void* workspace, size_t workspace_bytes,
                    int32_t* host_status, void* stream)
{
    if (!plan || !workspace || !host_status || T < 0 || T > plan->shape.max_tokens)
        return MOE_ERR_INVALID_ARG;
    const Layout L = make_layout(plan->shape, T);
    if (workspace_bytes < L.status + 4 * sizeof(int32_t))
        return MOE_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(host_status, static_cast<const char*>(workspace) + L.status,
                       4 * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
        return MOE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

}  // extern "C"
