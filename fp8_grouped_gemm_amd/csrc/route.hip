// Routing planner: per-expert histogram, aligned prefix sum and a stable
// slot assignment into per-expert contiguous pool segments.
//
// "07 · MegaMoE" §7 counts the tokens of every expert on the device, skips
// masked slots (id < 0), and §4 lays the pool out expert by expert with
// every segment aligned to the row tile, the segment start being the prefix
// sum of the aligned segment sizes; nothing is copied back to the host.
// The pages fill a segment in atomic-ticket order and say the order inside
// a segment does not change the result; here the rows of an expert hold its
// slots in ascending flat index f = t*K + j, which makes the plan
// deterministic and lets it be compared bit for bit.
//
// Three launches, no host synchronisation:
//   route_count  : one 1024-slot chunk per block, LDS histogram
//   route_scan   : one block, totals, aligned exclusive scan, per-chunk bases,
//                  padding rows and the row-block -> expert table
//   route_assign : one chunk per block, rank of each slot among the earlier
//                  slots of the same expert in its chunk, scatter
#include "moe_internal.h"

namespace moe {

// Maximum of v over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int wave_max(int v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v = max(v, __shfl_xor(v, d));
    return v;
}

__global__ __launch_bounds__(kRouteThreads) void route_count(RouteArgs a)
{
    extern __shared__ int32_t hist[];  // [E+1]; hist[E] counts ids >= E
    for (int e = threadIdx.x; e <= a.E; e += kRouteThreads)
        hist[e] = 0;
    __syncthreads();
    const int f = blockIdx.x * kRouteThreads + threadIdx.x;
    if (f < a.TK) {
        const int e = a.idx[f];
        if (e >= a.E)
            atomicAdd(&hist[a.E], 1);
        else if (e >= 0)
            atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    int32_t* out = a.blk + (size_t)blockIdx.x * (a.E + 1);
    for (int e = threadIdx.x; e <= a.E; e += kRouteThreads)
        out[e] = hist[e];
}

__global__ __launch_bounds__(kRouteThreads) void route_scan(RouteArgs a)
{
    __shared__ int32_t scan[kRouteThreads];
    __shared__ int32_t bad_sh;
    const int e = threadIdx.x;  // E <= 1024: one expert per thread
    int total = 0, seg = 0;
    // Column sums of the per-chunk counts, 16 loads in flight at a time.
    auto column_sum = [&](int col) {
        int sum = 0;
        for (int b0 = 0; b0 < a.NB; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                c[i] = (b0 + i < a.NB) ? a.blk[(size_t)(b0 + i) * (a.E + 1) + col] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sum += c[i];
        }
        return sum;
    };
    if (e < a.E) {
        total = column_sum(e);
        seg = (total + a.row_align - 1) / a.row_align * a.row_align;
        a.counts[e] = total;
    }
    if (e == 0)
        bad_sh = column_sum(a.E);
    // Inclusive Hillis-Steele scan of the aligned segment sizes.
    scan[e] = seg;
    __syncthreads();
    for (int d = 1; d < kRouteThreads; d <<= 1) {
        int v = (e >= d) ? scan[e - d] : 0;
        __syncthreads();
        scan[e] += v;
        __syncthreads();
    }
    const int start = scan[e] - seg;
    const int used = scan[kRouteThreads - 1];
    // the largest segment (status[3]: the prefill tiles' walk reads it)
    __shared__ int32_t seg_max;
    if (e == 0)
        seg_max = 0;
    __syncthreads();
    const int wmax = wave_max(seg);  // one LDS atomic per wave
    if ((e & 63) == 0 && wmax > 0)
        atomicMax(&seg_max, wmax);
    __syncthreads();
    if (e < a.E) {
        a.offsets[e] = start;
        // Per-chunk base row of this expert's slots (the chunk counts are
        // loaded 16 at a time, so their latencies overlap).
        int run = start;
        int32_t* col = a.blk + e;
        const size_t ld = (size_t)a.E + 1;
        for (int b0 = 0; b0 < a.NB; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                c[i] = (b0 + i < a.NB) ? col[(size_t)(b0 + i) * ld] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (b0 + i < a.NB) {
                    col[(size_t)(b0 + i) * ld] = run;
                    run += c[i];
                }
            }
        }
        // Padding rows at the end of the segment.
        for (int r = start + total; r < start + seg; ++r)
            a.row_src[r] = -1;
        if (a.mblock_expert) {
            for (int m = start / a.row_align; m < (start + seg) / a.row_align; ++m)
                a.mblock_expert[m] = e;
        }
    }
    if (e == 0) {
        a.offsets[a.E] = used;
        a.status[0] = bad_sh > 0 ? 1 : 0;
        a.status[1] = bad_sh;
        a.status[2] = used;
        a.status[3] = seg_max;
    }
    for (int r = used + e; r < a.r_cap; r += kRouteThreads)
        a.row_src[r] = -1;
    if (a.mblock_expert) {
        for (int m = used / a.row_align + e; m < a.mb_cap; m += kRouteThreads)
            a.mblock_expert[m] = -1;
    }
    if (a.sync) {
        for (int i = e; i < a.n_sync; i += kRouteThreads)
            a.sync[i] = 0;
    }
}

__global__ __launch_bounds__(kRouteThreads) void route_assign(RouteArgs a)
{
    extern __shared__ int32_t wave_cnt[];  // [16][E]: per-wave counts, then per-wave bases
    constexpr int kWaves = kRouteThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kWaves * a.E; i += kRouteThreads)
        wave_cnt[i] = 0;
    __syncthreads();
    const int f = blockIdx.x * kRouteThreads + threadIdx.x;
    const int e = (f < a.TK) ? a.idx[f] : -1;
    const bool valid = e >= 0 && e < a.E;
    const int key = valid ? e : -1;
    // Rank among the earlier lanes of this wave with the same expert.
    int rank = 0;
    if (__ballot(valid)) {  // a wave with no routed slot (past the last one) skips it
        for (int j = 0; j < 64; ++j) {
            const int other = __shfl(key, j);
            rank += (j < lane && other == key) ? 1 : 0;
        }
    }
    if (valid)
        atomicAdd(&wave_cnt[wave * a.E + e], 1);
    __syncthreads();
    for (int x = threadIdx.x; x < a.E; x += kRouteThreads) {
        int run = 0;
        for (int w = 0; w < kWaves; ++w) {
            const int c = wave_cnt[w * a.E + x];
            wave_cnt[w * a.E + x] = run;
            run += c;
        }
    }
    __syncthreads();
    if (f < a.TK) {
        if (valid) {
            const int pos = a.blk[(size_t)blockIdx.x * (a.E + 1) + e] + wave_cnt[wave * a.E + e] + rank;
            a.row_src[pos] = f;
            a.src_row[f] = pos;
        } else {
            a.src_row[f] = -1;
        }
    }
}

// All three steps in one block when every slot fits in one chunk
// (T*K <= 1024, the decode case): one launch instead of three.
__global__ __launch_bounds__(kRouteThreads) void route_small(RouteArgs a)
{
    extern __shared__ int32_t wave_cnt[];  // [16][E]: per-wave counts, then per-wave bases
    __shared__ int32_t scan[kRouteThreads];
    __shared__ int32_t bad_sh;
    constexpr int kWaves = kRouteThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kWaves * a.E; i += kRouteThreads)
        wave_cnt[i] = 0;
    if (threadIdx.x == 0)
        bad_sh = 0;
    __syncthreads();
    const int f = threadIdx.x;
    const int e = (f < a.TK) ? a.idx[f] : -1;
    const bool valid = e >= 0 && e < a.E;
    const int key = valid ? e : -1;
    int rank = 0;
    if (__ballot(valid)) {  // a wave with no routed slot (past the last one) skips it
        for (int j = 0; j < 64; ++j) {
            const int other = __shfl(key, j);
            rank += (j < lane && other == key) ? 1 : 0;
        }
    }
    if (valid)
        atomicAdd(&wave_cnt[wave * a.E + e], 1);
    else if (f < a.TK && e >= a.E)
        atomicAdd(&bad_sh, 1);
    __syncthreads();
    // Thread x owns expert x: total, per-wave bases, aligned segment.
    const int x = threadIdx.x;
    int total = 0, seg = 0;
    if (x < a.E) {
        for (int w = 0; w < kWaves; ++w) {
            const int c = wave_cnt[w * a.E + x];
            wave_cnt[w * a.E + x] = total;
            total += c;
        }
        seg = (total + a.row_align - 1) / a.row_align * a.row_align;
        a.counts[x] = total;
    }
    // Inclusive prefix sum of seg over the block: within each wave by
    // shuffles, then the 16 wave totals by wave 0 (integer adds: the same
    // result in any order).
    __shared__ int32_t wave_sum[kWaves];
    int incl = seg;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d)
            incl += v;
    }
    if (lane == 63)
        wave_sum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kWaves ? wave_sum[lane] : 0;
#pragma unroll
        for (int d = 1; d < kWaves; d <<= 1) {
            const int v = __shfl_up(w, d);
            if (lane >= d)
                w += v;
        }
        if (lane < kWaves)
            wave_sum[lane] = w;  // inclusive over waves 0 .. lane
    }
    __syncthreads();
    scan[x] = incl + (wave > 0 ? wave_sum[wave - 1] : 0);
    const int start = scan[x] - seg;
    const int used = wave_sum[kWaves - 1];
    __shared__ int32_t seg_max;  // the largest segment (status[3])
    if (x == 0)
        seg_max = 0;
    __syncthreads();
    const int wmax = wave_max(seg);  // one LDS atomic per wave
    if (lane == 0 && wmax > 0)
        atomicMax(&seg_max, wmax);
    __syncthreads();
    if (x < a.E) {
        a.offsets[x] = start;
        for (int r = start + total; r < start + seg; ++r)
            a.row_src[r] = -1;
        if (a.mblock_expert) {
            for (int m = start / a.row_align; m < (start + seg) / a.row_align; ++m)
                a.mblock_expert[m] = x;
        }
    }
    if (x == 0) {
        a.offsets[a.E] = used;
        a.status[0] = bad_sh > 0 ? 1 : 0;
        a.status[1] = bad_sh;
        a.status[2] = used;
        a.status[3] = seg_max;
    }
    for (int r = used + x; r < a.r_cap; r += kRouteThreads)
        a.row_src[r] = -1;
    if (a.mblock_expert) {
        for (int m = used / a.row_align + x; m < a.mb_cap; m += kRouteThreads)
            a.mblock_expert[m] = -1;
    }
    if (a.sync) {
        for (int i = x; i < a.n_sync; i += kRouteThreads)
            a.sync[i] = 0;
    }
    __syncthreads();  // scan[] holds inclusive ends: start of expert e = scan[e] - seg(e)
    if (f < a.TK) {
        if (valid) {
            const int seg_e = scan[e] - (e > 0 ? scan[e - 1] : 0);
            const int pos = scan[e] - seg_e + wave_cnt[wave * a.E + e] + rank;
            a.row_src[pos] = f;
            a.src_row[f] = pos;
        } else {
            a.src_row[f] = -1;
        }
    }
}

// Stream of the single launch with a ring pool (DeepGEMM PR #440 "How it
// works"): units of up to kUnitBlocks consecutive row blocks of one expert,
// in pool order; the L2 tiles of unit group j (kStreamGroup units) follow
// the L1 tiles of unit G j + G - 1 + lag (or, when that unit does not
// exist, the last L1 unit).  In closed form, with U units, G = kStreamGroup
// and L = lag: L1 of unit u is entry u + min(U, G max(0, floor((u - L) / G)))
// and L2 of unit u is entry u + 1 + min(G floor(u / G) + G - 1 + L, U - 1).
// One block: per-expert unit counts and their scan, the unit table, each
// unit's two entries with their item counts (row blocks x column tiles),
// the exclusive scan of those counts and the item table.
__global__ __launch_bounds__(kRouteThreads) void route_stream(FwdArgs a)
{
    __shared__ int32_t scan[kRouteThreads];
    const int tid = threadIdx.x;
    const int BM = a.BM;
    auto block_scan = [&](int v) {  // inclusive scan over the block
        scan[tid] = v;
        __syncthreads();
        for (int d = 1; d < kRouteThreads; d <<= 1) {
            const int w = tid >= d ? scan[tid - d] : 0;
            __syncthreads();
            scan[tid] += w;
            __syncthreads();
        }
        return scan[tid];
    };
    int first = 0, nu = 0;
    if (tid < a.E) {
        first = a.offsets[tid] / BM;
        const int nb = (a.offsets[tid + 1] - a.offsets[tid]) / BM;
        nu = (nb + kUnitBlocks - 1) / kUnitBlocks;
    }
    const int ubase = block_scan(nu) - nu;
    const int U = scan[kRouteThreads - 1];
    __syncthreads();
    for (int k = 0; k < nu; ++k)
        a.unit_mb[ubase + k] = first + kUnitBlocks * k;
    if (tid == 0)
        a.unit_mb[U] = a.offsets[a.E] / BM;
    __syncthreads();  // the unit table is visible to the whole block
    // Used row blocks that fit the ring never share a slot: single-wave
    // order (a lag of U units puts every L1 unit before every L2 unit).
    // Otherwise the host's lag.  (Lengthening it on the device to the
    // longest the ring holds for the routed unit sizes was measured slower:
    // L1 tiles then wait on the slots' previous L2 tiles.)
    const int RB = a.ring_blocks, G = kStreamGroup;
    const int L = a.unit_mb[U] <= RB ? U : a.lag_units;
    const int NT1 = a.I / 128, NT2 = (a.H + 255) / 256;
    for (int u = tid; u < U; u += kRouteThreads) {
        const int nbu = a.unit_mb[u + 1] - a.unit_mb[u];
        const int c = u >= L ? (u - L) / G : 0;
        const int p1 = u + min(U, G * c);
        const int p2 = u + 1 + min(G * (u / G) + G - 1 + L, U - 1);
        a.stream_start[p1] = nbu * NT1;
        a.stream_desc[p1] = u;
        a.stream_start[p2] = nbu * NT2;
        a.stream_desc[p2] = u | kStreamL2;
    }
    __syncthreads();
    // exclusive scan of the 2U item counts, in place, 1024 at a time
    int carry = 0;
    for (int base = 0; base < 2 * U; base += kRouteThreads) {
        const int i = base + tid;
        const int v = i < 2 * U ? a.stream_start[i] : 0;
        const int incl = block_scan(v);
        const int total = scan[kRouteThreads - 1];
        if (i < 2 * U)
            a.stream_start[i] = carry + incl - v;
        carry += total;
        __syncthreads();
    }
    if (tid == 0) {
        a.stream_start[2 * U] = carry;
        a.sync[kSyncStreamItems] = carry;
        a.sync[kSyncUnits] = U;
    }
    __syncthreads();
    // item table: one wave per stream entry, its items in consecutive words
    const int lane = tid & 63, wave = tid >> 6;
    for (int p = wave; p < 2 * U; p += kRouteThreads / 64) {
        const int d = a.stream_desc[p];
        const bool l2 = (d & kStreamL2) != 0;
        const int tile0 = a.unit_mb[d & kStreamUnitMask] * (l2 ? NT2 : NT1);
        const int q0 = a.stream_start[p], n = a.stream_start[p + 1] - q0;
        for (int i = lane; i < n; i += 64)
            a.item_tab[q0 + i] = (tile0 + i) | (l2 ? kItemL2 : 0);
    }
}

hipError_t launch_route_stream(const FwdArgs& a, hipStream_t s)
{
    if (a.E > kRouteThreads || !a.offsets || !a.unit_mb || !a.stream_start || !a.stream_desc ||
        !a.item_tab || !a.sync || a.ring_blocks <= 0 || a.lag_units < 1)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_stream, dim3(1), dim3(kRouteThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s)
{
    if (a.NB == 1 && a.E <= 512) {
        hipLaunchKernelGGL(route_small, dim3(1), dim3(kRouteThreads),
                           sizeof(int32_t) * 16 * a.E, s, a);
        return hipGetLastError();
    }
    const size_t lds_hist = sizeof(int32_t) * (a.E + 1);
    const size_t lds_wave = sizeof(int32_t) * 16 * a.E;
    if (a.NB > 0)
        hipLaunchKernelGGL(route_count, dim3(a.NB), dim3(kRouteThreads), lds_hist, s, a);
    hipLaunchKernelGGL(route_scan, dim3(1), dim3(kRouteThreads), 0, s, a);
    if (a.NB > 0)
        hipLaunchKernelGGL(route_assign, dim3(a.NB), dim3(kRouteThreads), lds_wave, s, a);
    return hipGetLastError();
}

}  // namespace moe
