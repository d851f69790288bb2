// Stable arg-sort of the assignment vector on gfx950 (paper digest, "argsort与分段规约": only
// the 1-D vector of cluster ids is sorted, the N x D points are never permuted; the digest's
// "独立分析的弱点" suggests a radix sort for this key range).
//
// LSD counting passes over digits of the cluster id.  Per pass:
//   1. hist:    each workgroup counts the digits of its tile of 4096 keys in LDS and writes
//               one column of the [bins][tiles] table of its problem;
//   2. offsets: where a problem has few tiles (<= SORT_INLINE_TILES) the table is stored
//               tile-major and every scatter workgroup derives its own offsets from it (sum over
//               earlier tiles plus an exclusive scan of the digit totals); otherwise the table is
//               digit-major, one scan workgroup per (problem, digit) turns its row into the
//               digit's offsets over the tiles and records the digit's total, and every scatter
//               workgroup adds the exclusive scan of the totals;
//   3. scatter: each wave ranks its keys 64 at a time, in index order: lanes holding the same
//               digit are found with one ballot per digit bit (the digit width is a template
//               parameter, so these unroll); a lane's rank = earlier peers
//               in the round + the wave's running count of that digit (LDS).  The tile is
//               then laid out in LDS in (digit, index) order and written out with consecutive
//               lanes on consecutive positions of each digit's run.  Result: stable.
// All tiles of one problem run on one XCD, so the short runs that neighbouring tiles write
// into the same cache lines meet in that XCD's L2 instead of being written back piecemeal.
// The single-pass case (all of the id in one digit) also yields the per-cluster counts and
// each cluster's first sorted position (the update's segment starts).
//
// Labels outside [0, K) are not sorted and not counted; the call cannot report them when it
// returns (it does not wait for the GPU), so the kernels raise bits of a status word that the
// first counting kernel of the call clears: 1 = a label outside [0, K), 2 = a destination outside
// the output rows (a digit table that does not count the keys it is used with).  The output
// positions past the sorted valid labels are then left unwritten.
#include "common.h"
#include "plan.h"

namespace fkm {

// the scatter workgroup: 8 waves, each ranking 8 rounds of 64 keys of the tile
constexpr int SORT_WAVES = 8;
constexpr int SORT_THREADS = SORT_WAVES * 64;
constexpr int SORT_ROUNDS = SORT_TILE / SORT_THREADS;  // 8
static_assert(SORT_ROUNDS * SORT_THREADS == SORT_TILE, "a tile is whole rounds of the workgroup");

// tile_major: the table is [tiles][bins] (each workgroup writes one contiguous row); otherwise
// [bins][tiles] (one column per workgroup, the order the scan kernel needs).
__global__ __launch_bounds__(256) void sort_hist_kernel(const int32_t *__restrict__ keys, int N, int ntiles,
                                                        int shift, int bins, int32_t *__restrict__ hist,
                                                        int tile_major, int K, int32_t *__restrict__ status) {
    extern __shared__ int32_t s_h[];
    if (status && shift == 0 && blockIdx.x == 0 && threadIdx.x == 0) *status = 0;  // the call's first kernel
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lb / ntiles, t = lb - b * ntiles;
    for (int i = threadIdx.x; i < bins; i += 256) s_h[i] = 0;
    __syncthreads();
    const int32_t *kb = keys + (size_t)b * N;
    const int lo = t * SORT_TILE, hi = min(N, lo + SORT_TILE);
    const uint32_t mask = (uint32_t)bins - 1u;
    // all 16 keys of the thread are loaded before the first count
    constexpr int PER = SORT_TILE / 256;
    int32_t kv[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int i = lo + r * 256 + (int)threadIdx.x;
        kv[r] = i < hi ? kb[i] : -1;
    }
#pragma unroll
    for (int r = 0; r < PER; ++r)
        if ((uint32_t)kv[r] < (uint32_t)K) atomicAdd(&s_h[((uint32_t)kv[r] >> shift) & mask], 1);
    __syncthreads();
    int32_t *hb = hist + (size_t)b * bins * ntiles;
    if (tile_major)
        for (int i = threadIdx.x; i < bins; i += 256) hb[(size_t)t * bins + i] = s_h[i];
    else
        for (int i = threadIdx.x; i < bins; i += 256) hb[(size_t)i * ntiles + t] = s_h[i];
}

// Exclusive scan of one row of a problem's digit-major [bins][tiles] table, in place; the row's
// total goes to totals[problem][digit].  One 256-thread workgroup per (problem, digit); each pass
// covers 256 x 8 consecutive entries (8 independent loads per thread), scanned with wave
// shuffles and one LDS step, carried to the next pass.
constexpr int SCAN_ITEMS = 8;

__global__ __launch_bounds__(256) void sort_rowscan_kernel(int32_t *__restrict__ hist, int bins, int ntiles,
                                                           int32_t *__restrict__ totals) {
    __shared__ int32_t s_wave[4];
    __shared__ int32_t s_carry;
    const int row = blockIdx.x;  // problem * bins + digit
    int32_t *hb = hist + (size_t)row * ntiles;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    if (t == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < ntiles; base += 256 * SCAN_ITEMS) {
        const int lo = base + t * SCAN_ITEMS;
        int32_t v[SCAN_ITEMS];
#pragma unroll
        for (int i = 0; i < SCAN_ITEMS; ++i) v[i] = lo + i < ntiles ? hb[lo + i] : 0;
        int32_t sum = 0;
#pragma unroll
        for (int i = 0; i < SCAN_ITEMS; ++i) sum += v[i];
        // inclusive scan of the thread sums within the wave
        int32_t inc = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t o = __shfl_up(inc, off);
            if (lane >= off) inc += o;
        }
        if (lane == 63) s_wave[w] = inc;
        __syncthreads();
        int32_t wbase = 0;
        for (int i = 0; i < w; ++i) wbase += s_wave[i];
        int32_t run = s_carry + wbase + inc - sum;
#pragma unroll
        for (int i = 0; i < SCAN_ITEMS; ++i) {
            if (lo + i < ntiles) hb[lo + i] = run;
            run += v[i];
        }
        __syncthreads();
        if (t == 255) s_carry = run;
        __syncthreads();
    }
    if (t == 0) totals[row] = s_carry;
    (void)bins;
}

// In-place exclusive scan of s[0, n) (n <= 1024) by a workgroup of NT threads.
static_assert(SORT_MAX_BITS <= 10, "block_exscan_1024 covers at most 1024 bins");

template <int NT>
__device__ inline void block_exscan_1024(int32_t *s, int n, int32_t *s_wsum) {
    static_assert(NT % 64 == 0 && 1024 % NT == 0, "whole waves, whole elements per thread");
    constexpr int PER = 1024 / NT;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int32_t v[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = t * PER + i;
        v[i] = idx < n ? s[idx] : 0;
        sum += v[i];
    }
    int32_t inc = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    if (lane == 63) s_wsum[w] = inc;
    __syncthreads();
    int32_t run = inc - sum;
    for (int i = 0; i < w; ++i) run += s_wsum[i];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = t * PER + i;
        if (idx < n) s[idx] = run;
        run += v[i];
    }
    __syncthreads();
}

// Stable scatter of one pass.  vals_in == NULL means the values are the point indices.
// INLINE: `hist` holds the raw [tiles][bins] counts and each workgroup derives its offsets;
// otherwise `hist` holds each digit's offsets over the tiles ([bins][tiles], scanned per row)
// and `totals` the digit totals, whose exclusive scan each workgroup adds.  For counts != NULL
// the workgroup of tile 0 writes the per-bin totals.
template <bool INLINE, int BITS>
__global__ __launch_bounds__(SORT_THREADS) void sort_scatter_kernel(const int32_t *__restrict__ keys_in,
                                                           const int32_t *__restrict__ vals_in,
                                                           const int32_t *__restrict__ hist,
                                                           const int32_t *__restrict__ totals, int N, int ntiles,
                                                           int shift, int bits, int32_t *__restrict__ keys_out,
                                                           int32_t *__restrict__ vals_out,
                                                           int32_t *__restrict__ counts, int K,
                                                           int32_t *__restrict__ offs,
                                                           int32_t *__restrict__ status) {
    extern __shared__ int32_t s_mem[];
    __shared__ int32_t s_wsum[SORT_WAVES];
    __shared__ int32_t s_nvalid;
    const int bins = 1 << bits;
    // [SORT_WAVES][bins] running counts of each wave, then their exclusive prefix over the waves
    // (at most SORT_TILE, so 16 bits hold them)
    uint16_t *s_wc = (uint16_t *)s_mem;
    int32_t *s_off = s_mem + SORT_WAVES * bins / 2;  // [bins] this tile's global offset of each digit
    int32_t *s_ls = s_off + bins;                 // [bins] start of each digit inside the tile
    int32_t *s_k = s_ls + bins;                   // [SORT_TILE] keys in (digit, index) order
    int32_t *s_v = s_k + SORT_TILE;               // [SORT_TILE] values, same order
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lb / ntiles, t = lb - b * ntiles;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int32_t *hb = hist + (size_t)b * bins * ntiles;
    // this wave's keys and values, loaded first: their memory latency overlaps the offsets below
    const size_t base = (size_t)b * N;
    const int tile0 = t * SORT_TILE + w * (SORT_ROUNDS * 64);
    int32_t key[SORT_ROUNDS], val[SORT_ROUNDS], pos[SORT_ROUNDS];
#pragma unroll
    for (int r = 0; r < SORT_ROUNDS; ++r) {
        const int i = tile0 + r * 64 + lane;
        const bool ok = i < N;
        key[r] = ok ? keys_in[base + i] : -1;
        val[r] = ok ? (vals_in ? vals_in[base + i] : i) : 0;
    }
    for (int i = tid; i < SORT_WAVES * bins / 2; i += SORT_THREADS) s_mem[i] = 0;  // s_wc
    if (tid == 0) s_nvalid = 0;
    if constexpr (INLINE) {
        // `hist` is [tiles][bins]: thread tid sums the rows of its four consecutive digits
        // (16-byte loads, all issued before the sums): the total over all tiles and the sum over
        // the tiles before this one
        const int i0 = 4 * tid;
        int32_t tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
        if (i0 < bins) {
            for (int tt0 = 0; tt0 < ntiles; tt0 += 16) {
                int4 hv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    hv[u] = tt0 + u < ntiles ? *(const int4 *)(hb + (size_t)(tt0 + u) * bins + i0)
                                             : make_int4(0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const bool before = tt0 + u < t;
                    tot[0] += hv[u].x;
                    tot[1] += hv[u].y;
                    tot[2] += hv[u].z;
                    tot[3] += hv[u].w;
                    pre[0] += before ? hv[u].x : 0;
                    pre[1] += before ? hv[u].y : 0;
                    pre[2] += before ? hv[u].z : 0;
                    pre[3] += before ? hv[u].w : 0;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s_off[i0 + e] = tot[e];
                if (counts && t == 0 && i0 + e < K) counts[(size_t)b * K + i0 + e] = tot[e];
            }
        }
        __syncthreads();
        block_exscan_1024<SORT_THREADS>(s_off, bins, s_wsum);
        if (i0 < bins) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s_off[i0 + e] += pre[e];
        }
    } else {
        const int32_t *tb = totals + (size_t)b * bins;
        for (int i = tid; i < bins; i += SORT_THREADS) {
            s_off[i] = tb[i];
            if (counts && t == 0 && i < K) counts[(size_t)b * K + i] = tb[i];
        }
        __syncthreads();
        block_exscan_1024<SORT_THREADS>(s_off, bins, s_wsum);
        for (int i = tid; i < bins; i += SORT_THREADS) s_off[i] += hb[(size_t)i * ntiles + t];
    }
    __syncthreads();
    // tile 0 starts every digit at its global offset: the clusters' first sorted positions
    if (offs && t == 0)
        for (int i = tid; i < bins && i < K; i += SORT_THREADS) offs[(size_t)b * K + i] = s_off[i];

    const uint32_t mask = (uint32_t)bins - 1u;
    const uint64_t lt = lanemask_lt();
    uint16_t *wc = s_wc + w * bins;
    int nvalid = 0;
    bool bad = false;
#pragma unroll
    for (int r = 0; r < SORT_ROUNDS; ++r) {
        const int i = tile0 + r * 64 + lane;
        const bool ok = (uint32_t)key[r] < (uint32_t)K;  // in range (positions past N hold -1)
        bad |= i < N && !ok;
        const uint32_t dg = ((uint32_t)key[r] >> shift) & mask;
        // peers: the lanes whose digit equals this lane's, one ballot per digit bit; a lane
        // keeps the ballot where its bit is set and its complement where it is clear
        const uint64_t okm = __ballot(ok);
        nvalid += __popcll(okm);
        uint32_t p_lo = (uint32_t)okm, p_hi = (uint32_t)(okm >> 32);
#pragma unroll
        for (int bit = 0; bit < BITS; ++bit) {
            const uint32_t sx = (uint32_t)__builtin_amdgcn_sbfe((int)dg, bit, 1);  // 0 or all ones
            const uint64_t bal = __ballot(sx != 0u);
            p_lo &= ~((uint32_t)bal ^ sx);
            p_hi &= ~((uint32_t)(bal >> 32) ^ sx);
        }
        const uint64_t peers = ((uint64_t)p_hi << 32) | p_lo;
        const int before = __popcll(peers & lt);
        // LDS accesses of one wave complete in order and the store depends on the load, so
        // every lane reads its base before the group's lowest lane bumps it.
        const int32_t wbase = ok ? (int32_t)wc[dg] : 0;
        if (ok && before == 0) wc[dg] = (uint16_t)(wbase + __popcll(peers));
        pos[r] = wbase + before;
    }
    if (lane == 0) atomicAdd(&s_nvalid, nvalid);
    if (status && __ballot(bad) != 0ull && lane == 0) atomicOr(status, 1);
    __syncthreads();
    // exclusive prefix over waves, per digit; the digit's total in this tile
    for (int i = tid; i < bins; i += SORT_THREADS) {
        int32_t run = 0;
#pragma unroll
        for (int ww = 0; ww < SORT_WAVES; ++ww) {
            const int32_t v = s_wc[ww * bins + i];
            s_wc[ww * bins + i] = (uint16_t)run;
            run += v;
        }
        s_ls[i] = run;
    }
    __syncthreads();
    block_exscan_1024<SORT_THREADS>(s_ls, bins, s_wsum);
    // lay the tile out in (digit, index) order
#pragma unroll
    for (int r = 0; r < SORT_ROUNDS; ++r) {
        if ((uint32_t)key[r] < (uint32_t)K) {
            const uint32_t dg = ((uint32_t)key[r] >> shift) & mask;
            const int lp = s_ls[dg] + wc[dg] + pos[r];
            s_k[lp] = key[r];
            s_v[lp] = val[r];
        }
    }
    __syncthreads();
    const int tile_n = s_nvalid;  // the valid keys of the tile, laid out above
#pragma unroll 4
    for (int e = tid; e < tile_n; e += SORT_THREADS) {
        const int32_t k = s_k[e];
        const uint32_t dg = ((uint32_t)k >> shift) & mask;
        const int dst = s_off[dg] + (e - s_ls[dg]);
        // in range whenever the table counts the keys it is used with; a table that does not
        // (keys changed between the kernels by a concurrent writer) raises status bit 2 instead
        // of writing outside the rows
        if ((unsigned)dst < (unsigned)N) {
            keys_out[base + dst] = k;
            vals_out[base + dst] = s_v[e];
        } else if (status) {
            atomicOr(status, 2);
        }
    }
}

// Counts per cluster from the sorted ids: +end at a segment's last position, -start at its
// first (each cluster gets exactly one of each, so integer atomics give an exact result); the
// first position itself is the cluster's segment start.  Each thread takes SEGC_E consecutive
// positions of the flattened [B][N] ids (two 16-byte loads, plus the positions just before and
// after for the edges): with one position per thread, 2^24 ids took 46 us, latency-bound.
constexpr int SEGC_E = 8;
__global__ __launch_bounds__(256) void segment_counts_kernel(const int32_t *__restrict__ sids, int64_t total, int N,
                                                             int K, int32_t *__restrict__ counts,
                                                             int32_t *__restrict__ offs) {
    const int64_t g0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * SEGC_E;
    if (g0 >= total) return;
    int64_t b = g0 / N;
    int p = (int)(g0 - b * N);
    int32_t v[SEGC_E + 2];  // v[e + 1] = sids[g0 + e]; v[0] and v[SEGC_E + 1] the neighbours (-1 past the ends)
    v[0] = g0 > 0 ? sids[g0 - 1] : -1;
    if (g0 + SEGC_E <= total && ((uintptr_t)(sids + g0) & 15) == 0) {  // 16-byte loads where aligned
        const int4 lo = *(const int4 *)(sids + g0), hi = *(const int4 *)(sids + g0 + 4);
        v[1] = lo.x; v[2] = lo.y; v[3] = lo.z; v[4] = lo.w;
        v[5] = hi.x; v[6] = hi.y; v[7] = hi.z; v[8] = hi.w;
    } else {
#pragma unroll
        for (int e = 0; e < SEGC_E; ++e) v[e + 1] = g0 + e < total ? sids[g0 + e] : -1;
    }
    v[SEGC_E + 1] = g0 + SEGC_E < total ? sids[g0 + SEGC_E] : -1;
#pragma unroll
    for (int e = 0; e < SEGC_E; ++e) {
        if (g0 + e >= total) break;
        const int32_t k = v[e + 1];
        if (k >= 0 && k < K) {
            int32_t *cb = counts + b * K;
            // a problem's last position ends its segment; its first starts one (the neighbour
            // values there belong to the adjacent problem and are not compared)
            if (p == N - 1 || v[e + 2] != k) atomicAdd(&cb[k], p + 1);
            if (p == 0 || v[e] != k) {
                atomicSub(&cb[k], p);
                if (offs) offs[b * K + k] = p;
            }
        }
        if (++p == N) {
            p = 0;
            ++b;
        }
    }
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t *__restrict__ p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    fill_i32_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(p, n, v);
    return hipGetLastError();
}

// The scatter kernel for `bits` bits per digit (1..SORT_MAX_BITS): the ballot loop unrolls.
template <bool INLINE>
static hipError_t launch_scatter(int bits, dim3 grid, size_t lds, hipStream_t s, const int32_t *kin, const int32_t *vin,
                           const int32_t *hist, const int32_t *totals, int N, int ntiles, int shift, int32_t *ko,
                           int32_t *vo, int32_t *cnt, int K, int32_t *offs, int32_t *status) {
#define FKM_SCATTER(B_)                                                                                            \
    case B_:                                                                                                       \
        sort_scatter_kernel<INLINE, B_><<<grid, dim3(SORT_THREADS), lds, s>>>(kin, vin, hist, totals, N, ntiles, shift, bits, \
                                                                      ko, vo, cnt, K, offs, status);               \
        break;
    static_assert(SORT_MAX_BITS == 10, "one instance per digit width");
    switch (bits) {
        FKM_SCATTER(1) FKM_SCATTER(2) FKM_SCATTER(3) FKM_SCATTER(4) FKM_SCATTER(5)
        FKM_SCATTER(6) FKM_SCATTER(7) FKM_SCATTER(8) FKM_SCATTER(9) FKM_SCATTER(10)
        default: return hipErrorInvalidValue;  // the plan never asks for another width
    }
#undef FKM_SCATTER
    return hipGetLastError();
}

size_t sort_ws_bytes(int64_t B, int64_t N, int64_t K) {
    const SortCfg c = plan_sort(N, K);
    size_t bytes = align256((size_t)B * c.bins * c.ntiles * 4) + align256((size_t)B * c.bins * 4);
    if (c.passes > 1) bytes += 2 * align256((size_t)B * N * 4);
    return bytes;
}

// keys [B][N] -> sorted keys / point indices; counts, first positions ([B][K], only with
// counts) and the status word optional.
hipError_t launch_argsort(const int32_t *keys, int B, int N, int K, int32_t *out_keys, int32_t *out_vals,
                          int32_t *counts, int32_t *offs, int32_t *status, void *ws, hipStream_t s) {
    const SortCfg c = plan_sort(N, K);
    char *wp = (char *)ws;
    int32_t *hist = (int32_t *)wp;
    wp += align256((size_t)B * c.bins * c.ntiles * 4);
    int32_t *totals = (int32_t *)wp;
    wp += align256((size_t)B * c.bins * 4);
    int32_t *tk = nullptr, *tv = nullptr;
    if (c.passes > 1) {
        tk = (int32_t *)wp;
        wp += align256((size_t)B * N * 4);
        tv = (int32_t *)wp;
    }
    const int32_t *kin = keys;
    const int32_t *vin = nullptr;
    for (int pass = 0; pass < c.passes; ++pass) {
        const int shift = pass * c.bits;
        // the last pass writes the outputs; earlier passes alternate so that holds
        const bool to_out = ((c.passes - 1 - pass) % 2) == 0;
        int32_t *ko = to_out ? out_keys : tk;
        int32_t *vo = to_out ? out_vals : tv;
        int32_t *cnt_out = (counts && c.passes == 1) ? counts : nullptr;
        int32_t *offs_out = (offs && c.passes == 1) ? offs : nullptr;
        int32_t *st = pass == 0 ? status : nullptr;
        const size_t lds = (size_t)SORT_WAVES * c.bins * 2 + ((size_t)2 * c.bins + 2 * SORT_TILE) * 4;
        const bool inline_offsets = c.bins >= 4 && c.ntiles <= SORT_INLINE_TILES;
        sort_hist_kernel<<<dim3(B * c.ntiles), dim3(256), c.bins * 4, s>>>(kin, N, c.ntiles, shift, c.bins, hist,
                                                                            inline_offsets ? 1 : 0, K, st);
        if (inline_offsets) {
            const hipError_t e = launch_scatter<true>(c.bits, dim3(B * c.ntiles), lds, s, kin, vin, hist, nullptr, N,
                                                      c.ntiles, shift, ko, vo, cnt_out, K, offs_out, st);
            if (e != hipSuccess) return e;
        } else {
            sort_rowscan_kernel<<<dim3(B * c.bins), dim3(256), 0, s>>>(hist, c.bins, c.ntiles, totals);
            const hipError_t e = launch_scatter<false>(c.bits, dim3(B * c.ntiles), lds, s, kin, vin, hist, totals, N,
                                                       c.ntiles, shift, ko, vo, cnt_out, K, offs_out, st);
            if (e != hipSuccess) return e;
        }
        kin = ko;
        vin = vo;
    }
    if (counts && c.passes > 1) {
        hipError_t e = launch_fill_i32(counts, (int64_t)B * K, 0, s);
        if (e != hipSuccess) return e;
        const int64_t total = (int64_t)B * N;
        const int64_t threads = (total + SEGC_E - 1) / SEGC_E;
        segment_counts_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s>>>(out_keys, total, N, K,
                                                                                           counts, offs);
    }
    return hipGetLastError();
}

}  // namespace fkm
