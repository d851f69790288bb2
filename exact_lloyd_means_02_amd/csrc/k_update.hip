// Sort-inverse update on gfx950 (paper summary, "Method"; paper digest, "方法步骤详情" step (2)):
// the sorted order is cut into chunks; each wave takes one chunk, walks its cluster-id
// segments, gathers the rows of the unpermuted x through sorted_idx, sums each segment on
// chip in fp32, and writes once per segment.  The digest issues one atomic per segment; here
// a segment that lies inside one chunk (or ends in the next one) is finished by its wave
// (c_k = s_k / n_k written directly).  A longer segment leaves one fp32 partial per chunk; the
// waves of its chunks count their arrivals with an integer atomic per group of chunks, and the
// last wave to arrive adds the group's partials in chunk order, then (for segments over more
// than one group) the last group to arrive adds the group sums in group order and finishes the
// cluster.  The order of every float sum is fixed by the chunk layout alone, not by which wave
// arrives last, so the result is deterministic; there are no float atomics and no second kernel.
//
// Lane layout: a row is covered by `lanes` lanes (a power of two) holding 16-byte vectors
// (or scalars when D is not a multiple of the vector width); one wave load instruction
// therefore reads 64/lanes rows.  A window of 64 sorted positions is read with one
// coalesced load of ids and indices; the rows of the current segment inside the window are
// a prefix of it (ids are sorted), counted with one ballot.
#include "common.h"
#include "plan.h"

namespace fkm {

hipError_t launch_sum_f64_rows(const double *part, int rows, int64_t len, double *out, hipStream_t s,
                               int accumulate = 0);

// Row loads issued before any is consumed: 8 vectors per lane in flight (8 KiB per wave).  With
// 16 the kernel needs more than 128 VGPRs and only 3 waves fit a SIMD instead of 4; more waves
// with shallower queues gather faster (measured on the headline shape).
template <int VPL>
constexpr int upd_unroll() { return 8 / VPL; }

struct UpdArgs {
    const void *x;
    const int32_t *sids, *sidx, *counts;
    int N, D, K, R, nch, lanes, ncb, cb_elems;
    int mode;          // 0: finish c_k in place; 1: accumulate into sums / cnt (streamed chunks)
    int dt;
    float *C;          // [B][K][D] in/out (mode 0)
    // optional fp64 partials of sum_k ||c_new - c_old||^2, each written once (no atomics):
    // mode 0: [B*nch][2*ncb]: slot cb, the clusters a chunk's wave finished in column block cb;
    // slot ncb + cb, the long segment that starts in the chunk (written by the wave that
    // finishes it, 0 when none starts there); finalize: [B][K], one per cluster.
    double *shp;
    float *sums;       // [B][K][D] (mode 1)
    int32_t *cnt;      // [B][K]    (mode 1)
    float *part;       // [B*nch][2][D]: slot 0, the segment cut on entry; slot 1, cut on exit
    const int32_t *offs;  // [B][K] first sorted position of each cluster's segment
    int32_t *gcnt;     // [B*nch][2][ncb] arrivals per chunk group (zero between launches)
    int32_t *scnt;     // [B][K][ncb] arrivals of group sums per long segment (zero between launches)
    // optional (mode 0): refresh the assign kernels' prepared centroids for every finished
    // cluster (same layout as the prep kernel); clusters without points keep theirs.
    void *cprep;
    float *cnh;
    int DP, KT;
    int zero_norm;     // similarity metrics: the refreshed norm terms are 0
    int normalize;     // finalize (cosine k-means): c_k <- sums_k / ||sums_k|| instead of / cnt_k
};

// The half-norm term the assign kernels add to a refreshed centroid's scores.
__device__ inline float refreshed_half_norm(const UpdArgs &a, float cn2) { return a.zero_norm ? 0.f : 0.5f * cn2; }

// Store element d of -c~ (c~ = dtype(c), nearest even) into the prepared layout; returns c~^2.
__device__ inline float prep_store_elem(const UpdArgs &a, int b, int k, int d, float c) {
    const int VW = a.dt == DT_F32 ? 4 : 8;
    const int gi = d / VW;
    const int q = gi >> 1, hh = gi & 1, e = d - gi * VW;
    const size_t word = (((size_t)b * a.KT + (k >> 5)) * (a.DP / (2 * VW)) + q) * 64 + (k & 31) + 32 * hh;
    float r;
    if (a.dt == DT_F32) {
        r = c;
        ((float *)a.cprep)[word * 4 + e] = -r;
    } else if (a.dt == DT_F16) {
        const uint32_t hb = f32_to_f16_bits(c);
        r = f16_bits_to_f32(hb);
        ((uint16_t *)a.cprep)[word * 8 + e] = (uint16_t)(hb ^ 0x8000u);
    } else {
        const uint32_t bb = f32_to_bf16_bits(c);
        r = bf16_bits_to_f32(bb);
        ((uint16_t *)a.cprep)[word * 8 + e] = (uint16_t)(bb ^ 0x8000u);
    }
    return r * r;
}

// Same for a whole 16-byte group starting at element d0 (d0 % VW == 0, all in range).
template <int DT>
__device__ inline float prep_store_group(const UpdArgs &a, int b, int k, int d0, const float *c) {
    constexpr int VW = DT == DT_F32 ? 4 : 8;
    const int gi = d0 / VW;
    const int q = gi >> 1, hh = gi & 1;
    const size_t word = (((size_t)b * a.KT + (k >> 5)) * (a.DP / (2 * VW)) + q) * 64 + (k & 31) + 32 * hh;
    uint32_t w[4];
    float ss = 0.f;
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] = __float_as_uint(-c[e]);
            ss += c[e] * c[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t lo, hi;
            float rl, rh;
            if constexpr (DT == DT_F16) {
                lo = f32_to_f16_bits(c[2 * e]);
                hi = f32_to_f16_bits(c[2 * e + 1]);
                rl = f16_bits_to_f32(lo);
                rh = f16_bits_to_f32(hi);
            } else {
                lo = f32_to_bf16_bits(c[2 * e]);
                hi = f32_to_bf16_bits(c[2 * e + 1]);
                rl = bf16_bits_to_f32(lo);
                rh = bf16_bits_to_f32(hi);
            }
            w[e] = ((lo ^ 0x8000u) & 0xFFFFu) | (((hi ^ 0x8000u) & 0xFFFFu) << 16);
            ss += rl * rl + rh * rh;
        }
    }
    ((uint4 *)a.cprep)[word] = make_uint4(w[0], w[1], w[2], w[3]);
    return ss;
}

// Load the lane's vectors of row `row` within column block starting at element `c0`.
template <int DT, int V, int VPL>
__device__ inline void load_row(const UpdArgs &a, size_t row_elem0, int c0, int r, float (&out)[VPL][V], bool ok) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e0 = c0 + (r + i * a.lanes) * V;
        if constexpr (V == 1) {
            out[i][0] = (ok && e0 < a.D) ? load_elem<DT>(a.x, row_elem0 + e0) : 0.f;
        } else {
            if (ok && e0 < a.D) {
                const uint4 v = *(const uint4 *)((const char *)a.x + (row_elem0 + e0) * (DT == DT_F32 ? 4 : 2));
                widen16<DT>(v, out[i]);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) out[i][e] = 0.f;
            }
        }
    }
}

// Finish cluster k from the row sum held by the lanes of one row group (lane index r < lanes).
// mode 0: c_k <- s / n (fp32, IEEE division); when shift partials are wanted returns
//         sum (c_new - c_old)^2 over the lane's columns (c_old prefetched in `cold`); adds
//         sum c~^2 to cn2 when the prepared centroids are refreshed.
// mode 1: sums_k += s, cnt_k += n.
// With a.normalize (mode 0, cosine k-means) c_k <- s / ||s|| (fp32 norm over the row, IEEE
// division) instead of s / n, and a cluster whose sum is the zero vector keeps its centroid.  The
// norm is reduced over the row group's lanes, so it needs one column block per row (ncb == 1).
template <int DT, int V, int VPL, bool SHIFT>
__device__ inline float finish_cluster(const UpdArgs &a, int b, int k, int c0, int r, const float (&s)[VPL][V], int n,
                                       const float (&cold)[VPL][V], bool write_cnt, float &cn2) {
    float d2 = 0.f;
    const size_t rowo = ((size_t)b * a.K + k) * a.D;
    float den = (float)n;
    if (a.mode == 0 && a.normalize) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e0 = c0 + (r + i * a.lanes) * V;
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (e0 + e < a.D) ss += s[i][e] * s[i][e];
        }
        for (int off = 1; off < a.lanes; off <<= 1) ss += __shfl_xor(ss, off);  // the row group's lanes
        den = sqrtf(ss);
        if (!(den > 0.f)) return 0.f;  // uniform over the row group: the centroid is kept
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e0 = c0 + (r + i * a.lanes) * V;
        if (a.mode == 0 && V > 1) {
            // whole 16-byte vectors (D is a multiple of V here): the new row goes out with
            // 16-byte stores
            if (e0 < a.D) {
                float nw[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    nw[e] = s[i][e] / den;
                    if (SHIFT) {
                        const float df = nw[e] - cold[i][e];
                        d2 += df * df;
                    }
                }
#pragma unroll
                for (int q = 0; q < V / 4; ++q)
                    *(float4 *)(a.C + rowo + e0 + 4 * q) =
                        make_float4(nw[4 * q], nw[4 * q + 1], nw[4 * q + 2], nw[4 * q + 3]);
                if (a.cprep) cn2 += prep_store_group<DT>(a, b, k, e0, nw);
            }
        } else if (a.mode == 0) {
            float nw[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int d = e0 + e;
                nw[e] = 0.f;
                if (d < a.D) {
                    nw[e] = s[i][e] / den;
                    a.C[rowo + d] = nw[e];
                    if (SHIFT) {
                        const float df = nw[e] - cold[i][e];
                        d2 += df * df;
                    }
                }
            }
            if (a.cprep && e0 < a.D) cn2 += prep_store_elem(a, b, k, e0, nw[0]);  // V == 1 here
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const int d = e0 + e;
                if (d < a.D) a.sums[rowo + d] += s[i][e];
            }
        }
    }
    if (a.mode == 1 && write_cnt && r == 0) a.cnt[(size_t)b * a.K + k] += n;
    return d2;
}

// Finish column d of cluster k of problem b from its sum `s` (a long segment's finishing wave).
// den: n_k, or ||s_k|| with a.normalize (mode 0).  Returns (c_new - c_old)^2 (mode 0).
__device__ inline float finish_col(const UpdArgs &a, int b, int k, size_t rowo, int d, float s, float den,
                                   float &cn2) {
    if (a.mode == 0) {
        const float old = a.C[rowo + d];
        const float nw = s / den;
        a.C[rowo + d] = nw;
        if (a.cprep) cn2 += prep_store_elem(a, b, k, d, nw);
        return (nw - old) * (nw - old);
    }
    a.sums[rowo + d] += s;
    return 0.f;
}

// Chunks per first-level group of a long segment's partials.
constexpr int UPD_GROUP = 32;

// The partial records and group sums pass between waves of different XCDs.  They are written and
// read with device-scope (agent) atomic stores and loads, which the memory system keeps coherent
// across the XCDs' L2 caches, so no device-wide cache write-back or invalidation is needed: a
// wave waits until its record stores are acknowledged (vmcnt 0) before its arrival (an integer
// atomic, also device scope), and the wave that sees the last arrival reads the records after it.
// The empty asm statements keep the compiler from moving memory operations across these points.
__device__ inline void rec_store(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float rec_load(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Count this wave's arrival (lane 0) once its earlier record stores are complete; returns the
// count before it (wave-uniform).
__device__ inline int arrive(int32_t *ctr, int lane) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0);
    asm volatile("" ::: "memory");
    return old;
}

// Column d of the sum of m partial records: those of chunks first, first + stride, ... of the
// problem whose chunk 0 is `cbase` (the segment's first chunk c_first holds it in slot 1, every
// later chunk in slot 0), added in that order; eight loads in flight.
__device__ inline float sum_pieces(const UpdArgs &a, size_t cbase, int c_first, int first, int stride, int m,
                                   int d) {
    float s = 0.f;
    int i = 0;
    for (; i + 8 <= m; i += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int ch = first + (i + u) * stride;
            v[u] = rec_load(a.part + ((cbase + ch) * 2 + (ch == c_first ? 1 : 0)) * a.D + d);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; i < m; ++i) {
        const int ch = first + i * stride;
        s += rec_load(a.part + ((cbase + ch) * 2 + (ch == c_first ? 1 : 0)) * a.D + d);
    }
    return s;
}

// Finish long segment k (n points) in column block cbi from the sum of its m partial records
// (first, stride as in sum_pieces).  The whole wave calls it; lanes take the block's columns.
__device__ inline void finish_long(const UpdArgs &a, int b, int k, int cbi, int n, size_t cbase, int c_first,
                                   int first, int stride, int m, int lane) {
    const int c0 = cbi * a.cb_elems;
    const int c1 = min(a.D, c0 + a.cb_elems);
    const size_t rowo = ((size_t)b * a.K + k) * a.D;
    double *shp_slot = a.shp ? a.shp + (cbase + c_first) * (2 * a.ncb) + a.ncb + cbi : nullptr;
    float den = (float)n;
    if (a.mode == 0 && a.normalize) {
        // the mean direction needs ||s|| first (one column block per row here): one pass for the
        // norm, then the same sums again
        float ss = 0.f;
        for (int d = c0 + lane; d < c1; d += 64) {
            const float v = sum_pieces(a, cbase, c_first, first, stride, m, d);
            ss += v * v;
        }
        for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
        den = sqrtf(ss);
        if (!(den > 0.f)) {  // uniform over the wave: the zero sum keeps the centroid
            if (shp_slot && lane == 0) *shp_slot = 0.0;
            return;
        }
    }
    float d2 = 0.f, cn2 = 0.f;
    for (int d = c0 + lane; d < c1; d += 64)
        d2 += finish_col(a, b, k, rowo, d, sum_pieces(a, cbase, c_first, first, stride, m, d), den, cn2);
    if (a.mode == 0) {
        for (int off = 1; off < 64; off <<= 1) {
            d2 += __shfl_xor(d2, off);
            cn2 += __shfl_xor(cn2, off);
        }
        if (shp_slot && lane == 0) *shp_slot = (double)d2;
        if (a.cprep && lane == 0) a.cnh[(size_t)b * a.KT * 32 + k] = refreshed_half_norm(a, cn2);
    } else if (cbi == 0 && lane == 0) {
        a.cnt[(size_t)b * a.K + k] += n;
    }
}

// Called by the whole wave of chunk c (problem b, column block cbi) right after it wrote its
// partial record of long segment k.  The segment's chunks c_first..c_last form groups of
// UPD_GROUP; the last wave of a group to arrive adds the group's partials.  With one group that
// wave finishes the cluster; otherwise it leaves the group sum in the record of the group's first
// chunk, and the last group to arrive adds the group sums and finishes the cluster.  Records
// pass between the waves as rec_store / rec_load describe.  The counters return to zero for the
// next launch.
__device__ inline void arrive_long(const UpdArgs &a, int b, int c, int cbi, int k, int lane) {
    // counts and first positions come from the arg-sort of the same labels; clamped so that
    // inconsistent inputs give wrong numbers, not accesses outside the records and counters
    const int n = max(1, a.counts[(size_t)b * a.K + k]);
    const int s0 = min(max(a.offs[(size_t)b * a.K + k], 0), a.N - 1);
    const int c_first = s0 / a.R;
    const int c_last = (int)min((int64_t)a.nch - 1, ((int64_t)s0 + n - 1) / a.R);
    if (c < c_first || c > c_last) return;
    const int P = c_last - c_first + 1;
    const int j = (c - c_first) / UPD_GROUP;
    const int gfirst = c_first + j * UPD_GROUP;
    const int m = min(UPD_GROUP, P - j * UPD_GROUP);
    const int gslot = j == 0 ? 1 : 0;
    const size_t cbase = (size_t)b * a.nch;
    int32_t *ctr = a.gcnt + ((cbase + gfirst) * 2 + gslot) * a.ncb + cbi;
    if (arrive(ctr, lane) != m - 1) return;
    if (lane == 0) *ctr = 0;
    const int ngroups = (P + UPD_GROUP - 1) / UPD_GROUP;
    if (ngroups == 1) {
        finish_long(a, b, k, cbi, n, cbase, c_first, c_first, 1, P, lane);
        return;
    }
    const int c0 = cbi * a.cb_elems;
    const int c1 = min(a.D, c0 + a.cb_elems);
    float *grec = a.part + ((cbase + gfirst) * 2 + gslot) * a.D;
    for (int d = c0 + lane; d < c1; d += 64) {
        const float v = sum_pieces(a, cbase, c_first, gfirst, 1, m, d);
        rec_store(grec + d, v);  // every piece of the group (this record too) was read above
    }
    int32_t *sctr = a.scnt + ((size_t)b * a.K + k) * a.ncb + cbi;
    if (arrive(sctr, lane) != ngroups - 1) return;
    if (lane == 0) *sctr = 0;
    finish_long(a, b, k, cbi, n, cbase, c_first, c_first, UPD_GROUP, ngroups, lane);
}

// SHIFT: a.shp is set (mode 0 with shift partials wanted); a separate instance keeps the
// register budget of the common case free of the old-centroid prefetch.
// BUF (16-byte vectors, a problem's rows at most 2 GiB): rows are gathered with raw buffer loads
// over the problem's rows: 32-bit offsets, and a lane without a row takes an offset past the end,
// which the buffer's range check turns into zeros without a memory access, so the loads of a
// batch go out back to back with no branches around them.
template <int DT, int V, int VPL, bool SHIFT, bool BUF>
__global__ __launch_bounds__(256) void upd_segsum_kernel(UpdArgs a, int64_t total_waves) {
    const int lane = threadIdx.x & 63;
    // the wave's index, in a scalar register: everything derived from it (problem, chunk,
    // positions, the row buffer) is then wave-uniform to the compiler too
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t gw = (int64_t)xcd_remap_rev(blockIdx.x, gridDim.x) * 4 + wave;
    if (gw >= total_waves) return;
    const int cbi = (int)(gw % a.ncb);
    const int64_t chunk = gw / a.ncb;
    const int b = (int)(chunk / a.nch);
    const int c = (int)(chunk - (int64_t)b * a.nch);
    const int G = 64 / a.lanes;
    const int g = lane / a.lanes, r = lane - g * a.lanes;
    const int c0 = cbi * a.cb_elems;
    const int N = a.N;
    const int p0 = c * a.R, p1 = min(N, p0 + a.R);
    const int32_t *sb = a.sids + (size_t)b * N;
    const int32_t *ib = a.sidx + (size_t)b * N;
    const size_t xb = (size_t)b * N;
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    const uint32_t rowbytes = (uint32_t)a.D * ES;
    const uint32_t x_end = BUF ? (uint32_t)N * rowbytes : 0u;  // the problem's bytes: an offset there reads zeros
    // the byte offsets of the rows at the 64 positions of the current view, one LDS row per wave
    // (written and read by the same wave: its LDS accesses complete in order, no barrier)
    __shared__ __align__(16) uint32_t s_xo[4][64];
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (char *)const_cast<void *>(a.x) + xb * rowbytes, (short)0, (int)x_end, 0x00020000);

    // Sorted ids / indices are read through a sliding window of 192 positions held in three
    // register pairs per lane ([wp, wp+64), [wp+64, wp+128), [wp+128, wp+192)).  When the walk
    // passes wp+64 the window moves on by 64 and the 64 positions after it are loaded: two
    // windows ahead of their first read, so that load overlaps the row gathers in between
    // instead of stalling the next view.
    int wp = p0, cs, ci, ns, ni, fs, fi;
    auto load_ids = [&](int q, int &s_, int &i_) {
        s_ = q < N ? sb[q] : -1;
        i_ = q < N ? ib[q] : 0;
    };
    load_ids(p0 + lane, cs, ci);
    load_ids(p0 + 64 + lane, ns, ni);
    load_ids(p0 + 128 + lane, fs, fi);
    auto slide_if_past = [&](int pos) {  // keep pos - wp < 64 (pos advanced by at most 64)
        if (pos - wp >= 64) {
            wp += 64;
            cs = ns;
            ci = ni;
            ns = fs;
            ni = fi;
            load_ids(wp + 128 + lane, fs, fi);
        }
    };
    // the 64 positions from pos: lane l takes window slot pos - wp + l of the first 128
    auto view = [&](int pos, int &sid, int &idx) {
        const int q = pos - wp + lane;
        const int s_lo = __shfl(cs, q & 63), s_hi = __shfl(ns, q & 63);
        const int i_lo = __shfl(ci, q & 63), i_hi = __shfl(ni, q & 63);
        sid = q < 64 ? s_lo : s_hi;
        idx = q < 64 ? i_lo : i_hi;
    };
    // positions of id k from pos on (at most 64, stopping at lim), given the view at pos
    auto run_len = [&](int pos, int sid, int k, int lim) -> int {
        const uint64_t eq = __ballot(pos + lane < lim && sid == k);
        return (~eq == 0ull) ? 64 : (int)__builtin_ctzll(~eq);
    };
    auto clampk = [&](int kr) { return kr < 0 ? 0 : (kr >= a.K ? a.K - 1 : kr); };

    // The ids around the chunk edges, read with the first window: they settle which wave sums a
    // segment cut by an edge without waiting for the walk to reach it.
    const int id_prev = p0 > 0 ? sb[p0 - 1] : -1;                    // before the chunk
    const int id_prev2 = p0 - a.R - 1 >= 0 ? sb[p0 - a.R - 1] : -1;  // before the previous chunk
    const int id_last = sb[p1 - 1];                                  // the chunk's last
    const int id_next = p1 < N ? sb[p1] : -1;                        // after the chunk
    const bool next2_in = (int64_t)p1 + a.R < N;
    const int id_next2 = next2_in ? sb[p1 + a.R] : -1;               // after the next chunk

    int p = p0, plim = p1;
    int sid, idx;
    view(p, sid, idx);
    int kraw = __shfl(sid, 0);
    bool cin = p0 > 0 && id_prev == kraw;
    // Segment ownership: a segment that ends within the chunk after the one where it starts is
    // summed entirely by the wave of its first chunk (which runs past its chunk end for it);
    // only segments spanning three or more chunks leave partials (the long segments).  A wave
    // whose chunk starts inside a segment that began in the previous chunk (the id before that
    // chunk differs) and ends in this one (the chunk's last id differs, or the id after it does)
    // walks past it without gathering.
    bool done = false;
    if (cin) {
        const bool ends_here = id_last != kraw || p1 == N || id_next != kraw;
        const bool began_prev = !(p0 - a.R - 1 >= 0 && id_prev2 == kraw);
        if (ends_here && began_prev) {
            int e = p;
            while (true) {
                const int m = run_len(e, sid, kraw, p1);
                e += m;
                slide_if_past(e);
                if (m < 64 || e >= p1) break;
                view(e, sid, idx);
            }
            p = e;
            if (p >= p1) {
                done = true;
            } else {
                view(p, sid, idx);
                kraw = __shfl(sid, 0);
                cin = false;
            }
        }
    }
    // old centroid columns of the current segment's cluster, fetched when the segment starts
    // (only for the shift partials), so the read overlaps the segment's row gathers
    float cold[VPL][V];
    auto fetch_cold = [&](int kr) {
        if (SHIFT && g == 0) {
            const size_t rowo = ((size_t)b * a.K + clampk(kr)) * a.D;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int e0 = c0 + (r + i * a.lanes) * V;
#pragma unroll
                for (int e = 0; e < V; ++e) cold[i][e] = e0 + e < a.D ? a.C[rowo + e0 + e] : 0.f;
            }
        }
    };
    fetch_cold(kraw);
    int seg_start = p;
    // long segments this chunk holds a partial of: cut on entry (k_in), cut on exit (k_out); the
    // wave arrives at them after its walk, when the walk's registers are free
    int k_in = -1, k_out = -1;
    float d2acc = 0.f;
    float acc[VPL][V];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[i][e] = 0.f;

    // The summed segment ends: add the row groups and finish the cluster, or, for a segment cut
    // by a chunk edge (cin / cout), write this chunk's partial.
    auto end_segment = [&](int kr, int n, bool s_cout) {
        // sum the row groups: lanes r, r + lanes, r + 2*lanes, ... hold the same columns
        for (int off = a.lanes; off < 64; off <<= 1) {
#pragma unroll
            for (int i = 0; i < VPL; ++i)
#pragma unroll
                for (int e = 0; e < V; ++e) acc[i][e] += __shfl_xor(acc[i][e], off);
        }
        const int k = clampk(kr);
        if (!cin && !s_cout) {
            float cn2 = 0.f;
            if (g == 0) d2acc += finish_cluster<DT, V, VPL, SHIFT>(a, b, k, c0, r, acc, n, cold, cbi == 0, cn2);
            if (a.cprep) {  // mode 0, ncb == 1
                for (int off = 1; off < a.lanes; off <<= 1) cn2 += __shfl_xor(cn2, off);
                if (lane == 0) a.cnh[(size_t)b * a.KT * 32 + k] = refreshed_half_norm(a, cn2);
            }
        } else {
            const int slot = cin ? 0 : 1;
            if (g == 0) {
                float *dst = a.part + ((size_t)chunk * 2 + slot) * a.D;
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int e0 = c0 + (r + i * a.lanes) * V;
#pragma unroll
                    for (int e = 0; e < V; ++e)
                        if (e0 + e < a.D) rec_store(dst + e0 + e, acc[i][e]);
                }
            }
            if (slot == 0) k_in = k;
            else k_out = k;
        }
    };
    constexpr int U = upd_unroll<VPL>();

    while (!done) {
        // m == 0 is a normal case: a segment whose length is a multiple of 64 ends at a window
        // boundary, and the next view starts on the next segment's id
        const int m = run_len(p, sid, kraw, plim);
        // the rows' byte offsets in the problem (buffer path; a garbage index wraps within the
        // 32-bit offsets, and the range check keeps the load inside the problem's rows)
        if constexpr (BUF && V > 1) s_xo[wave][lane] = (uint32_t)idx * rowbytes;
        for (int base = 0; base < m; base += G * U) {
            if constexpr (V == 1) {
                float tmp[U][VPL][V];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int rr = base + u * G + g;
                    int row = __shfl(idx, rr & 63);
                    row = row < 0 ? 0 : (row >= N ? N - 1 : row);
                    load_row<DT, V, VPL>(a, (xb + row) * a.D, c0, r, tmp[u], rr < m);
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int i = 0; i < VPL; ++i) acc[i][0] += tmp[u][i][0];
            } else if constexpr (BUF) {
                // row group g takes the U consecutive positions base + g*U ...: their byte offsets
                // come from the wave's LDS row of offsets in one or two vector reads, then the
                // loads go out back to back
                uint32_t off[U];
                const int i0 = (base + g * U) & 63;  // a multiple of U; rows at or past m are masked
                if constexpr (U % 4 == 0) {
#pragma unroll
                    for (int q = 0; q < U / 4; ++q) {
                        const uint4 v4 = *(const uint4 *)&s_xo[wave][i0 + 4 * q];
                        off[4 * q] = v4.x;
                        off[4 * q + 1] = v4.y;
                        off[4 * q + 2] = v4.z;
                        off[4 * q + 3] = v4.w;
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) off[u] = s_xo[wave][i0 + u];
                }
#pragma unroll
                for (int u = 0; u < U; ++u) off[u] = base + g * U + u < m ? off[u] : x_end;
                uint4 raw[U][VPL];
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int i = 0; i < VPL; ++i) {
                        const int e0 = c0 + (r + i * a.lanes) * V;
                        const uint32_t o = e0 < a.D ? off[u] + (uint32_t)e0 * ES : x_end;
                        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
                        const v4u t = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)o, 0, 2 /* nt */);
                        raw[u][i] = make_uint4(t.x, t.y, t.z, t.w);
                    }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int i = 0; i < VPL; ++i) {
                        float fv[V];
                        widen16<DT>(raw[u][i], fv);
#pragma unroll
                        for (int e = 0; e < V; ++e) acc[i][e] += fv[e];
                    }
            } else {
                // keep the raw 16-byte vectors in flight; widen while accumulating
                uint4 raw[U][VPL];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int rr = base + u * G + g;
                    int row = __shfl(idx, rr & 63);
                    row = row < 0 ? 0 : (row >= N ? N - 1 : row);
                    const size_t e_row = (xb + row) * a.D;
#pragma unroll
                    for (int i = 0; i < VPL; ++i) {
                        const int e0 = c0 + (r + i * a.lanes) * V;
                        raw[u][i] = (rr < m && e0 < a.D)
                                        ? load16_nt((const char *)a.x + (e_row + e0) * (DT == DT_F32 ? 4 : 2))
                                        : make_uint4(0u, 0u, 0u, 0u);
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int i = 0; i < VPL; ++i) {
                        float fv[V];
                        widen16<DT>(raw[u][i], fv);
#pragma unroll
                        for (int e = 0; e < V; ++e) acc[i][e] += fv[e];
                    }
            }
        }
        const int next_k = __shfl(sid, m & 63);  // id at p + m (when m < 64)
        p += m;
        slide_if_past(p);
        bool ended = (m < 64) || (p >= plim);
        bool cout = false;
        if (p >= plim && plim == p1 && p1 < N && id_next == kraw) {
            // the segment runs past the chunk end: take all of it when it started in this chunk
            // and ends within the next one (the id after the next chunk differs, or there is
            // none); the walk then stops where the id changes
            if (!cin && (!next2_in || id_next2 != kraw)) {
                plim = next2_in ? p1 + a.R : N;
                ended = false;
            } else {
                cout = true;
            }
        }
        if (ended) {
            end_segment(kraw, p - seg_start, cout);
            // the chunk is done, or the segment taken past its end was (the walk stopped where
            // its id changed, short of the limit)
            if (p >= plim || plim != p1) break;
            kraw = next_k;
            fetch_cold(kraw);
            cin = false;
            seg_start = p;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
#pragma unroll
                for (int e = 0; e < V; ++e) acc[i][e] = 0.f;
        }
        view(p, sid, idx);
    }
    if (SHIFT) {  // mode 0
        double d = (double)d2acc;
        for (int off = 1; off < 64; off <<= 1) d += __shfl_xor(d, off);
        if (lane == 0) {
            a.shp[(size_t)chunk * (2 * a.ncb) + cbi] = d;
            // a long segment starting here has its shift written by the wave that finishes it
            if (k_out < 0) a.shp[(size_t)chunk * (2 * a.ncb) + a.ncb + cbi] = 0.0;
        }
    }
    if (k_in >= 0) arrive_long(a, b, c, cbi, k_in, lane);
    if (k_out >= 0) arrive_long(a, b, c, cbi, k_out, lane);
}

// After the accumulating update (streamed chunks, or the cosine fit): c_k <- sums_k / cnt_k
// where cnt_k > 0 (else keep), shift += ||c_new - c_old||^2, prepared centroids refreshed.
// With a.normalize (cosine k-means, the mean direction) c_k <- sums_k / ||sums_k|| (fp32 norm
// over the row, IEEE division), and a cluster whose sum is the zero vector keeps its centroid
// too.  One wave per cluster.
__global__ __launch_bounds__(256) void upd_finalize_acc_kernel(UpdArgs a, int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int b = (int)(row / a.K), k = (int)(row - (int64_t)b * a.K);
    const int n = a.cnt[row];
    const int D = a.D;
    float den = (float)n;
    if (a.normalize && n > 0) {
        float ss = 0.f;
        for (int d = lane; d < D; d += 64) {
            const float v = a.sums[row * D + d];
            ss += v * v;
        }
        for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
        den = sqrtf(ss);
    }
    if (n <= 0 || !(den > 0.f)) {  // wave-uniform: the centroid is kept
        if (lane == 0 && a.shp) a.shp[row] = 0.0;
        return;
    }
    float d2 = 0.f, cn2 = 0.f;
    for (int d = lane; d < D; d += 64) {
        const float old = a.C[row * D + d];
        const float nw = a.sums[row * D + d] / den;
        a.C[row * D + d] = nw;
        d2 += (nw - old) * (nw - old);
        if (a.cprep) cn2 += prep_store_elem(a, b, k, d, nw);
    }
    for (int off = 1; off < 64; off <<= 1) {
        d2 += __shfl_xor(d2, off);
        cn2 += __shfl_xor(cn2, off);
    }
    if (lane == 0 && a.shp) a.shp[row] = (double)d2;
    if (lane == 0 && a.cprep) a.cnh[(size_t)b * a.KT * 32 + k] = refreshed_half_norm(a, cn2);
}

// Update memory: the arrival counters (zero between launches), the segments' first positions
// and a scratch region for the partial records and shift partials.
size_t update_ctr_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    const UpdCfg u = plan_update(dt, B, N, D, K);
    const int64_t chunks = B * u.nch;
    return align256((size_t)chunks * 2 * u.ncb * 4) + align256((size_t)B * K * u.ncb * 4);
}

size_t update_scratch_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    const UpdCfg u = plan_update(dt, B, N, D, K);
    const int64_t chunks = B * u.nch;
    (void)K;
    return align256((size_t)chunks * 2 * u.ncb * 8) + align256((size_t)chunks * 2 * D * 4);
}

// A caller's update workspace: counters, first positions [B][K], scratch.
size_t update_ws_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    return update_ctr_bytes(dt, B, N, D, K) + align256((size_t)B * K * 4) + update_scratch_bytes(dt, B, N, D, K);
}

template <int DT, bool SHIFT>
static void launch_segsum_shift(const UpdArgs &a, int vec, int vpl, int64_t waves, hipStream_t s) {
    dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    constexpr int VV = DT == DT_F32 ? 4 : 8;
    // the buffer path needs each problem's rows within 2 GiB (offsets plus a vector never wrap)
    const bool buf = (int64_t)a.N * a.D * (DT == DT_F32 ? 4 : 2) <= ((int64_t)1 << 31);
    if (vec == 1) {
        if (vpl == 1) upd_segsum_kernel<DT, 1, 1, SHIFT, false><<<grid, block, 0, s>>>(a, waves);
        else if (vpl == 2) upd_segsum_kernel<DT, 1, 2, SHIFT, false><<<grid, block, 0, s>>>(a, waves);
        else upd_segsum_kernel<DT, 1, 4, SHIFT, false><<<grid, block, 0, s>>>(a, waves);
    } else if (buf) {
        if (vpl == 1) upd_segsum_kernel<DT, VV, 1, SHIFT, true><<<grid, block, 0, s>>>(a, waves);
        else if (vpl == 2) upd_segsum_kernel<DT, VV, 2, SHIFT, true><<<grid, block, 0, s>>>(a, waves);
        else upd_segsum_kernel<DT, VV, 4, SHIFT, true><<<grid, block, 0, s>>>(a, waves);
    } else {
        if (vpl == 1) upd_segsum_kernel<DT, VV, 1, SHIFT, false><<<grid, block, 0, s>>>(a, waves);
        else if (vpl == 2) upd_segsum_kernel<DT, VV, 2, SHIFT, false><<<grid, block, 0, s>>>(a, waves);
        else upd_segsum_kernel<DT, VV, 4, SHIFT, false><<<grid, block, 0, s>>>(a, waves);
    }
}

template <int DT>
static hipError_t launch_segsum_dt(const UpdArgs &a, int vec, int vpl, int64_t waves, hipStream_t s) {
    if (a.shp) launch_segsum_shift<DT, true>(a, vec, vpl, waves, s);
    else launch_segsum_shift<DT, false>(a, vec, vpl, waves, s);
    return hipGetLastError();
}

static UpdArgs make_args(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                         int B, int N, int D, int K, int mode, float *C, bool want_shift, float *sums, int32_t *cnt,
                         const UpdRefresh &ref, const UpdMem &mem) {
    const UpdCfg u = plan_update(dt, mem.plan_B > B ? mem.plan_B : B, N, D, K);
    const int64_t chunks = (int64_t)B * u.nch;
    char *wp = (char *)mem.scratch;
    UpdArgs a{};
    a.shp = (mode == 0 && want_shift) ? (double *)wp : nullptr;
    wp += align256((size_t)chunks * 2 * u.ncb * 8);
    a.part = (float *)wp;
    a.gcnt = mem.ctr;
    a.scnt = mem.ctr + align256((size_t)chunks * 2 * u.ncb * 4) / 4;
    a.offs = mem.offs;
    a.x = x;
    a.sids = sids;
    a.sidx = sidx;
    a.counts = counts;
    a.N = N;
    a.D = D;
    a.K = K;
    a.R = u.rows;
    a.nch = (int)u.nch;
    a.lanes = u.lanes;
    a.ncb = u.ncb;
    a.cb_elems = u.cb_elems;
    a.mode = mode;
    a.dt = dt;
    a.C = C;
    a.sums = sums;
    a.cnt = cnt;
    // the fused refresh needs one column block per row (each cluster finished by one lane group)
    a.cprep = (ref.cprep && u.ncb == 1) ? ref.cprep : nullptr;
    a.cnh = ref.cnh;
    a.DP = ref.DP;
    a.KT = ref.KT;
    a.zero_norm = ref.zero_norm;
    return a;
}

// (the column blocks do not depend on K)
bool update_refreshes_prep(int dt, int64_t B, int64_t N, int64_t D) { return plan_update(dt, B, N, D, 1).ncb == 1; }

// Before an update whose caller has no first positions from the arg-sort: each cluster's first
// sorted position (where the sorted id changes; clusters without points get none, and none is
// read for them), and the arrival counters set to zero.
__global__ __launch_bounds__(256) void upd_prologue_kernel(const int32_t *__restrict__ sids, int64_t total, int N,
                                                           int K, int32_t *__restrict__ offs,
                                                           int32_t *__restrict__ ctr, int64_t nctr) {
    const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = gi; i < nctr; i += stride) ctr[i] = 0;
    if (gi >= total) return;
    const int64_t b = gi / N;
    const int p = (int)(gi - b * N);
    const int32_t k = sids[gi];
    if (k < 0 || k >= K) return;
    if (p == 0 || sids[gi - 1] != k) offs[b * K + k] = p;
}

// The same from the counts when the cluster table is small next to the points: one workgroup per
// problem takes the exclusive scan of its counts (1024 at a time, carried), and every workgroup
// clears a share of the counters.
__global__ __launch_bounds__(256) void upd_prologue_counts_kernel(const int32_t *__restrict__ counts, int K,
                                                                  int32_t *__restrict__ offs,
                                                                  int32_t *__restrict__ ctr, int64_t nctr) {
    __shared__ int32_t s_w[4];
    __shared__ int32_t s_carry;
    const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
    for (int64_t i = (int64_t)b * 256 + t; i < nctr; i += (int64_t)gridDim.x * 256) ctr[i] = 0;
    const int32_t *cb = counts + (size_t)b * K;
    int32_t *ob = offs + (size_t)b * K;
    if (t == 0) s_carry = 0;
    __syncthreads();
    for (int k0 = 0; k0 < K; k0 += 1024) {
        int32_t v[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + 4 * t + i;
            v[i] = k < K ? cb[k] : 0;
            sum += v[i];
        }
        int32_t inc = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t o = __shfl_up(inc, off);
            if (lane >= off) inc += o;
        }
        if (lane == 63) s_w[w] = inc;
        __syncthreads();
        int32_t run = s_carry + inc - sum;
        for (int i = 0; i < w; ++i) run += s_w[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + 4 * t + i;
            if (k < K) ob[k] = run;
            run += v[i];
        }
        __syncthreads();
        if (t == 255) s_carry = run;
        __syncthreads();
    }
}

hipError_t launch_update_prologue(const int32_t *sids, const int32_t *counts, int B, int N, int K, int32_t *offs,
                                  int32_t *ctr, size_t ctr_bytes, hipStream_t s) {
    const int64_t total = (int64_t)B * N;
    const int64_t nctr = (int64_t)(ctr_bytes / 4);
    if ((int64_t)K * 64 <= N) {  // scanning K counts per problem is cheaper than reading N ids
        upd_prologue_counts_kernel<<<dim3((unsigned)B), dim3(256), 0, s>>>(counts, K, offs, ctr, nctr);
        return hipGetLastError();
    }
    const int64_t work = total > nctr ? total : nctr;
    const int64_t blocks = (work + 255) / 256 < 65536 ? (work + 255) / 256 : 65536;
    upd_prologue_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(sids, total, N, K, offs, ctr, nctr);
    return hipGetLastError();
}

// mode 0: in-core update of C; shift (optional, [B]) receives sum_k ||c_new - c_old||^2 in fp64,
// summed in a fixed order.  mode 1: accumulate into sums / cnt.  `ref` optionally names the
// prepared centroids to refresh.  mem: first positions (from the arg-sort or the prologue),
// zeroed counters (left zero) and scratch.
// normalize (mode 0, one column block per row): c_k <- s_k / ||s_k||, the cosine mean direction.
hipError_t launch_update(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                         int B, int N, int D, int K, int mode, float *C, double *shift, float *sums, int32_t *cnt,
                         const UpdRefresh &ref, const UpdMem &mem, hipStream_t s, int normalize) {
    const UpdCfg u = plan_update(dt, mem.plan_B > B ? mem.plan_B : B, N, D, K);
    const int64_t chunks = (int64_t)B * u.nch;
    if (normalize && (mode != 0 || u.ncb != 1)) return hipErrorInvalidValue;
    UpdArgs a = make_args(dt, x, sids, sidx, counts, B, N, D, K, mode, C, shift != nullptr, sums, cnt,
                          mode == 0 ? ref : UpdRefresh{}, mem);
    a.normalize = normalize;
    hipError_t e;
    const int64_t waves = chunks * u.ncb;
    if (dt == DT_F32) e = launch_segsum_dt<DT_F32>(a, u.vec, u.vpl, waves, s);
    else if (dt == DT_F16) e = launch_segsum_dt<DT_F16>(a, u.vec, u.vpl, waves, s);
    else e = launch_segsum_dt<DT_BF16>(a, u.vec, u.vpl, waves, s);
    if (e != hipSuccess || !a.shp) return e;
    return launch_sum_f64_rows(a.shp, B, u.nch * 2 * u.ncb, shift, s);
}

// A standalone update in a caller's workspace (update_ws_bytes): the prologue, then the update.
hipError_t launch_update_ws(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                            int B, int N, int D, int K, float *C, double *shift, void *ws, hipStream_t s) {
    const size_t cb = update_ctr_bytes(dt, B, N, D, K);
    char *wp = (char *)ws;
    UpdMem mem;
    mem.ctr = (int32_t *)wp;
    int32_t *offs = (int32_t *)(wp + cb);
    mem.offs = offs;
    mem.scratch = wp + cb + align256((size_t)B * K * 4);
    hipError_t e = launch_update_prologue(sids, counts, B, N, K, offs, mem.ctr, cb, s);
    if (e != hipSuccess) return e;
    return launch_update(dt, x, sids, sidx, counts, B, N, D, K, 0, C, shift, nullptr, nullptr, UpdRefresh{}, mem, s, 0);
}

// shk: [B][K] doubles of scratch for the per-cluster shifts (optional, with shift).
hipError_t launch_finalize_acc(int dt, const float *sums, const int32_t *cnt, float *C, double *shift, double *shk,
                               const UpdRefresh &ref, int B, int K, int D, hipStream_t s, int normalize) {
    UpdArgs a{};
    a.zero_norm = ref.zero_norm;
    a.normalize = normalize;
    a.dt = dt;
    a.D = D;
    a.K = K;
    a.C = C;
    a.shp = shift ? shk : nullptr;
    a.sums = (float *)sums;
    a.cnt = (int32_t *)cnt;
    a.cprep = ref.cprep;
    a.cnh = ref.cnh;
    a.DP = ref.DP;
    a.KT = ref.KT;
    const int64_t rows = (int64_t)B * K;
    upd_finalize_acc_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(a, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !shift) return e;
    return launch_sum_f64_rows(shk, B, K, shift, s);
}

}  // namespace fkm
