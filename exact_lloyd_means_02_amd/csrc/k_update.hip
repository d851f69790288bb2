// Sort-inverse update on gfx950 (paper summary, "Method"; paper digest, "方法步骤详情" step (2)):
// the sorted order is cut into chunks; each wave takes one chunk, walks its cluster-id
// segments, gathers the rows of the unpermuted x through sorted_idx, sums each segment on
// chip in fp32, and writes once per segment.  The digest issues one atomic per segment; here
// a segment that lies inside one chunk is finished by its wave (c_k = s_k / n_k written
// directly), and a segment cut by chunk edges leaves one fp32 partial per chunk that a
// second kernel adds in chunk order.  No float atomics, so the result is deterministic.
//
// Lane layout: a row is covered by `lanes` lanes (a power of two) holding 16-byte vectors
// (or scalars when D is not a multiple of the vector width); one wave load instruction
// therefore reads 64/lanes rows.  A window of 64 sorted positions is read with one
// coalesced load of ids and indices; the rows of the current segment inside the window are
// a prefix of it (ids are sorted), counted with one ballot.
#include "common.h"
#include "plan.h"

namespace fkm {

hipError_t launch_sum_f64_rows(const double *part, int rows, int64_t len, double *out, hipStream_t s);

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
    // mode 0: [B*nch][ncb + 1] (column block of a chunk's wave; last slot: the chunk's cut
    // segment, finished by the combine kernel); finalize: [B][K], one per cluster.
    double *shp;
    float *sums;       // [B][K][D] (mode 1)
    int32_t *cnt;      // [B][K]    (mode 1)
    float *part;       // [B*nch][2][D]
    int32_t *rec;      // [B*nch][4]: cluster of slot 0 (cut on entry), of slot 1 (cut on exit), start of slot 1
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

// SHIFT: a.shp is set (mode 0 with shift partials wanted); a separate instance keeps the
// register budget of the common case free of the old-centroid prefetch.
template <int DT, int V, int VPL, bool SHIFT>
__global__ __launch_bounds__(256) void upd_segsum_kernel(UpdArgs a, int64_t total_waves) {
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)xcd_remap_rev(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
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

    // Sorted ids / indices are read through a sliding window of 128 positions held in two
    // registers per lane ([wp, wp+64) and [wp+64, wp+128)); the next 64 are loaded as soon as
    // the walk passes wp+64, so that load overlaps the row gathers of the segments in between.
    int wp = p0, cs, ci, ns, ni;
    auto load_window = [&](int pos) {
        wp = pos;
        const int q0 = wp + lane, q1 = wp + 64 + lane;
        cs = q0 < N ? sb[q0] : -1;
        ci = q0 < N ? ib[q0] : 0;
        ns = q1 < N ? sb[q1] : -1;
        ni = q1 < N ? ib[q1] : 0;
    };
    auto slide_if_past = [&](int pos) {  // keep pos - wp < 64 (pos advanced by at most 64)
        if (pos - wp >= 64) {
            wp += 64;
            cs = ns;
            ci = ni;
            const int q1 = wp + 64 + lane;
            ns = q1 < N ? sb[q1] : -1;
            ni = q1 < N ? ib[q1] : 0;
        }
    };
    // the 64 positions from pos: lane l takes window slot pos - wp + l of the 128
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

    load_window(p0);
    int p = p0, plim = p1;
    int sid, idx;
    view(p, sid, idx);
    int kraw = __shfl(sid, 0);
    bool cin = p0 > 0 && sb[p0 - 1] == kraw;
    // Segment ownership: a segment that ends within the chunk after the one where it starts is
    // summed entirely by the wave of its first chunk (which runs past its chunk end for it);
    // only segments spanning three or more chunks leave partials for the combine kernel.  A
    // wave whose chunk starts inside a segment finds the segment's end from the ids alone and
    // its start from the count, and skips it when the previous chunk's wave owns it.
    bool done = false;
    if (cin) {
        int e = p;
        while (true) {
            const int m = run_len(e, sid, kraw, p1);
            e += m;
            slide_if_past(e);
            if (m < 64 || e >= p1) break;
            view(e, sid, idx);
        }
        const bool ends_here = e < p1 || p1 == N || sb[p1] != kraw;
        const int s_start = e - a.counts[(size_t)b * a.K + clampk(kraw)];
        if (ends_here && s_start >= p0 - a.R) {
            p = e;
            if (p >= p1) {
                done = true;
            } else {
                view(p, sid, idx);
                kraw = __shfl(sid, 0);
                cin = false;
            }
        } else {
            load_window(p0);  // shared segment: sum this chunk's part after all
            view(p, sid, idx);
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
    int rec0 = -1, rec1 = -1, recps = 0;
    float d2acc = 0.f;
    float acc[VPL][V];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[i][e] = 0.f;

    // The summed segment ends: add the row groups and finish the cluster, or leave a partial
    // for the combine kernel when the segment is cut by a chunk edge (cin / cout).
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
                        if (e0 + e < a.D) dst[e0 + e] = acc[i][e];
                }
            }
            if (slot == 0) rec0 = k; else { rec1 = k; recps = seg_start; }
        }
    };
    constexpr int U = upd_unroll<VPL>();

    while (!done) {
        // m == 0 is a normal case: a segment whose length is a multiple of 64 ends at a window
        // boundary, and the next view starts on the next segment's id
        const int m = run_len(p, sid, kraw, plim);
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
                                        ? *(const uint4 *)((const char *)a.x + (e_row + e0) * (DT == DT_F32 ? 4 : 2))
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
        if (p >= plim && plim == p1 && p1 < N && sb[p1] == kraw) {
            // the segment runs past the chunk end: take all of it when it ends within the
            // next chunk and started in this one
            const int e = seg_start + a.counts[(size_t)b * a.K + clampk(kraw)];
            if (!cin && e <= p1 + a.R) {
                plim = e;
                ended = false;
            } else {
                cout = true;
            }
        }
        if (ended) {
            end_segment(kraw, p - seg_start, cout);
            if (p >= plim) break;
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
        if (lane == 0) a.shp[(size_t)chunk * (a.ncb + 1) + cbi] = d;
    }
    if (cbi == 0 && lane == 0) {
        int32_t *rc = a.rec + chunk * 4;
        rc[0] = rec0;
        rc[1] = rec1;
        rc[2] = recps;
        rc[3] = 0;
    }
}

// Finish column d of cluster k of problem b from its sum `s`, within a combine kernel.
// den: n_k, or ||s_k|| with a.normalize (mode 0).
__device__ inline float combine_finish_col(const UpdArgs &a, int b, int k, size_t rowo, int d, float s, float den,
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

// Segments that span three or more chunks: add the chunk partials in chunk order and finish
// the cluster.  A workgroup covers COMBINE_CHUNKS consecutive chunks; their records are read
// at once (most chunks start no such segment).  A segment spread over at most 8 chunks is
// finished by one wave (lanes over columns, pieces in order); a longer one by the whole
// workgroup (piece groups x columns, fixed-order tree).  Deterministic either way.
constexpr int COMBINE_WAVE_MAX = 8;
constexpr int COMBINE_CHUNKS = 16;

__global__ __launch_bounds__(256) void upd_combine_kernel(UpdArgs a, int64_t nchunks) {
    __shared__ float s_red[256];
    __shared__ int s_kk[COMBINE_CHUNKS], s_np[COMBINE_CHUNKS], s_nk[COMBINE_CHUNKS];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t chunk0 = (int64_t)blockIdx.x * COMBINE_CHUNKS;
    if (t < COMBINE_CHUNKS) {
        int kv = -1, npv = 0, nkv = 1;
        const int64_t chunk = chunk0 + t;
        if (chunk < nchunks) {
            const int32_t *rc = a.rec + chunk * 4;
            const int k = rc[1];
            if (k >= 0) {
                const int b = (int)(chunk / a.nch);
                const int c = (int)(chunk - (int64_t)b * a.nch);
                int nk = a.counts[(size_t)b * a.K + k];
                nk = nk < 1 ? 1 : nk;
                int c_last = (int)(((int64_t)rc[2] + nk - 1) / a.R);
                c_last = c_last > a.nch - 1 ? a.nch - 1 : (c_last < c ? c : c_last);
                kv = k;
                npv = c_last - c + 1;
                nkv = nk;
            }
        }
        s_kk[t] = kv;
        s_np[t] = npv;
        s_nk[t] = nkv;
    }
    __syncthreads();
    const int D = a.D;
    // long segments: the whole workgroup
    for (int i = 0; i < COMBINE_CHUNKS; ++i) {
        const int kk = s_kk[i], np = s_np[i], nkk = s_nk[i];
        if (kk < 0 || np <= COMBINE_WAVE_MAX) continue;  // uniform over the workgroup
        const int64_t chunk = chunk0 + i;
        const int b = (int)(chunk / a.nch);
        const size_t rowo = ((size_t)b * a.K + kk) * D;
        int DC = 1;
        while (DC < D && DC < 256) DC <<= 1;
        const int PG = 256 / DC;
        const int pg = t / DC, dcol = t - pg * DC;
        // column d's sum over the pieces, left in s_red[dcol] (fixed-order tree; every thread calls)
        auto column_sum = [&](int d) {
            float sum = 0.f;
            if (d < D) {
                // pieces pg, pg + PG, ... in order; eight loads in flight before they are added
                int j = pg;
                for (; j + 7 * PG < np; j += 8 * PG) {
                    float pv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int jj = j + u * PG;
                        pv[u] = a.part[((size_t)(chunk + jj) * 2 + (jj == 0 ? 1 : 0)) * D + d];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) sum += pv[u];
                }
                for (; j < np; j += PG) sum += a.part[((size_t)(chunk + j) * 2 + (j == 0 ? 1 : 0)) * D + d];
            }
            s_red[t] = sum;
            __syncthreads();
            for (int off = PG / 2; off >= 1; off >>= 1) {
                if (pg < off) s_red[t] += s_red[t + off * DC];
                __syncthreads();
            }
        };
        const int dend = ((D + DC - 1) / DC) * DC;
        float den = (float)nkk;
        if (a.mode == 0 && a.normalize) {
            // the mean direction needs ||s|| first: one pass for the norm, then the same sums again
            float ss = 0.f;
            for (int d = dcol; d < dend; d += DC) {
                column_sum(d);
                if (pg == 0 && d < D) ss += s_red[dcol] * s_red[dcol];
                __syncthreads();
            }
            s_red[t] = ss;
            __syncthreads();
            for (int off = 128; off >= 1; off >>= 1) {
                if (t < off) s_red[t] += s_red[t + off];
                __syncthreads();
            }
            den = sqrtf(s_red[0]);
            __syncthreads();
            if (!(den > 0.f)) {  // uniform: the zero sum keeps the centroid
                if (t == 0 && a.shp) a.shp[(size_t)chunk * (a.ncb + 1) + a.ncb] = 0.0;
                continue;
            }
        }
        float d2 = 0.f, cn2 = 0.f;
        for (int d = dcol; d < dend; d += DC) {
            column_sum(d);
            if (pg == 0 && d < D) d2 += combine_finish_col(a, b, kk, rowo, d, s_red[dcol], den, cn2);
            __syncthreads();
        }
        if (a.mode == 0) {
            s_red[t] = d2;
            __syncthreads();
            for (int off = 128; off >= 1; off >>= 1) {
                if (t < off) s_red[t] += s_red[t + off];
                __syncthreads();
            }
            if (t == 0 && a.shp) a.shp[(size_t)chunk * (a.ncb + 1) + a.ncb] = (double)s_red[0];
            __syncthreads();
            s_red[t] = cn2;
            __syncthreads();
            for (int off = 128; off >= 1; off >>= 1) {
                if (t < off) s_red[t] += s_red[t + off];
                __syncthreads();
            }
            if (t == 0 && a.cprep) a.cnh[(size_t)b * a.KT * 32 + kk] = refreshed_half_norm(a, s_red[0]);
            __syncthreads();
        } else if (t == 0) {
            a.cnt[(size_t)b * a.K + kk] += nkk;
        }
    }
    // short segments (and the shift slot of every chunk): one wave each
    for (int i = w; i < COMBINE_CHUNKS; i += 4) {  // 4 waves per workgroup
        const int64_t chunk = chunk0 + i;
        if (chunk >= nchunks) break;
        const int kk = s_kk[i], np = s_np[i], nkk = s_nk[i];
        if (kk < 0) {
            if (a.shp && lane == 0) a.shp[(size_t)chunk * (a.ncb + 1) + a.ncb] = 0.0;
            continue;
        }
        if (np > COMBINE_WAVE_MAX) continue;
        const int b = (int)(chunk / a.nch);
        const size_t rowo = ((size_t)b * a.K + kk) * D;
        // column d's sum over the pieces, in chunk order; every piece is loaded before the sum
        auto column_sum = [&](int d) {
            float pv[COMBINE_WAVE_MAX];
            pv[0] = a.part[((size_t)chunk * 2 + 1) * D + d];
#pragma unroll
            for (int j = 1; j < COMBINE_WAVE_MAX; ++j)
                pv[j] = j < np ? a.part[((size_t)(chunk + j) * 2) * D + d] : 0.f;
            float sum = pv[0];
#pragma unroll
            for (int j = 1; j < COMBINE_WAVE_MAX; ++j)
                if (j < np) sum += pv[j];
            return sum;
        };
        float den = (float)nkk;
        if (a.mode == 0 && a.normalize) {
            float ss = 0.f;
            for (int d = lane; d < D; d += 64) {
                const float sum = column_sum(d);
                ss += sum * sum;
            }
            for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
            den = sqrtf(ss);
            if (!(den > 0.f)) {  // uniform: the zero sum keeps the centroid
                if (lane == 0 && a.shp) a.shp[(size_t)chunk * (a.ncb + 1) + a.ncb] = 0.0;
                continue;
            }
        }
        float d2 = 0.f, cn2 = 0.f;
        for (int d = lane; d < D; d += 64) d2 += combine_finish_col(a, b, kk, rowo, d, column_sum(d), den, cn2);
        if (a.mode == 0) {
            for (int off = 1; off < 64; off <<= 1) {
                d2 += __shfl_xor(d2, off);
                cn2 += __shfl_xor(cn2, off);
            }
            if (lane == 0 && a.shp) a.shp[(size_t)chunk * (a.ncb + 1) + a.ncb] = (double)d2;
            if (lane == 0 && a.cprep) a.cnh[(size_t)b * a.KT * 32 + kk] = refreshed_half_norm(a, cn2);
        } else if (lane == 0) {
            a.cnt[(size_t)b * a.K + kk] += nkk;
        }
    }
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

size_t update_ws_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    const UpdCfg u = plan_update(dt, B, N, D);
    const int64_t chunks = B * u.nch;
    (void)K;
    return align256((size_t)chunks * 2 * D * 4) + align256((size_t)chunks * 4 * 4) +
           align256((size_t)chunks * (u.ncb + 1) * 8);
}

template <int DT, bool SHIFT>
static void launch_segsum_shift(const UpdArgs &a, int vec, int vpl, int64_t waves, hipStream_t s) {
    dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    constexpr int VV = DT == DT_F32 ? 4 : 8;
    if (vec == 1) {
        if (vpl == 1) upd_segsum_kernel<DT, 1, 1, SHIFT><<<grid, block, 0, s>>>(a, waves);
        else if (vpl == 2) upd_segsum_kernel<DT, 1, 2, SHIFT><<<grid, block, 0, s>>>(a, waves);
        else upd_segsum_kernel<DT, 1, 4, SHIFT><<<grid, block, 0, s>>>(a, waves);
    } else {
        if (vpl == 1) upd_segsum_kernel<DT, VV, 1, SHIFT><<<grid, block, 0, s>>>(a, waves);
        else if (vpl == 2) upd_segsum_kernel<DT, VV, 2, SHIFT><<<grid, block, 0, s>>>(a, waves);
        else upd_segsum_kernel<DT, VV, 4, SHIFT><<<grid, block, 0, s>>>(a, waves);
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
                         const UpdRefresh &ref, void *ws) {
    const UpdCfg u = plan_update(dt, B, N, D);
    const int64_t chunks = (int64_t)B * u.nch;
    char *wp = (char *)ws;
    UpdArgs a{};
    a.part = (float *)wp;
    wp += align256((size_t)chunks * 2 * D * 4);
    a.rec = (int32_t *)wp;
    wp += align256((size_t)chunks * 4 * 4);
    a.shp = (mode == 0 && want_shift) ? (double *)wp : nullptr;
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

bool update_refreshes_prep(int dt, int64_t B, int64_t N, int64_t D) { return plan_update(dt, B, N, D).ncb == 1; }

// mode 0: in-core update of C; shift (optional, [B]) receives sum_k ||c_new - c_old||^2 in fp64,
// summed in a fixed order.  mode 1: accumulate into sums / cnt.  `ref` optionally names the
// prepared centroids to refresh.
// normalize (mode 0, one column block per row): c_k <- s_k / ||s_k||, the cosine mean direction.
hipError_t launch_update(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                         int B, int N, int D, int K, int mode, float *C, double *shift, float *sums, int32_t *cnt,
                         const UpdRefresh &ref, void *ws, hipStream_t s, int normalize) {
    const UpdCfg u = plan_update(dt, B, N, D);
    const int64_t chunks = (int64_t)B * u.nch;
    if (normalize && (mode != 0 || u.ncb != 1)) return hipErrorInvalidValue;
    UpdArgs a = make_args(dt, x, sids, sidx, counts, B, N, D, K, mode, C, shift != nullptr, sums, cnt,
                          mode == 0 ? ref : UpdRefresh{}, ws);
    a.normalize = normalize;
    hipError_t e;
    const int64_t waves = chunks * u.ncb;
    if (dt == DT_F32) e = launch_segsum_dt<DT_F32>(a, u.vec, u.vpl, waves, s);
    else if (dt == DT_F16) e = launch_segsum_dt<DT_F16>(a, u.vec, u.vpl, waves, s);
    else e = launch_segsum_dt<DT_BF16>(a, u.vec, u.vpl, waves, s);
    if (e != hipSuccess) return e;
    upd_combine_kernel<<<dim3((unsigned)((chunks + COMBINE_CHUNKS - 1) / COMBINE_CHUNKS)), dim3(256), 0, s>>>(a, chunks);
    e = hipGetLastError();
    if (e != hipSuccess || !a.shp) return e;
    return launch_sum_f64_rows(a.shp, B, u.nch * (u.ncb + 1), shift, s);
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
