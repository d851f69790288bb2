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

constexpr int UPD_UNROLL = 4;

struct UpdArgs {
    const void *x;
    const int32_t *sids, *sidx, *counts;
    int N, D, K, R, nch, lanes, ncb, cb_elems;
    int mode;          // 0: finish c_k in place; 1: accumulate into sums / cnt (streamed chunks)
    float *C;          // [B][K][D] in/out (mode 0)
    float *shiftk;     // [B][ncb][K] (mode 0; zeroed by the caller)
    float *sums;       // [B][K][D] (mode 1)
    int32_t *cnt;      // [B][K]    (mode 1)
    float *part;       // [B*nch][2][D]
    int32_t *rec;      // [B*nch][4]: cluster of slot 0 (cut on entry), of slot 1 (cut on exit), start of slot 1
};

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
// mode 0: c_k <- s / n (fp32, IEEE division), shift_k contribution = sum (c_new - c_old)^2.
// mode 1: sums_k += s, cnt_k += n.
template <int V, int VPL>
__device__ inline float finish_cluster(const UpdArgs &a, int b, int k, int c0, int r, const float (&s)[VPL][V], int n,
                                       bool write_cnt) {
    float d2 = 0.f;
    const size_t rowo = ((size_t)b * a.K + k) * a.D;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e0 = c0 + (r + i * a.lanes) * V;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const int d = e0 + e;
            if (d < a.D) {
                if (a.mode == 0) {
                    const float old = a.C[rowo + d];
                    const float nw = s[i][e] / (float)n;
                    a.C[rowo + d] = nw;
                    const float df = nw - old;
                    d2 += df * df;
                } else {
                    a.sums[rowo + d] += s[i][e];
                }
            }
        }
    }
    if (a.mode == 1 && write_cnt && r == 0) a.cnt[(size_t)b * a.K + k] += n;
    return d2;
}

template <int DT, int V, int VPL>
__global__ __launch_bounds__(256) void upd_segsum_kernel(UpdArgs a, int64_t total_waves) {
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
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

    int p = p0;
    int kraw = sb[p0];
    bool cin = p0 > 0 && sb[p0 - 1] == kraw;
    int seg_start = p0;
    int rec0 = -1, rec1 = -1, recps = 0;
    float acc[VPL][V];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[i][e] = 0.f;

    while (true) {
        const int pos = p + lane;
        const bool have = pos < p1;
        const int sid = have ? sb[pos] : -1;
        const int idx = have ? ib[pos] : 0;
        const uint64_t eq = __ballot(have && sid == kraw);
        const int m = (~eq == 0ull) ? 64 : (int)__builtin_ctzll(~eq);
        for (int base = 0; base < m; base += G * UPD_UNROLL) {
            float tmp[UPD_UNROLL][VPL][V];
#pragma unroll
            for (int u = 0; u < UPD_UNROLL; ++u) {
                const int rr = base + u * G + g;
                const bool ok = rr < m;
                int row = __shfl(idx, rr & 63);
                row = row < 0 ? 0 : (row >= N ? N - 1 : row);
                load_row<DT, V, VPL>(a, (xb + row) * a.D, c0, r, tmp[u], ok);
            }
#pragma unroll
            for (int u = 0; u < UPD_UNROLL; ++u)
#pragma unroll
                for (int i = 0; i < VPL; ++i)
#pragma unroll
                    for (int e = 0; e < V; ++e) acc[i][e] += tmp[u][i][e];
        }
        p += m;
        const bool ended = (m < 64) || (p >= p1);
        if (ended) {
            // sum the row groups: lanes r, r + lanes, r + 2*lanes, ... hold the same columns
            for (int off = a.lanes; off < 64; off <<= 1) {
#pragma unroll
                for (int i = 0; i < VPL; ++i)
#pragma unroll
                    for (int e = 0; e < V; ++e) acc[i][e] += __shfl_xor(acc[i][e], off);
            }
            const int k = kraw < 0 ? 0 : (kraw >= a.K ? a.K - 1 : kraw);
            const bool cout = (p >= p1) && (p1 < N) && (sb[p1] == kraw);
            const int n = p - seg_start;
            if (!cin && !cout) {
                float d2 = 0.f;
                if (g == 0) d2 = finish_cluster<V, VPL>(a, b, k, c0, r, acc, n, cbi == 0);
                if (a.mode == 0) {
                    for (int off = 1; off < a.lanes; off <<= 1) d2 += __shfl_xor(d2, off);
                    if (lane == 0) a.shiftk[((size_t)b * a.ncb + cbi) * a.K + k] = d2;
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
            if (p >= p1) break;
            kraw = __shfl(sid, m & 63);
            cin = false;
            seg_start = p;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
#pragma unroll
                for (int e = 0; e < V; ++e) acc[i][e] = 0.f;
        }
    }
    if (cbi == 0 && lane == 0) {
        int32_t *rc = a.rec + chunk * 4;
        rc[0] = rec0;
        rc[1] = rec1;
        rc[2] = recps;
        rc[3] = 0;
    }
}

// One workgroup per chunk: if a segment starts in this chunk and runs past its end, add the
// chunk partials of that segment in chunk order and finish the cluster.
__global__ __launch_bounds__(256) void upd_combine_kernel(UpdArgs a) {
    __shared__ float s_red[256];
    const int64_t chunk = blockIdx.x;
    const int32_t *rc = a.rec + chunk * 4;
    const int k = rc[1];
    if (k < 0) return;
    const int b = (int)(chunk / a.nch);
    const int c = (int)(chunk - (int64_t)b * a.nch);
    const int ps = rc[2];
    int nk = a.counts[(size_t)b * a.K + k];
    if (nk < 1) nk = 1;
    int c_last = (int)(((int64_t)ps + nk - 1) / a.R);
    if (c_last > a.nch - 1) c_last = a.nch - 1;
    if (c_last < c) c_last = c;
    const int npieces = c_last - c + 1;
    const int D = a.D;
    // threads = PG piece groups x DC columns
    int DC = 1;
    while (DC < D && DC < 256) DC <<= 1;
    const int PG = 256 / DC;
    const int t = threadIdx.x, pg = t / DC, dcol = t - pg * DC;
    const size_t rowo = ((size_t)b * a.K + k) * D;
    float d2 = 0.f;
    for (int d = dcol; d < ((D + DC - 1) / DC) * DC; d += DC) {
        float sum = 0.f;
        if (d < D) {
            for (int j = pg; j < npieces; j += PG) {
                const int slot = j == 0 ? 1 : 0;
                sum += a.part[((size_t)(chunk + j) * 2 + slot) * D + d];
            }
        }
        s_red[t] = sum;
        __syncthreads();
        for (int off = PG / 2; off >= 1; off >>= 1) {
            if (pg < off) s_red[t] += s_red[t + off * DC];
            __syncthreads();
        }
        if (pg == 0 && d < D) {
            const float s = s_red[dcol];
            if (a.mode == 0) {
                const float old = a.C[rowo + d];
                const float nw = s / (float)nk;
                a.C[rowo + d] = nw;
                d2 += (nw - old) * (nw - old);
            } else {
                a.sums[rowo + d] += s;
            }
        }
        __syncthreads();
    }
    if (a.mode == 0) {
        s_red[t] = pg == 0 ? d2 : 0.f;
        __syncthreads();
        for (int off = 128; off >= 1; off >>= 1) {
            if (t < off) s_red[t] += s_red[t + off];
            __syncthreads();
        }
        if (t == 0) a.shiftk[((size_t)b * a.ncb) * a.K + k] = s_red[0];
    } else if (t == 0) {
        a.cnt[(size_t)b * a.K + k] += a.counts[(size_t)b * a.K + k];
    }
}

// Streamed path, after the last chunk: c_k <- sums_k / cnt_k where cnt_k > 0 (else keep),
// shift_k = ||c_new - c_old||^2.  One wave per cluster.
__global__ __launch_bounds__(256) void upd_finalize_acc_kernel(const float *__restrict__ sums,
                                                               const int32_t *__restrict__ cnt, float *__restrict__ C,
                                                               float *__restrict__ shiftk, int64_t rows, int D) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int n = cnt[row];
    float d2 = 0.f;
    if (n > 0) {
        for (int d = lane; d < D; d += 64) {
            const float old = C[row * D + d];
            const float nw = sums[row * D + d] / (float)n;
            C[row * D + d] = nw;
            d2 += (nw - old) * (nw - old);
        }
    }
    for (int off = 1; off < 64; off <<= 1) d2 += __shfl_xor(d2, off);
    if (lane == 0) shiftk[row] = d2;
}

size_t update_ws_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    const UpdCfg u = plan_update(dt, B, N, D);
    const int64_t chunks = B * u.nch;
    return align256((size_t)chunks * 2 * D * 4) + align256((size_t)chunks * 4 * 4) +
           align256((size_t)B * u.ncb * K * 4);
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);

template <int DT>
static hipError_t launch_segsum_dt(const UpdArgs &a, int vec, int vpl, int64_t waves, hipStream_t s) {
    dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    constexpr int VV = DT == DT_F32 ? 4 : 8;
    if (vec == 1) {
        if (vpl == 1) upd_segsum_kernel<DT, 1, 1><<<grid, block, 0, s>>>(a, waves);
        else if (vpl == 2) upd_segsum_kernel<DT, 1, 2><<<grid, block, 0, s>>>(a, waves);
        else upd_segsum_kernel<DT, 1, 4><<<grid, block, 0, s>>>(a, waves);
    } else {
        if (vpl == 1) upd_segsum_kernel<DT, VV, 1><<<grid, block, 0, s>>>(a, waves);
        else if (vpl == 2) upd_segsum_kernel<DT, VV, 2><<<grid, block, 0, s>>>(a, waves);
        else upd_segsum_kernel<DT, VV, 4><<<grid, block, 0, s>>>(a, waves);
    }
    return hipGetLastError();
}

// mode 0: in-core update of C (shiftk gets per-cluster shifts); mode 1: accumulate into sums / cnt.
hipError_t launch_update(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                         int B, int N, int D, int K, int mode, float *C, float *sums, int32_t *cnt, void *ws,
                         float **shiftk_out, int *ncb_out, hipStream_t s) {
    const UpdCfg u = plan_update(dt, B, N, D);
    const int64_t chunks = (int64_t)B * u.nch;
    char *wp = (char *)ws;
    float *part = (float *)wp;
    wp += align256((size_t)chunks * 2 * D * 4);
    int32_t *rec = (int32_t *)wp;
    wp += align256((size_t)chunks * 4 * 4);
    float *shiftk = (float *)wp;
    if (shiftk_out) *shiftk_out = shiftk;
    if (ncb_out) *ncb_out = u.ncb;
    UpdArgs a;
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
    a.C = C;
    a.shiftk = shiftk;
    a.sums = sums;
    a.cnt = cnt;
    a.part = part;
    a.rec = rec;
    hipError_t e;
    if (mode == 0) {
        e = launch_fill_i32((int32_t *)shiftk, (int64_t)B * u.ncb * K, 0, s);  // 0.0f has all-zero bits
        if (e != hipSuccess) return e;
    }
    const int64_t waves = chunks * u.ncb;
    if (dt == DT_F32) e = launch_segsum_dt<DT_F32>(a, u.vec, u.vpl, waves, s);
    else if (dt == DT_F16) e = launch_segsum_dt<DT_F16>(a, u.vec, u.vpl, waves, s);
    else e = launch_segsum_dt<DT_BF16>(a, u.vec, u.vpl, waves, s);
    if (e != hipSuccess) return e;
    upd_combine_kernel<<<dim3((unsigned)chunks), dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_finalize_acc(const float *sums, const int32_t *cnt, float *C, float *shiftk, int B, int K, int D,
                               hipStream_t s) {
    const int64_t rows = (int64_t)B * K;
    upd_finalize_acc_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(sums, cnt, C, shiftk, rows, D);
    return hipGetLastError();
}

}  // namespace fkm
