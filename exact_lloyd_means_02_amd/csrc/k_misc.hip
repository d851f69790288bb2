// Row norms (paper digest, "方法步骤详情" step (1): ||x_i||^2 precomputed before the centroid
// scan) and the fp64 reductions behind the loop control (inertia and centroid shift).
#include "common.h"
#include "plan.h"

namespace fkm {

// One row per `lanes` lanes; each lane sums squares of 16-byte vectors (or scalars) of the row
// in fp32, then a butterfly over the row's lanes.  Rows are dispatched in waves of 64/lanes.
template <int DT, int V>
__global__ __launch_bounds__(256) void row_norms_kernel(const void *__restrict__ x, float *__restrict__ out,
                                                        int64_t rows, int D, int lanes) {
    const int lane = threadIdx.x & 63;
    const int G = 64 / lanes;
    const int g = lane / lanes, r = lane - g * lanes;
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * G + g;
    const bool ok = row < rows;
    const size_t e0 = (size_t)(ok ? row : 0) * D;
    float s = 0.f;
    if (ok) {
        if constexpr (V == 1) {
            for (int d = r; d < D; d += lanes) {
                const float v = load_elem<DT>(x, e0 + d);
                s += v * v;
            }
        } else {
            constexpr int S = DT == DT_F32 ? 4 : 2;
            for (int d = r * V; d < D; d += lanes * V) {
                const uint4 u = *(const uint4 *)((const char *)x + (e0 + d) * S);
                float f[V];
                widen16<DT>(u, f);
#pragma unroll
                for (int e = 0; e < V; ++e) s += f[e] * f[e];
            }
        }
    }
    for (int off = 1; off < lanes; off <<= 1) s += __shfl_xor(s, off);
    if (ok && r == 0) out[row] = s;
}

// Rows of at most 64 16-byte vectors (D * s <= 1 KiB, D a multiple of the vector width): a
// row takes `lanes` lanes with one vector each, and a wave takes ROW_STEPS groups of 64/lanes
// rows, all of whose loads are issued before the first is used (4 loads in flight per lane).
// NORMALIZE = false: out (float*) = ||x_i||^2.  NORMALIZE = true: out (dtype) =
// dtype(x_i / ||x_i||), from the vector already in registers (out may alias x).
constexpr int ROW_STEPS = 4;

template <int DT, bool NORMALIZE>
__global__ __launch_bounds__(256) void rows_short_kernel(const void *x, void *out, int64_t rows, int D, int lanes) {
    constexpr int S = DT == DT_F32 ? 4 : 2;
    constexpr int V = 16 / S;
    const int lane = threadIdx.x & 63;
    const int G = 64 / lanes;
    const int g = lane / lanes, r = lane - g * lanes;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool has_vec = r * V < D;
    uint4 u[ROW_STEPS];
#pragma unroll
    for (int st = 0; st < ROW_STEPS; ++st) {
        const int64_t row = (wave * ROW_STEPS + st) * G + g;
        u[st] = make_uint4(0u, 0u, 0u, 0u);
        if (row < rows && has_vec) u[st] = *(const uint4 *)((const char *)x + ((size_t)row * D + r * V) * S);
    }
#pragma unroll
    for (int st = 0; st < ROW_STEPS; ++st) {
        const int64_t row = (wave * ROW_STEPS + st) * G + g;
        float f[V];
        widen16<DT>(u[st], f);
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) sq += f[e] * f[e];
        for (int off = 1; off < lanes; off <<= 1) sq += __shfl_xor(sq, off);
        if (row >= rows) continue;
        if constexpr (!NORMALIZE) {
            if (r == 0) ((float *)out)[row] = sq;
        } else {
            if (!has_vec) continue;
            const float n = sqrtf(sq);
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < V; ++e) f[e] = n > 0.f ? f[e] / n : 0.f;
            if constexpr (DT == DT_F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(f[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = DT == DT_F16 ? f32_to_f16_bits(f[2 * e]) : f32_to_bf16_bits(f[2 * e]);
                    const uint32_t hi = DT == DT_F16 ? f32_to_f16_bits(f[2 * e + 1]) : f32_to_bf16_bits(f[2 * e + 1]);
                    w[e] = (lo & 0xFFFFu) | ((hi & 0xFFFFu) << 16);
                }
            }
            *(uint4 *)((char *)out + ((size_t)row * D + r * V) * S) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// Launches rows_short_kernel when the row fits (returns true), else leaves it to the caller.
template <bool NORMALIZE>
static bool launch_rows_short(int dt, const void *x, void *out, int64_t rows, int D, hipStream_t s, hipError_t *err) {
    const int v16 = dt == DT_F32 ? 4 : 8;
    if (D % v16 != 0 || D / v16 > 64) return false;
    const int nvec = D / v16;
    int lanes = 1;
    while (lanes < nvec) lanes <<= 1;
    const int64_t per_wave = (int64_t)ROW_STEPS * (64 / lanes);
    const int64_t waves = (rows + per_wave - 1) / per_wave;
    dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (dt == DT_F32) rows_short_kernel<DT_F32, NORMALIZE><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    else if (dt == DT_F16) rows_short_kernel<DT_F16, NORMALIZE><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    else rows_short_kernel<DT_BF16, NORMALIZE><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    *err = hipGetLastError();
    return true;
}

hipError_t launch_row_norms(int dt, const void *x, float *out, int64_t rows, int D, hipStream_t s) {
    hipError_t err;
    if (launch_rows_short<false>(dt, x, out, rows, D, s, &err)) return err;
    const int v16 = dt == DT_F32 ? 4 : 8;
    const bool vec = (D % v16) == 0;
    const int nvec = vec ? D / v16 : D;
    int lanes = 1;
    while (lanes < nvec && lanes < 64) lanes <<= 1;
    const int G = 64 / lanes;
    const int64_t waves = (rows + G - 1) / G;
    dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (dt == DT_F32) {
        if (vec) row_norms_kernel<DT_F32, 4><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
        else row_norms_kernel<DT_F32, 1><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    } else if (dt == DT_F16) {
        if (vec) row_norms_kernel<DT_F16, 8><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
        else row_norms_kernel<DT_F16, 1><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    } else {
        if (vec) row_norms_kernel<DT_BF16, 8><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
        else row_norms_kernel<DT_BF16, 1><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Unit rows for cosine k-means (the project README, "CuTe backend", names cosine k-means as a
// mode; spherical k-means works on x / ||x||): out_i = dtype(x_i / ||x_i||), the norm summed
// in fp32 over the row's lanes as in row_norms_kernel, each element divided by it (IEEE fp32
// division) and rounded to the storage dtype (nearest even).  A zero row stays zero.  The
// lane layout is row_norms_kernel's; every lane reads its own elements again for the quotient
// and writes only those, so `out` may alias `x`.
// ------------------------------------------------------------------------------------------
template <int DT>
__device__ inline void store_elem(void *base, size_t i, float v) {
    if constexpr (DT == DT_F32) {
        ((float *)base)[i] = v;
    } else if constexpr (DT == DT_F16) {
        ((uint16_t *)base)[i] = (uint16_t)f32_to_f16_bits(v);
    } else {
        ((uint16_t *)base)[i] = (uint16_t)f32_to_bf16_bits(v);
    }
}

template <int DT, int V>
__global__ __launch_bounds__(256) void normalize_rows_kernel(const void *x, void *out, int64_t rows, int D,
                                                             int lanes) {
    constexpr int S = DT == DT_F32 ? 4 : 2;
    const int lane = threadIdx.x & 63;
    const int G = 64 / lanes;
    const int g = lane / lanes, r = lane - g * lanes;
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * G + g;
    const bool ok = row < rows;
    const size_t e0 = (size_t)(ok ? row : 0) * D;
    float s = 0.f;
    if (ok) {
        if constexpr (V == 1) {
            for (int d = r; d < D; d += lanes) {
                const float v = load_elem<DT>(x, e0 + d);
                s += v * v;
            }
        } else {
            for (int d = r * V; d < D; d += lanes * V) {
                const uint4 u = *(const uint4 *)((const char *)x + (e0 + d) * S);
                float f[V];
                widen16<DT>(u, f);
#pragma unroll
                for (int e = 0; e < V; ++e) s += f[e] * f[e];
            }
        }
    }
    for (int off = 1; off < lanes; off <<= 1) s += __shfl_xor(s, off);
    const float n = sqrtf(s);
    if (!ok) return;
    if constexpr (V == 1) {
        for (int d = r; d < D; d += lanes) {
            const float v = load_elem<DT>(x, e0 + d);
            store_elem<DT>(out, e0 + d, n > 0.f ? v / n : 0.f);
        }
    } else {
        for (int d = r * V; d < D; d += lanes * V) {
            const uint4 u = *(const uint4 *)((const char *)x + (e0 + d) * S);
            float f[V];
            widen16<DT>(u, f);
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < V; ++e) f[e] = n > 0.f ? f[e] / n : 0.f;
            if constexpr (DT == DT_F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(f[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = DT == DT_F16 ? f32_to_f16_bits(f[2 * e]) : f32_to_bf16_bits(f[2 * e]);
                    const uint32_t hi = DT == DT_F16 ? f32_to_f16_bits(f[2 * e + 1]) : f32_to_bf16_bits(f[2 * e + 1]);
                    w[e] = (lo & 0xFFFFu) | ((hi & 0xFFFFu) << 16);
                }
            }
            *(uint4 *)((char *)out + (e0 + d) * S) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

hipError_t launch_normalize_rows(int dt, const void *x, void *out, int64_t rows, int D, hipStream_t s) {
    hipError_t err;
    if (launch_rows_short<true>(dt, x, out, rows, D, s, &err)) return err;
    const int v16 = dt == DT_F32 ? 4 : 8;
    const bool vec = (D % v16) == 0;
    const int nvec = vec ? D / v16 : D;
    int lanes = 1;
    while (lanes < nvec && lanes < 64) lanes <<= 1;
    const int G = 64 / lanes;
    const int64_t waves = (rows + G - 1) / G;
    dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (dt == DT_F32) {
        if (vec) normalize_rows_kernel<DT_F32, 4><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
        else normalize_rows_kernel<DT_F32, 1><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    } else if (dt == DT_F16) {
        if (vec) normalize_rows_kernel<DT_F16, 8><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
        else normalize_rows_kernel<DT_F16, 1><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    } else {
        if (vec) normalize_rows_kernel<DT_BF16, 8><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
        else normalize_rows_kernel<DT_BF16, 1><<<grid, block, 0, s>>>(x, out, rows, D, lanes);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Deterministic fp64 sums of partials, one row per workgroup in a fixed order.
// ------------------------------------------------------------------------------------------
// out[r] = sum_j part[r * len + j] (fp64), one workgroup per row, fixed order; with accumulate,
// out[r] += that sum.  Rows run to a few hundred thousand partials (one per assign wave of a
// 2^24-point problem), so each thread keeps SUM_U independent loads in flight (a strided slot
// each: thread t, slot u reads j = t + T (U i + u)) and adds them into SUM_U accumulators; the
// accumulators, then the threads, are added in a fixed tree.  With one load in flight per thread a
// 262144-partial row took about 400 us (latency-bound).  Long rows take T = 1024 threads; short
// ones T = 256 (four waves, which find room on a CU beside a running assign where sixteen do
// not).  T is a function of len, so the order depends on len only.
constexpr int SUM_U = 16;
constexpr int64_t SUM_LONG = 16384;  // rows at least this long take 1024 threads
template <int T>
__global__ __launch_bounds__(T) void sum_f64_rows_kernel(const double *__restrict__ part, int64_t len,
                                                         double *__restrict__ out, int accumulate) {
    __shared__ double s[T];
    const double *p = part + (size_t)blockIdx.x * len;
    const int t = threadIdx.x;
    double a[SUM_U];
#pragma unroll
    for (int u = 0; u < SUM_U; ++u) a[u] = 0.0;
    int64_t i = t;
    for (; i + (int64_t)(SUM_U - 1) * T < len; i += (int64_t)SUM_U * T) {
        double v[SUM_U];
#pragma unroll
        for (int u = 0; u < SUM_U; ++u) v[u] = p[i + (int64_t)u * T];
#pragma unroll
        for (int u = 0; u < SUM_U; ++u) a[u] += v[u];
    }
    for (; i < len; i += T) a[0] += p[i];
#pragma unroll
    for (int w = SUM_U / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int u = 0; u < w; ++u) a[u] += a[u + w];
    s[t] = a[0];
    __syncthreads();
    for (int off = T / 2; off >= 1; off >>= 1) {
        if (t < off) s[t] += s[t + off];
        __syncthreads();
    }
    if (t == 0) out[blockIdx.x] = accumulate ? out[blockIdx.x] + s[0] : s[0];
}

hipError_t launch_sum_f64_rows(const double *part, int rows, int64_t len, double *out, hipStream_t s,
                               int accumulate) {
    if (rows <= 0) return hipSuccess;
    if (len >= SUM_LONG) sum_f64_rows_kernel<1024><<<dim3(rows), dim3(1024), 0, s>>>(part, len, out, accumulate);
    else sum_f64_rows_kernel<256><<<dim3(rows), dim3(256), 0, s>>>(part, len, out, accumulate);
    return hipGetLastError();
}

}  // namespace fkm
