// C-ABI layer of libflashkm: argument validation (before any HIP call), workspace layout,
// launch sequencing, Lloyd's loop and the streamed (pinned host) pipeline.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/flashkm.h"
#include "common.h"
#include "plan.h"

namespace fkm {
// kernels (k_*.hip)
hipError_t launch_prep_centroids(int dt, const float *C, void *cprep, float *cnh, int B, int K, int D, int DP,
                                 hipStream_t stream, int zero_norm);
hipError_t launch_assign(int dt, const AssignCfg &cfg, const void *x, const void *cprep, const float *cnh,
                         const float *xn, int32_t *a, float *md, double *wgi, int B, int N, int D, int K,
                         hipStream_t s);
size_t sort_ws_bytes(int64_t B, int64_t N, int64_t K);
hipError_t launch_argsort(const int32_t *keys, int B, int N, int K, int32_t *out_keys, int32_t *out_vals,
                          int32_t *counts, void *ws, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);
size_t update_ws_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K);
bool update_refreshes_prep(int dt, int64_t B, int64_t N, int64_t D);
hipError_t launch_update(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                         int B, int N, int D, int K, int mode, float *C, double *shift, float *sums, int32_t *cnt,
                         const UpdRefresh &ref, void *ws, hipStream_t s, int normalize = 0);
hipError_t launch_finalize_acc(int dt, const float *sums, const int32_t *cnt, float *C, double *shift, double *shk,
                               const UpdRefresh &ref, int B, int K, int D, hipStream_t s, int normalize);
hipError_t launch_row_norms(int dt, const void *x, float *out, int64_t rows, int D, hipStream_t s);
hipError_t launch_normalize_rows(int dt, const void *x, void *out, int64_t rows, int D, hipStream_t s);
size_t reduce_ws_bytes(int64_t B);
hipError_t launch_sum_f32(const float *v, int B, int64_t n, double *out, int accumulate, void *ws, hipStream_t s);
hipError_t launch_sum_f64_rows(const double *part, int rows, int64_t len, double *out, hipStream_t s);
}  // namespace fkm

using namespace fkm;

namespace {

thread_local std::string g_err;

km_status_t fail(km_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

km_status_t ok() { return KM_OK; }

#define KM_HIP(call)                                                                                      \
    do {                                                                                                  \
        hipError_t e_ = (call);                                                                           \
        if (e_ != hipSuccess) return fail(KM_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));    \
    } while (0)

constexpr int64_t MAX_N = (int64_t)1 << 31;
constexpr int64_t MAX_D = 4096;
constexpr int64_t MAX_K = (int64_t)1 << 24;
constexpr int RING = 16;  // iterations of inertia / shift kept on the device between host reads
constexpr int64_t DEFAULT_CHUNK = (int64_t)1 << 24;

bool dt_ok(int dt) { return dt == KM_F32 || dt == KM_F16 || dt == KM_BF16; }
bool metric_ok(int m) { return m == KM_METRIC_L2 || m == KM_METRIC_DOT || m == KM_METRIC_COSINE; }

km_status_t check_shape(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    if (!dt_ok(dt)) return fail(KM_ERR_INVALID, "unknown dtype %d", dt);
    if (B < 1 || N < 1 || D < 1 || K < 1) return fail(KM_ERR_INVALID, "B, N, D, K must be >= 1 (got %lld %lld %lld %lld)",
                                                      (long long)B, (long long)N, (long long)D, (long long)K);
    if (K > N) return fail(KM_ERR_INVALID, "K (%lld) > N (%lld)", (long long)K, (long long)N);
    if (N >= MAX_N || B * N >= MAX_N) return fail(KM_ERR_INVALID, "B*N must be < 2^31");
    if (D > MAX_D) return fail(KM_ERR_INVALID, "D (%lld) > %lld", (long long)D, (long long)MAX_D);
    if (K > MAX_K) return fail(KM_ERR_INVALID, "K (%lld) > 2^24", (long long)K);
    return ok();
}

km_status_t check_ptr(const void *p, const char *name) {
    if (!p) return fail(KM_ERR_INVALID, "%s is NULL", name);
    return ok();
}

km_status_t check_ws(const void *ws, size_t ws_bytes, size_t need) {
    if (need == 0) return ok();
    if (!ws) return fail(KM_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (((uintptr_t)ws & 255) != 0) return fail(KM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(KM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    return ok();
}

// --------------------------------------------------------------------------------------------
// workspace layouts
// --------------------------------------------------------------------------------------------
size_t assign_ws(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    const AssignCfg c = plan_assign(dt, B, N, D, K);
    const int64_t KT = (int64_t)assign_tiles(K);
    return align256((size_t)B * KT * 32 * c.d_pad * elem_bytes(dt)) + align256((size_t)B * KT * 32 * 4);
}

size_t argsort_ws(int64_t B, int64_t N, int64_t K) { return sort_ws_bytes(B, N, K); }

size_t update_ws(int dt, int64_t B, int64_t N, int64_t D, int64_t K) { return update_ws_bytes(dt, B, N, D, K); }

int64_t assign_wgs_per_problem(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    return ceil_div(N, plan_assign(dt, B, N, D, K).block_n);
}

struct FitLayout {
    size_t xn, a, sids, sidx, counts, prep, ring_part, ring_j, ring_s, xhat, sums, cnt, shk, scratch, total;
};

// Device-resident x.  The prepared centroids persist across iterations (the update refreshes
// them); the arg-sort and update scratch share one region.  Cosine k-means adds the unit rows
// x^ [B][N][D] (input dtype) and, where rows need several column blocks, the accumulating
// update's sums [B][K][D], counts [B][K] and per-cluster shifts [B][K].
FitLayout fit_layout(int dt, int64_t B, int64_t N, int64_t D, int64_t K, int metric = KM_METRIC_L2) {
    FitLayout L{};
    size_t o = 0;
    const size_t bn4 = align256((size_t)B * N * 4);
    L.xn = o; o += bn4;
    L.a = o; o += bn4;
    L.sids = o; o += bn4;
    L.sidx = o; o += bn4;
    L.counts = o; o += align256((size_t)B * K * 4);
    L.prep = o; o += assign_ws(dt, B, N, D, K);
    L.ring_part = o; o += align256((size_t)RING * B * assign_wgs_per_problem(dt, B, N, D, K) * 8);
    L.ring_j = o; o += align256((size_t)RING * B * 8);
    L.ring_s = o; o += align256((size_t)RING * B * 8);
    if (metric == KM_METRIC_COSINE) {
        L.xhat = o; o += align256((size_t)B * N * D * elem_bytes(dt));
        if (!update_refreshes_prep(dt, B, N, D)) {  // the accumulating update (wide rows) only
            L.sums = o; o += align256((size_t)B * K * D * 4);
            L.cnt = o; o += align256((size_t)B * K * 4);
            L.shk = o; o += align256((size_t)B * K * 8);
        }
    }
    L.scratch = o;
    const size_t s2 = argsort_ws(B, N, K), s3 = update_ws(dt, B, N, D, K);
    o += s2 > s3 ? s2 : s3;
    L.total = o;
    return L;
}

struct HostLayout {
    size_t stage_buf[2], cprep, xn, md, a, sids, sidx, counts, sums, cnt, shk, ring_j, ring_s, red, scratch, total;
    int64_t chunk;
};

int64_t host_chunk(int64_t N, int64_t chunk_points) {
    int64_t c = chunk_points > 0 ? chunk_points : DEFAULT_CHUNK;
    if (c > N) c = N;
    return c;
}

// Pinned-host x: two staging buffers, per-chunk arrays, [B][K][D] sums and [B][K] counts.
HostLayout host_layout(int dt, int64_t B, int64_t N, int64_t D, int64_t K, int64_t chunk_points) {
    HostLayout L{};
    const int64_t c = host_chunk(N, chunk_points);
    L.chunk = c;
    size_t o = 0;
    const size_t sb = align256((size_t)c * D * elem_bytes(dt));
    L.stage_buf[0] = o; o += sb;
    L.stage_buf[1] = o; o += sb;
    L.cprep = o; o += assign_ws(dt, B, N, D, K);
    const size_t c4 = align256((size_t)c * 4);
    L.xn = o; o += c4;
    L.md = o; o += c4;
    L.a = o; o += c4;
    L.sids = o; o += c4;
    L.sidx = o; o += c4;
    L.counts = o; o += align256((size_t)K * 4);
    L.sums = o; o += align256((size_t)B * K * D * 4);
    L.cnt = o; o += align256((size_t)B * K * 4);
    L.shk = o; o += align256((size_t)B * K * 8);
    L.ring_j = o; o += align256((size_t)RING * B * 8);
    L.ring_s = o; o += align256((size_t)RING * B * 8);
    L.red = o; o += reduce_ws_bytes(B);
    L.scratch = o;
    size_t sc = argsort_ws(1, c, K);
    const size_t u = update_ws(dt, 1, c, D, K);
    if (u > sc) sc = u;
    o += sc;
    L.total = o;
    return L;
}

// --------------------------------------------------------------------------------------------
// device / pointer checks (HIP calls: only after argument validation)
// --------------------------------------------------------------------------------------------
enum PtrKind { PTR_DEVICE, PTR_PINNED_HOST, PTR_PAGEABLE };

PtrKind pointer_kind(const void *p) {
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return PTR_PAGEABLE;
    }
    if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) return PTR_DEVICE;
    if (attr.type == hipMemoryTypeHost) return PTR_PINNED_HOST;
    return PTR_PAGEABLE;
}

km_status_t require_device(const void *p, const char *name) {
    if (!p) return ok();
    const PtrKind k = pointer_kind(p);
    if (k != PTR_DEVICE)
        return fail(KM_ERR_UNSUPPORTED, "%s must be device memory (got %s)", name,
                    k == PTR_PINNED_HOST ? "pinned host memory" : "pageable/unknown host memory");
    return ok();
}

km_status_t check_device_arch() {
    static thread_local int checked_dev = -1;
    int dev = 0;
    KM_HIP(hipGetDevice(&dev));
    if (checked_dev == dev) return ok();
    hipDeviceProp_t prop;
    KM_HIP(hipGetDeviceProperties(&prop, dev));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(KM_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev,
                    prop.gcnArchName);
    checked_dev = dev;
    return ok();
}

#define KM_TRY(expr)                          \
    do {                                      \
        km_status_t st_ = (expr);             \
        if (st_ != KM_OK) return st_;         \
    } while (0)

// --------------------------------------------------------------------------------------------
// stage bodies (validated arguments)
// --------------------------------------------------------------------------------------------
// The prepared operand: c~ in tile order, then ||c~||^2 / 2 (assign_ws bytes in all).
float *prep_norms(int dt, char *cprep, int64_t B, int64_t D, int64_t K, int d_pad) {
    (void)D;
    return (float *)(cprep + align256((size_t)B * assign_tiles(K) * 32 * d_pad * elem_bytes(dt)));
}

km_status_t do_prepare(int dt, const float *C, int64_t B, int64_t N, int64_t D, int64_t K, void *cprep,
                       hipStream_t s, int metric = KM_METRIC_L2) {
    const AssignCfg cfg = plan_assign(dt, B, N, D, K);
    KM_HIP(launch_prep_centroids(dt, C, cprep, prep_norms(dt, (char *)cprep, B, D, K, cfg.d_pad), (int)B, (int)K,
                                 (int)D, cfg.d_pad, s, metric != KM_METRIC_L2));
    return ok();
}

km_status_t do_assign_prepared(int dt, const void *x, const void *cprep, int64_t B, int64_t N, int64_t D, int64_t K,
                               const float *xn, int32_t *a, float *md, hipStream_t s) {
    const AssignCfg cfg = plan_assign(dt, B, N, D, K);
    const float *cnh = prep_norms(dt, (char *)cprep, B, D, K, cfg.d_pad);
    KM_HIP(launch_assign(dt, cfg, x, cprep, cnh, xn, a, md, nullptr, (int)B, (int)N, (int)D, (int)K, s));
    return ok();
}

km_status_t do_assign(int dt, const void *x, const float *C, int64_t B, int64_t N, int64_t D, int64_t K,
                      const float *xn, int32_t *a, float *md, void *ws, hipStream_t s) {
    KM_TRY(do_prepare(dt, C, B, N, D, K, ws, s));
    return do_assign_prepared(dt, x, ws, B, N, D, K, xn, a, md, s);
}

km_status_t do_update(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                      int64_t B, int64_t N, int64_t D, int64_t K, float *C, double *shift, void *ws, hipStream_t s) {
    KM_HIP(launch_update(dt, x, sids, sidx, counts, (int)B, (int)N, (int)D, (int)K, 0, C, shift, nullptr, nullptr,
                         UpdRefresh{}, ws, s));
    return ok();
}

}  // namespace

extern "C" {

const char *kmeans_last_error(void) { return g_err.c_str(); }

km_status_t kmeans_plan(km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K, km_plan_t *out) {
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(out, "out"));
    const AssignCfg a = plan_assign(dt, B, N, D, K);
    const SortCfg so = plan_sort(N, K);
    const UpdCfg u = plan_update(dt, B, N, D);
    out->path = a.path;
    out->d_pad = a.d_pad;
    out->point_blocks = a.pb;
    out->waves = ASSIGN_WAVES;
    out->block_n = a.block_n;
    out->block_k = a.path == 0 ? a.tps * 32 : SPLITD_KB * 32;
    out->block_d = a.bd;
    out->lds_bytes = a.lds;
    out->vgpr_est = a.vgpr;
    out->assign_wgs = (int32_t)(B * ceil_div(N, a.block_n));
    out->sort_bits = so.bits;
    out->sort_passes = so.passes;
    out->sort_tile = SORT_TILE;
    out->upd_rows = u.rows;
    out->upd_vec = u.vec;
    out->upd_lanes = u.lanes;
    return ok();
}

size_t kmeans_workspace_bytes(int op, km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K,
                              int64_t chunk_points) {
    if (check_shape(dt, B, N, D, K) != KM_OK) return 0;
    switch (op) {
        case KM_OP_ASSIGN: return assign_ws(dt, B, N, D, K);
        case KM_OP_ARGSORT: return argsort_ws(B, N, K);
        case KM_OP_UPDATE: return update_ws(dt, B, N, D, K);
        case KM_OP_FIT: return fit_layout(dt, B, N, D, K).total;
        case KM_OP_FIT_HOST: return host_layout(dt, B, N, D, K, chunk_points).total;
        case KM_OP_FIT_DOT: return fit_layout(dt, B, N, D, K, KM_METRIC_DOT).total;
        case KM_OP_FIT_COSINE: return fit_layout(dt, B, N, D, K, KM_METRIC_COSINE).total;
        default: g_err = "unknown workspace op"; return 0;
    }
}

km_status_t kmeans_row_norms(const void *x, km_dtype_t dt, int64_t B, int64_t N, int64_t D, float *x_norms,
                             void *stream) {
    if (!dt_ok(dt)) return fail(KM_ERR_INVALID, "unknown dtype %d", dt);
    if (B < 1 || N < 1 || D < 1 || D > MAX_D || B * N >= MAX_N) return fail(KM_ERR_INVALID, "bad shape");
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(x_norms, "x_norms"));
    if (((uintptr_t)x & 15) != 0) return fail(KM_ERR_INVALID, "x must be 16-byte aligned");
    KM_TRY(check_device_arch());
    KM_TRY(require_device(x, "x"));
    KM_TRY(require_device(x_norms, "x_norms"));
    KM_HIP(launch_row_norms(dt, x, x_norms, B * N, (int)D, (hipStream_t)stream));
    return ok();
}

km_status_t kmeans_assign(const void *x, km_dtype_t dt, const float *centroids, int64_t B, int64_t N, int64_t D,
                          int64_t K, const float *x_norms, int32_t *assign, float *min_dist, void *ws,
                          size_t ws_bytes, void *stream) {
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(centroids, "centroids"));
    KM_TRY(check_ptr(assign, "assign"));
    if (min_dist && !x_norms) return fail(KM_ERR_INVALID, "min_dist requires x_norms");
    if (((uintptr_t)x & 15) != 0) return fail(KM_ERR_INVALID, "x must be 16-byte aligned");
    KM_TRY(check_ws(ws, ws_bytes, assign_ws(dt, B, N, D, K)));
    KM_TRY(check_device_arch());
    KM_TRY(require_device(x, "x"));
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(assign, "assign"));
    KM_TRY(require_device(min_dist, "min_dist"));
    KM_TRY(require_device(x_norms, "x_norms"));
    KM_TRY(require_device(ws, "ws"));
    return do_assign(dt, x, centroids, B, N, D, K, x_norms, assign, min_dist, ws, (hipStream_t)stream);
}

km_status_t kmeans_prepare_centroids(const float *centroids, km_dtype_t dt, int64_t B, int64_t N, int64_t D,
                                     int64_t K, void *c_prep, size_t c_prep_bytes, void *stream) {
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(centroids, "centroids"));
    KM_TRY(check_ptr(c_prep, "c_prep"));
    KM_TRY(check_ws(c_prep, c_prep_bytes, assign_ws(dt, B, N, D, K)));
    KM_TRY(check_device_arch());
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(c_prep, "c_prep"));
    return do_prepare(dt, centroids, B, N, D, K, c_prep, (hipStream_t)stream);
}

km_status_t kmeans_assign_prepared(const void *x, km_dtype_t dt, const void *c_prep, size_t c_prep_bytes, int64_t B,
                                   int64_t N, int64_t D, int64_t K, const float *x_norms, int32_t *assign,
                                   float *min_dist, void *stream) {
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(c_prep, "c_prep"));
    KM_TRY(check_ptr(assign, "assign"));
    if (min_dist && !x_norms) return fail(KM_ERR_INVALID, "min_dist requires x_norms");
    if (((uintptr_t)x & 15) != 0) return fail(KM_ERR_INVALID, "x must be 16-byte aligned");
    KM_TRY(check_ws(c_prep, c_prep_bytes, assign_ws(dt, B, N, D, K)));
    KM_TRY(check_device_arch());
    KM_TRY(require_device(x, "x"));
    KM_TRY(require_device(c_prep, "c_prep"));
    KM_TRY(require_device(assign, "assign"));
    KM_TRY(require_device(min_dist, "min_dist"));
    KM_TRY(require_device(x_norms, "x_norms"));
    return do_assign_prepared(dt, x, c_prep, B, N, D, K, x_norms, assign, min_dist, (hipStream_t)stream);
}

km_status_t kmeans_normalize_rows(const void *x, km_dtype_t dt, int64_t rows, int64_t D, void *out, void *stream) {
    if (!dt_ok(dt)) return fail(KM_ERR_INVALID, "unknown dtype %d", dt);
    if (rows < 1 || D < 1 || D > MAX_D || rows >= MAX_N) return fail(KM_ERR_INVALID, "bad shape");
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(out, "out"));
    if (((uintptr_t)x & 15) != 0 || ((uintptr_t)out & 15) != 0)
        return fail(KM_ERR_INVALID, "x and out must be 16-byte aligned");
    KM_TRY(check_device_arch());
    KM_TRY(require_device(x, "x"));
    KM_TRY(require_device(out, "out"));
    KM_HIP(launch_normalize_rows(dt, x, out, rows, (int)D, (hipStream_t)stream));
    return ok();
}

km_status_t kmeans_prepare_centroids_metric(const float *centroids, km_dtype_t dt, km_metric_t metric, int64_t B,
                                            int64_t N, int64_t D, int64_t K, void *c_prep, size_t c_prep_bytes,
                                            void *stream) {
    if (!metric_ok(metric)) return fail(KM_ERR_INVALID, "unknown metric %d", (int)metric);
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(centroids, "centroids"));
    KM_TRY(check_ptr(c_prep, "c_prep"));
    KM_TRY(check_ws(c_prep, c_prep_bytes, assign_ws(dt, B, N, D, K)));
    KM_TRY(check_device_arch());
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(c_prep, "c_prep"));
    return do_prepare(dt, centroids, B, N, D, K, c_prep, (hipStream_t)stream, (int)metric);
}

km_status_t kmeans_argsort_ids(const int32_t *assign, int64_t B, int64_t N, int64_t K, int32_t *sorted_ids,
                               int32_t *sorted_idx, int32_t *counts, void *ws, size_t ws_bytes, void *stream) {
    KM_TRY(check_shape(KM_F32, B, N, 1, K));
    KM_TRY(check_ptr(assign, "assign"));
    KM_TRY(check_ptr(sorted_ids, "sorted_ids"));
    KM_TRY(check_ptr(sorted_idx, "sorted_idx"));
    KM_TRY(check_ws(ws, ws_bytes, argsort_ws(B, N, K)));
    KM_TRY(check_device_arch());
    KM_TRY(require_device(assign, "assign"));
    KM_TRY(require_device(sorted_ids, "sorted_ids"));
    KM_TRY(require_device(sorted_idx, "sorted_idx"));
    KM_TRY(require_device(counts, "counts"));
    KM_TRY(require_device(ws, "ws"));
    KM_HIP(launch_argsort(assign, (int)B, (int)N, (int)K, sorted_ids, sorted_idx, counts, ws, (hipStream_t)stream));
    return ok();
}

km_status_t kmeans_update(const void *x, km_dtype_t dt, const int32_t *sorted_ids, const int32_t *sorted_idx,
                          const int32_t *counts, int64_t B, int64_t N, int64_t D, int64_t K, float *centroids,
                          double *shift, void *ws, size_t ws_bytes, void *stream) {
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(sorted_ids, "sorted_ids"));
    KM_TRY(check_ptr(sorted_idx, "sorted_idx"));
    KM_TRY(check_ptr(counts, "counts"));
    KM_TRY(check_ptr(centroids, "centroids"));
    if (((uintptr_t)centroids & 15) != 0) return fail(KM_ERR_INVALID, "centroids must be 16-byte aligned");
    if (((uintptr_t)x & 15) != 0) return fail(KM_ERR_INVALID, "x must be 16-byte aligned");
    KM_TRY(check_ws(ws, ws_bytes, update_ws(dt, B, N, D, K)));
    KM_TRY(check_device_arch());
    KM_TRY(require_device(x, "x"));
    KM_TRY(require_device(sorted_ids, "sorted_ids"));
    KM_TRY(require_device(sorted_idx, "sorted_idx"));
    KM_TRY(require_device(counts, "counts"));
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(shift, "shift"));
    KM_TRY(require_device(ws, "ws"));
    return do_update(dt, x, sorted_ids, sorted_idx, counts, B, N, D, K, centroids, shift, ws, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Copy the first `n` iterations of a device ring [RING][B] into host[t0*B ...].
km_status_t ring_to_host(const double *ring, double *host, int t0, int n, int64_t B, hipStream_t s) {
    if (!host || n <= 0) return ok();
    KM_HIP(hipMemcpyAsync(host + (size_t)t0 * B, ring, (size_t)n * B * 8, hipMemcpyDeviceToHost, s));
    KM_HIP(hipStreamSynchronize(s));
    return ok();
}

km_status_t read_shift_max(const double *dev, int64_t B, double *out, hipStream_t s) {
    double tmp[64];
    double m = 0.0;
    for (int64_t b0 = 0; b0 < B; b0 += 64) {
        const int64_t nb = B - b0 < 64 ? B - b0 : 64;
        KM_HIP(hipMemcpyAsync(tmp, dev + b0, (size_t)nb * 8, hipMemcpyDeviceToHost, s));
        KM_HIP(hipStreamSynchronize(s));
        for (int64_t i = 0; i < nb; ++i) m = tmp[i] > m ? tmp[i] : m;
    }
    *out = m;
    return ok();
}

// metric: KM_METRIC_L2 (Lloyd), KM_METRIC_DOT (similarity x.c, mean update) or KM_METRIC_COSINE
// (unit rows, mean-direction update).  For the similarity metrics the assign kernels get zero
// norm terms (scores -x.c~) and zero point norms, so their per-point "distance" is
// -2 x.c~ and the per-iteration value returned is -1/2 of its sum: the total similarity.
km_status_t fit_device(int dt, const void *x, int64_t B, int64_t N, int64_t D, int64_t K, int iters, float tol,
                       float *C, int32_t *assign, double *inertia, int32_t *iters_done, char *ws, hipStream_t s,
                       int metric = KM_METRIC_L2) {
    const FitLayout L = fit_layout(dt, B, N, D, K, metric);
    const bool simm = metric != KM_METRIC_L2;
    const bool cosine = metric == KM_METRIC_COSINE;
    const AssignCfg cfg = plan_assign(dt, B, N, D, K);
    const int64_t KT = assign_tiles(K);
    const int64_t wpb = assign_wgs_per_problem(dt, B, N, D, K);
    float *xn = (float *)(ws + L.xn);
    int32_t *a = assign ? assign : (int32_t *)(ws + L.a);
    int32_t *sids = (int32_t *)(ws + L.sids);
    int32_t *sidx = (int32_t *)(ws + L.sidx);
    int32_t *counts = (int32_t *)(ws + L.counts);
    char *cprep = ws + L.prep;
    float *cnh = (float *)(cprep + align256((size_t)B * KT * 32 * cfg.d_pad * elem_bytes(dt)));
    double *ring_part = (double *)(ws + L.ring_part);
    double *ring_j = (double *)(ws + L.ring_j);
    double *ring_s = (double *)(ws + L.ring_s);
    void *scratch = ws + L.scratch;
    const bool fused_prep = update_refreshes_prep(dt, B, N, D);
    const UpdRefresh full_ref{cprep, cnh, cfg.d_pad, (int)KT, simm ? 1 : 0};
    const UpdRefresh ref = fused_prep ? full_ref : UpdRefresh{};

    // the points the iterations use: x, or its unit rows for cosine k-means (whose centroids
    // are made unit rows too, in place)
    const void *xa = x;
    if (cosine) {
        KM_HIP(launch_normalize_rows(dt, x, ws + L.xhat, B * N, (int)D, s));
        KM_HIP(launch_normalize_rows(KM_F32, C, C, B * K, (int)D, s));
        xa = ws + L.xhat;
    }
    // the small-D assign kernel computes the point norms it needs from its own registers; the
    // split-D kernel reads them.  The similarity metrics take zeros instead.
    const float *xn_in = simm ? xn : (cfg.path == 0 ? nullptr : xn);
    if (simm) KM_HIP(launch_fill_i32((int32_t *)xn, B * N, 0, s));
    else if (xn_in) KM_HIP(launch_row_norms(dt, x, xn, B * N, (int)D, s));
    KM_HIP(launch_prep_centroids(dt, C, cprep, cnh, (int)B, (int)K, (int)D, cfg.d_pad, s, simm ? 1 : 0));
    int done = 0, flushed = 0;
    for (int t = 0; t < iters; ++t) {
        const int slot = t - flushed;
        // one iteration: assign (+ per-workgroup inertia partials), arg-sort, update (+ shift,
        // + the next iteration's prepared centroids)
        KM_HIP(launch_assign(dt, cfg, xa, cprep, cnh, xn_in, a, nullptr, ring_part + (size_t)slot * B * wpb, (int)B,
                             (int)N, (int)D, (int)K, s));
        KM_HIP(launch_argsort(a, (int)B, (int)N, (int)K, sids, sidx, counts, scratch, s));
        if (cosine && fused_prep) {
            // one column block per row: the update finishes each cluster in place with the mean
            // direction s_k / ||s_k|| (and the shift and the refresh), like the Euclidean finish
            KM_HIP(launch_update(dt, xa, sids, sidx, counts, (int)B, (int)N, (int)D, (int)K, 0, C,
                                 tol > 0.f ? ring_s + (size_t)slot * B : nullptr, nullptr, nullptr, full_ref, scratch,
                                 s, 1));
        } else if (cosine) {
            // sums and counts per cluster, then the mean direction (with shift and refresh)
            float *sums = (float *)(ws + L.sums);
            int32_t *cnt = (int32_t *)(ws + L.cnt);
            KM_HIP(launch_fill_i32((int32_t *)sums, B * K * D, 0, s));
            KM_HIP(launch_fill_i32(cnt, B * K, 0, s));
            KM_HIP(launch_update(dt, xa, sids, sidx, counts, (int)B, (int)N, (int)D, (int)K, 1, nullptr, nullptr,
                                 sums, cnt, UpdRefresh{}, scratch, s));
            KM_HIP(launch_finalize_acc(dt, sums, cnt, C, tol > 0.f ? ring_s + (size_t)slot * B : nullptr,
                                       (double *)(ws + L.shk), full_ref, (int)B, (int)K, (int)D, s, 1));
        } else {
            KM_HIP(launch_update(dt, xa, sids, sidx, counts, (int)B, (int)N, (int)D, (int)K, 0, C,
                                 tol > 0.f ? ring_s + (size_t)slot * B : nullptr, nullptr, nullptr, ref, scratch, s));
            if (!fused_prep && t + 1 < iters)
                KM_HIP(launch_prep_centroids(dt, C, cprep, cnh, (int)B, (int)K, (int)D, cfg.d_pad, s, simm ? 1 : 0));
        }
        done = t + 1;
        bool stop = false;
        if (tol > 0.f) {
            double smax = 0.0;
            KM_TRY(read_shift_max(ring_s + (size_t)slot * B, B, &smax, s));
            stop = smax < (double)tol;
        }
        if (slot + 1 == RING || stop || t + 1 == iters) {
            KM_HIP(launch_sum_f64_rows(ring_part, (slot + 1) * (int)B, wpb, ring_j, s));
            KM_TRY(ring_to_host(ring_j, inertia, flushed, slot + 1, B, s));
            flushed = t + 1;
        }
        if (stop) break;
    }
    KM_HIP(hipStreamSynchronize(s));
    if (simm && inertia)
        for (int64_t i = 0; i < (int64_t)done * B; ++i) inertia[i] *= -0.5;
    if (iters_done) *iters_done = done;
    return ok();
}

struct StreamedPipe {
    hipStream_t cs = nullptr;
    hipEvent_t ev_copy[2] = {nullptr, nullptr};
    hipEvent_t ev_free[2] = {nullptr, nullptr};
    ~StreamedPipe() {
        for (int i = 0; i < 2; ++i) {
            if (ev_copy[i]) (void)hipEventDestroy(ev_copy[i]);
            if (ev_free[i]) (void)hipEventDestroy(ev_free[i]);
        }
        if (cs) (void)hipStreamDestroy(cs);
    }
};

// metric as in fit_device.  Cosine k-means turns each staged chunk into unit rows in place (the
// staging buffer is a device copy of x) before its assign and update.
km_status_t fit_host(int dt, const void *xh, int64_t B, int64_t N, int64_t D, int64_t K, int iters, float tol,
                     int64_t chunk_points, float *C, int32_t *assign, double *inertia, int32_t *iters_done, char *ws,
                     hipStream_t s, int metric = KM_METRIC_L2) {
    const HostLayout L = host_layout(dt, B, N, D, K, chunk_points);
    const bool simm = metric != KM_METRIC_L2;
    const bool cosine = metric == KM_METRIC_COSINE;
    const int64_t chunk = L.chunk;
    const int64_t nchunk = ceil_div(N, chunk);
    const size_t es = elem_bytes(dt);
    char *stage_buf[2] = {ws + L.stage_buf[0], ws + L.stage_buf[1]};
    char *cprep = ws + L.cprep;
    const AssignCfg cfg = plan_assign(dt, B, N, D, K);
    const int64_t KT = (int64_t)assign_tiles(K);
    const size_t cprep_bytes = align256((size_t)B * KT * 32 * cfg.d_pad * es);
    float *cnh = (float *)(cprep + cprep_bytes);
    const size_t cprep_per_b = (size_t)KT * 32 * cfg.d_pad * es;
    float *xn = (float *)(ws + L.xn);
    float *md = (float *)(ws + L.md);
    int32_t *a_ws = (int32_t *)(ws + L.a);
    int32_t *sids = (int32_t *)(ws + L.sids);
    int32_t *sidx = (int32_t *)(ws + L.sidx);
    int32_t *counts = (int32_t *)(ws + L.counts);
    float *sums = (float *)(ws + L.sums);
    int32_t *cnt = (int32_t *)(ws + L.cnt);
    double *ring_j = (double *)(ws + L.ring_j);
    double *ring_s = (double *)(ws + L.ring_s);
    void *red = ws + L.red;
    void *scratch = ws + L.scratch;
    const UpdRefresh ref{cprep, cnh, cfg.d_pad, (int)KT, simm ? 1 : 0};

    StreamedPipe P;
    KM_HIP(hipStreamCreateWithFlags(&P.cs, hipStreamNonBlocking));
    for (int i = 0; i < 2; ++i) {
        KM_HIP(hipEventCreateWithFlags(&P.ev_copy[i], hipEventDisableTiming));
        KM_HIP(hipEventCreateWithFlags(&P.ev_free[i], hipEventDisableTiming));
    }
    // chunk sequence (iteration-major), copies run one chunk ahead, across iteration borders
    const int64_t per_iter = B * nchunk;
    auto chunk_rows = [&](int64_t q, int64_t *b, int64_t *lo, int64_t *n) {
        const int64_t r = q % per_iter;
        *b = r / nchunk;
        *lo = (r % nchunk) * chunk;
        *n = N - *lo < chunk ? N - *lo : chunk;
    };
    auto issue_copy = [&](int64_t q) -> km_status_t {
        int64_t b, lo, n;
        chunk_rows(q, &b, &lo, &n);
        const int buf = (int)(q & 1);
        KM_HIP(hipStreamWaitEvent(P.cs, P.ev_free[buf], 0));
        KM_HIP(hipMemcpyAsync(stage_buf[buf], (const char *)xh + ((size_t)b * N + lo) * D * es, (size_t)n * D * es,
                              hipMemcpyHostToDevice, P.cs));
        KM_HIP(hipEventRecord(P.ev_copy[buf], P.cs));
        return ok();
    };
    // the copy stream must not start before work already queued on `s` that it depends on
    KM_HIP(hipEventRecord(P.ev_free[0], s));
    KM_HIP(hipEventRecord(P.ev_free[1], s));
    KM_TRY(issue_copy(0));
    if (cosine) KM_HIP(launch_normalize_rows(KM_F32, C, C, B * K, (int)D, s));
    // the similarity metrics take zero point norms (their per-point value is then -2 x.c~)
    if (simm) KM_HIP(launch_fill_i32((int32_t *)xn, chunk, 0, s));
    KM_HIP(launch_prep_centroids(dt, C, cprep, cnh, (int)B, (int)K, (int)D, cfg.d_pad, s, simm ? 1 : 0));
    int64_t q = 0;
    int done = 0, flushed = 0;
    for (int t = 0; t < iters; ++t) {
        const int slot = t - flushed;
        KM_HIP(launch_fill_i32((int32_t *)sums, B * K * D, 0, s));
        KM_HIP(launch_fill_i32(cnt, B * K, 0, s));
        KM_HIP(launch_fill_i32((int32_t *)(ring_j + (size_t)slot * B), 2 * B, 0, s));
        for (int64_t i = 0; i < per_iter; ++i, ++q) {
            const bool more = (t + 1 < iters) || (i + 1 < per_iter);
            if (more) KM_TRY(issue_copy(q + 1));
            int64_t b, lo, n;
            chunk_rows(q, &b, &lo, &n);
            const int buf = (int)(q & 1);
            const void *xc = stage_buf[buf];
            KM_HIP(hipStreamWaitEvent(s, P.ev_copy[buf], 0));
            int32_t *ac = assign ? assign + (size_t)b * N + lo : a_ws;
            if (cosine) KM_HIP(launch_normalize_rows(dt, xc, stage_buf[buf], n, (int)D, s));
            if (cfg.path != 0 && !simm) KM_HIP(launch_row_norms(dt, xc, xn, n, (int)D, s));
            KM_HIP(launch_assign(dt, cfg, xc, cprep + (size_t)b * cprep_per_b, cnh + (size_t)b * KT * 32,
                                 (cfg.path == 0 && !simm) ? nullptr : xn, ac, md,
                                 nullptr, 1, (int)n, (int)D, (int)K, s));
            KM_HIP(launch_sum_f32(md, 1, n, ring_j + (size_t)slot * B + b, 1, red, s));
            KM_HIP(launch_argsort(ac, 1, (int)n, (int)K, sids, sidx, counts, scratch, s));
            KM_HIP(launch_update(dt, xc, sids, sidx, counts, 1, (int)n, (int)D, (int)K, 1, nullptr, nullptr,
                                 sums + (size_t)b * K * D, cnt + (size_t)b * K, UpdRefresh{}, scratch, s));
            KM_HIP(hipEventRecord(P.ev_free[buf], s));
        }
        KM_HIP(launch_finalize_acc(dt, sums, cnt, C, tol > 0.f ? ring_s + (size_t)slot * B : nullptr,
                                   (double *)(ws + L.shk), ref, (int)B, (int)K, (int)D, s, cosine ? 1 : 0));
        done = t + 1;
        bool stop = false;
        if (tol > 0.f) {
            double smax = 0.0;
            KM_TRY(read_shift_max(ring_s + (size_t)slot * B, B, &smax, s));
            stop = smax < (double)tol;
        }
        if (slot + 1 == RING || stop || t + 1 == iters) {
            KM_TRY(ring_to_host(ring_j, inertia, flushed, slot + 1, B, s));
            flushed = t + 1;
        }
        if (stop) break;
    }
    KM_HIP(hipStreamSynchronize(s));
    KM_HIP(hipStreamSynchronize(P.cs));
    if (simm && inertia)
        for (int64_t i = 0; i < (int64_t)done * B; ++i) inertia[i] *= -0.5;
    if (iters_done) *iters_done = done;
    return ok();
}

}  // namespace

extern "C" km_status_t kmeans_fit_metric(const void *x, km_dtype_t dt, km_metric_t metric, int64_t B, int64_t N,
                                         int64_t D, int64_t K, int32_t iters, float tol, int64_t chunk_points,
                                         float *centroids, int32_t *assign, double *objective, int32_t *iters_done,
                                         void *ws, size_t ws_bytes, void *stream) {
    if (!metric_ok(metric)) return fail(KM_ERR_INVALID, "unknown metric %d", (int)metric);
    if (metric == KM_METRIC_L2)
        return kmeans_fit(x, dt, B, N, D, K, iters, tol, chunk_points, centroids, assign, objective, iters_done, ws,
                          ws_bytes, stream);
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(centroids, "centroids"));
    if (iters < 1) return fail(KM_ERR_INVALID, "iters must be >= 1");
    if (!(tol >= 0.f)) return fail(KM_ERR_INVALID, "tol must be >= 0");
    if (chunk_points < 0) return fail(KM_ERR_INVALID, "chunk_points must be >= 0");
    if (((uintptr_t)centroids & 15) != 0) return fail(KM_ERR_INVALID, "centroids must be 16-byte aligned");
    if (((uintptr_t)x & 15) != 0) return fail(KM_ERR_INVALID, "x must be 16-byte aligned");
    if (!ws) return fail(KM_ERR_WORKSPACE, "workspace is NULL");
    KM_TRY(check_device_arch());
    const PtrKind xk = pointer_kind(x);
    if (xk == PTR_PAGEABLE)
        return fail(KM_ERR_UNSUPPORTED, "x is pageable host memory; pass device memory or pinned host memory");
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(assign, "assign"));
    KM_TRY(require_device(ws, "ws"));
    if (xk == PTR_DEVICE) {
        KM_TRY(check_ws(ws, ws_bytes, fit_layout(dt, B, N, D, K, (int)metric).total));
        return fit_device(dt, x, B, N, D, K, iters, tol, centroids, assign, objective, iters_done, (char *)ws,
                          (hipStream_t)stream, (int)metric);
    }
    KM_TRY(check_ws(ws, ws_bytes, host_layout(dt, B, N, D, K, chunk_points).total));
    return fit_host(dt, x, B, N, D, K, iters, tol, chunk_points, centroids, assign, objective, iters_done,
                    (char *)ws, (hipStream_t)stream, (int)metric);
}

extern "C" km_status_t kmeans_fit(const void *x, km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K,
                                  int32_t iters, float tol, int64_t chunk_points, float *centroids, int32_t *assign,
                                  double *inertia, int32_t *iters_done, void *ws, size_t ws_bytes, void *stream) {
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(centroids, "centroids"));
    if (iters < 1) return fail(KM_ERR_INVALID, "iters must be >= 1");
    if (!(tol >= 0.f)) return fail(KM_ERR_INVALID, "tol must be >= 0");
    if (chunk_points < 0) return fail(KM_ERR_INVALID, "chunk_points must be >= 0");
    if (((uintptr_t)centroids & 15) != 0) return fail(KM_ERR_INVALID, "centroids must be 16-byte aligned");
    if (((uintptr_t)x & 15) != 0) return fail(KM_ERR_INVALID, "x must be 16-byte aligned");
    if (!ws) return fail(KM_ERR_WORKSPACE, "workspace is NULL");
    KM_TRY(check_device_arch());
    const PtrKind xk = pointer_kind(x);
    if (xk == PTR_PAGEABLE)
        return fail(KM_ERR_UNSUPPORTED, "x is pageable host memory; pass device memory or pinned host memory");
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(assign, "assign"));
    KM_TRY(require_device(ws, "ws"));
    hipStream_t s = (hipStream_t)stream;
    if (xk == PTR_DEVICE) {
        KM_TRY(check_ws(ws, ws_bytes, fit_layout(dt, B, N, D, K).total));
        return fit_device(dt, x, B, N, D, K, iters, tol, centroids, assign, inertia, iters_done, (char *)ws, s);
    }
    KM_TRY(check_ws(ws, ws_bytes, host_layout(dt, B, N, D, K, chunk_points).total));
    return fit_host(dt, x, B, N, D, K, iters, tol, chunk_points, centroids, assign, inertia, iters_done, (char *)ws,
                    s);
}
