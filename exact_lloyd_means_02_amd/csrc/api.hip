// C-ABI layer of libflashkm: argument validation (before any HIP call), workspace layout,
// launch sequencing, Lloyd's loop and the streamed (pinned host) pipeline.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/flashkm.h"
#include "common.h"
#include "plan.h"

namespace fkm {
// kernels (k_*.hip)
hipError_t launch_prep_centroids(int dt, const float *C, void *cprep, float *cnh, int B, int K, int D, int DP,
                                 hipStream_t stream, int zero_norm);
hipError_t launch_assign(int dt, const AssignCfg &cfg, const void *x, const void *cprep, const float *cnh,
                         const float *xn, int32_t *a, float *md, double *wgi, int B, int N, int D, int K,
                         hipStream_t s, const AssignSplit &sp);
size_t sort_ws_bytes(int64_t B, int64_t N, int64_t K);
hipError_t launch_argsort(const int32_t *keys, int B, int N, int K, int32_t *out_keys, int32_t *out_vals,
                          int32_t *counts, int32_t *offs, int32_t *status, void *ws, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);
size_t update_ws_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K);
size_t update_ctr_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K);
size_t update_scratch_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K);
bool update_refreshes_prep(int dt, int64_t B, int64_t N, int64_t D);
hipError_t launch_update(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                         int B, int N, int D, int K, int mode, float *C, double *shift, float *sums, int32_t *cnt,
                         const UpdRefresh &ref, const UpdMem &mem, hipStream_t s, int normalize = 0);
hipError_t launch_update_ws(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                            int B, int N, int D, int K, float *C, double *shift, void *ws, hipStream_t s);
hipError_t launch_finalize_acc(int dt, const float *sums, const int32_t *cnt, float *C, double *shift, double *shk,
                               const UpdRefresh &ref, int B, int K, int D, hipStream_t s, int normalize);
hipError_t launch_row_norms(int dt, const void *x, float *out, int64_t rows, int D, hipStream_t s);
hipError_t launch_normalize_rows(int dt, const void *x, void *out, int64_t rows, int D, hipStream_t s);
hipError_t launch_sum_f64_rows(const double *part, int rows, int64_t len, double *out, hipStream_t s,
                               int accumulate = 0);
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

// The arg-sort's status word (see k_sort.hip): 0, or bits for labels outside [0, K) (1) and a
// digit table that did not count the keys (2).
km_status_t status_word(int32_t st, const char *who) {
    if (st == 0) return KM_OK;
    return fail(KM_ERR_INVALID, "%s met %s%s%s", who, (st & 1) ? "labels outside [0, K)" : "",
                (st & 3) == 3 ? " and " : "",
                (st & 2) ? "sorted destinations outside the rows (labels changed while it ran)" : "");
}

#define KM_HIP(call)                                                                                      \
    do {                                                                                                  \
        hipError_t e_ = (call);                                                                           \
        if (e_ != hipSuccess) return fail(KM_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));    \
    } while (0)

constexpr int64_t MAX_N = (int64_t)1 << 31;
constexpr int64_t MAX_D = 4096;
constexpr int64_t MAX_K = (int64_t)1 << 24;
// Iterations of inertia / shift kept on the device between host reads.  A read waits for the
// stream to drain, and the next iteration's kernels are only launched after it, so each read
// leaves the GPU idle for the host's round trip (about 75 us); 64 slots keep that to the end of
// fits of up to 64 iterations (with tol = 0) for 8 * 64 * B * (workgroups per problem + 2) bytes.
constexpr int RING = 64;
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
// The prepared centroid operand: c~ in tile order, then ||c~||^2 / 2.
size_t prep_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    const AssignCfg c = plan_assign(dt, B, N, D, K);
    const int64_t KT = (int64_t)assign_tiles(dt, D, K);
    return align256((size_t)B * KT * 32 * c.d_pad * elem_bytes(dt)) + align256((size_t)B * KT * 32 * 4);
}

// Buffers of a K-split assign (see AssignSplit), 0 when the plan does not split.
size_t split_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    if (plan_assign(dt, B, N, D, K).nsplit <= 1) return 0;
    return align256((size_t)B * N * 8) + align256((size_t)B * N * 4);
}

// kmeans_assign's workspace: the prepared operand, then the split buffers.
size_t assign_ws(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    return prep_bytes(dt, B, N, D, K) + split_bytes(dt, B, N, D, K);
}

AssignSplit split_at(int dt, int64_t B, int64_t N, int64_t D, int64_t K, char *buf) {
    AssignSplit sp;
    sp.nsplit = plan_assign(dt, B, N, D, K).nsplit;
    if (sp.nsplit > 1) {
        sp.packed = (unsigned long long *)buf;
        sp.xn = (float *)(buf + align256((size_t)B * N * 8));
    }
    return sp;
}

// A caller's arg-sort workspace: the status word (first 256 bytes), then the digit tables.
constexpr size_t STATUS_BYTES = 256;
size_t argsort_ws(int64_t B, int64_t N, int64_t K) { return STATUS_BYTES + sort_ws_bytes(B, N, K); }

size_t update_ws(int dt, int64_t B, int64_t N, int64_t D, int64_t K) { return update_ws_bytes(dt, B, N, D, K); }

int64_t assign_wgs_per_problem(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    return ceil_div(N, plan_assign(dt, B, N, D, K).block_n);
}

struct FitLayout {
    size_t xn, a, sids, sidx, counts, offs, status, updctr, prep, split, ring_part, ring_j, ring_s, xhat, sums, cnt,
        shk, scratch, total;
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
    L.offs = o; o += align256((size_t)B * K * 4);
    L.status = o; o += STATUS_BYTES;
    L.updctr = o; o += update_ctr_bytes(dt, B, N, D, K);
    L.prep = o; o += prep_bytes(dt, B, N, D, K);
    L.split = o; o += split_bytes(dt, B, N, D, K);
    L.ring_part = o; o += align256((size_t)RING * B * assign_wgs_per_problem(dt, B, N, D, K) * ASSIGN_WAVES * 8);
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
    const size_t s2 = sort_ws_bytes(B, N, K), s3 = update_scratch_bytes(dt, B, N, D, K);
    o += s2 > s3 ? s2 : s3;
    L.total = o;
    return L;
}

size_t fit_ws_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K, int metric);

struct HostLayout {
    size_t stage_buf[2], cprep, xn, part, a, sids, sidx, counts, offs, status, updctr, sums, cnt, shk, ring_j,
        ring_s, scratch, total;
    int64_t chunk;
};

int64_t host_chunk(int64_t N, int64_t chunk_points) {
    int64_t c = chunk_points > 0 ? chunk_points : DEFAULT_CHUNK;
    if (c > N) c = N;
    return c;
}

// One half of kmeans_fit_staged's pinned buffer: a chunk of rows, rounded up to 256 bytes.
size_t stage_half_bytes(int dt, int64_t N, int64_t D, int64_t chunk_points) {
    return align256((size_t)host_chunk(N, chunk_points) * (size_t)D * elem_bytes(dt));
}

// Per-chunk regions of the streamed path, sized for every chunk: chunks hold `c` points except
// the last, which holds N - (nchunk-1) c.  The update's plan is not monotonic in the point count
// (its rows per wave are a power of two derived from the count, so a shorter chunk can have more
// partial records and counters), so each region covers both sizes.
//   host_scratch: the arg-sort tables or the update's partial records of one staged chunk;
//   host_updctr:  the update's arrival counters.
size_t host_scratch(int dt, int64_t N, int64_t D, int64_t K, int64_t c) {
    auto need = [&](int64_t n) {
        const size_t s2 = sort_ws_bytes(1, n, K), s3 = update_scratch_bytes(dt, 1, n, D, K);
        return s2 > s3 ? s2 : s3;
    };
    size_t sc = need(c);
    const int64_t last = N - (ceil_div(N, c) - 1) * c;
    if (last != c) {
        const size_t sl = need(last);
        if (sl > sc) sc = sl;
    }
    return sc;
}

size_t host_updctr(int dt, int64_t N, int64_t D, int64_t K, int64_t c) {
    size_t sc = update_ctr_bytes(dt, 1, c, D, K);
    const int64_t last = N - (ceil_div(N, c) - 1) * c;
    if (last != c) {
        const size_t sl = update_ctr_bytes(dt, 1, last, D, K);
        if (sl > sc) sc = sl;
    }
    return sc;
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
    L.cprep = o; o += prep_bytes(dt, B, N, D, K);
    const size_t c4 = align256((size_t)c * 4);
    L.xn = o; o += c4;
    // the assign's per-wave inertia partials of one chunk (a shorter last chunk has fewer)
    L.part = o; o += align256((size_t)assign_wgs_per_problem(dt, 1, c, D, K) * ASSIGN_WAVES * 8);
    L.a = o; o += c4;
    L.sids = o; o += c4;
    L.sidx = o; o += c4;
    L.counts = o; o += align256((size_t)K * 4);
    L.offs = o; o += align256((size_t)K * 4);
    L.status = o; o += STATUS_BYTES;
    L.updctr = o; o += host_updctr(dt, N, D, K, c);
    L.sums = o; o += align256((size_t)B * K * D * 4);
    L.cnt = o; o += align256((size_t)B * K * 4);
    L.shk = o; o += align256((size_t)B * K * 8);
    L.ring_j = o; o += align256((size_t)RING * B * 8);
    L.ring_s = o; o += align256((size_t)RING * B * 8);
    L.scratch = o;
    o += host_scratch(dt, N, D, K, c);
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
    return (float *)(cprep + align256((size_t)B * assign_tiles(dt, D, K) * 32 * d_pad * elem_bytes(dt)));
}

km_status_t do_prepare(int dt, const float *C, int64_t B, int64_t N, int64_t D, int64_t K, void *cprep,
                       hipStream_t s, int metric = KM_METRIC_L2) {
    const AssignCfg cfg = plan_assign(dt, B, N, D, K);
    KM_HIP(launch_prep_centroids(dt, C, cprep, prep_norms(dt, (char *)cprep, B, D, K, cfg.d_pad), (int)B, (int)K,
                                 (int)D, cfg.d_pad, s, metric != KM_METRIC_L2));
    return ok();
}

// sp: the K split and its buffers (nsplit 1: one scan per point tile, as kmeans_assign_prepared runs).
km_status_t do_assign_prepared(int dt, const void *x, const void *cprep, int64_t B, int64_t N, int64_t D, int64_t K,
                               const float *xn, int32_t *a, float *md, hipStream_t s,
                               const AssignSplit &sp = AssignSplit{}) {
    const AssignCfg cfg = plan_assign(dt, B, N, D, K);
    const float *cnh = prep_norms(dt, (char *)cprep, B, D, K, cfg.d_pad);
    KM_HIP(launch_assign(dt, cfg, x, cprep, cnh, xn, a, md, nullptr, (int)B, (int)N, (int)D, (int)K, s, sp));
    return ok();
}

// kmeans_assign in workspace ws (assign_ws bytes): the prepared operand, then (for a K-split
// plan) the keys, set to all ones here, and the norms.
km_status_t do_assign(int dt, const void *x, const float *C, int64_t B, int64_t N, int64_t D, int64_t K,
                      const float *xn, int32_t *a, float *md, void *ws, hipStream_t s) {
    KM_TRY(do_prepare(dt, C, B, N, D, K, ws, s));
    const AssignSplit sp = split_at(dt, B, N, D, K, (char *)ws + prep_bytes(dt, B, N, D, K));
    if (sp.nsplit > 1) KM_HIP(launch_fill_i32((int32_t *)sp.packed, 2 * B * N, -1, s));
    return do_assign_prepared(dt, x, ws, B, N, D, K, xn, a, md, s, sp);
}

km_status_t do_update(int dt, const void *x, const int32_t *sids, const int32_t *sidx, const int32_t *counts,
                      int64_t B, int64_t N, int64_t D, int64_t K, float *C, double *shift, void *ws, hipStream_t s) {
    KM_HIP(launch_update_ws(dt, x, sids, sidx, counts, (int)B, (int)N, (int)D, (int)K, C, shift, ws, s));
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
    const UpdCfg u = plan_update(dt, B, N, D, K);
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
    out->assign_splits = a.nsplit;
    return ok();
}

size_t kmeans_workspace_bytes(int op, km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K,
                              int64_t chunk_points) {
    if (check_shape(dt, B, N, D, K) != KM_OK) return 0;
    switch (op) {
        case KM_OP_ASSIGN: return assign_ws(dt, B, N, D, K);
        case KM_OP_ARGSORT: return argsort_ws(B, N, K);
        case KM_OP_UPDATE: return update_ws(dt, B, N, D, K);
        case KM_OP_FIT: return fit_ws_bytes(dt, B, N, D, K, KM_METRIC_L2);
        case KM_OP_FIT_HOST: return host_layout(dt, B, N, D, K, chunk_points).total;
        case KM_OP_FIT_DOT: return fit_ws_bytes(dt, B, N, D, K, KM_METRIC_DOT);
        case KM_OP_FIT_COSINE: return fit_ws_bytes(dt, B, N, D, K, KM_METRIC_COSINE);
        case KM_OP_STAGE_PINNED: return 2 * stage_half_bytes(dt, N, D, chunk_points);
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
    KM_TRY(check_ws(c_prep, c_prep_bytes, prep_bytes(dt, B, N, D, K)));
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
    KM_TRY(check_ws(c_prep, c_prep_bytes, prep_bytes(dt, B, N, D, K)));
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
    KM_TRY(check_ws(c_prep, c_prep_bytes, prep_bytes(dt, B, N, D, K)));
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
    KM_HIP(launch_argsort(assign, (int)B, (int)N, (int)K, sorted_ids, sorted_idx, counts, nullptr, (int32_t *)ws,
                          (char *)ws + STATUS_BYTES, (hipStream_t)stream));
    return ok();
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// The assignment without a caller workspace, for callers that cannot allocate: its scratch (the
// prepared centroid operand) lives in one static device array per GPU, whose address each device
// gets once from hipGetSymbolAddress; host code passes only that address, never the array's name.
// ------------------------------------------------------------------------------------------------
namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

km_status_t scratch_for_current_device(void **out) {
    int dev = 0;
    KM_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(KM_ERR_UNSUPPORTED, "device index %d beyond %d", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        KM_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return fail(KM_ERR_HIP, "hipGetSymbolAddress returned a null scratch address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ok();
}

}  // namespace

extern "C" {

km_status_t kmeans_assign_noalloc(const void *x, km_dtype_t dt, const float *centroids, int64_t B, int64_t N,
                                  int64_t D, int64_t K, const float *x_norms, int32_t *assign, float *min_dist,
                                  void *stream) {
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(centroids, "centroids"));
    KM_TRY(check_ptr(assign, "assign"));
    if (min_dist && !x_norms) return fail(KM_ERR_INVALID, "min_dist requires x_norms");
    if (((uintptr_t)x & 15) != 0) return fail(KM_ERR_INVALID, "x must be 16-byte aligned");
    const size_t need = assign_ws(dt, B, N, D, K);
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(KM_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; kmeans_assign_noalloc holds %zu",
                    need, NOALLOC_SCRATCH_BYTES);
    KM_TRY(check_device_arch());
    KM_TRY(require_device(x, "x"));
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(assign, "assign"));
    KM_TRY(require_device(min_dist, "min_dist"));
    KM_TRY(require_device(x_norms, "x_norms"));
    void *ws = nullptr;
    KM_TRY(scratch_for_current_device(&ws));
    // the prepare kernel writes every byte of the operand the assign kernel reads (padding
    // included), so nothing from an earlier call needs clearing
    return do_assign(dt, x, centroids, B, N, D, K, x_norms, assign, min_dist, ws, (hipStream_t)stream);
}

km_status_t kmeans_argsort_status(const void *ws, size_t ws_bytes, void *stream) {
    KM_TRY(check_ptr(ws, "ws"));
    if (((uintptr_t)ws & 255) != 0) return fail(KM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < STATUS_BYTES) return fail(KM_ERR_WORKSPACE, "workspace too small: %zu bytes", ws_bytes);
    KM_TRY(check_device_arch());
    KM_TRY(require_device(ws, "ws"));
    int32_t st = 0;
    KM_HIP(hipMemcpyAsync(&st, ws, 4, hipMemcpyDeviceToHost, (hipStream_t)stream));
    KM_HIP(hipStreamSynchronize((hipStream_t)stream));
    return status_word(st, "the arg-sort");
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

// Copy the first `n` iterations of a device ring [RING][B] into host[t0*B ...]; with `st_dev`,
// also the arg-sort's status word into *st_host (one wait for both).
km_status_t ring_to_host(const double *ring, double *host, int t0, int n, int64_t B, hipStream_t s,
                         const int32_t *st_dev = nullptr, int32_t *st_host = nullptr) {
    if (st_dev) KM_HIP(hipMemcpyAsync(st_host, st_dev, 4, hipMemcpyDeviceToHost, s));
    if (host && n > 0) KM_HIP(hipMemcpyAsync(host + (size_t)t0 * B, ring, (size_t)n * B * 8, hipMemcpyDeviceToHost, s));
    if (st_dev || (host && n > 0)) KM_HIP(hipStreamSynchronize(s));
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

// One chain of the device fit: a contiguous range of the problems with its own workspace layout
// and stream.
struct FitChain {
    int64_t B = 0, b0 = 0;
    hipStream_t s = nullptr;
    FitLayout L{};
    char *ws = nullptr;
    AssignCfg cfg{};
    int64_t wpb = 0;
    const void *xa = nullptr;
    float *C = nullptr, *xn = nullptr, *cnh = nullptr;
    const float *xn_in = nullptr;
    int32_t *a = nullptr, *sids = nullptr, *sidx = nullptr, *counts = nullptr, *status = nullptr;
    char *cprep = nullptr;
    double *ring_part = nullptr, *ring_j = nullptr, *ring_s = nullptr;
    void *scratch = nullptr;
    UpdMem mem;
    AssignSplit sp;
    bool fused_prep = false;
    UpdRefresh full_ref{}, ref{};
    int32_t st_host = 0;
    std::vector<double> j_host;  // two chains: this chain's inertia rows, read at a flush
};

// Two half-batch chains (see fit_device) where the iterations stop at `iters` (tol = 0), the batch
// has at least two problems, and each half runs the small-D assign without a K split (its grid
// fills the chip).
bool fit_two_chains(int dt, int64_t B, int64_t N, int64_t D, int64_t K) {
    if (B < 2) return false;
    for (const int64_t bh : {B / 2, B - B / 2}) {
        const AssignCfg c = plan_assign(dt, bh, N, D, K);
        if (c.path != 0 || c.nsplit != 1) return false;
    }
    return true;
}

// The device fit's workspace: one chain's layout, or, where two chains may run, the larger of that
// and the two halves' layouts one after the other.
size_t fit_ws_bytes(int dt, int64_t B, int64_t N, int64_t D, int64_t K, int metric) {
    size_t t = fit_layout(dt, B, N, D, K, metric).total;
    if (fit_two_chains(dt, B, N, D, K)) {
        const size_t t2 = fit_layout(dt, B / 2, N, D, K, metric).total + fit_layout(dt, B - B / 2, N, D, K, metric).total;
        t = t2 > t ? t2 : t;
    }
    return t;
}

// A chain's pointers, and its setup on its stream (point norms or unit rows, prepared centroids,
// zeroed counters).
km_status_t fit_chain_setup(FitChain &c, int dt, const void *x, int64_t B_all, int64_t N, int64_t D, int64_t K,
                            float *C, int32_t *assign, int metric) {
    const bool simm = metric != KM_METRIC_L2;
    const bool cosine = metric == KM_METRIC_COSINE;
    const int64_t B = c.B;
    const FitLayout &L = c.L;
    char *ws = c.ws;
    c.cfg = plan_assign(dt, B, N, D, K);
    const int64_t KT = assign_tiles(dt, D, K);
    c.wpb = assign_wgs_per_problem(dt, B, N, D, K) * ASSIGN_WAVES;  // inertia partials per problem
    c.C = C + c.b0 * K * D;
    c.xn = (float *)(ws + L.xn);
    c.a = assign ? assign + c.b0 * N : (int32_t *)(ws + L.a);
    c.sids = (int32_t *)(ws + L.sids);
    c.sidx = (int32_t *)(ws + L.sidx);
    c.counts = (int32_t *)(ws + L.counts);
    c.status = (int32_t *)(ws + L.status);
    c.cprep = ws + L.prep;
    c.cnh = (float *)(c.cprep + align256((size_t)B * KT * 32 * c.cfg.d_pad * elem_bytes(dt)));
    c.ring_part = (double *)(ws + L.ring_part);
    c.ring_j = (double *)(ws + L.ring_j);
    c.ring_s = (double *)(ws + L.ring_s);
    c.scratch = ws + L.scratch;
    c.mem.offs = (const int32_t *)(ws + L.offs);
    c.mem.ctr = (int32_t *)(ws + L.updctr);
    c.mem.scratch = c.scratch;
    c.mem.plan_B = B_all;  // each problem's update chunked as in a launch over the whole batch
    c.sp = split_at(dt, B, N, D, K, ws + L.split);
    c.fused_prep = update_refreshes_prep(dt, B, N, D);
    c.full_ref = UpdRefresh{c.cprep, c.cnh, c.cfg.d_pad, (int)KT, simm ? 1 : 0};
    c.ref = c.fused_prep ? c.full_ref : UpdRefresh{};
    const hipStream_t s = c.s;
    const void *xc = (const char *)x + (size_t)c.b0 * N * D * elem_bytes(dt);
    // the points the iterations use: x, or its unit rows for cosine k-means (whose centroids
    // are made unit rows too, in place)
    c.xa = xc;
    if (cosine) {
        KM_HIP(launch_normalize_rows(dt, xc, ws + L.xhat, B * N, (int)D, s));
        KM_HIP(launch_normalize_rows(KM_F32, c.C, c.C, B * K, (int)D, s));
        c.xa = ws + L.xhat;
    }
    // the small-D assign kernel computes the point norms it needs from its own registers; the
    // split-D kernel reads them.  The similarity metrics take zeros instead.
    c.xn_in = simm ? c.xn : (c.cfg.path == 0 ? nullptr : c.xn);
    if (simm) KM_HIP(launch_fill_i32((int32_t *)c.xn, B * N, 0, s));
    else if (c.xn_in) KM_HIP(launch_row_norms(dt, xc, c.xn, B * N, (int)D, s));
    KM_HIP(launch_prep_centroids(dt, c.C, c.cprep, c.cnh, (int)B, (int)K, (int)D, c.cfg.d_pad, s, simm ? 1 : 0));
    // the update's arrival counters start at zero and the split assign's keys at all ones; every
    // update and every split finish leave them so
    KM_HIP(launch_fill_i32(c.mem.ctr, (int64_t)(update_ctr_bytes(dt, B, N, D, K) / 4), 0, s));
    if (c.sp.nsplit > 1) KM_HIP(launch_fill_i32((int32_t *)c.sp.packed, 2 * B * N, -1, s));
    return ok();
}

// One Lloyd iteration of a chain after its assign: arg-sort (+ counts and the clusters' first
// positions), update (+ shift, + the next iteration's prepared centroids).
km_status_t fit_chain_rest(FitChain &c, int dt, int64_t N, int64_t D, int64_t K, float tol, int slot, bool more,
                           int metric) {
    const bool simm = metric != KM_METRIC_L2;
    const bool cosine = metric == KM_METRIC_COSINE;
    const int64_t B = c.B;
    const hipStream_t s = c.s;
    KM_HIP(launch_argsort(c.a, (int)B, (int)N, (int)K, c.sids, c.sidx, c.counts, (int32_t *)c.mem.offs, c.status,
                          c.scratch, s));
    double *shift = tol > 0.f ? c.ring_s + (size_t)slot * B : nullptr;
    if (cosine && c.fused_prep) {
        // one column block per row: the update finishes each cluster in place with the mean
        // direction s_k / ||s_k|| (and the shift and the refresh), like the Euclidean finish
        KM_HIP(launch_update(dt, c.xa, c.sids, c.sidx, c.counts, (int)B, (int)N, (int)D, (int)K, 0, c.C, shift,
                             nullptr, nullptr, c.full_ref, c.mem, s, 1));
    } else if (cosine) {
        // sums and counts per cluster, then the mean direction (with shift and refresh)
        float *sums = (float *)(c.ws + c.L.sums);
        int32_t *cnt = (int32_t *)(c.ws + c.L.cnt);
        KM_HIP(launch_fill_i32((int32_t *)sums, B * K * D, 0, s));
        KM_HIP(launch_fill_i32(cnt, B * K, 0, s));
        KM_HIP(launch_update(dt, c.xa, c.sids, c.sidx, c.counts, (int)B, (int)N, (int)D, (int)K, 1, nullptr, nullptr,
                             sums, cnt, UpdRefresh{}, c.mem, s));
        KM_HIP(launch_finalize_acc(dt, sums, cnt, c.C, shift, (double *)(c.ws + c.L.shk), c.full_ref, (int)B,
                                   (int)K, (int)D, s, 1));
    } else {
        KM_HIP(launch_update(dt, c.xa, c.sids, c.sidx, c.counts, (int)B, (int)N, (int)D, (int)K, 0, c.C, shift,
                             nullptr, nullptr, c.ref, c.mem, s));
        if (!c.fused_prep && more)
            KM_HIP(launch_prep_centroids(dt, c.C, c.cprep, c.cnh, (int)B, (int)K, (int)D, c.cfg.d_pad, s,
                                         simm ? 1 : 0));
    }
    return ok();
}

// The second chain's stream: created once per device and kept until the process ends, so that its
// hardware queue stays the same from call to call (a stream made per call can land on the queue of
// the caller's stream, and the chains then run one after the other).  Fits that run at the same
// time on one device share it: their second chains queue behind each other, each still waiting
// only for its own events.
std::mutex g_chain_mu;
hipStream_t g_chain_stream[64] = {};

km_status_t chain_stream(hipStream_t *out) {
    int dev = 0;
    KM_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return fail(KM_ERR_UNSUPPORTED, "device index %d beyond 64", dev);
    std::lock_guard<std::mutex> lock(g_chain_mu);
    if (!g_chain_stream[dev]) KM_HIP(hipStreamCreateWithFlags(&g_chain_stream[dev], hipStreamNonBlocking));
    *out = g_chain_stream[dev];
    return ok();
}

struct ChainSync {
    hipStream_t s2 = nullptr;
    hipEvent_t after_assign[2] = {nullptr, nullptr};
    hipEvent_t done2 = nullptr;
    ~ChainSync() {
        for (auto &e : after_assign)
            if (e) (void)hipEventDestroy(e);
        if (done2) (void)hipEventDestroy(done2);
    }
};

// metric: KM_METRIC_L2 (Lloyd), KM_METRIC_DOT (similarity x.c, mean update) or KM_METRIC_COSINE
// (unit rows, mean-direction update).  For the similarity metrics the assign kernels get zero
// norm terms (scores -x.c~) and zero point norms, so their per-point "distance" is
// -2 x.c~ and the per-iteration value returned is -1/2 of its sum: the total similarity.
//
// The iterations of different problems are independent, so where fit_two_chains holds the batch
// runs as two half-batch chains: the first on the caller's stream, the second on the library's
// stream for the device (chain_stream), with three events of this call.  Their FlashAssign launches alternate (each waits for the other chain's previous one) and
// never overlap, while each chain's arg-sort and update run beside the other chain's FlashAssign:
// MFMA-bound and memory-bound work share the chip.  Per problem every kernel does the work of the
// one-chain fit (the updates are planned for the whole batch), so the results are bit-identical.
km_status_t fit_device(int dt, const void *x, int64_t B, int64_t N, int64_t D, int64_t K, int iters, float tol,
                       float *C, int32_t *assign, double *inertia, int32_t *iters_done, char *ws, hipStream_t s,
                       int metric = KM_METRIC_L2) {
    const bool simm = metric != KM_METRIC_L2;
    const int nch = (tol <= 0.f && fit_two_chains(dt, B, N, D, K)) ? 2 : 1;
    FitChain ch[2];
    ChainSync sync;
    if (nch == 1) {
        ch[0].B = B;
        ch[0].L = fit_layout(dt, B, N, D, K, metric);
        ch[0].ws = ws;
        ch[0].s = s;
    } else {
        ch[0].B = B / 2;
        ch[1].B = B - B / 2;
        ch[1].b0 = B / 2;
        ch[0].L = fit_layout(dt, ch[0].B, N, D, K, metric);
        ch[1].L = fit_layout(dt, ch[1].B, N, D, K, metric);
        ch[0].ws = ws;
        ch[1].ws = ws + ch[0].L.total;
        ch[0].s = s;
        KM_TRY(chain_stream(&sync.s2));
        for (auto &e : sync.after_assign) KM_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        KM_HIP(hipEventCreateWithFlags(&sync.done2, hipEventDisableTiming));
        ch[1].s = sync.s2;
        // the second chain starts after the caller's earlier work on its stream
        KM_HIP(hipEventRecord(sync.done2, s));
        KM_HIP(hipStreamWaitEvent(sync.s2, sync.done2, 0));
    }
    for (int h = 0; h < nch; ++h) KM_TRY(fit_chain_setup(ch[h], dt, x, B, N, D, K, C, assign, metric));
    int done = 0, flushed = 0;
    for (int t = 0; t < iters; ++t) {
        const int slot = t - flushed;
        const bool more = t + 1 < iters;
        for (int h = 0; h < nch; ++h) {
            FitChain &c = ch[h];
            // two chains: this FlashAssign after the other chain's latest one
            if (nch == 2 && (h == 1 || t > 0)) KM_HIP(hipStreamWaitEvent(c.s, sync.after_assign[1 - h], 0));
            KM_HIP(launch_assign(dt, c.cfg, c.xa, c.cprep, c.cnh, c.xn_in, c.a, nullptr,
                                 c.ring_part + (size_t)slot * c.B * c.wpb, (int)c.B, (int)N, (int)D, (int)K, c.s,
                                 c.sp));
            if (nch == 2) KM_HIP(hipEventRecord(sync.after_assign[h], c.s));
            KM_TRY(fit_chain_rest(c, dt, N, D, K, tol, slot, more, metric));
        }
        done = t + 1;
        bool stop = false;
        if (tol > 0.f) {  // one chain
            double smax = 0.0;
            KM_TRY(read_shift_max(ch[0].ring_s + (size_t)slot * B, B, &smax, s));
            stop = smax < (double)tol;
        }
        if (slot + 1 == RING || stop || t + 1 == iters) {
            const bool last = stop || t + 1 == iters;
            for (int h = 0; h < nch; ++h) {
                FitChain &c = ch[h];
                KM_HIP(launch_sum_f64_rows(c.ring_part, (slot + 1) * (int)c.B, c.wpb, c.ring_j, c.s));
                if (last) KM_HIP(hipMemcpyAsync(&c.st_host, c.status, 4, hipMemcpyDeviceToHost, c.s));
                if (inertia && nch == 1)
                    KM_HIP(hipMemcpyAsync(inertia + (size_t)flushed * B, c.ring_j, (size_t)(slot + 1) * B * 8,
                                          hipMemcpyDeviceToHost, c.s));
                else if (inertia) {
                    // each chain into a host buffer of its own: copies from the two streams into
                    // interleaved columns of the caller's (pageable) rows are staged by the runtime
                    // and can overwrite each other's columns
                    c.j_host.resize((size_t)(slot + 1) * c.B);
                    KM_HIP(hipMemcpyAsync(c.j_host.data(), c.ring_j, (size_t)(slot + 1) * c.B * 8,
                                          hipMemcpyDeviceToHost, c.s));
                }
            }
            for (int h = 0; h < nch; ++h) KM_HIP(hipStreamSynchronize(ch[h].s));
            if (inertia && nch == 2)  // the chains' columns of the [iteration][problem] rows
                for (int h = 0; h < nch; ++h)
                    for (int i = 0; i <= slot; ++i)
                        std::copy_n(ch[h].j_host.data() + (size_t)i * ch[h].B, ch[h].B,
                                    inertia + (size_t)(flushed + i) * B + ch[h].b0);
            flushed = t + 1;
        }
        if (stop) break;
    }
    if (nch == 2) {  // the caller's stream waits for the second chain
        KM_HIP(hipEventRecord(sync.done2, sync.s2));
        KM_HIP(hipStreamWaitEvent(s, sync.done2, 0));
    }
    KM_HIP(hipStreamSynchronize(s));
    if (simm && inertia)
        for (int64_t i = 0; i < (int64_t)done * B; ++i) inertia[i] *= -0.5;
    if (iters_done) *iters_done = done;
    int32_t st = 0;
    for (int h = 0; h < nch; ++h) st |= ch[h].st_host;
    return status_word(st, "the fit's arg-sort");
}

struct StreamedPipe {
    hipStream_t cs = nullptr;
    hipEvent_t ev_copy[2] = {nullptr, nullptr};
    hipEvent_t ev_free[2] = {nullptr, nullptr};
    hipEvent_t ev_pin[2] = {nullptr, nullptr};  // staged source: a pinned half's device copy done
    ~StreamedPipe() {
        for (int i = 0; i < 2; ++i) {
            if (ev_copy[i]) (void)hipEventDestroy(ev_copy[i]);
            if (ev_free[i]) (void)hipEventDestroy(ev_free[i]);
            if (ev_pin[i]) (void)hipEventDestroy(ev_pin[i]);
        }
        if (cs) (void)hipStreamDestroy(cs);
    }
};

// Where the streamed path finds the points: one contiguous pinned [B, N, D] array, or (B = 1) the
// rows of one problem split over pinned blocks, block j holding rows [base[j], base[j+1]).
struct HostSource {
    const void *x = nullptr;            // contiguous, or nullptr
    const void *const *blocks = nullptr;
    const int64_t *base = nullptr;      // nblocks + 1 row offsets
    int nblocks = 0;
    size_t row_bytes = 0;
    // staged source (pageable x): two pinned chunk buffers that host threads fill before each
    // chunk's copy to the device; nullptr when x itself is pinned
    char *pin[2] = {nullptr, nullptr};
    // rows [lo, lo + n) of problem b lie in one block (the blocks hold whole chunks)
    const char *rows(int64_t b, int64_t N, int64_t lo) const {
        if (x) return (const char *)x + ((size_t)b * N + lo) * row_bytes;
        int j = 0;
        while (j + 1 < nblocks && base[j + 1] <= lo) ++j;
        return (const char *)blocks[j] + (size_t)(lo - base[j]) * row_bytes;
    }
};

// memcpy over up to 16 host threads (contiguous 4 KiB-aligned slices; one thread below 8 MiB).  A
// slice whose thread cannot be started is copied by the calling thread (no exception leaves here).
void parallel_copy(void *dst, const void *src, size_t bytes) {
    const unsigned hw = std::thread::hardware_concurrency();
    const size_t nt = std::max<size_t>(1, std::min<size_t>(16, hw ? hw : 1));
    if (nt == 1 || bytes < ((size_t)8 << 20)) {
        memcpy(dst, src, bytes);
        return;
    }
    const size_t per = (bytes / nt + 4095) & ~(size_t)4095;
    std::vector<std::thread> th;
    th.reserve(nt);
    for (size_t i = 0; i < nt && i * per < bytes; ++i) {
        const size_t lo = i * per, n = std::min(per, bytes - lo);
        try {
            th.emplace_back([=] { memcpy((char *)dst + lo, (const char *)src + lo, n); });
        } catch (...) {
            memcpy((char *)dst + lo, (const char *)src + lo, n);
        }
    }
    for (auto &t : th) t.join();
}

// metric as in fit_device.  Cosine k-means turns each staged chunk into unit rows in place (the
// staging buffer is a device copy of x) before its assign and update.
//
// A staged source (src.pin set, x in pageable memory) runs two chunks ahead instead of one: right
// after chunk q's kernels are queued, host threads copy chunk q + 2 into the pinned half that chunk
// q's device copy has left (waiting for that copy to end), and its device copy is queued behind
// chunk q's kernels, into the device buffer they free.  During chunk q's kernels the copy engine
// moves chunk q + 1 and the host copies chunk q + 2, so the GPU waits only where one of the copies
// takes longer than a chunk's kernels.
km_status_t fit_host(int dt, const HostSource &src, int64_t B, int64_t N, int64_t D, int64_t K, int iters, float tol,
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
    const int64_t KT = (int64_t)assign_tiles(dt, D, K);
    const size_t cprep_bytes = align256((size_t)B * KT * 32 * cfg.d_pad * es);
    float *cnh = (float *)(cprep + cprep_bytes);
    const size_t cprep_per_b = (size_t)KT * 32 * cfg.d_pad * es;
    float *xn = (float *)(ws + L.xn);
    double *part = (double *)(ws + L.part);
    int32_t *a_ws = (int32_t *)(ws + L.a);
    int32_t *sids = (int32_t *)(ws + L.sids);
    int32_t *sidx = (int32_t *)(ws + L.sidx);
    int32_t *counts = (int32_t *)(ws + L.counts);
    int32_t *status = (int32_t *)(ws + L.status);
    float *sums = (float *)(ws + L.sums);
    int32_t *cnt = (int32_t *)(ws + L.cnt);
    double *ring_j = (double *)(ws + L.ring_j);
    double *ring_s = (double *)(ws + L.ring_s);
    void *scratch = ws + L.scratch;
    UpdMem mem;
    mem.offs = (const int32_t *)(ws + L.offs);
    mem.ctr = (int32_t *)(ws + L.updctr);
    mem.scratch = scratch;
    const UpdRefresh ref{cprep, cnh, cfg.d_pad, (int)KT, simm ? 1 : 0};

    StreamedPipe P;
    KM_HIP(hipStreamCreateWithFlags(&P.cs, hipStreamNonBlocking));
    const bool staged = src.pin[0] != nullptr;
    for (int i = 0; i < 2; ++i) {
        KM_HIP(hipEventCreateWithFlags(&P.ev_copy[i], hipEventDisableTiming));
        KM_HIP(hipEventCreateWithFlags(&P.ev_free[i], hipEventDisableTiming));
        if (staged) {
            KM_HIP(hipEventCreateWithFlags(&P.ev_pin[i], hipEventDisableTiming));
            KM_HIP(hipEventRecord(P.ev_pin[i], P.cs));  // both halves free at the start
        }
    }
    // chunk sequence (iteration-major); copies run one chunk ahead (two for a staged source), across
    // iteration borders
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
        const size_t bytes = (size_t)n * D * es;
        const void *from = src.rows(b, N, lo);
        if (staged) {  // into pinned half `buf`, once its previous device copy (chunk q - 2) is done
            KM_HIP(hipEventSynchronize(P.ev_pin[buf]));
            parallel_copy(src.pin[buf], from, bytes);
            from = src.pin[buf];
        }
        KM_HIP(hipStreamWaitEvent(P.cs, P.ev_free[buf], 0));
        KM_HIP(hipMemcpyAsync(stage_buf[buf], from, bytes, hipMemcpyHostToDevice, P.cs));
        KM_HIP(hipEventRecord(P.ev_copy[buf], P.cs));
        if (staged) KM_HIP(hipEventRecord(P.ev_pin[buf], P.cs));
        return ok();
    };
    const int64_t total_q = (int64_t)iters * per_iter;  // chunks of a fit that runs all iterations
    // the copy stream must not start before work already queued on `s` that it depends on
    KM_HIP(hipEventRecord(P.ev_free[0], s));
    KM_HIP(hipEventRecord(P.ev_free[1], s));
    KM_TRY(issue_copy(0));
    if (staged && total_q > 1) KM_TRY(issue_copy(1));
    if (cosine) KM_HIP(launch_normalize_rows(KM_F32, C, C, B * K, (int)D, s));
    // the similarity metrics take zero point norms (their per-point value is then -2 x.c~)
    if (simm) KM_HIP(launch_fill_i32((int32_t *)xn, chunk, 0, s));
    KM_HIP(launch_prep_centroids(dt, C, cprep, cnh, (int)B, (int)K, (int)D, cfg.d_pad, s, simm ? 1 : 0));
    // the update's arrival counters start at zero; every update leaves them zero
    KM_HIP(launch_fill_i32(mem.ctr, (int64_t)(host_updctr(dt, N, D, K, chunk) / 4), 0, s));
    int64_t q = 0;
    int done = 0, flushed = 0;
    int32_t st_host = 0;
    for (int t = 0; t < iters; ++t) {
        const int slot = t - flushed;
        KM_HIP(launch_fill_i32((int32_t *)sums, B * K * D, 0, s));
        KM_HIP(launch_fill_i32(cnt, B * K, 0, s));
        KM_HIP(launch_fill_i32((int32_t *)(ring_j + (size_t)slot * B), 2 * B, 0, s));
        for (int64_t i = 0; i < per_iter; ++i, ++q) {
            const bool more = (t + 1 < iters) || (i + 1 < per_iter);
            if (more && !staged) KM_TRY(issue_copy(q + 1));
            int64_t b, lo, n;
            chunk_rows(q, &b, &lo, &n);
            const int buf = (int)(q & 1);
            const void *xc = stage_buf[buf];
            KM_HIP(hipStreamWaitEvent(s, P.ev_copy[buf], 0));
            int32_t *ac = assign ? assign + (size_t)b * N + lo : a_ws;
            if (cosine) KM_HIP(launch_normalize_rows(dt, xc, stage_buf[buf], n, (int)D, s));
            if (cfg.path != 0 && !simm) KM_HIP(launch_row_norms(dt, xc, xn, n, (int)D, s));
            // one scan per point tile: chunks of 2^24 points fill the chip by themselves
            KM_HIP(launch_assign(dt, cfg, xc, cprep + (size_t)b * cprep_per_b, cnh + (size_t)b * KT * 32,
                                 (cfg.path == 0 && !simm) ? nullptr : xn, ac, nullptr, part, 1, (int)n, (int)D,
                                 (int)K, s, AssignSplit{}));
            // the chunk's inertia: its per-wave partials in order, added to the problem's sum
            KM_HIP(launch_sum_f64_rows(part, 1, ceil_div(n, (int64_t)cfg.block_n) * ASSIGN_WAVES,
                                       ring_j + (size_t)slot * B + b, s, 1));
            KM_HIP(launch_argsort(ac, 1, (int)n, (int)K, sids, sidx, counts, (int32_t *)mem.offs, status, scratch, s));
            KM_HIP(launch_update(dt, xc, sids, sidx, counts, 1, (int)n, (int)D, (int)K, 1, nullptr, nullptr,
                                 sums + (size_t)b * K * D, cnt + (size_t)b * K, UpdRefresh{}, mem, s));
            KM_HIP(hipEventRecord(P.ev_free[buf], s));
            if (staged && q + 2 < total_q) KM_TRY(issue_copy(q + 2));
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
            const bool last = stop || t + 1 == iters;
            KM_TRY(ring_to_host(ring_j, inertia, flushed, slot + 1, B, s, last ? status : nullptr, &st_host));
            flushed = t + 1;
        }
        if (stop) break;
    }
    KM_HIP(hipStreamSynchronize(s));
    KM_HIP(hipStreamSynchronize(P.cs));
    if (simm && inertia)
        for (int64_t i = 0; i < (int64_t)done * B; ++i) inertia[i] *= -0.5;
    if (iters_done) *iters_done = done;
    return status_word(st_host, "the fit's arg-sort");
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
        KM_TRY(check_ws(ws, ws_bytes, fit_ws_bytes(dt, B, N, D, K, (int)metric)));
        return fit_device(dt, x, B, N, D, K, iters, tol, centroids, assign, objective, iters_done, (char *)ws,
                          (hipStream_t)stream, (int)metric);
    }
    KM_TRY(check_ws(ws, ws_bytes, host_layout(dt, B, N, D, K, chunk_points).total));
    HostSource src;
    src.x = x;
    src.row_bytes = (size_t)D * elem_bytes(dt);
    return fit_host(dt, src, B, N, D, K, iters, tol, chunk_points, centroids, assign, objective, iters_done,
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
        KM_TRY(check_ws(ws, ws_bytes, fit_ws_bytes(dt, B, N, D, K, KM_METRIC_L2)));
        return fit_device(dt, x, B, N, D, K, iters, tol, centroids, assign, inertia, iters_done, (char *)ws, s);
    }
    KM_TRY(check_ws(ws, ws_bytes, host_layout(dt, B, N, D, K, chunk_points).total));
    HostSource src;
    src.x = x;
    src.row_bytes = (size_t)D * elem_bytes(dt);
    return fit_host(dt, src, B, N, D, K, iters, tol, chunk_points, centroids, assign, inertia, iters_done, (char *)ws,
                    s);
}

extern "C" km_status_t kmeans_fit_blocks(const void *const *x_blocks, const int64_t *block_points, int32_t nblocks,
                                         km_dtype_t dt, int64_t D, int64_t K, int32_t iters, float tol,
                                         int64_t chunk_points, float *centroids, int32_t *assign, double *inertia,
                                         int32_t *iters_done, void *ws, size_t ws_bytes, void *stream) {
    if (!x_blocks || !block_points) return fail(KM_ERR_INVALID, "x_blocks and block_points must not be NULL");
    if (nblocks < 1 || nblocks > 4096) return fail(KM_ERR_INVALID, "nblocks must be in [1, 4096] (got %d)", nblocks);
    if (chunk_points < 0) return fail(KM_ERR_INVALID, "chunk_points must be >= 0");
    int64_t N = 0;
    for (int j = 0; j < nblocks; ++j) {
        if (!x_blocks[j]) return fail(KM_ERR_INVALID, "block %d is NULL", j);
        if (block_points[j] < 1) return fail(KM_ERR_INVALID, "block %d holds %lld points", j, (long long)block_points[j]);
        if (((uintptr_t)x_blocks[j] & 15) != 0) return fail(KM_ERR_INVALID, "block %d must be 16-byte aligned", j);
        N += block_points[j];
        if (N >= MAX_N) return fail(KM_ERR_INVALID, "the blocks hold 2^31 points or more");
    }
    KM_TRY(check_shape(dt, 1, N, D, K));
    const int64_t c = host_chunk(N, chunk_points);
    for (int j = 0; j + 1 < nblocks; ++j)
        if (block_points[j] % c != 0)
            return fail(KM_ERR_INVALID, "block %d holds %lld points, not a multiple of the %lld-point chunk", j,
                        (long long)block_points[j], (long long)c);
    KM_TRY(check_ptr(centroids, "centroids"));
    if (iters < 1) return fail(KM_ERR_INVALID, "iters must be >= 1");
    if (!(tol >= 0.f)) return fail(KM_ERR_INVALID, "tol must be >= 0");
    if (((uintptr_t)centroids & 15) != 0) return fail(KM_ERR_INVALID, "centroids must be 16-byte aligned");
    if (!ws) return fail(KM_ERR_WORKSPACE, "workspace is NULL");
    KM_TRY(check_ws(ws, ws_bytes, host_layout(dt, 1, N, D, K, chunk_points).total));
    KM_TRY(check_device_arch());
    for (int j = 0; j < nblocks; ++j)
        if (pointer_kind(x_blocks[j]) != PTR_PINNED_HOST)
            return fail(KM_ERR_UNSUPPORTED, "block %d is not pinned host memory", j);
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(assign, "assign"));
    KM_TRY(require_device(ws, "ws"));
    std::vector<int64_t> base((size_t)nblocks + 1, 0);
    for (int j = 0; j < nblocks; ++j) base[(size_t)j + 1] = base[(size_t)j] + block_points[j];
    HostSource src;
    src.blocks = x_blocks;
    src.base = base.data();
    src.nblocks = nblocks;
    src.row_bytes = (size_t)D * elem_bytes(dt);
    return fit_host(dt, src, 1, N, D, K, iters, tol, chunk_points, centroids, assign, inertia, iters_done, (char *)ws,
                    (hipStream_t)stream);
}

extern "C" km_status_t kmeans_fit_staged(const void *x, km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K,
                                         int32_t iters, float tol, int64_t chunk_points, void *pinned_stage,
                                         size_t pinned_bytes, float *centroids, int32_t *assign, double *inertia,
                                         int32_t *iters_done, void *ws, size_t ws_bytes, void *stream) {
    KM_TRY(check_shape(dt, B, N, D, K));
    KM_TRY(check_ptr(x, "x"));
    KM_TRY(check_ptr(pinned_stage, "pinned_stage"));
    KM_TRY(check_ptr(centroids, "centroids"));
    if (iters < 1) return fail(KM_ERR_INVALID, "iters must be >= 1");
    if (!(tol >= 0.f)) return fail(KM_ERR_INVALID, "tol must be >= 0");
    if (chunk_points < 0) return fail(KM_ERR_INVALID, "chunk_points must be >= 0");
    if (((uintptr_t)centroids & 15) != 0) return fail(KM_ERR_INVALID, "centroids must be 16-byte aligned");
    if (((uintptr_t)x & 15) != 0) return fail(KM_ERR_INVALID, "x must be 16-byte aligned");
    if (((uintptr_t)pinned_stage & 15) != 0) return fail(KM_ERR_INVALID, "pinned_stage must be 16-byte aligned");
    const size_t half = stage_half_bytes(dt, N, D, chunk_points);
    if (pinned_bytes < 2 * half)
        return fail(KM_ERR_WORKSPACE, "pinned_stage too small: %zu < %zu bytes", pinned_bytes, 2 * half);
    if (!ws) return fail(KM_ERR_WORKSPACE, "workspace is NULL");
    KM_TRY(check_ws(ws, ws_bytes, host_layout(dt, B, N, D, K, chunk_points).total));
    KM_TRY(check_device_arch());
    if (pointer_kind(x) == PTR_DEVICE) return fail(KM_ERR_INVALID, "x must be host memory (got device memory)");
    if (pointer_kind(pinned_stage) != PTR_PINNED_HOST)
        return fail(KM_ERR_UNSUPPORTED, "pinned_stage is not pinned host memory");
    KM_TRY(require_device(centroids, "centroids"));
    KM_TRY(require_device(assign, "assign"));
    KM_TRY(require_device(ws, "ws"));
    HostSource src;
    src.x = x;
    src.row_bytes = (size_t)D * elem_bytes(dt);
    src.pin[0] = (char *)pinned_stage;
    src.pin[1] = (char *)pinned_stage + half;
    return fit_host(dt, src, B, N, D, K, iters, tol, chunk_points, centroids, assign, inertia, iters_done, (char *)ws,
                    (hipStream_t)stream);
}
