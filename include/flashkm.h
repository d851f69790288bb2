/*
 * flashkm.h -- C-ABI of an MI355X (gfx950) library for batched Lloyd k-means:
 * FlashAssign (streaming x.c^T contraction with an online arg-min) and the
 * sort-inverse update (stable arg-sort of the assignment vector, segmented
 * per-cluster sums, one write per segment).
 *
 * Sources are the Flash-KMeans pages:
 *   - paper summary "Flash-KMeans: Fast and Memory-Efficient Exact K-Means",
 *     sections "Key claims" and "Method";
 *   - paper digest "Flash-KMeans：快速且内存高效精确K-Means聚类", sections
 *     "argsort与分段规约", "核心方法" and "方法步骤详情" (steps (1)-(3));
 *   - the flash-kmeans README, sections "Usage", "Large tensor Benchmark" and
 *     "Large-D and dtype support".
 *
 * Conventions shared by every call:
 *   - Arrays are dense, row-major, C-contiguous.  "Device" means memory the
 *     GPU can address directly (hipMalloc / PyTorch CUDA tensors); "pinned
 *     host" means page-locked host memory from hipHostMalloc or
 *     torch.empty(..., pin_memory=True).
 *   - B independent problems share K.  Shapes: x [B, N, D]; centroids
 *     [B, K, D] float32; assign / sorted arrays [B, N] int32; counts [B, K]
 *     int32.  x, and the centroids that an update or a fit writes, are
 *     16-byte aligned.
 *   - The caller owns every buffer.  The library allocates no device memory:
 *     temporary storage comes from the caller's workspace `ws` of `ws_bytes`
 *     bytes, sized by kmeans_workspace_bytes() and 256-byte aligned.  Calls on
 *     one stream run in order and may share one workspace; calls that may run
 *     at the same time (other streams) need workspaces of their own, as their
 *     intermediate arrays (labels, digit tables, partial sums) live there.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue their
 *     kernels on it and return without waiting, except kmeans_fit (see there).
 *   - Errors are explicit: every call returns a km_status_t; there is no
 *     silent fallback.  Argument validation happens before any HIP call, so
 *     invalid arguments are reported even on a machine without a GPU.
 *     kmeans_last_error() returns a message for the calling thread's last
 *     non-OK status.
 *   - Preconditions: finite input values (not checked).  The arg-sort skips
 *     labels outside [0, K) and reports them through kmeans_argsort_status
 *     (kmeans_fit through its return value).  kmeans_update needs sorted arrays
 *     and counts produced by kmeans_argsort_ids from one assignment; it does
 *     not check that, and clamps every index it derives from them, so
 *     inconsistent inputs give wrong numbers, not accesses out of bounds.
 *   - Limits: 1 <= B, 1 <= K <= N < 2^31, 1 <= D <= 4096, B*N < 2^31,
 *     K <= 2^24.
 */
#ifndef FLASHKM_H
#define FLASHKM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KM_F32 = 0, KM_F16 = 1, KM_BF16 = 2 } km_dtype_t;

typedef enum {
    KM_OK = 0,
    KM_ERR_INVALID = -1,      /* bad shape, null required pointer, unknown dtype/op, bad iters/tol */
    KM_ERR_UNSUPPORTED = -2,  /* e.g. pageable host memory, host pointer where device memory is required */
    KM_ERR_WORKSPACE = -3,    /* ws too small or misaligned */
    KM_ERR_HIP = -4           /* a HIP runtime call failed; message carries hipGetErrorString */
} km_status_t;

typedef enum {
    KM_OP_ASSIGN = 1,
    KM_OP_ARGSORT = 2,
    KM_OP_UPDATE = 3,
    KM_OP_FIT = 4,            /* kmeans_fit with device-resident x */
    KM_OP_FIT_HOST = 5,       /* kmeans_fit with x in pinned host memory (streamed path) */
    KM_OP_FIT_DOT = 6,        /* kmeans_fit_metric, KM_METRIC_DOT, device-resident x */
    KM_OP_FIT_COSINE = 7,     /* kmeans_fit_metric, KM_METRIC_COSINE, device-resident x */
    KM_OP_STAGE_PINNED = 8    /* kmeans_fit_staged: bytes of its pinned host staging buffer (its
                                 device workspace is that of KM_OP_FIT_HOST) */
} km_op_t;

/* Similarity of a point and a centroid (see kmeans_fit_metric). */
typedef enum {
    KM_METRIC_L2 = 0,         /* squared Euclidean distance: Lloyd's k-means */
    KM_METRIC_DOT = 1,        /* dot product x.c, maximised */
    KM_METRIC_COSINE = 2      /* cosine x.c / (||x|| ||c||), maximised (spherical k-means) */
} km_metric_t;

/*
 * Tile plan chosen by the analytic heuristic (paper summary, "Key claims": a
 * cache-aware heuristic picks kernel configurations from cache sizes and the
 * problem shape instead of an exhaustive autotune).  Derived from gfx950 LDS
 * (160 KiB per CU), register file (512 VGPRs per lane per SIMD), L2 (4 MiB
 * per XCD) and (B, N, K, D, dtype); no timing runs.
 */
typedef struct {
    int32_t path;          /* 0: small-D (points held in registers); 1: split-D (D tiled through LDS) */
    int32_t d_pad;         /* D rounded up to the kernel's register tile */
    int32_t point_blocks;  /* 32-point MFMA column blocks per wave */
    int32_t waves;         /* waves per workgroup */
    int32_t block_n;       /* points per workgroup */
    int32_t block_k;       /* centroids per LDS stage (small-D) or per register group (split-D) */
    int32_t block_d;       /* split-D: elements of D per LDS stage; 0 for small-D */
    int32_t lds_bytes;     /* LDS per assign workgroup */
    int32_t vgpr_est;      /* estimated VGPRs per lane of the assign kernel */
    int32_t assign_wgs;    /* assign workgroups per launch */
    int32_t sort_bits;     /* radix digit width */
    int32_t sort_passes;   /* counting-sort passes */
    int32_t sort_tile;     /* keys per sort workgroup */
    int32_t upd_rows;      /* sorted rows per update wave */
    int32_t upd_vec;       /* elements per update vector load */
    int32_t upd_lanes;     /* lanes covering one row in the update */
    int32_t assign_splits; /* small-D: workgroups per point tile, each scanning a share of the
                              centroids (> 1 when B * ceil(N / block_n) cannot fill the chip) */
} km_plan_t;

/* Fill *out with the plan for this problem.  Host only; no HIP call. */
km_status_t kmeans_plan(km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K, km_plan_t *out);

/*
 * Workspace bytes needed by `op` (a km_op_t) for this shape.  `chunk_points`
 * is used by KM_OP_FIT_HOST only (0 = default of 2^24 points, clamped to N).
 * Returns 0 for invalid arguments.  Host only; no HIP call.
 */
size_t kmeans_workspace_bytes(int op, km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K,
                              int64_t chunk_points);

/*
 * ||x_i||^2 for every point (paper digest, "方法步骤详情" step (1): the squared
 * norms of the points are computed before the centroid scan).
 *   x        device [B, N, D] of dtype dt
 *   x_norms  device [B, N] float32 out (fp32 accumulation)
 */
km_status_t kmeans_row_norms(const void *x, km_dtype_t dt, int64_t B, int64_t N, int64_t D,
                             float *x_norms, void *stream);

/*
 * FlashAssign (paper summary, "Method"; paper digest, "核心方法" and step (1)):
 * for every point, a_i = argmin_k ||c~_k||^2 - 2 x_i . c~_k, scanning
 * centroids tile by tile with a running (min, index) per point, never
 * writing the N x K distance matrix.  c~ = dtype(fp32 centroids), rounded to
 * nearest even; the contraction runs on MFMA in dt with fp32 accumulation.
 * Ties go to the lowest centroid index.
 *   x          device [B, N, D] dtype dt
 *   centroids  device [B, K, D] float32 (the master copy; read only)
 *   x_norms    device [B, N] float32 or NULL; required when min_dist != NULL
 *   assign     device [B, N] int32 out
 *   min_dist   device [B, N] float32 out or NULL: x_norms_i + min score
 *              (the squared distance to the chosen centroid, in fp32)
 *   ws         workspace >= kmeans_workspace_bytes(KM_OP_ASSIGN, ...)
 */
km_status_t kmeans_assign(const void *x, km_dtype_t dt, const float *centroids, int64_t B, int64_t N,
                          int64_t D, int64_t K, const float *x_norms, int32_t *assign,
                          float *min_dist, void *ws, size_t ws_bytes, void *stream);

/*
 * kmeans_assign without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as kmeans_assign, minus ws.
 * Its scratch (the prepared centroids, kmeans_workspace_bytes(KM_OP_ASSIGN,
 * ...) bytes) lives in one static device array of 32 MiB per GPU, which the
 * library holds until the process ends; larger shapes return
 * KM_ERR_WORKSPACE.  Every call on a GPU uses that GPU's array: calls that
 * may overlap on one GPU (other streams, other threads) race and must not be
 * made.  The call allocates nothing.
 */
km_status_t kmeans_assign_noalloc(const void *x, km_dtype_t dt, const float *centroids, int64_t B, int64_t N,
                                  int64_t D, int64_t K, const float *x_norms, int32_t *assign,
                                  float *min_dist, void *stream);

/*
 * The two halves of kmeans_assign, for callers that assign repeatedly against
 * the same centroids (and to time the FlashAssign kernel on its own).
 *
 * kmeans_prepare_centroids: the centroid side of the contraction (paper
 * digest, "核心方法": ||x - c||^2 = ||x||^2 + ||c||^2 - 2 x.c, so only c~ and
 * ||c~||^2 are needed per centroid): c~ = dtype(fp32 centroids) (nearest
 * even), laid out in the assign kernel's tile order, followed by ||c~||^2 / 2
 * in fp32 computed from c~.
 *   centroids  device [B, K, D] float32 (read only)
 *   c_prep     device out, opaque, c_prep_bytes >= kmeans_workspace_bytes(
 *              KM_OP_ASSIGN, dt, B, N, D, K) for any N (N = K is enough),
 *              256-byte aligned; valid for calls with the same (dt, B, D, K)
 *
 * kmeans_assign_prepared: FlashAssign as kmeans_assign, from a c_prep written
 * by kmeans_prepare_centroids for the same (dt, B, D, K).  It always runs one
 * scan of all centroids per point tile (no K split, see km_plan_t), so its
 * result is the same as kmeans_assign's.
 */
km_status_t kmeans_prepare_centroids(const float *centroids, km_dtype_t dt, int64_t B, int64_t N, int64_t D,
                                     int64_t K, void *c_prep, size_t c_prep_bytes, void *stream);
km_status_t kmeans_assign_prepared(const void *x, km_dtype_t dt, const void *c_prep, size_t c_prep_bytes,
                                   int64_t B, int64_t N, int64_t D, int64_t K, const float *x_norms,
                                   int32_t *assign, float *min_dist, void *stream);

/*
 * Stable ascending arg-sort of each problem's assignment vector (paper
 * digest, "argsort与分段规约": [3,1,2,1,3,2] -> ids [1,1,2,2,3,3], indices
 * [1,3,2,5,0,4]); a hand-written LDS counting/radix sort keyed by cluster id.
 *   assign      device [B, N] int32, values in [0, K)
 *   sorted_ids  device [B, N] int32 out: assign[b, sorted_idx[b, j]]
 *   sorted_idx  device [B, N] int32 out: 0-based point indices, equal ids in
 *               increasing index order
 *   counts      device [B, K] int32 out or NULL: points per cluster
 *   ws          workspace >= kmeans_workspace_bytes(KM_OP_ARGSORT, ...); its
 *               first 4 bytes become the call's status word (below)
 * Labels outside [0, K) are left out of the sort and the counts (the outputs
 * are then unspecified, and no access leaves the output rows) and the status
 * word records them.  The call returns without waiting for the GPU, so it
 * cannot return that as its status; kmeans_argsort_status does.
 */
km_status_t kmeans_argsort_ids(const int32_t *assign, int64_t B, int64_t N, int64_t K,
                               int32_t *sorted_ids, int32_t *sorted_idx, int32_t *counts, void *ws,
                               size_t ws_bytes, void *stream);

/*
 * Waits for `stream` and reports the status word of the last
 * kmeans_argsort_ids call made with workspace `ws` on it: KM_OK, or
 * KM_ERR_INVALID when that call met labels outside [0, K) (or a label array
 * that changed while it ran).  Same digest section as kmeans_argsort_ids.
 *   ws, ws_bytes  the workspace passed to kmeans_argsort_ids (device)
 */
km_status_t kmeans_argsort_status(const void *ws, size_t ws_bytes, void *stream);

/*
 * Sort-inverse update (paper summary, "Method"; paper digest, step (2)):
 * each wave takes a contiguous chunk of the sorted order, gathers the rows
 * of the unpermuted x through sorted_idx, sums each cluster-id segment on
 * chip in fp32, and writes once per segment; a segment spread over three or
 * more chunks leaves one partial per chunk, and the last of its waves to
 * finish adds them in chunk order (deterministic, no float atomics, one
 * integer atomic per chunk of such a segment).  Then c_k <- s_k / n_k; a
 * cluster with n_k == 0 keeps its centroid.
 *   x           device [B, N, D] dtype dt
 *   sorted_ids, sorted_idx, counts   from kmeans_argsort_ids for the same
 *               assignment
 *   centroids   device [B, K, D] float32 in: C_t, out: C_{t+1}
 *   shift       device [B] double out or NULL: sum_k ||C_{t+1,k} - C_{t,k}||^2
 */
km_status_t kmeans_update(const void *x, km_dtype_t dt, const int32_t *sorted_ids,
                          const int32_t *sorted_idx, const int32_t *counts, int64_t B, int64_t N,
                          int64_t D, int64_t K, float *centroids, double *shift, void *ws,
                          size_t ws_bytes, void *stream);

/*
 * Lloyd's loop (README, "Usage": batch_kmeans_Euclid(x, n_clusters,
 * max_iters, tol, init_centroids)): row norms once, then per iteration
 * assign -> inertia -> arg-sort -> update.  With tol > 0 the run stops after
 * iteration t when max_b shift_t[b] < tol (one host read per iteration);
 * with tol == 0 all `iters` iterations run without a host wait until the end.
 * Returns KM_ERR_INVALID (after the run) if the arg-sort of the last
 * iteration met labels outside [0, K), which the fit's own assignment never
 * produces.
 * If x is pinned host memory, the streamed path runs instead (README,
 * "Large tensor Benchmark"; paper digest, step (3)): each iteration streams
 * x in chunks of `chunk_points` points with hipMemcpyAsync into two device
 * staging buffers, overlapping the copy of chunk i+1 with assign / arg-sort
 * / partial update of chunk i, and divides after the last chunk.  x is never
 * cached on the device across iterations.
 *   x            device or pinned host [B, N, D] dtype dt (pageable host
 *                memory -> KM_ERR_UNSUPPORTED; kmeans_fit_staged takes it)
 *   iters        maximum iterations (>= 1); tol >= 0
 *   chunk_points streamed path only (0 = 2^24, clamped to N)
 *   centroids    device [B, K, D] float32 in: init, out: final
 *   assign       device [B, N] int32 out or NULL: labels of the last assignment
 *   inertia      host double [iters * B] out or NULL: per iteration and
 *                problem, sum_i ||x_i - c~_{a_i}||^2 (fp32 terms, fp64 sum)
 *   iters_done   host int32 out or NULL
 * Returns after the work has finished (it synchronises `stream`).  The
 * streamed path creates one copy stream and four events for the call and
 * destroys them before it returns.  With device x, tol = 0 and a batch whose
 * halves each fill the GPU, the fit runs the two halves as two chains (their
 * assignments alternating, each half's arg-sort and update running beside
 * the other half's assignment; the results are bit-identical to one chain):
 * the second half on a stream the library creates once per device and keeps
 * until the process ends, with three events created for the call.
 */
km_status_t kmeans_fit(const void *x, km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K,
                       int32_t iters, float tol, int64_t chunk_points, float *centroids,
                       int32_t *assign, double *inertia, int32_t *iters_done, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * The streamed path for one problem whose points lie in several pinned host
 * blocks, for point sets too large for one pinned allocation (README, "Large
 * tensor Benchmark"; paper digest, step (3)).  The same as kmeans_fit on
 * pinned host x with B = 1, where x is the concatenation of the blocks.
 *   x_blocks      nblocks pointers to pinned host [block_points[j], D] arrays of
 *                 dtype dt, 16-byte aligned; every block but the last holds a
 *                 multiple of the chunk (chunk_points, 0 = 2^24, clamped to the
 *                 total), so no staged chunk straddles two blocks
 *   block_points  host int64 [nblocks]; their sum N < 2^31
 *   centroids     device [1, K, D] float32 in: init, out: final
 *   assign        device [1, N] int32 out or NULL (point order: block 0 first)
 *   ws            >= kmeans_workspace_bytes(KM_OP_FIT_HOST, dt, 1, N, D, K,
 *                 chunk_points)
 * Other arguments and the return as kmeans_fit.
 */
km_status_t kmeans_fit_blocks(const void *const *x_blocks, const int64_t *block_points, int32_t nblocks,
                              km_dtype_t dt, int64_t D, int64_t K, int32_t iters, float tol,
                              int64_t chunk_points, float *centroids, int32_t *assign, double *inertia,
                              int32_t *iters_done, void *ws, size_t ws_bytes, void *stream);

/*
 * The streamed path for points in pageable host memory, staged through a
 * pinned host buffer that the caller provides: for hosts that cannot pin the
 * whole point set (README, "Large tensor Benchmark"; paper digest, step (3):
 * data that does not fit the GPU streams through it chunk by chunk).  Host
 * threads of the call copy chunk q + 2 into one half of the pinned buffer
 * while the GPU works on chunk q and the copy engine moves chunk q + 1 to the
 * device, so where those copies keep up the iteration tracks the GPU's work.
 * The result is that of kmeans_fit on pinned host x with the same chunk,
 * bit for bit.
 *   x             host [B, N, D] of dtype dt (pageable or pinned), 16-byte
 *                 aligned; read by host threads during the call
 *   pinned_stage  pinned host memory (hipHostMalloc or a pinned allocation),
 *                 16-byte aligned, of at least
 *                 kmeans_workspace_bytes(KM_OP_STAGE_PINNED, dt, B, N, D, K,
 *                 chunk_points) bytes: two chunk buffers; overwritten
 *   ws            device, >= kmeans_workspace_bytes(KM_OP_FIT_HOST, ...)
 * Other arguments and the return as kmeans_fit (KM_ERR_INVALID for device x,
 * KM_ERR_UNSUPPORTED for a pinned_stage that is not pinned host memory).  It
 * creates one copy stream and six events for the call, and up to 16 host
 * threads per chunk copy, and returns after the work has finished.
 */
km_status_t kmeans_fit_staged(const void *x, km_dtype_t dt, int64_t B, int64_t N, int64_t D, int64_t K,
                              int32_t iters, float tol, int64_t chunk_points, void *pinned_stage,
                              size_t pinned_bytes, float *centroids, int32_t *assign, double *inertia,
                              int32_t *iters_done, void *ws, size_t ws_bytes, void *stream);

/*
 * Dot-product and cosine k-means.  The project README ("CuTe backend") names
 * both as modes of the library without defining them; the readings taken:
 *   KM_METRIC_DOT: a_i = the lowest k maximising x_i.c~_k; the update is the
 *     mean of the members (a cluster without points keeps its centroid).
 *   KM_METRIC_COSINE (spherical k-means): the points are used as unit rows
 *     x^_i = dtype(x_i / ||x_i||) (kmeans_normalize_rows; a zero row stays
 *     zero) and the initial centroids are made unit rows in place; a_i = the
 *     lowest k maximising x^_i.c~_k; the update is the mean direction
 *     c_k = S_k / ||S_k||, S_k = sum_{a_i = k} x^_i (fp32), and a cluster
 *     without points, or with S_k = 0, keeps its centroid.
 *   KM_METRIC_L2: exactly kmeans_fit.
 * Both similarity metrics run on the same kernels as Lloyd's loop: the
 * assign kernels get zero norm terms, so they take the arg-max of x.c~ with
 * ties to the lowest index.
 *
 * kmeans_normalize_rows: out_i = dtype(x_i / ||x_i||) for `rows` rows of D
 *   elements (fp32 norm and IEEE division, nearest-even rounding); out may
 *   equal x.  x and out: device, 16-byte aligned.
 * kmeans_prepare_centroids_metric: kmeans_prepare_centroids with the norm
 *   terms 0 for KM_METRIC_DOT / KM_METRIC_COSINE (the centroids are taken as
 *   given: unit rows are the caller's business here); the result feeds
 *   kmeans_assign_prepared, whose min_dist then holds x_norms_i - 2 x_i.c~_a.
 * kmeans_fit_metric: kmeans_fit for a metric, with the same arguments.
 *   Device-resident x takes ws from kmeans_workspace_bytes(KM_OP_FIT /
 *   KM_OP_FIT_DOT / KM_OP_FIT_COSINE). Pinned host x selects the streamed
 *   path, which takes ws from KM_OP_FIT_HOST; cosine then turns each staged
 *   chunk into unit rows in place.
 *   `objective` (host double [iters * B] or NULL): for KM_METRIC_L2 the
 *   inertia; otherwise the total similarity sum_i x_i.c~_{a_i} (x^ for
 *   cosine) of each iteration's assignment (fp32 terms, fp64 sum).
 */
km_status_t kmeans_normalize_rows(const void *x, km_dtype_t dt, int64_t rows, int64_t D, void *out,
                                  void *stream);
km_status_t kmeans_prepare_centroids_metric(const float *centroids, km_dtype_t dt, km_metric_t metric,
                                            int64_t B, int64_t N, int64_t D, int64_t K, void *c_prep,
                                            size_t c_prep_bytes, void *stream);
km_status_t kmeans_fit_metric(const void *x, km_dtype_t dt, km_metric_t metric, int64_t B, int64_t N,
                              int64_t D, int64_t K, int32_t iters, float tol, int64_t chunk_points,
                              float *centroids, int32_t *assign, double *objective,
                              int32_t *iters_done, void *ws, size_t ws_bytes, void *stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *kmeans_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHKM_H */
