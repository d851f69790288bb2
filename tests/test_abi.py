"""C-ABI checks that need no GPU: the library loads, exports every symbol the header declares,
rejects invalid arguments before touching HIP, sizes workspaces consistently and plans tiles
that fit gfx950 (LDS, VGPR) for every workload."""
import ctypes
import os
import re

import pytest

from exact_lloyd_means_02_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashkm.h")


@pytest.fixture(scope="module")
def fk():
    from exact_lloyd_means_02_amd import flashkm
    return flashkm


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kmeans_\w+)\s*\(", text)))


def test_exports_match_header(fk):
    names = header_functions()
    assert names == sorted(fk.EXPORTS)
    for n in names:
        assert hasattr(fk.LIB, n), n


P = ctypes.c_void_p(256)   # a non-null pointer value: never dereferenced on the paths tested


@pytest.mark.parametrize("args,err", [
    ((None, 2, 1, 10, 10, P, None), "x is NULL"),
    ((P, 7, 1, 10, 10, P, None), "unknown dtype"),
    ((P, 2, 0, 10, 10, P, None), "bad shape"),
    ((P, 2, 1, 10, 5000, P, None), "bad shape"),
    ((P, 2, 1, 10, 10, None, None), "x_norms is NULL"),
    ((ctypes.c_void_p(258), 2, 1, 10, 10, P, None), "16-byte aligned"),
])
def test_row_norms_validation(fk, args, err):
    assert fk.LIB.kmeans_row_norms(*args) == fk.KM_ERR_INVALID
    assert err in fk.last_error()


def _assign(fk, **kw):
    a = dict(x=P, dt=2, c=P, B=1, N=100, D=16, K=10, xn=None, out=P, md=None, ws=P, wsb=1 << 30)
    a.update(kw)
    return fk.LIB.kmeans_assign(a["x"], a["dt"], a["c"], a["B"], a["N"], a["D"], a["K"], a["xn"], a["out"], a["md"],
                                a["ws"], a["wsb"], None)


def test_assign_validation(fk):
    assert _assign(fk, K=101) == fk.KM_ERR_INVALID and "K (101) > N (100)" in fk.last_error()
    assert _assign(fk, K=0) == fk.KM_ERR_INVALID
    assert _assign(fk, N=1 << 31) == fk.KM_ERR_INVALID
    assert _assign(fk, B=2, N=1 << 30) == fk.KM_ERR_INVALID
    assert _assign(fk, D=4097) == fk.KM_ERR_INVALID
    assert _assign(fk, dt=3) == fk.KM_ERR_INVALID
    assert _assign(fk, c=None) == fk.KM_ERR_INVALID and "centroids" in fk.last_error()
    assert _assign(fk, out=None) == fk.KM_ERR_INVALID
    assert _assign(fk, md=P) == fk.KM_ERR_INVALID and "x_norms" in fk.last_error()
    assert _assign(fk, ws=None) == fk.KM_ERR_WORKSPACE
    assert _assign(fk, ws=ctypes.c_void_p(256 + 128)) == fk.KM_ERR_WORKSPACE
    assert _assign(fk, wsb=16) == fk.KM_ERR_WORKSPACE and "too small" in fk.last_error()


def test_prepared_assign_validation(fk):
    L = fk.LIB
    assert L.kmeans_prepare_centroids(None, 2, 1, 100, 16, 10, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert L.kmeans_prepare_centroids(P, 2, 1, 100, 16, 10, None, 1 << 20, None) == fk.KM_ERR_INVALID
    assert L.kmeans_prepare_centroids(P, 2, 1, 100, 16, 10, P, 16, None) == fk.KM_ERR_WORKSPACE
    assert L.kmeans_prepare_centroids(P, 2, 1, 100, 16, 101, P, 1 << 20, None) == fk.KM_ERR_INVALID
    args = [P, 2, P, 1 << 20, 1, 100, 16, 10, None, P, None, None]
    bad = list(args); bad[2] = None
    assert L.kmeans_assign_prepared(*bad) == fk.KM_ERR_INVALID and "c_prep" in fk.last_error()
    bad = list(args); bad[3] = 16
    assert L.kmeans_assign_prepared(*bad) == fk.KM_ERR_WORKSPACE
    bad = list(args); bad[10] = P
    assert L.kmeans_assign_prepared(*bad) == fk.KM_ERR_INVALID and "x_norms" in fk.last_error()
    bad = list(args); bad[0] = ctypes.c_void_p(258)
    assert L.kmeans_assign_prepared(*bad) == fk.KM_ERR_INVALID


def test_argsort_update_fit_validation(fk):
    L = fk.LIB
    assert L.kmeans_argsort_ids(None, 1, 10, 3, P, P, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert L.kmeans_argsort_ids(P, 1, 10, 11, P, P, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert L.kmeans_argsort_ids(P, 1, 10, 3, P, P, None, P, 0, None) == fk.KM_ERR_WORKSPACE
    assert L.kmeans_update(P, 2, P, P, None, 1, 10, 4, 3, P, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert L.kmeans_update(P, 2, P, P, P, 1, 10, 4, 3, None, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert L.kmeans_fit(P, 2, 1, 10, 4, 3, 0, 0.0, 0, P, None, None, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert "iters" in fk.last_error()
    assert L.kmeans_fit(P, 2, 1, 10, 4, 3, 5, -1.0, 0, P, None, None, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert L.kmeans_fit(P, 2, 1, 10, 4, 3, 5, 0.0, -5, P, None, None, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert L.kmeans_fit(P, 2, 1, 10, 4, 3, 5, 0.0, 0, P, None, None, None, None, 1 << 20, None) == fk.KM_ERR_WORKSPACE


def test_fit_blocks_validation(fk):
    L = fk.LIB
    VP, I64 = ctypes.c_void_p, ctypes.c_int64

    def call(ptrs, npts, nb=None, chunk=0, K=3, iters=2, tol=0.0, ws=P):
        pa = (VP * len(ptrs))(*ptrs)
        na = (I64 * len(npts))(*npts)
        return L.kmeans_fit_blocks(pa, na, len(ptrs) if nb is None else nb, 1, 8, K, iters, tol, chunk, P, None, None,
                                   None, ws, 1 << 30, None)
    assert call([256, 256], [4096, 100], nb=0) == fk.KM_ERR_INVALID and "nblocks" in fk.last_error()
    assert call([256, None], [4096, 100]) == fk.KM_ERR_INVALID and "block 1 is NULL" in fk.last_error()
    assert call([256, 256], [4096, 0]) == fk.KM_ERR_INVALID and "block 1 holds 0" in fk.last_error()
    assert call([258, 256], [4096, 100]) == fk.KM_ERR_INVALID and "16-byte" in fk.last_error()
    assert call([256, 256], [3000, 100], chunk=2048) == fk.KM_ERR_INVALID and "not a multiple" in fk.last_error()
    assert call([256, 256], [1 << 30, 1 << 30]) == fk.KM_ERR_INVALID and "2^31" in fk.last_error()
    assert call([256], [2], K=3) == fk.KM_ERR_INVALID and "K (3) > N (2)" in fk.last_error()
    assert call([256], [4096], iters=0) == fk.KM_ERR_INVALID
    assert call([256], [4096], tol=-1.0) == fk.KM_ERR_INVALID
    assert call([256], [4096], ws=None) == fk.KM_ERR_WORKSPACE


def test_fit_staged_validation(fk):
    """kmeans_fit_staged rejects bad arguments before any HIP call; its pinned buffer holds two
    chunks of rows, each rounded up to 256 bytes."""
    L = fk.LIB
    half = lambda n, d, c, es: -(-min(c if c > 0 else 1 << 24, n) * d * es // 256) * 256
    assert fk.kmeans_workspace_bytes(fk.KM_OP_STAGE_PINNED, 1, 1, 1 << 20, 64, 100, 1 << 18) == 2 * half(1 << 20, 64, 1 << 18, 2)
    assert fk.kmeans_workspace_bytes(fk.KM_OP_STAGE_PINNED, 0, 2, 5000, 37, 10, 0) == 2 * half(5000, 37, 0, 4)
    need = fk.kmeans_workspace_bytes(fk.KM_OP_STAGE_PINNED, 2, 1, 4096, 16, 8, 0)

    def call(x=P, iters=2, tol=0.0, chunk=0, stage=P, sbytes=None, ws=P, C=P, K=8):
        return L.kmeans_fit_staged(x, 2, 1, 4096, 16, K, iters, tol, chunk, stage, need if sbytes is None else sbytes,
                                   C, None, None, None, ws, 1 << 30, None)
    assert call(x=None) == fk.KM_ERR_INVALID and "x" in fk.last_error()
    assert call(stage=None) == fk.KM_ERR_INVALID and "pinned_stage" in fk.last_error()
    assert call(C=None) == fk.KM_ERR_INVALID
    assert call(K=5000) == fk.KM_ERR_INVALID and "K (5000) > N (4096)" in fk.last_error()
    assert call(iters=0) == fk.KM_ERR_INVALID
    assert call(tol=-1.0) == fk.KM_ERR_INVALID
    assert call(chunk=-1) == fk.KM_ERR_INVALID
    assert call(x=ctypes.c_void_p(264)) == fk.KM_ERR_INVALID and "16-byte" in fk.last_error()
    assert call(stage=ctypes.c_void_p(264)) == fk.KM_ERR_INVALID and "16-byte" in fk.last_error()
    assert call(sbytes=need - 1) == fk.KM_ERR_WORKSPACE and "pinned_stage too small" in fk.last_error()
    assert call(ws=None) == fk.KM_ERR_WORKSPACE


def test_workspace_sizes(fk):
    for op in (fk.KM_OP_ASSIGN, fk.KM_OP_ARGSORT, fk.KM_OP_UPDATE, fk.KM_OP_FIT, fk.KM_OP_FIT_HOST):
        assert fk.kmeans_workspace_bytes(op, 2, 1, 10, 4, 11) == 0          # K > N: invalid
        small = fk.kmeans_workspace_bytes(op, 2, 1, 4096, 16, 8)
        big = fk.kmeans_workspace_bytes(op, 2, 4, 65536, 128, 1024)
        assert 0 < small <= big and small % 256 == 0
    assert fk.kmeans_workspace_bytes(99, 2, 1, 10, 4, 3) == 0
    # the fit workspace covers every stage's workspace
    fit = fk.kmeans_workspace_bytes(fk.KM_OP_FIT, 2, 32, 65536, 128, 1024)
    for op in (fk.KM_OP_ASSIGN, fk.KM_OP_ARGSORT, fk.KM_OP_UPDATE):
        assert fk.kmeans_workspace_bytes(op, 2, 32, 65536, 128, 1024) < fit
    # streamed: two staging buffers of chunk_points rows
    host = fk.kmeans_workspace_bytes(fk.KM_OP_FIT_HOST, 1, 1, 1 << 26, 64, 32768, 1 << 24)
    assert host >= 2 * (1 << 24) * 64 * 2


def _sort_need(fk, dt, n, D, K):
    """Digit tables of one arg-sort of n labels (the standalone workspace less its status word)."""
    return fk.kmeans_workspace_bytes(fk.KM_OP_ARGSORT, dt, 1, n, D, K) - 256


def _update_need(fk, dt, n, D, K):
    """Counters and scratch of one update of n points (the standalone workspace less the
    clusters' first positions, which the streamed layout keeps at a fixed size)."""
    return fk.kmeans_workspace_bytes(fk.KM_OP_UPDATE, dt, 1, n, D, K) - (-(-4 * K // 256) * 256)


@pytest.mark.parametrize("dt,D,K", [(2, 128, 64), (1, 64, 512), (2, 256, 64), (0, 1024, 32), (1, 64, 32768)])
def test_streamed_scratch_covers_the_last_chunk(fk, dt, D, K):
    """The streamed path keeps the arg-sort tables, the update's partial records and its arrival
    counters of one staged chunk.  The update's plan is not monotonic in the point count, so a
    ragged last chunk can need more than a full one: the workspace must cover both.  Only those
    regions of the streamed layout depend on N (for a fixed chunk), so the growth of the workspace
    from N = m c (all chunks full) to N = m c + r bounds what the r-point chunk may need beyond a
    full one: at least u(r) - u(c) - s(c) and s(r) - s(c) - u(c), with u the update's counters and
    scratch and s the arg-sort's tables (the two share the scratch region)."""
    chunks = [1 << 14, 50000, 532480, 786432, 1 << 20, (1 << 24) - 4096, 1 << 24]
    rests = [1, 100, 12345, 31072, 262144, 524288, 532479, 782336, (1 << 20) - 1]
    checked = 0
    for c in chunks:
        for m in (1, 2):
            full = fk.kmeans_workspace_bytes(fk.KM_OP_FIT_HOST, dt, 1, m * c, D, K, c)
            uc, sc = _update_need(fk, dt, c, D, K), _sort_need(fk, dt, c, D, K)
            for r in rests:
                if r >= c or r < K:
                    continue
                ws = fk.kmeans_workspace_bytes(fk.KM_OP_FIT_HOST, dt, 1, m * c + r, D, K, c)
                ur, sr = _update_need(fk, dt, r, D, K), _sort_need(fk, dt, r, D, K)
                assert ws - full >= ur - uc - sc, (c, m, r, ws - full, ur - uc - sc)
                assert ws - full >= sr - sc - uc, (c, m, r, ws - full, sr - sc - uc)
                checked += 1
    assert checked > 0
    # a case where it matters: 786432-point chunks (192 points per wave slot, 256 rows per update
    # chunk) and a last chunk of 782336 points (191 per slot, rounded to 128 rows: twice the
    # chunks), D=128, K=64; the shorter chunk's update needs megabytes more than the full chunk's
    # update and sort together
    if (dt, D, K) == (2, 128, 64):
        c, r = 786432, 782336
        assert _update_need(fk, dt, r, D, K) - _update_need(fk, dt, c, D, K) - _sort_need(fk, dt, c, D, K) > 1 << 20


DT = {"f32": 0, "f16": 1, "bf16": 2}


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_plan_fits_gfx950(fk, name):
    w = W.WORKLOADS[name]
    n = min(w.N, w.chunk) if w.host else w.N
    p = fk.kmeans_plan(DT[w.dtype], w.B, n, w.D, w.K)
    assert p["lds_bytes"] <= 160 * 1024
    assert p["vgpr_est"] <= 256
    assert p["d_pad"] >= w.D
    assert p["path"] == (0 if w.D <= (128 if w.dtype == "f32" else 256) else 1)
    assert p["block_n"] == p["waves"] * p["point_blocks"] * 32
    assert (1 << (p["sort_bits"] * p["sort_passes"])) >= w.K
    assert p["sort_bits"] <= 10
    assert p["upd_rows"] >= 64 and p["upd_lanes"] in (1, 2, 4, 8, 16, 32, 64)
    assert p["assign_wgs"] == w.B * -(-n // p["block_n"])


def test_plan_headline_values(fk):
    p = fk.kmeans_plan(2, 32, 65536, 128, 1024)
    assert (p["path"], p["d_pad"], p["point_blocks"], p["block_n"]) == (0, 128, 2, 256)
    assert (p["sort_bits"], p["sort_passes"]) == (10, 1)
    s = fk.kmeans_plan(0, 1, 262144, 1024, 512)      # split-D fp32
    assert s["path"] == 1 and s["block_d"] == 16    # 16 fp32 dimensions per LDS chunk
    c5 = fk.kmeans_plan(1, 1, 1 << 24, 64, 32768)    # one streamed chunk: two counting passes
    assert c5["sort_passes"] == 2


def test_plan_update_rows(fk):
    """The update's sorted positions per wave: about 4 waves per SIMD over the launch (1024 SIMDs),
    to the nearest power of two, within 64..4096, halved when the chunk lies between a quarter of and
    twice the mean segment length N/K."""
    rows = lambda dt, B, N, D, K: fk.kmeans_plan(dt, B, N, D, K)["upd_rows"]
    assert rows(2, 32, 65536, 128, 1024) == 512         # 2^21 / 4096 positions
    assert rows(1, 32, 75600, 128, 1000) == 512         # 590.6 -> 512 (nearest power of two)
    assert rows(2, 1, 1 << 24, 128, 64) == 4096         # mean segment 262144: no halving
    assert rows(2, 1, 1 << 24, 128, 4096) == 2048       # mean segment 4096: 4096 halved
    assert rows(0, 1, 262144, 1024, 512) == 64          # 64 (the floor)
    assert rows(2, 1, 4096 * 255, 128, 64) == 256       # 255 -> 256
    assert rows(2, 1, 4096 * 191, 128, 64) == 128       # 191 -> 128 (below three quarters of 256)
    assert rows(2, 1, 1 << 30, 128, 2) == 4096          # the ceiling


def test_workload_generators_are_seeded():
    w = W.small("headline_bf16", B=2, N=500, K=20)
    x1, c1, _ = W.make(w)
    x2, c2, _ = W.make(w)
    assert (x1 == x2).all() and (c1 == c2).all()
    assert x1.dtype == W.NP_STORAGE["bf16"] and x1.shape == (2, 500, 128)
    idx = W.init_indices(w)
    assert all(len(set(r.tolist())) == w.K for r in idx)          # distinct init points
    w2 = W.small("skew_bf16_k64", N=40000, K=64)
    x, c, mu = W.make(w2)
    assert mu is not None and abs(mu[0, :4].mean() - 64.0) < 2.0   # the +64 channels, centred away
    assert abs(W.storage_to_f64(x, "bf16")[0, :, :4].mean()) < 0.5


def test_metric_entry_validation(fk):
    L = fk.LIB
    # kmeans_normalize_rows(x, dt, rows, D, out, stream)
    assert L.kmeans_normalize_rows(None, 2, 10, 16, P, None) == fk.KM_ERR_INVALID and "x is NULL" in fk.last_error()
    assert L.kmeans_normalize_rows(P, 2, 10, 16, None, None) == fk.KM_ERR_INVALID
    assert L.kmeans_normalize_rows(P, 9, 10, 16, P, None) == fk.KM_ERR_INVALID and "dtype" in fk.last_error()
    assert L.kmeans_normalize_rows(P, 2, 0, 16, P, None) == fk.KM_ERR_INVALID
    assert L.kmeans_normalize_rows(P, 2, 10, 5000, P, None) == fk.KM_ERR_INVALID
    assert L.kmeans_normalize_rows(P, 2, 10, 16, ctypes.c_void_p(264), None) == fk.KM_ERR_INVALID
    assert "aligned" in fk.last_error()
    # kmeans_prepare_centroids_metric(c, dt, metric, B, N, D, K, c_prep, bytes, stream)
    assert L.kmeans_prepare_centroids_metric(P, 2, 3, 1, 100, 16, 10, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert "metric" in fk.last_error()
    assert L.kmeans_prepare_centroids_metric(P, 2, 1, 1, 100, 16, 10, P, 16, None) == fk.KM_ERR_WORKSPACE
    assert L.kmeans_prepare_centroids_metric(None, 2, 2, 1, 100, 16, 10, P, 1 << 20, None) == fk.KM_ERR_INVALID
    # kmeans_fit_metric(x, dt, metric, B, N, D, K, iters, tol, chunk_points, C, assign, obj, done, ws, bytes, stream)
    def fit(**kw):
        a = dict(x=P, dt=2, m=1, B=1, N=10, D=4, K=3, it=5, tol=0.0, C=P, ws=P, wsb=1 << 20)
        a.update(kw)
        return L.kmeans_fit_metric(a["x"], a["dt"], a["m"], a["B"], a["N"], a["D"], a["K"], a["it"], a["tol"],
                                   a.get("cp", 0), a["C"], None, None, None, a["ws"], a["wsb"], None)
    assert fit(m=-1) == fk.KM_ERR_INVALID and "metric" in fk.last_error()
    assert fit(it=0) == fk.KM_ERR_INVALID and "iters" in fk.last_error()
    assert fit(tol=-1.0) == fk.KM_ERR_INVALID
    assert fit(K=11) == fk.KM_ERR_INVALID
    assert fit(C=None) == fk.KM_ERR_INVALID
    assert fit(x=ctypes.c_void_p(258), m=2) == fk.KM_ERR_INVALID
    assert fit(ws=None, m=2) == fk.KM_ERR_WORKSPACE
    assert fit(cp=-1, m=1) == fk.KM_ERR_INVALID and "chunk_points" in fk.last_error()
    # the L2 metric is kmeans_fit: same validation
    assert fit(m=0, it=0) == fk.KM_ERR_INVALID and "iters" in fk.last_error()


def test_metric_workspace_sizes(fk):
    B, N, K = 2, 5000, 100
    # (dtype, bytes per element, D, whether the update needs several column blocks per row):
    # one block covers 64 lanes x 4 vectors x 16 bytes, i.e. 2048 2-byte or 1024 fp32 columns
    for dt, s, D, wide in ((0, 4, 64, False), (1, 2, 64, False), (2, 2, 64, False), (2, 2, 4096, True),
                           (0, 4, 2048, True)):
        base = fk.kmeans_workspace_bytes(fk.KM_OP_FIT, dt, B, N, D, K)
        dot = fk.kmeans_workspace_bytes(fk.KM_OP_FIT_DOT, dt, B, N, D, K)
        cos = fk.kmeans_workspace_bytes(fk.KM_OP_FIT_COSINE, dt, B, N, D, K)
        assert dot == base
        # the unit rows come on top; the accumulating update's sums, counts and per-cluster shifts
        # only where a row needs several column blocks (else the update finishes in place)
        extra = B * N * D * s + ((B * K * D * 4 + B * K * 4 + B * K * 8) if wide else 0)
        assert base + extra <= cos <= base + extra + 4 * 256
    assert fk.kmeans_workspace_bytes(99, 2, B, N, 64, K) == 0


def test_wrapper_validation_without_gpu(fk):
    import torch
    km = fk.FlashKMeans(d=8, k=5, niter=2, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError, match="must be"):
        km.fit(torch.zeros(100, 7))
    with pytest.raises(ValueError, match="k \\(5\\) > number of points"):
        km.fit(torch.zeros(4, 8))
    with pytest.raises(ValueError, match="fit / train first"):
        km.predict(torch.zeros(10, 8))
    with pytest.raises(ValueError, match="unknown metric"):
        fk.FlashKMeans(d=8, k=5, metric="manhattan", device="cuda:0")
    with pytest.raises(ValueError):
        fk.FlashKMeans(d=8, k=0, device="cuda:0")
    with pytest.raises(ValueError, match="dtype"):
        fk.FlashKMeans(d=8, k=5, dtype=torch.float64, device="cuda:0")
    with pytest.raises(ValueError, match="host_streaming"):
        fk.FlashKMeans(d=8, k=5, metric="cosine", host_streaming=True, device="cuda:0")


def test_centroid_alignment_validation(fk):
    L = fk.LIB
    C = ctypes.c_void_p(256 + 4)
    assert L.kmeans_update(P, 2, P, P, P, 1, 10, 8, 3, C, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert "centroids must be 16-byte aligned" in fk.last_error()
    assert L.kmeans_fit(P, 2, 1, 10, 8, 3, 2, 0.0, 0, C, None, None, None, P, 1 << 20, None) == fk.KM_ERR_INVALID
    assert "centroids" in fk.last_error()
    assert L.kmeans_fit_metric(P, 2, 2, 1, 10, 8, 3, 2, 0.0, 0, C, None, None, None, P, 1 << 20,
                               None) == fk.KM_ERR_INVALID


def test_workspace_cache_is_per_stream(fk):
    """Calls on different streams may overlap, so the binding never hands them the same scratch
    memory; calls on one stream run in order and share it (host tensors stand in for the device)."""
    fk.clear_workspaces()
    try:
        a = fk.workspace(fk.KM_OP_FIT, fk.KM_BF16, 2, 4096, 64, 32, "cpu", stream=ctypes.c_void_p(0x1000))
        b = fk.workspace(fk.KM_OP_FIT, fk.KM_BF16, 2, 4096, 64, 32, "cpu", stream=ctypes.c_void_p(0x2000))
        a2 = fk.workspace(fk.KM_OP_FIT, fk.KM_BF16, 2, 4096, 64, 32, "cpu", stream=ctypes.c_void_p(0x1000))
        assert a.untyped_storage().data_ptr() != b.untyped_storage().data_ptr()
        assert a.untyped_storage().data_ptr() == a2.untyped_storage().data_ptr()
        assert a.data_ptr() % 256 == 0 and b.data_ptr() % 256 == 0
    finally:
        fk.clear_workspaces()
