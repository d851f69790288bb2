"""Thin ctypes binding of libflashkm (include/flashkm.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.  Torch
tensors supply device memory and the current HIP stream; the workspace the C-ABI asks for is
a torch uint8 tensor (the library itself allocates nothing).  If the library is missing the
import raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FLASHKM_LIB") or os.path.join(HERE, "libflashkm.so")

KM_F32, KM_F16, KM_BF16 = 0, 1, 2
DT_CODES = {"f32": KM_F32, "f16": KM_F16, "bf16": KM_BF16}
KM_OK, KM_ERR_INVALID, KM_ERR_UNSUPPORTED, KM_ERR_WORKSPACE, KM_ERR_HIP = 0, -1, -2, -3, -4
KM_OP_ASSIGN, KM_OP_ARGSORT, KM_OP_UPDATE, KM_OP_FIT, KM_OP_FIT_HOST = 1, 2, 3, 4, 5
KM_OP_FIT_DOT, KM_OP_FIT_COSINE, KM_OP_STAGE_PINNED = 6, 7, 8
KM_METRIC_L2, KM_METRIC_DOT, KM_METRIC_COSINE = 0, 1, 2
METRICS = {"l2": KM_METRIC_L2, "euclid": KM_METRIC_L2, "dot": KM_METRIC_DOT, "cosine": KM_METRIC_COSINE}
STATUS_NAMES = {0: "KM_OK", -1: "KM_ERR_INVALID", -2: "KM_ERR_UNSUPPORTED", -3: "KM_ERR_WORKSPACE", -4: "KM_ERR_HIP"}

# every symbol the header declares
EXPORTS = ["kmeans_plan", "kmeans_workspace_bytes", "kmeans_row_norms", "kmeans_assign", "kmeans_assign_noalloc",
           "kmeans_prepare_centroids", "kmeans_assign_prepared", "kmeans_argsort_ids", "kmeans_argsort_status",
           "kmeans_update", "kmeans_fit", "kmeans_fit_blocks", "kmeans_fit_staged", "kmeans_normalize_rows",
           "kmeans_prepare_centroids_metric", "kmeans_fit_metric", "kmeans_last_error"]


class KmPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "path", "d_pad", "point_blocks", "waves", "block_n", "block_k", "block_d", "lds_bytes", "vgpr_est",
        "assign_wgs", "sort_bits", "sort_passes", "sort_tile", "upd_rows", "upd_vec", "upd_lanes", "assign_splits")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class FlashKMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), msg))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libflashkm.so is not built (%s); run exact_lloyd_means_02_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kmeans_plan.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.POINTER(KmPlan)]
    lib.kmeans_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, i64]
    lib.kmeans_workspace_bytes.restype = sz
    lib.kmeans_row_norms.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp]
    lib.kmeans_assign.argtypes = [vp, ctypes.c_int, vp, i64, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    lib.kmeans_assign_noalloc.argtypes = [vp, ctypes.c_int, vp, i64, i64, i64, i64, vp, vp, vp, vp]
    lib.kmeans_prepare_centroids.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, vp, sz, vp]
    lib.kmeans_assign_prepared.argtypes = [vp, ctypes.c_int, vp, sz, i64, i64, i64, i64, vp, vp, vp, vp]
    lib.kmeans_argsort_ids.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    lib.kmeans_argsort_status.argtypes = [vp, sz, vp]
    lib.kmeans_update.argtypes = [vp, ctypes.c_int, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, sz, vp]
    lib.kmeans_fit.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, i32, f32, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.kmeans_fit_blocks.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(i64), i32, ctypes.c_int, i64, i64, i32, f32,
                                      i64, vp, vp, vp, vp, vp, sz, vp]
    lib.kmeans_fit_staged.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, i32, f32, i64, vp, sz, vp, vp, vp, vp,
                                      vp, sz, vp]
    lib.kmeans_normalize_rows.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp]
    lib.kmeans_prepare_centroids_metric.argtypes = [vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, vp, sz, vp]
    lib.kmeans_fit_metric.argtypes = [vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, i32, f32, i64, vp, vp, vp,
                                      vp, vp, sz, vp]
    for n in ("kmeans_plan", "kmeans_row_norms", "kmeans_assign", "kmeans_assign_noalloc", "kmeans_prepare_centroids",
              "kmeans_assign_prepared", "kmeans_argsort_ids", "kmeans_argsort_status", "kmeans_update", "kmeans_fit",
              "kmeans_fit_blocks", "kmeans_fit_staged", "kmeans_normalize_rows",
              "kmeans_prepare_centroids_metric", "kmeans_fit_metric"):
        getattr(lib, n).restype = ctypes.c_int
    lib.kmeans_last_error.argtypes = []
    lib.kmeans_last_error.restype = ctypes.c_char_p
    return lib


LIB = _load()


def last_error() -> str:
    return LIB.kmeans_last_error().decode()


def _check(st: int):
    if st != KM_OK:
        raise FlashKMError(st, last_error())


# ------------------------------------------------------------------------------------------------
# torch marshalling
# ------------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: KM_F32, torch.float16: KM_F16, torch.bfloat16: KM_BF16}
    if t.dtype not in m:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return m[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream=None):
    torch = _torch()
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    if t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


_WS = {}


def workspace(op: int, dt: int, B: int, N: int, D: int, K: int, device, chunk_points: int = 0, stream=None):
    """A cached uint8 device tensor of the size the C-ABI asks for.

    One cache entry per (operation, device, stream): calls queued on one stream run in order and
    may share scratch memory, calls on different streams may run at the same time and must not.
    A growing entry replaces the old tensor only after the device has drained, so no queued kernel
    still uses the memory the allocator takes back."""
    torch = _torch()
    nbytes = LIB.kmeans_workspace_bytes(op, dt, B, N, D, K, chunk_points)
    if nbytes == 0:
        raise FlashKMError(KM_ERR_INVALID, last_error() or "bad shape for workspace")
    sid = stream.value if isinstance(stream, ctypes.c_void_p) else stream
    key = (op, str(device), sid)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            torch.cuda.synchronize(ws.device)
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        _WS[key] = ws
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


def clear_workspaces():
    _WS.clear()


def kmeans_plan(dt: int, B: int, N: int, D: int, K: int) -> dict:
    p = KmPlan()
    _check(LIB.kmeans_plan(dt, B, N, D, K, ctypes.byref(p)))
    return p.as_dict()


def kmeans_workspace_bytes(op: int, dt: int, B: int, N: int, D: int, K: int, chunk_points: int = 0) -> int:
    return int(LIB.kmeans_workspace_bytes(op, dt, B, N, D, K, chunk_points))


def kmeans_row_norms(x, out=None, stream=None):
    torch = _torch()
    _need(x.dim() == 3 and x.is_contiguous(), "x must be a contiguous [B, N, D] tensor")
    B, N, D = x.shape
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _need(out.is_contiguous() and out.dtype == torch.float32 and tuple(out.shape) == (B, N), "bad out")
    _check(LIB.kmeans_row_norms(_ptr(x), dtype_code(x), B, N, D, _ptr(out), _stream(x, stream)))
    return out


def kmeans_assign(x, centroids, x_norms=None, assign=None, min_dist=None, want_min_dist=False, stream=None):
    """Returns (assign int32 [B,N], min_dist float32 [B,N] or None)."""
    torch = _torch()
    _need(x.dim() == 3 and x.is_contiguous(), "x must be a contiguous [B, N, D] tensor")
    B, N, D = x.shape
    _need(centroids.dim() == 3 and centroids.is_contiguous() and centroids.dtype == torch.float32
          and centroids.shape[0] == B and centroids.shape[2] == D, "centroids must be contiguous f32 [B, K, D]")
    K = centroids.shape[1]
    if assign is None:
        assign = torch.empty((B, N), dtype=torch.int32, device=x.device)
    if want_min_dist and min_dist is None:
        min_dist = torch.empty((B, N), dtype=torch.float32, device=x.device)
    dt = dtype_code(x)
    st = _stream(x, stream)
    ws = workspace(KM_OP_ASSIGN, dt, B, N, D, K, x.device, stream=st)
    _check(LIB.kmeans_assign(_ptr(x), dt, _ptr(centroids), B, N, D, K, _ptr(x_norms), _ptr(assign), _ptr(min_dist),
                             _ptr(ws), ws.numel(), st))
    return assign, min_dist


def kmeans_assign_noalloc(x, centroids, x_norms=None, assign=None, min_dist=None, want_min_dist=False, stream=None):
    """kmeans_assign without a workspace (the library's static per-GPU scratch; see the header).
    Returns (assign int32 [B,N], min_dist float32 [B,N] or None)."""
    torch = _torch()
    _need(x.dim() == 3 and x.is_contiguous(), "x must be a contiguous [B, N, D] tensor")
    B, N, D = x.shape
    _need(centroids.dim() == 3 and centroids.is_contiguous() and centroids.dtype == torch.float32
          and centroids.shape[0] == B and centroids.shape[2] == D, "centroids must be contiguous f32 [B, K, D]")
    K = centroids.shape[1]
    if assign is None:
        assign = torch.empty((B, N), dtype=torch.int32, device=x.device)
    if want_min_dist and min_dist is None:
        min_dist = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _check(LIB.kmeans_assign_noalloc(_ptr(x), dtype_code(x), _ptr(centroids), B, N, D, K, _ptr(x_norms),
                                     _ptr(assign), _ptr(min_dist), _stream(x, stream)))
    return assign, min_dist


class PreparedCentroids:
    """The assign kernel's centroid operand (opaque device bytes) for one (dtype, B, D, K)."""

    def __init__(self, buf, dt: int, B: int, D: int, K: int):
        self.buf, self.dt, self.B, self.D, self.K = buf, dt, B, D, K


def metric_code(metric) -> int:
    if isinstance(metric, int) and metric in METRICS.values():
        return metric
    if metric not in METRICS:
        raise ValueError("unknown metric %r (one of %s)" % (metric, sorted(METRICS)))
    return METRICS[metric]


def kmeans_prepare_centroids(centroids, dtype, out=None, stream=None, metric="l2") -> PreparedCentroids:
    """c~ = dtype(centroids) in the assign kernel's layout plus ||c~||^2 / 2 (0 for the "dot" and
    "cosine" metrics).  `dtype` is the points' torch dtype (or a tensor of it)."""
    torch = _torch()
    _need(centroids.dim() == 3 and centroids.is_contiguous() and centroids.dtype == torch.float32,
          "centroids must be contiguous f32 [B, K, D]")
    B, K, D = centroids.shape
    dt = dtype_code(dtype) if hasattr(dtype, "dtype") else dtype_code(torch.empty(0, dtype=dtype))
    nbytes = LIB.kmeans_workspace_bytes(KM_OP_ASSIGN, dt, B, K, D, K, 0)
    if nbytes == 0:
        raise FlashKMError(KM_ERR_INVALID, last_error() or "bad shape")
    if out is None:
        raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=centroids.device)
        off = (-raw.data_ptr()) % 256
        out = raw[off:off + nbytes]
    _need(out.dtype == torch.uint8 and out.numel() >= nbytes, "out: uint8 device buffer too small")
    m = metric_code(metric)
    if m == KM_METRIC_L2:
        _check(LIB.kmeans_prepare_centroids(_ptr(centroids), dt, B, K, D, K, _ptr(out), out.numel(),
                                            _stream(centroids, stream)))
    else:
        _check(LIB.kmeans_prepare_centroids_metric(_ptr(centroids), dt, m, B, K, D, K, _ptr(out), out.numel(),
                                                   _stream(centroids, stream)))
    return PreparedCentroids(out, dt, B, D, K)


def kmeans_normalize_rows(x, out=None, stream=None):
    """Unit rows dtype(x_i / ||x_i||) over the last axis (zero rows stay zero); `out` may be `x`."""
    torch = _torch()
    _need(x.is_contiguous() and x.dim() >= 1, "x must be contiguous")
    D = x.shape[-1]
    rows = x.numel() // D
    if out is None:
        out = torch.empty_like(x)
    _need(out.shape == x.shape and out.dtype == x.dtype and out.is_contiguous(), "out: same shape and dtype")
    _check(LIB.kmeans_normalize_rows(_ptr(x), dtype_code(x), rows, D, _ptr(out), _stream(x, stream)))
    return out


def kmeans_assign_prepared(x, prep: PreparedCentroids, x_norms=None, assign=None, min_dist=None,
                           want_min_dist=False, stream=None):
    """FlashAssign from prepared centroids.  Returns (assign, min_dist or None)."""
    torch = _torch()
    _need(x.dim() == 3 and x.is_contiguous(), "x must be a contiguous [B, N, D] tensor")
    B, N, D = x.shape
    dt = dtype_code(x)
    _need((prep.dt, prep.B, prep.D) == (dt, B, D), "prepared centroids were made for another dtype/shape")
    if assign is None:
        assign = torch.empty((B, N), dtype=torch.int32, device=x.device)
    if want_min_dist and min_dist is None:
        min_dist = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _check(LIB.kmeans_assign_prepared(_ptr(x), dt, _ptr(prep.buf), prep.buf.numel(), B, N, D, prep.K, _ptr(x_norms),
                                      _ptr(assign), _ptr(min_dist), _stream(x, stream)))
    return assign, min_dist


def kmeans_argsort_ids(assign, K: int, sorted_ids=None, sorted_idx=None, counts=None, want_counts=True,
                       stream=None, check=False):
    """Returns (sorted_ids, sorted_idx, counts or None), all int32.  check=True waits for the
    sort and raises FlashKMError when it met labels outside [0, K) (kmeans_argsort_status)."""
    torch = _torch()
    _need(assign.dim() == 2 and assign.is_contiguous() and assign.dtype == torch.int32, "assign: int32 [B, N]")
    B, N = assign.shape
    if sorted_ids is None:
        sorted_ids = torch.empty_like(assign)
    if sorted_idx is None:
        sorted_idx = torch.empty_like(assign)
    if want_counts and counts is None:
        counts = torch.empty((B, K), dtype=torch.int32, device=assign.device)
    st = _stream(assign, stream)
    ws = workspace(KM_OP_ARGSORT, KM_F32, B, N, 1, K, assign.device, stream=st)
    _check(LIB.kmeans_argsort_ids(_ptr(assign), B, N, K, _ptr(sorted_ids), _ptr(sorted_idx), _ptr(counts),
                                  _ptr(ws), ws.numel(), st))
    if check:
        _check(LIB.kmeans_argsort_status(_ptr(ws), ws.numel(), st))
    return sorted_ids, sorted_idx, counts


def kmeans_update(x, sorted_ids, sorted_idx, counts, centroids, shift=None, want_shift=False, stream=None):
    """Updates `centroids` (f32 [B,K,D]) in place; returns shift (float64 [B]) or None."""
    torch = _torch()
    _need(x.dim() == 3 and x.is_contiguous(), "x must be a contiguous [B, N, D] tensor")
    B, N, D = x.shape
    _need(centroids.dim() == 3 and centroids.is_contiguous() and centroids.dtype == torch.float32, "centroids")
    K = centroids.shape[1]
    if want_shift and shift is None:
        shift = torch.empty((B,), dtype=torch.float64, device=x.device)
    dt = dtype_code(x)
    st = _stream(x, stream)
    ws = workspace(KM_OP_UPDATE, dt, B, N, D, K, x.device, stream=st)
    _check(LIB.kmeans_update(_ptr(x), dt, _ptr(sorted_ids), _ptr(sorted_idx), _ptr(counts), B, N, D, K,
                             _ptr(centroids), _ptr(shift), _ptr(ws), ws.numel(), st))
    return shift


def kmeans_fit(x, centroids, iters: int, tol: float = 0.0, chunk_points: int = 0, assign=None,
               want_assign=True, device=None, stream=None):
    """Lloyd's loop.  x: device tensor, or pinned host tensor (streamed path).  `centroids` (device
    f32 [B,K,D]) holds the init and receives the result.  Returns (assign, inertia [iters_done, B]
    numpy float64, iters_done)."""
    torch = _torch()
    import numpy as np
    _need(x.dim() == 3 and x.is_contiguous(), "x must be a contiguous [B, N, D] tensor")
    B, N, D = x.shape
    _need(centroids.is_cuda and centroids.dtype == torch.float32 and centroids.is_contiguous(), "centroids")
    K = centroids.shape[1]
    dev = centroids.device
    if want_assign and assign is None:
        assign = torch.empty((B, N), dtype=torch.int32, device=dev)
    dt = dtype_code(x)
    op = KM_OP_FIT if x.is_cuda else KM_OP_FIT_HOST
    st = _stream(centroids, stream)
    ws = workspace(op, dt, B, N, D, K, dev, chunk_points, stream=st)
    inertia = np.zeros((iters, B), dtype=np.float64)
    done = ctypes.c_int32(0)
    _check(LIB.kmeans_fit(_ptr(x), dt, B, N, D, K, int(iters), float(tol), int(chunk_points), _ptr(centroids),
                          _ptr(assign), inertia.ctypes.data_as(ctypes.c_void_p), ctypes.byref(done), _ptr(ws),
                          ws.numel(), st))
    return assign, inertia[: done.value], done.value


def kmeans_fit_blocks(blocks, centroids, iters: int, tol: float = 0.0, chunk_points: int = 0, assign=None,
                      want_assign=True, stream=None):
    """Lloyd's loop, streamed, for one problem whose points are split over pinned host tensors
    `blocks` ([n_j, D] each, one dtype; every block but the last a multiple of the chunk).
    `centroids` (device f32 [1, K, D]) holds the init and receives the result.  Returns (assign
    [1, N] or None, inertia [iters_done, 1] numpy float64, iters_done)."""
    torch = _torch()
    import numpy as np
    _need(len(blocks) >= 1, "at least one block")
    D = blocks[0].shape[-1]
    for t in blocks:
        _need(t.dim() == 2 and t.shape[1] == D and t.is_contiguous() and t.dtype == blocks[0].dtype
              and not t.is_cuda, "blocks: contiguous host [n, D] tensors of one dtype")
    _need(centroids.is_cuda and centroids.dtype == torch.float32 and centroids.is_contiguous()
          and centroids.dim() == 3 and centroids.shape[0] == 1, "centroids: device f32 [1, K, D]")
    K = centroids.shape[1]
    N = sum(int(t.shape[0]) for t in blocks)
    dev = centroids.device
    if want_assign and assign is None:
        assign = torch.empty((1, N), dtype=torch.int32, device=dev)
    dt = dtype_code(blocks[0])
    st = _stream(centroids, stream)
    ws = workspace(KM_OP_FIT_HOST, dt, 1, N, D, K, dev, chunk_points, stream=st)
    ptrs = (ctypes.c_void_p * len(blocks))(*[t.data_ptr() for t in blocks])
    npts = (ctypes.c_int64 * len(blocks))(*[int(t.shape[0]) for t in blocks])
    inertia = np.zeros((iters, 1), dtype=np.float64)
    done = ctypes.c_int32(0)
    _check(LIB.kmeans_fit_blocks(ptrs, npts, len(blocks), dt, D, K, int(iters), float(tol), int(chunk_points),
                                 _ptr(centroids), _ptr(assign), inertia.ctypes.data_as(ctypes.c_void_p),
                                 ctypes.byref(done), _ptr(ws), ws.numel(), st))
    return assign, inertia[: done.value], done.value


def stage_buffer(dt: int, B: int, N: int, D: int, K: int, chunk_points: int = 0):
    """A pinned host uint8 tensor of the size kmeans_fit_staged asks for (KM_OP_STAGE_PINNED)."""
    torch = _torch()
    nbytes = LIB.kmeans_workspace_bytes(KM_OP_STAGE_PINNED, dt, B, N, D, K, chunk_points)
    if nbytes == 0:
        raise FlashKMError(KM_ERR_INVALID, last_error() or "bad shape for the staging buffer")
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, pin_memory=True)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


def kmeans_fit_staged(x, centroids, iters: int, tol: float = 0.0, chunk_points: int = 0, stage=None, assign=None,
                      want_assign=True, stream=None):
    """Lloyd's loop, streamed from host memory that need not be pinned: x is a contiguous host
    tensor [B, N, D] (pageable or pinned); chunks pass through the pinned tensor `stage` (from
    stage_buffer, made here when None).  `centroids` (device f32 [B, K, D]) holds the init and
    receives the result.  Returns (assign or None, inertia [iters_done, B] numpy float64,
    iters_done)."""
    torch = _torch()
    import numpy as np
    _need(x.dim() == 3 and x.is_contiguous() and not x.is_cuda, "x must be a contiguous host [B, N, D] tensor")
    B, N, D = x.shape
    _need(centroids.is_cuda and centroids.dtype == torch.float32 and centroids.is_contiguous()
          and centroids.dim() == 3 and centroids.shape[0] == B and centroids.shape[2] == D,
          "centroids: device f32 [B, K, D]")
    K = centroids.shape[1]
    dt = dtype_code(x)
    dev = centroids.device
    if stage is None:
        stage = stage_buffer(dt, B, N, D, K, chunk_points)
    if want_assign and assign is None:
        assign = torch.empty((B, N), dtype=torch.int32, device=dev)
    st = _stream(centroids, stream)
    ws = workspace(KM_OP_FIT_HOST, dt, B, N, D, K, dev, chunk_points, stream=st)
    inertia = np.zeros((iters, B), dtype=np.float64)
    done = ctypes.c_int32(0)
    _check(LIB.kmeans_fit_staged(_ptr(x), dt, B, N, D, K, int(iters), float(tol), int(chunk_points), _ptr(stage),
                                 stage.numel(), _ptr(centroids), _ptr(assign), inertia.ctypes.data_as(ctypes.c_void_p),
                                 ctypes.byref(done), _ptr(ws), ws.numel(), st))
    return assign, inertia[: done.value], done.value


def kmeans_fit_metric(x, centroids, metric, iters: int, tol: float = 0.0, chunk_points: int = 0, assign=None,
                      want_assign=True, stream=None):
    """k-means under `metric` ("l2", "dot" or "cosine").  x: device tensor, or pinned host tensor
    (streamed path).  `centroids` (device f32 [B,K,D]) holds the init and receives the result (unit
    rows for cosine).  Returns (assign, objective [iters_done, B] numpy float64: inertia for "l2",
    total similarity otherwise, iters_done)."""
    torch = _torch()
    import numpy as np
    m = metric_code(metric)
    _need(x.dim() == 3 and x.is_contiguous(), "x must be a contiguous [B, N, D] tensor")
    B, N, D = x.shape
    _need(centroids.is_cuda and centroids.dtype == torch.float32 and centroids.is_contiguous(), "centroids")
    K = centroids.shape[1]
    dev = centroids.device
    if want_assign and assign is None:
        assign = torch.empty((B, N), dtype=torch.int32, device=dev)
    dt = dtype_code(x)
    if x.is_cuda:
        op = {KM_METRIC_L2: KM_OP_FIT, KM_METRIC_DOT: KM_OP_FIT_DOT, KM_METRIC_COSINE: KM_OP_FIT_COSINE}[m]
    else:
        op = KM_OP_FIT_HOST
    st = _stream(centroids, stream)
    ws = workspace(op, dt, B, N, D, K, dev, chunk_points, stream=st)
    obj = np.zeros((iters, B), dtype=np.float64)
    done = ctypes.c_int32(0)
    _check(LIB.kmeans_fit_metric(_ptr(x), dt, m, B, N, D, K, int(iters), float(tol), int(chunk_points),
                                 _ptr(centroids), _ptr(assign), obj.ctypes.data_as(ctypes.c_void_p),
                                 ctypes.byref(done), _ptr(ws), ws.numel(), st))
    return assign, obj[: done.value], done.value


def batch_kmeans_euclid(x, n_clusters: int, max_iters: int = 100, tol: float = 0.0, init_centroids=None,
                        chunk_points: int = 0, seed: int = 0):
    """README-style entry (flash-kmeans README, "Usage"): returns (cluster_ids, centers, inertia).
    Without init_centroids, K distinct points per problem are drawn with torch's generator.  x on
    the GPU, or in host memory: pinned (streamed fit) or pageable (staged streamed fit)."""
    torch = _torch()
    B, N, D = x.shape
    dev = x.device if x.is_cuda else torch.device("cuda", torch.cuda.current_device())
    if init_centroids is None:
        init_centroids = _seeded_init(x, n_clusters, seed)
    c = init_centroids.to(dev, dtype=torch.float32).contiguous().clone()
    if not x.is_cuda and not x.is_pinned():
        ids, inertia, _ = kmeans_fit_staged(x.contiguous(), c, max_iters, tol, chunk_points)
    else:
        ids, inertia, _ = kmeans_fit(x, c, max_iters, tol, chunk_points)
    return ids, c, inertia


def batch_kmeans_cosine(x, n_clusters: int, max_iters: int = 100, tol: float = 0.0, init_centroids=None, seed: int = 0):
    """Cosine (spherical) k-means, README-style: returns (cluster_ids, unit centers, objective)."""
    return _batch_metric(x, n_clusters, max_iters, tol, init_centroids, seed, "cosine")


def batch_kmeans_dot(x, n_clusters: int, max_iters: int = 100, tol: float = 0.0, init_centroids=None, seed: int = 0):
    """Dot-product k-means, README-style: returns (cluster_ids, centers, objective)."""
    return _batch_metric(x, n_clusters, max_iters, tol, init_centroids, seed, "dot")


def _seeded_init(x, n_clusters: int, seed: int):
    """K distinct points per problem, drawn with torch's CPU generator (fp32 copies)."""
    torch = _torch()
    B, N, _ = x.shape
    g = torch.Generator(device="cpu").manual_seed(seed)
    idx = torch.stack([torch.randperm(N, generator=g)[:n_clusters] for _ in range(B)])
    return torch.stack([x[b].index_select(0, idx[b].to(x.device)) for b in range(B)]).float()


def _batch_metric(x, n_clusters, max_iters, tol, init_centroids, seed, metric):
    """x on the GPU, in pinned host memory (streamed fit), or, for the Euclidean metric, in pageable
    host memory (staged streamed fit); the centroids live on the GPU (the current device for host x)."""
    torch = _torch()
    pageable = not x.is_cuda and not x.is_pinned()
    _need(not pageable or metric_code(metric) == KM_METRIC_L2,
          "x must be on the GPU or in pinned host memory (pageable host memory: Euclidean metric only)")
    if init_centroids is None:
        init_centroids = _seeded_init(x, n_clusters, seed)
    dev = x.device if x.is_cuda else torch.device("cuda", torch.cuda.current_device())
    c = init_centroids.to(dev, dtype=torch.float32).contiguous().clone()
    if pageable:
        ids, obj, _ = kmeans_fit_staged(x.contiguous(), c, max_iters, tol)
    else:
        ids, obj, _ = kmeans_fit_metric(x, c, metric, max_iters, tol)
    return ids, c, obj


class FlashKMeans:
    """faiss / scikit-learn style k-means object over the C-ABI (README: "an API interface similar to
    faiss/sklearn"; "FlashKMeans(d=..., k=..., niter=..., tol=..., dtype=...)", with train / fit /
    predict / fit_predict and init_centroids).

    Input: [N, d] (one problem) or [B, N, d] (B independent problems sharing k), on the GPU, or in
    host memory.  Pinned host memory selects the streamed path; other host tensors are copied to
    the GPU first, or, with `host_streaming=True` (Euclidean metric), fitted in place through the
    staged streamed path (kmeans_fit_staged: for point sets larger than the GPU's memory).  `dtype`
    is the compute dtype the points are cast to.
    After fitting: `centroids` (fp32 [B, k, d], or [k, d] for 2-D input), `labels_` (from the last
    assignment), `obj` (per-iteration inertia, or total similarity for "dot" / "cosine"),
    `iters_done`.  `cluster_centers_` and `inertia_` mirror scikit-learn's names."""

    def __init__(self, d: int, k: int, niter: int = 25, tol: float = 0.0, dtype=None, metric: str = "l2",
                 device=None, seed: int = 0, verbose: bool = False, chunk_points: int = 0,
                 host_streaming: bool = False):
        torch = _torch()
        _need(d >= 1 and k >= 1 and niter >= 1 and tol >= 0.0, "d, k, niter must be >= 1 and tol >= 0")
        metric_code(metric)
        self.d, self.k, self.niter, self.tol = int(d), int(k), int(niter), float(tol)
        self.dtype = dtype if dtype is not None else torch.float16
        _need(self.dtype in (torch.float32, torch.float16, torch.bfloat16), "dtype: float32, float16 or bfloat16")
        self.metric = metric
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.seed, self.verbose, self.chunk_points = int(seed), bool(verbose), int(chunk_points)
        _need(not host_streaming or metric_code(metric) == KM_METRIC_L2, "host_streaming: Euclidean metric only")
        self.host_streaming = bool(host_streaming)
        self.centroids = None
        self.labels_ = None
        self.obj = None
        self.iters_done = 0
        self._batched = True
        self._prep = None

    # -- input marshalling
    def _points(self, x, fitting=False):
        _need(x.dim() in (2, 3) and x.shape[-1] == self.d, "x must be [N, %d] or [B, N, %d]" % (self.d, self.d))
        if fitting:
            _need(self.k <= x.shape[-2], "k (%d) > number of points (%d)" % (self.k, x.shape[-2]))
        batched = x.dim() == 3
        x3 = x if batched else x.unsqueeze(0)
        if x3.dtype != self.dtype:
            x3 = x3.to(self.dtype)
        if not x3.is_cuda and not x3.is_pinned() and not (fitting and self.host_streaming):
            x3 = x3.to(self.device)
        return x3.contiguous(), batched

    def _out(self, t, batched):
        return t if batched else t[0]

    # -- faiss names
    def train(self, x, init_centroids=None):
        """Fits the centroids; returns self."""
        torch = _torch()
        x3, batched = self._points(x, fitting=True)
        B, N, _ = x3.shape
        if init_centroids is None:
            init = _seeded_init(x3, self.k, self.seed)
        else:
            init = init_centroids if init_centroids.dim() == 3 else init_centroids.unsqueeze(0)
            _need(tuple(init.shape) == (B, self.k, self.d), "init_centroids must be [B, k, d] or [k, d]")
        c = init.to(self.device, dtype=torch.float32).contiguous().clone()
        if not x3.is_cuda and not x3.is_pinned():   # host_streaming with pageable points
            a, obj, done = kmeans_fit_staged(x3, c, self.niter, self.tol, self.chunk_points)
        else:
            a, obj, done = kmeans_fit_metric(x3, c, self.metric, self.niter, self.tol, self.chunk_points)
        self.centroids = c
        self.labels_ = a
        self.obj = obj
        self.iters_done = done
        self._batched = batched
        self._prep = None
        if self.verbose:
            for t in range(done):
                print("iteration %d: %s" % (t, " ".join("%.6g" % v for v in obj[t])))
        return self

    def fit(self, x, init_centroids=None):
        return self.train(x, init_centroids)

    def predict(self, x):
        """Nearest (or most similar) fitted centroid of every point, through FlashAssign."""
        torch = _torch()
        _need(self.centroids is not None, "call fit / train first")
        x3, batched = self._points(x)
        if not x3.is_cuda:
            x3 = x3.to(self.device)
        _need(x3.shape[0] == self.centroids.shape[0], "x has %d problems, the model %d" % (
            x3.shape[0], self.centroids.shape[0]))
        if self._prep is None:
            self._prep = kmeans_prepare_centroids(self.centroids, x3.dtype, metric=self.metric)
        if self.metric == "cosine":
            x3 = kmeans_normalize_rows(x3)
        a, _ = kmeans_assign_prepared(x3, self._prep)
        return self._out(a, batched)

    def fit_predict(self, x, init_centroids=None):
        """Fits, then returns the labels of the last assignment."""
        self.train(x, init_centroids)
        return self._out(self.labels_, self._batched)

    # -- scikit-learn names
    @property
    def cluster_centers_(self):
        return None if self.centroids is None else self._out(self.centroids, self._batched)

    @property
    def inertia_(self):
        return None if self.obj is None or len(self.obj) == 0 else self.obj[-1]
