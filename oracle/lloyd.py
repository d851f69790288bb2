"""Oracle for batched Lloyd k-means (fp64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import or call this package.  It imports nothing from
the GPU package and the GPU package never imports it.

Sources (page, section):
  * paper summary "Flash-KMeans: Fast and Memory-Efficient Exact K-Means", "Method":
    a Lloyd iteration = assignment (squared distances to every centroid, row-wise
    arg-min) followed by update (average of the points assigned to each cluster);
    "Key claims": the output is exact Lloyd's k-means, not an approximation.
  * paper digest "Flash-KMeans：快速且内存高效精确K-Means聚类", "K-Means聚类算法":
    the objective  sum_i ||x_i - c_{a_i}||^2;  "argsort与分段规约": arg-sorting the
    assignment vector makes equal cluster ids contiguous (worked example
    [3,1,2,1,3,2] -> [1,1,2,2,3,3] with indices [1,3,2,5,0,4]);  "方法步骤详情":
    sums s and counts n per cluster, then c_k <- s_k / n_k.

Readings taken where the pages are silent (each is listed in the design notes):
  * ties in the arg-min go to the lowest centroid index;
  * a cluster that receives no point keeps its previous centroid;
  * the arg-sort is stable and 0-based (as the worked example is);
  * "modelled" mode: the assignment uses c~ = dtype(fp32(C)), the centroid master
    rounded to fp32 and then to the input dtype (the low-precision contraction consumes
    c~); "pure" mode uses C itself (exact Lloyd, used for invariants);
  * inertia J_t = sum_i ||x_i - c~_{a_i}||^2 against the centroids the assignment used;
  * shift_t = max over batches of sum_k ||C_{t+1,k} - C_{t,k}||^2; the run stops after
    iteration t when shift_t < tol.  The pages give only tol values, so this rule is
    "parity unpinned".

Every array is float64; batches are independent problems that share K.
"""
from __future__ import annotations

import ctypes

import numpy as np

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        from . import build as _build
        path = _build.build()
        lib = ctypes.CDLL(path)
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        lib.oracle_assign.argtypes = [f64p, f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      i64p, f64p, f64p]
        lib.oracle_assign.restype = None
        lib.oracle_dist_to.argtypes = [f64p, f64p, i64p, ctypes.c_int64, ctypes.c_int64, f64p]
        lib.oracle_dist_to.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def threads() -> int:
    """OpenMP threads the oracle's distance loops use."""
    return int(_lib().oracle_threads())


# ------------------------------------------------------------------------------------------
# step 1 (modelled mode): the centroid operand the low-precision contraction consumes
# ------------------------------------------------------------------------------------------
def _bf16_round(v32: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values.
    bfloat16 keeps the top 16 bits of the IEEE float32 pattern."""
    u = np.ascontiguousarray(v32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    rest = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    up = (rest > half) | ((rest == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    keep = keep + up.astype(np.uint64)
    return (keep << np.uint64(16)).astype(np.uint32).view(np.float32)


def centroid_operand(c: np.ndarray, dtype: str, mode: str = "modelled") -> np.ndarray:
    """c~ used by the assignment: dtype(fp32(c)) in modelled mode, c in pure mode."""
    c = np.asarray(c, dtype=np.float64)
    if mode == "pure":
        return c
    c32 = c.astype(np.float32)
    if dtype == "f32":
        return c32.astype(np.float64)
    if dtype == "f16":
        return c32.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        return _bf16_round(c32).astype(np.float64)
    raise ValueError(dtype)


# ------------------------------------------------------------------------------------------
# assignment
# ------------------------------------------------------------------------------------------
def row_norms(x: np.ndarray) -> np.ndarray:
    """||x_i||^2 in fp64 (the quantity the method precomputes before the scan)."""
    x = np.asarray(x, dtype=np.float64)
    return np.sum(x * x, axis=-1)


def assign(x: np.ndarray, c: np.ndarray):
    """One problem: x [N, D], c [K, D] -> (a [N] int64, d1 [N], d2 [N]).

    a_i = lowest k minimising ||x_i - c_k||^2; d1 the minimum, d2 the smallest distance to
    any other centroid (inf when K == 1)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    c = np.ascontiguousarray(c, dtype=np.float64)
    n, d = x.shape
    k = c.shape[0]
    assert c.shape[1] == d and k >= 1
    a = np.empty(n, dtype=np.int64)
    d1 = np.empty(n, dtype=np.float64)
    d2 = np.empty(n, dtype=np.float64)
    if n:
        _lib().oracle_assign(x, c, n, k, d, a, d1, d2)
    return a, d1, d2


def assign_batched(x: np.ndarray, c: np.ndarray):
    """x [B, N, D], c [B, K, D] -> (a, d1, d2) each [B, N]."""
    outs = [assign(x[b], c[b]) for b in range(x.shape[0])]
    return tuple(np.stack([o[j] for o in outs]) for j in range(3))


def dist_to(x: np.ndarray, c: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """||x_i - c_{sel_i}||^2 for one problem (fp64)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    c = np.ascontiguousarray(c, dtype=np.float64)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    assert sel.shape[0] == x.shape[0]
    assert sel.size == 0 or (sel.min() >= 0 and sel.max() < c.shape[0])
    out = np.empty(x.shape[0], dtype=np.float64)
    if x.shape[0]:
        _lib().oracle_dist_to(x, c, sel, x.shape[0], x.shape[1], out)
    return out


def near_mask(d1: np.ndarray, d2: np.ndarray, rel: float = 1e-3) -> np.ndarray:
    """Points whose top-2 distance gap is below rel * |best| (ties that rounding may flip)."""
    return (d2 - d1) < rel * np.abs(d1)


# ------------------------------------------------------------------------------------------
# sort-inverse update
# ------------------------------------------------------------------------------------------
def argsort_ids(a: np.ndarray, K: int):
    """One problem: stable ascending arg-sort of the assignment vector.

    Returns (sorted ids, sorted_idx, counts[K]) with sorted ids = a[sorted_idx]."""
    a = np.asarray(a, dtype=np.int64)
    assert a.size == 0 or (a.min() >= 0 and a.max() < K)
    sidx = np.argsort(a, kind="stable")
    counts = np.bincount(a, minlength=K)
    return a[sidx], sidx, counts


def segment_sums(x: np.ndarray, a: np.ndarray, K: int):
    """One problem (or one block of its points): s_k = sum_{a_i = k} x_i and
    n_k = |{i : a_i = k}|, in fp64.  Returns (sums [K, D], counts [K])."""
    x = np.asarray(x, dtype=np.float64)
    a = np.asarray(a, dtype=np.int64)
    sums = np.zeros((K, x.shape[1]), dtype=np.float64)
    np.add.at(sums, a, x)
    return sums, np.bincount(a, minlength=K)


def update(x: np.ndarray, a: np.ndarray, c_old: np.ndarray):
    """One problem: s_k = sum_{a_i = k} x_i, n_k = |{i : a_i = k}|,
    c_k = s_k / n_k, or the previous c_k when n_k == 0.  Returns (c_new, counts)."""
    c_old = np.asarray(c_old, dtype=np.float64)
    sums, counts = segment_sums(x, a, c_old.shape[0])
    c_new = c_old.copy()
    nz = counts > 0
    c_new[nz] = sums[nz] / counts[nz, None]
    return c_new, counts


def inertia(x: np.ndarray, c: np.ndarray, a: np.ndarray) -> float:
    """sum_i ||x_i - c_{a_i}||^2 for one problem."""
    return float(np.sum(dist_to(x, c, a)))


def shift(c_new: np.ndarray, c_old: np.ndarray) -> np.ndarray:
    """Per problem: sum_k ||c_new_k - c_old_k||^2 (batched input -> [B])."""
    diff = np.asarray(c_new, dtype=np.float64) - np.asarray(c_old, dtype=np.float64)
    return np.sum(diff * diff, axis=(-1, -2))


# ------------------------------------------------------------------------------------------
# the iteration and the loop
# ------------------------------------------------------------------------------------------
def lloyd_iteration(x: np.ndarray, c: np.ndarray, dtype: str = "f32", mode: str = "modelled"):
    """One batched iteration.  x [B, N, D] (exact values of the stored points), c [B, K, D]
    the centroid master.  Returns a dict with the operand c~, labels, d1, d2, inertia [B],
    sorted ids/idx, counts, new centroids and shift [B]."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    B, N, D = x.shape
    K = c.shape[1]
    ct = centroid_operand(c, dtype, mode)
    a, d1, d2 = assign_batched(x, ct)
    sids = np.empty((B, N), dtype=np.int64)
    sidx = np.empty((B, N), dtype=np.int64)
    counts = np.empty((B, K), dtype=np.int64)
    c_new = np.empty_like(c)
    for b in range(B):
        sids[b], sidx[b], counts[b] = argsort_ids(a[b], K)
        c_new[b], _ = update(x[b], a[b], c[b])
    if mode == "modelled":
        c_new = c_new.astype(np.float32).astype(np.float64)   # the master is kept in fp32
    return {
        "c_operand": ct, "a": a, "d1": d1, "d2": d2, "inertia": d1.sum(axis=1),
        "sorted_ids": sids, "sorted_idx": sidx, "counts": counts, "c_new": c_new,
        "shift": shift(c_new, c),
    }


def lloyd_fit(x: np.ndarray, c0: np.ndarray, iters: int, tol: float = 0.0, dtype: str = "f32",
              mode: str = "modelled"):
    """Free-running Lloyd from c0.  Returns a dict: labels (from the last assignment),
    centroids, inertia [T, B], shift [T], iterations done."""
    assert iters >= 1 and tol >= 0.0
    c = np.asarray(c0, dtype=np.float64).copy()
    J, S = [], []
    labels = None
    done = 0
    for _ in range(iters):
        it = lloyd_iteration(x, c, dtype, mode)
        labels = it["a"]
        J.append(it["inertia"])
        c = it["c_new"]
        s = float(np.max(it["shift"]))
        S.append(s)
        done += 1
        if s < tol:
            break
    return {"labels": labels, "centroids": c, "inertia": np.array(J), "shift": np.array(S),
            "iters_done": done}


__all__ = [
    "centroid_operand", "row_norms", "assign", "assign_batched", "dist_to", "near_mask", "segment_sums",
    "argsort_ids", "update", "inertia", "shift", "lloyd_iteration", "lloyd_fit", "threads",
]
