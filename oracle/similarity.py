"""Oracle for the similarity variants of batched Lloyd k-means: dot-product and cosine
k-means (fp64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import or call this module.  It imports nothing from the
GPU package and the GPU package never imports it.

Source (page, section): the project README ("Flash-KMeans" repository page, section "CuTe
backend") names cosine k-means and dot-product k-means as modes the library serves on its
Triton paths.  It defines neither.  Readings taken (each listed in the design notes):

  * dot-product k-means: the similarity of point x and centroid c is x.c.  The assignment
    is a_i = the lowest k maximising x_i.c~_k (c~ the centroid operand, modelled exactly as
    for Euclidean k-means: dtype(fp32(c))).  The update is the Euclidean one: the mean of the
    members, and a cluster without points keeps its centroid.
  * cosine k-means (spherical k-means): points enter as unit vectors
    x^_i = x_i / ||x_i|| (a zero row stays zero), rounded to the input dtype; centroids are
    unit vectors (the initial ones are normalised first).  The assignment is a_i = the lowest
    k maximising x^_i.c~_k.  The update is the mean direction c_k = S_k / ||S_k|| with
    S_k = sum_{a_i = k} x^_i; a cluster without points, or whose S_k is the zero vector,
    keeps its centroid.
  * the objective reported per iteration is the total similarity
    sum_i x_i.c~_{a_i} (x^ for cosine), which the method increases.
  * near tie (where rounding may flip the pick): s_(1) - s_(2) < 1e-3 * ||x_i|| * max_k ||c~_k||,
    the Cauchy-Schwarz scale of the scores (a relative band around s_(1) would collapse for
    scores near zero).

Every array is float64 unless stated.
"""
from __future__ import annotations

import numpy as np

from .lloyd import centroid_operand, segment_sums, argsort_ids, shift


def normalize_rows(x: np.ndarray) -> np.ndarray:
    """x_i / ||x_i|| in fp64; rows of norm zero stay zero (last axis is the feature axis)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    out = np.zeros_like(x)
    np.divide(x, n, out=out, where=n > 0)
    return out


def round_to_dtype(v: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values rounded to fp32 and then to the storage dtype (nearest even each time),
    returned as fp64: how a value computed in fp32 is stored in that dtype."""
    return centroid_operand(v, dtype, "modelled")


def similarity_assign(x: np.ndarray, c: np.ndarray, chunk: int = 8192):
    """One problem: x [N, D], c [K, D] -> (a [N] int64, s1 [N], s2 [N], scale [N]).

    a_i = the lowest k maximising x_i.c_k (np.argmax keeps the first maximum); s1 the
    maximum, s2 the largest similarity to any other centroid (-inf when K == 1); scale the
    score scale ||x_i|| * max_k ||c_k|| of the near-tie band.  The products are one fp64
    matrix product per chunk of points."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    n = x.shape[0]
    k = c.shape[0]
    a = np.empty(n, dtype=np.int64)
    s1 = np.empty(n)
    s2 = np.full(n, -np.inf)
    cmax = float(np.sqrt(np.max(np.sum(c * c, axis=1)))) if k else 0.0
    scale = np.sqrt(np.sum(x * x, axis=1)) * cmax
    for i0 in range(0, n, chunk):
        s = x[i0:i0 + chunk] @ c.T
        am = np.argmax(s, axis=1)
        rows = np.arange(s.shape[0])
        a[i0:i0 + chunk] = am
        s1[i0:i0 + chunk] = s[rows, am]
        if k > 1:
            s[rows, am] = -np.inf
            s2[i0:i0 + chunk] = np.max(s, axis=1)
    return a, s1, s2, scale


def similarity_near_mask(s1: np.ndarray, s2: np.ndarray, scale: np.ndarray, rel: float = 1e-3) -> np.ndarray:
    """Points whose top-2 similarity gap is inside the rounding band."""
    return (s1 - s2) < rel * scale


def mean_direction(x_hat: np.ndarray, a: np.ndarray, c_old: np.ndarray):
    """One problem: S_k = sum_{a_i = k} x^_i; c_k = S_k / ||S_k||, or the previous c_k when
    cluster k has no point or S_k = 0.  Returns (c_new, counts)."""
    c_old = np.asarray(c_old, dtype=np.float64)
    sums, counts = segment_sums(x_hat, a, c_old.shape[0])
    norms = np.sqrt(np.sum(sums * sums, axis=1))
    c_new = c_old.copy()
    ok = (counts > 0) & (norms > 0)
    c_new[ok] = sums[ok] / norms[ok, None]
    return c_new, counts


def mean_update(x: np.ndarray, a: np.ndarray, c_old: np.ndarray):
    """One problem: the Euclidean update (mean of the members; empties keep).  Returns
    (c_new, counts)."""
    c_old = np.asarray(c_old, dtype=np.float64)
    sums, counts = segment_sums(x, a, c_old.shape[0])
    c_new = c_old.copy()
    nz = counts > 0
    c_new[nz] = sums[nz] / counts[nz, None]
    return c_new, counts


def similarity_iteration(x: np.ndarray, c: np.ndarray, metric: str, dtype: str = "f32", mode: str = "modelled"):
    """One batched iteration of dot-product (metric "dot") or cosine (metric "cosine")
    k-means.  x [B, N, D]: the points as the contraction sees them (for cosine: already the
    unit rows x^ in the storage dtype); c [B, K, D] the fp32 centroid master (unit rows for
    cosine).  Returns a dict with the operand c~, labels, s1, s2, scale, objective [B],
    sorted ids/idx, counts, new centroids and shift [B]."""
    assert metric in ("dot", "cosine")
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    B, N, D = x.shape
    K = c.shape[1]
    ct = centroid_operand(c, dtype, mode)
    a = np.empty((B, N), dtype=np.int64)
    s1 = np.empty((B, N))
    s2 = np.empty((B, N))
    scale = np.empty((B, N))
    sids = np.empty((B, N), dtype=np.int64)
    sidx = np.empty((B, N), dtype=np.int64)
    counts = np.empty((B, K), dtype=np.int64)
    c_new = np.empty_like(c)
    for b in range(B):
        a[b], s1[b], s2[b], scale[b] = similarity_assign(x[b], ct[b])
        sids[b], sidx[b], counts[b] = argsort_ids(a[b], K)
        if metric == "dot":
            c_new[b], _ = mean_update(x[b], a[b], c[b])
        else:
            c_new[b], _ = mean_direction(x[b], a[b], c[b])
    if mode == "modelled":
        c_new = c_new.astype(np.float32).astype(np.float64)   # the master is kept in fp32
    return {
        "c_operand": ct, "a": a, "s1": s1, "s2": s2, "scale": scale, "objective": s1.sum(axis=1),
        "sorted_ids": sids, "sorted_idx": sidx, "counts": counts, "c_new": c_new,
        "shift": shift(c_new, c),
    }


def similarity_fit(x: np.ndarray, c0: np.ndarray, metric: str, iters: int, tol: float = 0.0, dtype: str = "f32",
                   mode: str = "modelled"):
    """Free-running dot-product or cosine k-means from c0.  For cosine, x is normalised and
    stored in the dtype (modelled mode; pure mode keeps fp64) and c0 is normalised first (and
    kept in fp32 in modelled mode).  Returns a dict: labels (from the last assignment),
    centroids, objective [T, B], shift [T], iterations done, and the x the iterations used."""
    assert iters >= 1 and tol >= 0.0
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c0, dtype=np.float64).copy()
    if metric == "cosine":
        x = normalize_rows(x)
        c = normalize_rows(c)
        if mode == "modelled":
            x = round_to_dtype(x, dtype)
            c = c.astype(np.float32).astype(np.float64)
    J, S = [], []
    labels = None
    done = 0
    for _ in range(iters):
        it = similarity_iteration(x, c, metric, dtype, mode)
        labels = it["a"]
        J.append(it["objective"])
        c = it["c_new"]
        s = float(np.max(it["shift"]))
        S.append(s)
        done += 1
        if s < tol:
            break
    return {"labels": labels, "centroids": c, "objective": np.array(J), "shift": np.array(S),
            "iters_done": done, "x_used": x}


__all__ = [
    "normalize_rows", "round_to_dtype", "similarity_assign", "similarity_near_mask", "mean_direction",
    "mean_update", "similarity_iteration", "similarity_fit",
]
