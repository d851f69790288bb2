"""Seeded synthetic workloads for batched Lloyd k-means: inputs only.

This module draws points, picks the initial centroid rows and casts values to
the storage dtype.  It holds none of the k-means arithmetic (no distances, no
arg-min, no means of clusters), so both the GPU path's tests/benchmark and the
CPU oracle can take their inputs from it without sharing method code.

Workload shapes restate the pages' workloads:
  * the README "Usage" example (B=32, N=75600, D=128, K=1000, fp16, tol=1e-4);
  * the paper digest's motivation shape (N=65536, K=1024, d=128, B=32);
  * the README "Centre your data" attention-sink shape (a few channels
    offset by +64) together with skewed (hot) clusters from the paper summary,
    "Key claims" (scatter contention on hot clusters);
  * the README "Large tensor Benchmark" (data in pinned CPU memory, K ~ sqrt(N))
    and "Large-D and dtype support" (D > 512 split-D path, fp32).

Recipe (all configurations):
  * seeds: ``np.random.SeedSequence(20260309 + seed_id)``; its children are
    (means, labels/noise blocks, init) and per batch / per block of 2**20 points;
  * values are drawn as float32: mixture means ``mean_std * N(0, I)``, unit
    variance noise, then cast round-to-nearest-even to the storage dtype;
  * bf16 values are stored as uint16 bit patterns (numpy has no bfloat16);
  * init centroids: the rows ``perm(N)[:K]`` of a seeded permutation, upcast
    exactly to float32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

BLOCK_POINTS = 1 << 20
BASE_SEED = 20260309


@dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int
    B: int
    N: int
    D: int
    K: int
    dtype: str            # "f32" | "f16" | "bf16"
    iters: int
    tol: float
    data: str             # "gmm" | "normal"
    M: int = 0            # mixture components
    mean_std: float = 0.0
    zipf_s: float = 0.0   # 0 -> uniform component weights
    offset: float = 0.0   # added to the first `offset_channels` channels
    offset_channels: int = 0
    center: bool = False  # subtract the (fp64) mean over points before clustering
    host: bool = False    # points live in pinned host memory (streamed path)
    chunk: int = 0        # points per streamed chunk

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny fp32 Lloyd run
    "tiny_f32": Workload("tiny_f32", 1, B=1, N=4096, D=16, K=8, dtype="f32", iters=10, tol=0.0,
                         data="gmm", M=8, mean_std=5.0),
    # batched fp16 run shaped like the README usage example
    "batched_f16": Workload("batched_f16", 2, B=32, N=75600, D=128, K=1000, dtype="f16", iters=10,
                            tol=1e-4, data="normal"),
    # headline bf16 kernel shape
    "headline_bf16": Workload("headline_bf16", 3, B=32, N=65536, D=128, K=1024, dtype="bf16", iters=10,
                              tol=0.0, data="gmm", M=1024, mean_std=2.0),
    # skewed large-N update stress (Zipf 1.2 weights, 4 channels offset by +64, centred)
    "skew_bf16_k64": Workload("skew_bf16_k64", 4, B=1, N=1 << 24, D=128, K=64, dtype="bf16", iters=5,
                              tol=0.0, data="gmm", M=64, mean_std=2.0, zipf_s=1.2, offset=64.0,
                              offset_channels=4, center=True),
    "skew_bf16_k4096": Workload("skew_bf16_k4096", 5, B=1, N=1 << 24, D=128, K=4096, dtype="bf16", iters=5,
                                tol=0.0, data="gmm", M=4096, mean_std=2.0, zipf_s=1.2, offset=64.0,
                                offset_channels=4, center=True),
    # host-resident streamed run (pinned host memory, chunks of 2**24 points)
    "streamed_f16": Workload("streamed_f16", 6, B=1, N=1 << 30, D=64, K=32768, dtype="f16", iters=3,
                             tol=0.0, data="gmm", M=32768, mean_std=2.0, host=True, chunk=1 << 24),
    # split-D check, fp32, device resident
    "splitd_f32": Workload("splitd_f32", 7, B=1, N=262144, D=1024, K=512, dtype="f32", iters=3, tol=0.0,
                           data="gmm", M=512, mean_std=2.0),
}


# --------------------------------------------------------------------------------------------
# dtype storage helpers (casts only)
# --------------------------------------------------------------------------------------------
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def cast_f32(v: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage dtype (round to nearest even)."""
    if dtype == "f32":
        return np.ascontiguousarray(v, dtype=np.float32)
    if dtype == "f16":
        return v.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    raise ValueError(dtype)


def storage_to_f32(s: np.ndarray, dtype: str) -> np.ndarray:
    """Storage dtype -> float32 (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(s)
    return np.asarray(s).astype(np.float32)


def storage_to_f64(s: np.ndarray, dtype: str) -> np.ndarray:
    return storage_to_f32(s, dtype).astype(np.float64)


def to_torch(s: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(s))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def from_torch(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# --------------------------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------------------------
def _weights(w: Workload) -> np.ndarray | None:
    if w.zipf_s <= 0.0:
        return None
    j = np.arange(1, w.M + 1, dtype=np.float64)
    p = j ** (-w.zipf_s)
    return p / p.sum()


def _draw_block(ss: np.random.SeedSequence, n: int, D: int, means: np.ndarray | None,
                p: np.ndarray | None, w: Workload, out: np.ndarray) -> None:
    rng = np.random.default_rng(ss)
    if means is not None:
        if p is None:
            lab = rng.integers(0, means.shape[0], size=n)
        else:
            lab = rng.choice(means.shape[0], size=n, p=p)
    v = rng.standard_normal((n, D), dtype=np.float32)
    if means is not None:
        v += means[lab]
    if w.offset_channels:
        v[:, : w.offset_channels] += np.float32(w.offset)
    out[...] = cast_f32(v, w.dtype)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def generate_points(w: Workload, out: np.ndarray | None = None, out_blocks=None) -> np.ndarray:
    """Points [B, N, D] in the storage dtype (uncentred).  `out` may be a preallocated
    (e.g. pinned-host) numpy view of that shape.  With `out_blocks` (B = 1: a list of [n_j, D]
    arrays holding consecutive rows, every one but the last a multiple of 2^20 rows) the same
    points are written into the blocks instead, and the list is returned."""
    ss = np.random.SeedSequence(BASE_SEED + w.seed_id)
    ss_means, ss_data, _ = ss.spawn(3)
    if out_blocks is not None:
        assert w.B == 1 and sum(bl.shape[0] for bl in out_blocks) == w.N
        assert all(bl.shape[0] % BLOCK_POINTS == 0 for bl in out_blocks[:-1])
        starts = np.cumsum([0] + [bl.shape[0] for bl in out_blocks])

        def dest(b, lo, hi):
            j = int(np.searchsorted(starts, lo, side="right")) - 1
            return out_blocks[j][lo - starts[j]:hi - starts[j]]
    else:
        if out is None:
            out = np.empty((w.B, w.N, w.D), dtype=NP_STORAGE[w.dtype])
        assert out.shape == (w.B, w.N, w.D)

        def dest(b, lo, hi):
            return out[b, lo:hi]
    p = _weights(w)
    jobs = []
    mean_children = ss_means.spawn(w.B)
    data_children = ss_data.spawn(w.B)
    nblk = -(-w.N // BLOCK_POINTS)
    for b in range(w.B):
        means = None
        if w.data == "gmm":
            rng = np.random.default_rng(mean_children[b])
            means = (np.float32(w.mean_std) * rng.standard_normal((w.M, w.D), dtype=np.float32))
        blocks = data_children[b].spawn(nblk)
        for j in range(nblk):
            lo, hi = j * BLOCK_POINTS, min(w.N, (j + 1) * BLOCK_POINTS)
            jobs.append((blocks[j], hi - lo, means, b, lo, hi))
    if len(jobs) == 1:
        s, n, means, b, lo, hi = jobs[0]
        _draw_block(s, n, w.D, means, p, w, dest(b, lo, hi))
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda j: _draw_block(j[0], j[1], w.D, j[2], p, w, dest(j[3], j[4], j[5])), jobs))
    return out if out_blocks is None else out_blocks


def center_points(w: Workload, x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Translation used by the attention-sink workload: mu = fp64 mean over points of the stored
    values; returns (dtype(fp32(x) - fp32(mu)), mu[B, D]).  k-means is translation invariant
    (README, "Centre your data"), so this is harness-side data preparation."""
    B, N, D = x.shape
    mu = np.zeros((B, D), dtype=np.float64)
    step = BLOCK_POINTS
    for b in range(B):
        acc = np.zeros(D, dtype=np.float64)
        for lo in range(0, N, step):
            acc += storage_to_f32(x[b, lo:lo + step], w.dtype).astype(np.float64).sum(axis=0)
        mu[b] = acc / N
    mu32 = mu.astype(np.float32)

    def job(args):
        b, lo = args
        blk = storage_to_f32(x[b, lo:lo + step], w.dtype) - mu32[b]
        x[b, lo:lo + step] = cast_f32(blk, w.dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, [(b, lo) for b in range(B) for lo in range(0, N, step)]))
    return x, mu


def init_indices(w: Workload) -> np.ndarray:
    """[B, K] distinct point indices per batch (first K entries of a seeded permutation)."""
    ss = np.random.SeedSequence(BASE_SEED + w.seed_id)
    _, _, ss_init = ss.spawn(3)
    kids = ss_init.spawn(w.B)
    out = np.empty((w.B, w.K), dtype=np.int64)
    for b in range(w.B):
        out[b] = np.random.default_rng(kids[b]).permutation(w.N)[: w.K]
    return out


def init_centroids(w: Workload, x: np.ndarray) -> np.ndarray:
    """[B, K, D] float32 copies of the chosen rows (exact upcast of the stored values)."""
    idx = init_indices(w)
    c = np.empty((w.B, w.K, w.D), dtype=np.float32)
    for b in range(w.B):
        c[b] = storage_to_f32(x[b, idx[b]], w.dtype)
    return c


def rows_of_blocks(blocks, idx: np.ndarray) -> np.ndarray:
    """Rows `idx` (global row numbers, any order) of the points split over `blocks`."""
    starts = np.cumsum([0] + [bl.shape[0] for bl in blocks])
    j = np.searchsorted(starts, idx, side="right") - 1
    out = np.empty((idx.size, blocks[0].shape[1]), dtype=blocks[0].dtype)
    for jj in np.unique(j):
        sel = j == jj
        out[sel] = blocks[jj][idx[sel] - starts[jj]]
    return out


def init_centroids_blocks(w: Workload, blocks) -> np.ndarray:
    """init_centroids for points split over blocks (B = 1)."""
    idx = init_indices(w)
    return storage_to_f32(rows_of_blocks(blocks, idx[0]), w.dtype)[None].astype(np.float32)


def make(w: Workload, out: np.ndarray | None = None):
    """Points (storage dtype, centred if the workload says so), init centroids f32 and the
    centring translation (None when not centred)."""
    x = generate_points(w, out)
    mu = None
    if w.center:
        x, mu = center_points(w, x)
    c0 = init_centroids(w, x)
    return x, c0, mu


def small(name: str, **kw) -> Workload:
    """A reduced copy of a named workload (same data recipe, smaller shape) for tests."""
    w = WORKLOADS[name]
    if "M" not in kw and w.data == "gmm" and "K" in kw:
        kw["M"] = max(1, min(w.M, kw["K"]))
    return w.scaled(**kw)


def nbytes(w: Workload) -> int:
    return w.B * w.N * w.D * ELEM_BYTES[w.dtype]


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [
    "Workload", "WORKLOADS", "make", "generate_points", "center_points", "init_indices", "init_centroids",
    "small", "cast_f32", "storage_to_f32", "storage_to_f64", "to_torch", "from_torch", "torch_dtype",
    "rows_of_blocks", "init_centroids_blocks",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "NP_STORAGE", "ELEM_BYTES", "nbytes", "ceil_div",
]
