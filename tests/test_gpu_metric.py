"""Parity of the dot-product and cosine k-means paths (HIP, through the C-ABI) against the fp64
similarity oracle on identical seeded inputs: unit rows, the arg-max assignment, one
teacher-forced iteration of each metric, free-running fits, and exactness properties."""
import sys

import numpy as np
import pytest

import oracle
from oracle import similarity as sim
from exact_lloyd_means_02_amd import workloads as W

from helpers import CENTROID_TOL, INERTIA_TOL, NEAR, U32, device, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    from exact_lloyd_means_02_amd import flashkm
    return flashkm


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.float32 else t.cpu().numpy().astype(np.float64)


def _ulps(a, b, dtype):
    """Distance in units in the last place of the storage dtype between two arrays of its values."""
    mant = {"f32": 23, "f16": 10, "bf16": 7}[dtype]
    m = np.maximum(np.abs(a), np.abs(b))
    e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    return np.abs(a - b) / np.exp2(e - mant)


# ---------------------------------------------------------------------------------------------
# unit rows
# ---------------------------------------------------------------------------------------------
NORM_CASES = [("bf16", 128), ("bf16", 100), ("f16", 64), ("f16", 24), ("f32", 16), ("f32", 1024), ("f32", 7)]


@pytest.mark.parametrize("dtype,D", NORM_CASES, ids=[f"{d}-D{n}" for d, n in NORM_CASES])
def test_normalize_rows(fk, dtype, D):
    _say(f"normalize rows {dtype} D={D}")
    r = np.random.default_rng(D)
    x64 = r.standard_normal((3001, D)) * r.uniform(0.01, 50.0, size=(3001, 1)) + 0.5
    x64[17] = 0.0                                             # a zero row stays zero
    xs = W.cast_f32(x64.astype(np.float32), dtype)
    xin = W.storage_to_f64(xs, dtype)
    xt = W.to_torch(xs, dtype).to(device())
    out = fk.kmeans_normalize_rows(xt)
    g = _f64(out)
    want = sim.round_to_dtype(sim.normalize_rows(xin), dtype)
    assert (g[17] == 0).all()
    u = _ulps(g, want, dtype)
    if dtype == "f32":
        # fp32 norm over D terms, one division: a few ulp per D
        assert u.max() <= D / 2 + 4, u.max()
    else:
        # the fp32 quotient is within a few fp32 ulps of the exact one, so the stored value is the
        # exact value rounded, or its neighbour when the exact value lies that close to a rounding
        # boundary
        assert u.max() <= 1.0
        assert (u > 0).mean() < 2e-3
    # in place
    x2 = xt.clone()
    fk.kmeans_normalize_rows(x2, out=x2)
    assert torch.equal(x2, out)


# ---------------------------------------------------------------------------------------------
# the arg-max assignment from prepared centroids with zero norm terms
# ---------------------------------------------------------------------------------------------
ASSIGN_CASES = [
    ("headline_bf16", dict(B=2, N=5000, K=1024)),
    ("headline_bf16", dict(B=1, N=3001, D=100, K=77)),
    ("batched_f16", dict(B=3, N=4097, K=200)),
    ("tiny_f32", dict()),
    ("splitd_f32", dict(N=2000, K=40)),
]


def _check_similarity_assign(x64, ct64, a_gpu, md_gpu=None):
    flips = 0
    D = x64.shape[2]
    for b in range(x64.shape[0]):
        a_or, s1, s2, scale = sim.similarity_assign(x64[b], ct64[b])
        ag = a_gpu[b].astype(np.int64)
        assert ag.min() >= 0 and ag.max() < ct64.shape[1]
        near = sim.similarity_near_mask(s1, s2, scale, NEAR)
        mism = ag != a_or
        bad = mism & ~near
        assert not bad.any(), "problem %d: %d picks differ outside the near-tie band" % (b, int(bad.sum()))
        sg = np.einsum("nd,nd->n", x64[b], ct64[b][ag])
        assert (sg >= s1 - NEAR * scale).all()
        flips += int(mism.sum())
        if md_gpu is not None:
            # min_dist = 0 - 2 x.c~_a in fp32: D products accumulated
            bound = (D + 8) * U32 * 2 * np.sqrt((x64[b] ** 2).sum(1) * (ct64[b][ag] ** 2).sum(1)) + 1e-30
            err = np.abs(md_gpu[b].astype(np.float64) + 2 * sg)
            assert (err <= bound).all(), "min_dist error %g" % err.max()
    return flips


@pytest.mark.parametrize("name,kw", ASSIGN_CASES, ids=[f"{n}-{kw}" for n, kw in ASSIGN_CASES])
def test_dot_assign(fk, name, kw):
    w = W.small(name, **kw)
    _say(f"dot assign {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    prep = fk.kmeans_prepare_centroids(ct, xt, metric="dot")
    zeros = torch.zeros((w.B, w.N), dtype=torch.float32, device=device())
    a, md = fk.kmeans_assign_prepared(xt, prep, x_norms=zeros, want_min_dist=True)
    torch.cuda.synchronize()
    ct64 = oracle.centroid_operand(c0.astype(np.float64), w.dtype)
    flips = _check_similarity_assign(x64, ct64, a.cpu().numpy(), md.cpu().numpy())
    _say(f"near-tie flips: {flips}")
    # the same prepared buffer with the Euclidean norm terms gives the Euclidean assignment
    prep2 = fk.kmeans_prepare_centroids(ct, xt, metric="l2", out=prep.buf)
    a2, _ = fk.kmeans_assign_prepared(xt, prep2)
    a3, _ = fk.kmeans_assign_prepared(xt, fk.kmeans_prepare_centroids(ct, xt))
    assert torch.equal(a2, a3)


# ---------------------------------------------------------------------------------------------
# one teacher-forced iteration of each metric
# ---------------------------------------------------------------------------------------------
STEP_CASES = [
    ("dot", "headline_bf16", dict(B=2, N=6000, K=300)),
    ("dot", "batched_f16", dict(B=2, N=3000, K=64)),
    ("dot", "tiny_f32", dict()),
    ("cosine", "headline_bf16", dict(B=2, N=6000, K=300)),
    ("cosine", "headline_bf16", dict(B=1, N=3000, D=240, K=48)),
    ("cosine", "batched_f16", dict(B=2, N=3000, K=64)),
    ("cosine", "tiny_f32", dict()),
    ("cosine", "splitd_f32", dict(N=2000, K=32)),
]


@pytest.mark.parametrize("metric,name,kw", STEP_CASES, ids=[f"{m}-{n}-{kw}" for m, n, kw in STEP_CASES])
def test_one_iteration(fk, metric, name, kw):
    w = W.small(name, **kw)
    _say(f"{metric} one iteration {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    c = ct.clone()
    a, obj, done = fk.kmeans_fit_metric(xt, c, metric, 1)
    assert done == 1
    if metric == "cosine":
        xa = _f64(fk.kmeans_normalize_rows(xt))               # the same kernel the fit runs
        c_start = _f64(fk.kmeans_normalize_rows(ct))
    else:
        xa = x64
        c_start = c0.astype(np.float64)
    ct64 = oracle.centroid_operand(c_start, w.dtype)
    ag = a.cpu().numpy().astype(np.int64)
    flips = _check_similarity_assign(xa, ct64, ag)
    _say(f"near-tie flips: {flips}")
    cg = c.cpu().numpy().astype(np.float64)
    tol = CENTROID_TOL[w.dtype]
    for b in range(w.B):
        if metric == "dot":
            c_or, counts = sim.mean_update(xa[b], ag[b], c_start[b])
        else:
            c_or, counts = sim.mean_direction(xa[b], ag[b], c_start[b])
        kept = counts == 0
        assert np.array_equal(cg[b][kept], c_start[b][kept].astype(np.float32).astype(np.float64))
        num = np.linalg.norm(cg[b] - c_or, axis=1)
        den = np.maximum(np.linalg.norm(c_or, axis=1), 1e-30)
        assert (num / den).max() <= tol, "centroid rel err %g" % (num / den).max()
        if metric == "cosine":
            nrm = np.linalg.norm(cg[b][~kept], axis=1)
            assert np.abs(nrm - 1).max() < 1e-5
        # the objective: the total similarity of the assignment the GPU made
        s = np.einsum("nd,nd->n", xa[b], ct64[b][ag[b]])
        assert abs(obj[0, b] - s.sum()) <= INERTIA_TOL * np.abs(s).sum()


# ---------------------------------------------------------------------------------------------
# free-running fits against the oracle loop
# ---------------------------------------------------------------------------------------------
FIT_CASES = [
    ("dot", "headline_bf16", dict(B=2, N=8192, K=256), 4),
    ("cosine", "headline_bf16", dict(B=2, N=8192, K=256), 6),
    ("cosine", "batched_f16", dict(B=2, N=5000, K=100), 4),
    ("cosine", "tiny_f32", dict(), 10),
    # rows of 1100 fp32 columns need two column blocks in the update, so cosine takes the
    # accumulating update and the mean-direction finalize instead of the in-place finish
    ("cosine", "splitd_f32", dict(N=3000, D=1100, K=40), 3),
]


@pytest.mark.parametrize("metric,name,kw,iters", FIT_CASES, ids=[f"{m}-{n}-{kw}" for m, n, kw, _ in FIT_CASES])
def test_fit_matches_oracle(fk, metric, name, kw, iters):
    w = W.small(name, **kw)
    _say(f"{metric} fit {w} iters={iters}")
    x, x64, c0, xt, ct = make_inputs(w)
    c = ct.clone()
    a, obj, done = fk.kmeans_fit_metric(xt, c, metric, iters)
    assert done == iters
    ref = sim.similarity_fit(x64, c0, metric, iters, dtype=w.dtype, mode="modelled")
    scale = np.abs(ref["objective"]).max(axis=0)
    rel = np.abs(obj - ref["objective"]) / scale
    _say(f"max objective rel diff {rel.max():.3g}")
    assert rel.max() <= INERTIA_TOL
    flips = (a.cpu().numpy() != ref["labels"]).mean()
    assert flips < 1e-3
    if metric == "cosine":
        # the objective of spherical k-means does not fall (up to the dtype rounding of x^ and c~)
        j = obj[:, 0]
        assert (np.diff(j) >= -1e-3 * np.abs(j[:-1])).all()


def test_l2_metric_is_kmeans_fit(fk):
    w = W.small("headline_bf16", B=2, N=4096, K=128)
    x, x64, c0, xt, ct = make_inputs(w)
    c1, c2 = ct.clone(), ct.clone()
    a1, j1, d1 = fk.kmeans_fit(xt, c1, 3)
    a2, j2, d2 = fk.kmeans_fit_metric(xt, c2, "l2", 3)
    assert d1 == d2 == 3
    assert torch.equal(a1, a2) and torch.equal(c1, c2)
    assert np.array_equal(j1, j2)


def test_cosine_exact_scale_invariance(fk):
    """Scaling rows by powers of two is exact in bf16 and leaves x^ bit-identical, so the whole
    cosine fit (labels and centroids) must be bit-identical."""
    w = W.small("headline_bf16", B=1, N=6000, K=64)
    x, x64, c0, xt, ct = make_inputs(w)
    sc = torch.tensor([2.0 ** float(k % 7 - 3) for k in range(w.N)], dtype=torch.float32, device=device())
    xs = (xt.float() * sc[None, :, None]).to(xt.dtype)
    assert torch.equal(fk.kmeans_normalize_rows(xs), fk.kmeans_normalize_rows(xt))
    c1, c2 = ct.clone(), (ct * 4.0).contiguous()
    a1, j1, _ = fk.kmeans_fit_metric(xt, c1, "cosine", 4)
    a2, j2, _ = fk.kmeans_fit_metric(xs, c2, "cosine", 4)
    assert torch.equal(a1, a2) and torch.equal(c1, c2)
    assert np.array_equal(j1, j2)


def test_cosine_zero_rows_and_repeat(fk):
    """A zero point scores 0 against every centroid (lowest index wins); two runs are identical."""
    w = W.small("headline_bf16", B=1, N=3000, K=40)
    x, x64, c0, xt, ct = make_inputs(w)
    xz = xt.clone()
    xz[0, :50] = 0
    runs = []
    for _ in range(2):
        c = ct.clone()
        a, j, _ = fk.kmeans_fit_metric(xz, c, "cosine", 3)
        runs.append((a.clone(), c.clone(), j.copy()))
    assert (runs[0][0][0, :50] == 0).all()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    assert np.array_equal(runs[0][2], runs[1][2])


@pytest.mark.parametrize("metric", ["cosine", "dot"])
def test_streamed_metric_matches_device(fk, metric):
    """Pinned host x (streamed in chunks, cosine: unit rows made per staged chunk) against the
    device-resident fit: the first assignment is identical (same points, same centroids); the
    centroids after it differ only by the fp32 order of the per-chunk sums."""
    w = W.small("headline_bf16", B=2, N=9000, K=48)
    _say(f"streamed {metric} {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    xh = xt.cpu().pin_memory()
    c_d, c_h = ct.clone(), ct.clone()
    a_d, o_d, _ = fk.kmeans_fit_metric(xt, c_d, metric, 1)
    a_h, o_h, _ = fk.kmeans_fit_metric(xh, c_h, metric, 1, chunk_points=4000)
    assert torch.equal(a_d, a_h)
    rel = (c_d - c_h).norm(dim=-1) / c_d.norm(dim=-1).clamp_min(1e-30)
    assert rel.max().item() < 1e-5
    assert np.abs(o_d - o_h).max() <= 1e-6 * np.abs(o_d).max()
    # a few more iterations: the objectives stay together
    c_d, c_h = ct.clone(), ct.clone()
    _, o_d, _ = fk.kmeans_fit_metric(xt, c_d, metric, 4)
    _, o_h, _ = fk.kmeans_fit_metric(xh, c_h, metric, 4, chunk_points=4000)
    assert (np.abs(o_d - o_h) / np.abs(o_d)).max() < 1e-4


def test_metric_degenerate_k(fk):
    """K = 1: every label 0; the centroid is the mean (dot) or the mean direction of the unit rows
    (cosine).  Cosine with K = N and the points as centroids: each point picks itself."""
    w = W.small("headline_bf16", B=2, N=2000, K=1)
    x, x64, c0, xt, ct = make_inputs(w)
    for metric in ("dot", "cosine"):
        c = ct.clone()
        a, obj, _ = fk.kmeans_fit_metric(xt, c, metric, 1)
        assert (a == 0).all()
        cg = c.cpu().numpy().astype(np.float64)
        xa = x64 if metric == "dot" else _f64(fk.kmeans_normalize_rows(xt))
        for b in range(w.B):
            want = xa[b].mean(axis=0) if metric == "dot" else xa[b].sum(axis=0) / np.linalg.norm(xa[b].sum(axis=0))
            assert np.linalg.norm(cg[b, 0] - want) / np.linalg.norm(want) < 1e-3
    w = W.small("headline_bf16", B=1, N=512, K=512)
    x, x64, c0, xt, ct = make_inputs(w)
    c = xt.float().contiguous().clone()                     # the points themselves as centroids
    a, _, _ = fk.kmeans_fit_metric(xt, c, "cosine", 1)
    assert torch.equal(a[0].cpu(), torch.arange(w.N, dtype=torch.int32))


def test_metric_tol_stop(fk):
    """The stopping rule is the same as Lloyd's: stop after iteration t when max_b shift_t < tol."""
    w = W.small("headline_bf16", B=2, N=4000, K=64)
    x, x64, c0, xt, ct = make_inputs(w)
    for metric in ("dot", "cosine"):
        c = ct.clone()
        _, obj, done = fk.kmeans_fit_metric(xt, c, metric, 5, tol=1e30)
        assert done == 1 and obj.shape == (1, w.B)
        # after the first iteration the centroids have moved off the sampled points: no stop
        c = ct.clone()
        _, obj, done = fk.kmeans_fit_metric(xt, c, metric, 2, tol=1e-30)
        assert done == 2
