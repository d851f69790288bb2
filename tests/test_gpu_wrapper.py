"""The faiss / scikit-learn style FlashKMeans object and the README-style batch functions: they
marshal arguments only, so their results must equal the C-ABI calls they wrap, bit for bit, and
predict must agree with the oracle's assignment from the fitted centroids."""
import sys

import numpy as np
import pytest

import oracle
from oracle import similarity as sim
from exact_lloyd_means_02_amd import workloads as W

from helpers import NEAR, device, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    from exact_lloyd_means_02_amd import flashkm
    return flashkm


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_fit_predict_equals_kmeans_fit(fk):
    w = W.small("headline_bf16", B=3, N=5000, K=64)
    _say(f"wrapper fit {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    km = fk.FlashKMeans(d=w.D, k=w.K, niter=5, dtype=torch.bfloat16, seed=3)
    labels = km.fit_predict(xt)
    init = fk._seeded_init(xt, w.K, 3)
    c = init.clone()
    a, J, done = fk.kmeans_fit(xt, c, 5)
    assert torch.equal(labels, a) and torch.equal(km.centroids, c)
    assert np.array_equal(km.obj, J) and km.iters_done == done == 5
    assert km.cluster_centers_.shape == (3, w.K, w.D)
    assert np.array_equal(km.inertia_, J[-1])
    # predict: FlashAssign from the fitted centroids, checked against the oracle
    p = km.predict(xt).cpu().numpy()
    ct64 = oracle.centroid_operand(km.centroids.cpu().numpy().astype(np.float64), "bf16")
    for b in range(w.B):
        a_or, d1, d2 = oracle.assign(x64[b], ct64[b])
        bad = (p[b] != a_or) & ~oracle.near_mask(d1, d2, NEAR)
        assert not bad.any()


def test_two_d_input_and_host_tensors(fk):
    w = W.small("batched_f16", B=1, N=4000, K=50)
    _say(f"wrapper 2-D {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    x2 = xt[0]
    km = fk.FlashKMeans(d=w.D, k=w.K, niter=4, dtype=torch.float16)
    lab = km.fit_predict(x2, init_centroids=ct[0])
    assert lab.shape == (w.N,) and km.cluster_centers_.shape == (w.K, w.D)
    # pageable host input: copied to the GPU, same result
    km2 = fk.FlashKMeans(d=w.D, k=w.K, niter=4, dtype=torch.float16)
    lab2 = km2.fit_predict(x2.cpu(), init_centroids=ct[0])
    assert torch.equal(lab, lab2) and torch.equal(km.centroids, km2.centroids)
    # fp32 input with a bf16 compute dtype: the points are cast first
    km3 = fk.FlashKMeans(d=w.D, k=w.K, niter=2, dtype=torch.bfloat16)
    km3.fit(x2.float(), init_centroids=ct[0])
    km4 = fk.FlashKMeans(d=w.D, k=w.K, niter=2, dtype=torch.bfloat16)
    km4.fit(x2.float().to(torch.bfloat16), init_centroids=ct[0])
    assert torch.equal(km3.centroids, km4.centroids)


def test_pinned_host_input_uses_streamed_path(fk):
    w = W.small("headline_bf16", B=1, N=9000, K=40)
    _say(f"wrapper pinned {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    xh = xt.cpu().pin_memory()
    km = fk.FlashKMeans(d=w.D, k=w.K, niter=3, dtype=torch.bfloat16, chunk_points=4096)
    lab_h = km.fit_predict(xh, init_centroids=ct)
    km_d = fk.FlashKMeans(d=w.D, k=w.K, niter=3, dtype=torch.bfloat16)
    lab_d = km_d.fit_predict(xt, init_centroids=ct)
    # same labels; centroids within fp32 summation-order differences
    assert (lab_h != lab_d).float().mean().item() < 1e-3
    rel = (km.centroids - km_d.centroids).norm(dim=-1) / km_d.centroids.norm(dim=-1).clamp_min(1e-30)
    assert rel.max().item() < 1e-5


def test_host_streaming_pageable_equals_pinned(fk):
    """host_streaming=True fits pageable host points in place through the staged path: the same chunk
    sequence as pinned host input, so the same labels and centroids, bit for bit."""
    w = W.small("headline_bf16", B=2, N=9000, K=40)
    _say(f"wrapper host streaming {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    xp = xt.cpu()
    assert not xp.is_pinned()
    km_s = fk.FlashKMeans(d=w.D, k=w.K, niter=3, dtype=torch.bfloat16, chunk_points=4096, host_streaming=True)
    lab_s = km_s.fit_predict(xp, init_centroids=ct)
    km_p = fk.FlashKMeans(d=w.D, k=w.K, niter=3, dtype=torch.bfloat16, chunk_points=4096)
    lab_p = km_p.fit_predict(xp.pin_memory(), init_centroids=ct)
    assert torch.equal(lab_s.cpu(), lab_p.cpu())
    assert torch.equal(km_s.centroids.cpu(), km_p.centroids.cpu())
    assert np.array_equal(km_s.obj, km_p.obj)


@pytest.mark.parametrize("metric", ["cosine", "dot"])
def test_metric_wrapper(fk, metric):
    w = W.small("headline_bf16", B=2, N=4000, K=32)
    _say(f"wrapper {metric} {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    km = fk.FlashKMeans(d=w.D, k=w.K, niter=3, dtype=torch.bfloat16, metric=metric)
    lab = km.fit_predict(xt, init_centroids=ct)
    c = ct.clone()
    a, obj, _ = fk.kmeans_fit_metric(xt, c, metric, 3)
    assert torch.equal(lab, a) and torch.equal(km.centroids, c) and np.array_equal(km.obj, obj)
    ids, cc, o2 = (fk.batch_kmeans_cosine if metric == "cosine" else fk.batch_kmeans_dot)(
        xt, w.K, 3, init_centroids=ct)
    assert torch.equal(ids, a) and torch.equal(cc, c)
    # predict against the oracle's arg-max from the fitted centroids
    xa = xt if metric == "dot" else fk.kmeans_normalize_rows(xt)
    xa64 = xa.float().cpu().numpy().astype(np.float64)
    ct64 = oracle.centroid_operand(km.centroids.cpu().numpy().astype(np.float64), "bf16")
    p = km.predict(xt).cpu().numpy()
    for b in range(w.B):
        a_or, s1, s2, scale = sim.similarity_assign(xa64[b], ct64[b])
        bad = (p[b] != a_or) & ~sim.similarity_near_mask(s1, s2, scale, NEAR)
        assert not bad.any()


def test_batch_kmeans_euclid_matches_fit(fk):
    w = W.small("batched_f16", B=2, N=3000, K=40)
    x, x64, c0, xt, ct = make_inputs(w)
    ids, c, J = fk.batch_kmeans_euclid(xt, w.K, max_iters=3, init_centroids=ct)
    c2 = ct.clone()
    a, J2, _ = fk.kmeans_fit(xt, c2, 3)
    assert torch.equal(ids, a) and torch.equal(c, c2) and np.array_equal(J, J2)


def test_batch_kmeans_euclid_host_inputs(fk):
    """Host x: pinned (streamed fit) and pageable (staged streamed fit) give the same result, bit for
    bit (the same chunks), with the centroids returned on the GPU."""
    w = W.small("batched_f16", B=2, N=3000, K=40)
    x, x64, c0, xt, ct = make_inputs(w)
    xp = xt.cpu()
    ids_p, c_p, J_p = fk.batch_kmeans_euclid(xp.pin_memory(), w.K, max_iters=3, init_centroids=ct.cpu())
    ids_s, c_s, J_s = fk.batch_kmeans_euclid(xp, w.K, max_iters=3, init_centroids=ct.cpu())
    assert c_p.is_cuda and c_s.is_cuda
    assert torch.equal(ids_p, ids_s) and torch.equal(c_p, c_s) and np.array_equal(J_p, J_s)
    ref = oracle.lloyd_fit(x64, c0, 3, 0.0, dtype=w.dtype, mode="modelled")
    assert (np.abs(J_s - ref["inertia"]) / ref["inertia"]).max() <= 1e-4
    with pytest.raises(ValueError, match="Euclidean metric only"):
        fk.batch_kmeans_cosine(xp, w.K, max_iters=1, init_centroids=ct.cpu())
