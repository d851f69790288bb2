"""Pins of the dot-product / cosine k-means oracle against things other than itself (CPU only).

What fixes each expected value: brute-force enumeration with exact integer arithmetic, the
identity ||x - c||^2 = ||x||^2 + ||c||^2 - 2 x.c (which ties the similarity assignment to the
independently pinned Euclidean oracle when the norms are equal), Cauchy-Schwarz (the mean
direction maximises the cluster's total cosine), invariances, and hand-computed cases.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import similarity as sim

RNG = np.random.default_rng(4321)


# ---------------------------------------------------------------------------------------------
# assignment
# ---------------------------------------------------------------------------------------------
def _joint_best_dot(x_int, c_int):
    """Lexicographically first joint assignment maximising sum_i x_i.c_{a_i}, by enumeration."""
    n, k = len(x_int), len(c_int)
    best_j, best_a = None, None
    for a in itertools.product(range(k), repeat=n):
        j = sum(sum(xv * cv for xv, cv in zip(x_int[i], c_int[a[i]])) for i in range(n))
        if best_j is None or j > best_j:
            best_j, best_a = j, a
    return best_j, list(best_a)


@pytest.mark.parametrize("seed", range(12))
def test_dot_assign_matches_enumeration(seed):
    r = np.random.default_rng(seed)
    n, k, d = int(r.integers(1, 7)), int(r.integers(1, 4)), int(r.integers(1, 4))
    x = r.integers(-3, 4, size=(n, d))
    c = r.integers(-3, 4, size=(k, d))
    if seed % 3 == 0 and k > 1:
        c[k - 1] = c[0]                                       # duplicate centroid: exact tie
    best_j, best_a = _joint_best_dot(x.tolist(), c.tolist())
    a, s1, s2, scale = sim.similarity_assign(x.astype(float), c.astype(float))
    assert a.tolist() == best_a
    assert float(s1.sum()) == best_j
    for i in range(n):
        others = [sum(int(xv) * int(cv) for xv, cv in zip(x[i], c[j])) for j in range(k) if j != a[i]]
        assert s2[i] == (max(others) if others else -np.inf)
        cmax = max(np.sqrt(float(sum(int(v) ** 2 for v in cc))) for cc in c)
        assert scale[i] == pytest.approx(np.sqrt(float(sum(int(v) ** 2 for v in x[i]))) * cmax, rel=1e-15)


def test_dot_equals_euclid_for_equal_norm_centroids():
    # centroids that are signed permutations of one vector have exactly equal norms, so
    # argmax x.c = argmin ||x - c||^2 (the Euclidean oracle is pinned on its own)
    base = np.array([3.0, -1.0, 2.0, 0.5, -4.0])
    c = []
    for p in itertools.permutations(range(5)):
        for sgn in (1.0, -1.0):
            c.append(sgn * base[list(p)])
            if len(c) == 60:
                break
        if len(c) == 60:
            break
    c = np.array(c)
    x = RNG.standard_normal((2000, 5)) * 2
    a_dot, s1, s2, _ = sim.similarity_assign(x, c)
    a_l2, d1, d2 = oracle.assign(x, c)
    clear = (s1 - s2) > 1e-9
    assert clear.mean() > 0.95
    assert (a_dot[clear] == a_l2[clear]).all()


def test_cosine_equals_euclid_on_unit_rows():
    # for unit vectors x.c = 1 - ||x - c||^2 / 2
    x = sim.normalize_rows(RNG.standard_normal((3000, 16)))
    c = sim.normalize_rows(RNG.standard_normal((50, 16)))
    a_cos, s1, s2, _ = sim.similarity_assign(x, c)
    a_l2, d1, _ = oracle.assign(x, c)
    clear = (s1 - s2) > 1e-9
    assert clear.mean() > 0.99
    assert (a_cos[clear] == a_l2[clear]).all()
    np.testing.assert_allclose(s1[clear], 1.0 - d1[clear] / 2.0, atol=1e-12)


def test_similarity_near_mask():
    s1 = np.array([1.0, 1.0, -0.5, 0.0])
    s2 = np.array([0.9995, 0.99, -0.5, -1e-4])
    scale = np.array([1.0, 1.0, 2.0, 0.2])
    assert sim.similarity_near_mask(s1, s2, scale).tolist() == [True, False, True, True]
    # a gap exactly at the band edge is not near (strict '<'); 1e-3 * 1000 is exactly 1.0
    assert sim.similarity_near_mask(np.array([3.0]), np.array([2.0]), np.array([1000.0])).tolist() == [False]


def test_assign_k1_and_chunking():
    x = RNG.standard_normal((20000, 8))
    c = RNG.standard_normal((1, 8))
    a, s1, s2, _ = sim.similarity_assign(x, c, chunk=777)
    assert (a == 0).all() and np.isinf(s2).all() and (s2 < 0).all()
    np.testing.assert_allclose(s1, x @ c[0], rtol=1e-14)
    c5 = RNG.standard_normal((5, 8))
    full = sim.similarity_assign(x, c5, chunk=1 << 20)
    small = sim.similarity_assign(x, c5, chunk=333)
    for u, v in zip(full, small):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------------------------------------
# normalisation
# ---------------------------------------------------------------------------------------------
def test_normalize_rows():
    x = RNG.standard_normal((500, 9)) * RNG.uniform(0.01, 100, size=(500, 1))
    x[7] = 0.0
    xh = sim.normalize_rows(x)
    n = np.sqrt((xh * xh).sum(axis=1))
    assert (xh[7] == 0).all()
    keep = np.ones(500, bool)
    keep[7] = False
    np.testing.assert_allclose(n[keep], 1.0, atol=1e-15)
    # the same direction: x = ||x|| * x^
    np.testing.assert_allclose(xh[keep] * np.sqrt((x[keep] ** 2).sum(axis=1))[:, None], x[keep], rtol=1e-13)
    assert np.allclose(sim.normalize_rows(3.5 * x), xh, rtol=1e-14, atol=0)
    assert sim.normalize_rows(np.array([[3.0, 4.0]])).tolist() == [[0.6, 0.8]]


def test_round_to_dtype_matches_torch_casts():
    import torch
    v = RNG.standard_normal(4000) * 0.3
    for name, td in (("bf16", torch.bfloat16), ("f16", torch.float16), ("f32", torch.float32)):
        want = torch.from_numpy(v.astype(np.float32)).to(td).to(torch.float64).numpy()
        assert np.array_equal(sim.round_to_dtype(v, name), want)


# ---------------------------------------------------------------------------------------------
# update
# ---------------------------------------------------------------------------------------------
def test_mean_direction_maximises_total_cosine():
    xh = sim.normalize_rows(RNG.standard_normal((600, 6)) + np.array([2.0, 0, 0, 0, 0, 0]))
    K = 5
    a = RNG.integers(0, K - 1, size=600)                      # cluster K-1 stays empty
    c_old = sim.normalize_rows(RNG.standard_normal((K, 6)))
    c_new, counts = sim.mean_direction(xh, a, c_old)
    assert counts[K - 1] == 0 and (c_new[K - 1] == c_old[K - 1]).all()
    for k in range(K - 1):
        m = xh[a == k]
        s = m.sum(axis=0)
        # Cauchy-Schwarz: max over unit c of sum_i x^_i.c is ||S||, reached at S / ||S||
        assert (m @ c_new[k]).sum() == pytest.approx(np.sqrt((s * s).sum()), rel=1e-13)
        assert abs(np.sqrt((c_new[k] ** 2).sum()) - 1.0) < 1e-15
        for _ in range(30):
            u = c_new[k] + RNG.standard_normal(6) * 0.05
            u /= np.sqrt((u * u).sum())
            assert (m @ u).sum() <= (m @ c_new[k]).sum() + 1e-12


def test_mean_direction_zero_sum_keeps():
    xh = np.array([[1.0, 0.0], [-1.0, 0.0], [0.0, 1.0]])
    a = np.array([0, 0, 1])
    c_old = np.array([[0.6, 0.8], [1.0, 0.0]])
    c_new, counts = sim.mean_direction(xh, a, c_old)
    assert counts.tolist() == [2, 1]
    assert c_new[0].tolist() == [0.6, 0.8]                   # members cancel: kept
    assert c_new[1].tolist() == [0.0, 1.0]


def test_mean_update_brute_force():
    x = RNG.standard_normal((50, 3))
    a = RNG.integers(0, 4, size=50)
    a[a == 2] = 1                                             # cluster 2 empty
    c_old = RNG.standard_normal((4, 3))
    c_new, counts = sim.mean_update(x, a, c_old)
    for k in range(4):
        rows = [x[i] for i in range(50) if a[i] == k]
        if rows:
            want = [sum(r[d] for r in rows) / len(rows) for d in range(3)]
            np.testing.assert_allclose(c_new[k], want, rtol=1e-13)
        else:
            assert (c_new[k] == c_old[k]).all()


def test_cosine_two_directions_by_hand():
    x = np.array([[[2.0, 0.0], [5.0, 0.0], [0.0, 3.0], [0.0, 0.5]]])
    c0 = np.array([[[1.0, 0.2], [0.1, 1.0]]])
    f = sim.similarity_fit(x, c0, "cosine", iters=2, mode="pure")
    assert f["labels"].tolist() == [[0, 0, 1, 1]]
    assert f["centroids"].tolist() == [[[1.0, 0.0], [0.0, 1.0]]]
    assert f["objective"][-1].tolist() == [4.0]


def test_dot_two_axes_by_hand():
    """Dot product: (2,0), (4,0) pick c0=(1,0); (0,3), (0,5) pick c1=(0,1).  Means (3,0) and (0,4);
    shift = 2^2 + 3^2 = 13; objective 2 + 4 + 3 + 5 = 14."""
    x = np.array([[[2.0, 0.0], [4.0, 0.0], [0.0, 3.0], [0.0, 5.0]]])
    c0 = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    it = sim.similarity_iteration(x, c0, "dot", mode="pure")
    assert it["a"].tolist() == [[0, 0, 1, 1]]
    assert it["c_new"].tolist() == [[[3.0, 0.0], [0.0, 4.0]]]
    assert it["shift"].tolist() == [13.0]
    assert it["objective"].tolist() == [14.0]
    f = sim.similarity_fit(x, c0, "dot", iters=4, tol=13.5, mode="pure")
    assert f["iters_done"] == 1                    # 13 < 13.5
    f = sim.similarity_fit(x, c0, "dot", iters=4, tol=13.0, mode="pure")
    assert f["iters_done"] == 2 and f["shift"].tolist() == [13.0, 0.0]


def test_dot_k1_one_step():
    x = RNG.standard_normal((1, 300, 4))
    c0 = RNG.standard_normal((1, 1, 4))
    it = sim.similarity_iteration(x, c0, "dot", mode="pure")
    assert (it["a"] == 0).all() and it["counts"].tolist() == [[300]]
    np.testing.assert_allclose(it["c_new"][0, 0], x[0].mean(axis=0), rtol=1e-13)
    np.testing.assert_allclose(it["objective"], [(x[0] @ c0[0, 0]).sum()], rtol=1e-13)


# ---------------------------------------------------------------------------------------------
# the whole iteration: monotone objective and invariances
# ---------------------------------------------------------------------------------------------
def _blobs(n, d, m, seed):
    r = np.random.default_rng(seed)
    mu = r.standard_normal((m, d)) * 3
    lab = r.integers(0, m, size=n)
    return mu[lab] + r.standard_normal((n, d))


@pytest.mark.parametrize("seed", range(3))
def test_spherical_objective_non_decreasing_pure(seed):
    x = _blobs(1500, 8, 10, seed)[None]
    c0 = x[:, np.random.default_rng(seed).permutation(1500)[:10]]
    f = sim.similarity_fit(x, c0, "cosine", iters=8, mode="pure")
    j = f["objective"][:, 0]
    assert (np.diff(j) >= -1e-12 * np.abs(j[:-1])).all()


def test_cosine_scale_invariance():
    x = _blobs(800, 5, 6, 11)[None]
    c0 = x[:, :6].copy()
    s = np.random.default_rng(3).uniform(0.1, 10.0, size=(1, 800, 1))
    f1 = sim.similarity_fit(x, c0, "cosine", iters=4, mode="pure")
    f2 = sim.similarity_fit(x * s, c0 * 2.5, "cosine", iters=4, mode="pure")
    assert np.array_equal(f1["labels"], f2["labels"])
    np.testing.assert_allclose(f1["centroids"], f2["centroids"], atol=1e-13)


def test_permutation_invariance_dot():
    x = _blobs(700, 4, 5, 5)[None]
    c0 = x[:, :5].copy()
    p = np.random.default_rng(9).permutation(700)
    f1 = sim.similarity_fit(x, c0, "dot", iters=3, mode="pure")
    f2 = sim.similarity_fit(x[:, p], c0, "dot", iters=3, mode="pure")
    assert np.array_equal(f1["labels"][:, p], f2["labels"])
    np.testing.assert_allclose(f1["centroids"], f2["centroids"], atol=1e-12)


def test_modelled_cosine_rounds_points_and_centroids():
    x = _blobs(300, 6, 4, 2)[None]
    c0 = x[:, :4].copy()
    f = sim.similarity_fit(x, c0, "cosine", iters=1, dtype="bf16")
    xu = f["x_used"]
    assert np.array_equal(xu, sim.round_to_dtype(sim.normalize_rows(x), "bf16"))
    # stored bf16 values carry at most 8 significant bits
    m, _ = np.frexp(xu[xu != 0])
    assert np.all((m * 256) == np.round(m * 256))
