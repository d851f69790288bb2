"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: the pages' worked example, brute-force
enumeration with exact integer arithmetic, closed forms, Lloyd's invariants, or an
independent library (scipy / scikit-learn / torch casts).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------------------------------------
# arg-sort: the pages' worked example and the stability property
# ---------------------------------------------------------------------------------------------
def test_argsort_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "argsort_worked_example.json")))
    sids, sidx, counts = oracle.argsort_ids(np.array(g["assign"]), g["K"])
    assert sids.tolist() == g["sorted_ids"]
    assert sidx.tolist() == g["sorted_idx"]
    assert counts.tolist() == g["counts"]


@pytest.mark.parametrize("n,K", [(1, 1), (257, 3), (5000, 17), (20000, 1000)])
def test_argsort_is_stable_permutation(n, K):
    a = RNG.integers(0, K, size=n)
    sids, sidx, counts = oracle.argsort_ids(a, K)
    assert sorted(sidx.tolist()) == list(range(n))          # a permutation
    assert (sids == a[sidx]).all()
    assert (np.diff(sids) >= 0).all()                        # ascending ids
    same = np.diff(sids) == 0
    assert (np.diff(sidx)[same] > 0).all()                   # equal ids keep index order
    for k in range(K):                                       # counts by direct counting
        assert counts[k] == sum(1 for v in a.tolist() if v == k)


# ---------------------------------------------------------------------------------------------
# assignment: exact enumeration with integer coordinates (so ties are exact)
# ---------------------------------------------------------------------------------------------
def _joint_best(x_int, c_int):
    """Lexicographically first joint assignment minimising the objective, by enumeration."""
    n, k = len(x_int), len(c_int)
    best_j, best_a = None, None
    for a in itertools.product(range(k), repeat=n):
        j = 0
        for i in range(n):
            j += sum((xv - cv) ** 2 for xv, cv in zip(x_int[i], c_int[a[i]]))
        if best_j is None or j < best_j:
            best_j, best_a = j, a
    return best_j, list(best_a)


@pytest.mark.parametrize("seed", range(12))
def test_assign_matches_enumeration(seed):
    r = np.random.default_rng(seed)
    n, k, d = int(r.integers(1, 7)), int(r.integers(1, 4)), int(r.integers(1, 4))
    x = r.integers(-3, 4, size=(n, d))
    c = r.integers(-3, 4, size=(k, d))
    if seed % 3 == 0 and k > 1:
        c[k - 1] = c[0]                                       # duplicate centroid: exact tie
    best_j, best_a = _joint_best(x.tolist(), c.tolist())
    a, d1, d2 = oracle.assign(x.astype(float), c.astype(float))
    assert a.tolist() == best_a
    assert float(d1.sum()) == best_j
    assert oracle.inertia(x.astype(float), c.astype(float), a) == best_j
    if k == 1:
        assert np.isinf(d2).all()
    else:
        for i in range(n):                                    # d2 = best over the other centroids
            others = [sum((xv - cv) ** 2 for xv, cv in zip(x[i], c[j])) for j in range(k) if j != a[i]]
            assert d2[i] == min(others)


def test_assign_matches_scipy_vq():
    from scipy.cluster.vq import vq
    x = RNG.standard_normal((3000, 24))
    c = RNG.standard_normal((37, 24))
    a, d1, _ = oracle.assign(x, c)
    code, dist = vq(x, c)
    assert (a == code).all()
    np.testing.assert_allclose(d1, dist ** 2, rtol=1e-12)


def test_row_norms_and_dist_closed_form():
    x = np.array([[3.0, 4.0], [1.0, -2.0], [0.0, 0.0]])
    assert oracle.row_norms(x).tolist() == [25.0, 5.0, 0.0]
    c = np.array([[0.0, 0.0], [3.0, 0.0]])
    assert oracle.dist_to(x, c, np.array([1, 0, 1])).tolist() == [16.0, 5.0, 9.0]


def test_near_mask():
    d1 = np.array([100.0, 100.0, 100.0, 0.0])
    d2 = np.array([100.05, 100.2, 100.0, 1.0])
    assert oracle.near_mask(d1, d2).tolist() == [True, False, True, False]


# ---------------------------------------------------------------------------------------------
# update: closed forms and the minimiser property
# ---------------------------------------------------------------------------------------------
def test_update_is_the_minimiser():
    x = RNG.standard_normal((400, 7)) * 3 + 1
    K = 9
    a = RNG.integers(0, K - 1, size=400)                      # cluster K-1 stays empty
    c_old = RNG.standard_normal((K, 7))
    c_new, counts = oracle.update(x, a, c_old)
    assert counts[K - 1] == 0
    assert (c_new[K - 1] == c_old[K - 1]).all()               # empty cluster keeps its centroid
    for k in range(K - 1):
        g = (x[a == k] - c_new[k]).sum(axis=0)                # gradient of the cluster SSE
        assert np.abs(g).max() < 1e-10 * max(1.0, np.abs(x[a == k]).sum())
        sse = ((x[a == k] - c_new[k]) ** 2).sum()
        for _ in range(20):
            p = c_new[k] + RNG.standard_normal(7) * 1e-3
            assert ((x[a == k] - p) ** 2).sum() >= sse


def test_update_matches_sklearn_one_step():
    from sklearn.cluster import KMeans
    rs = np.random.default_rng(7)
    centers = rs.standard_normal((6, 5)) * 6
    x = np.concatenate([centers[j] + rs.standard_normal((200, 5)) for j in range(6)])
    c0 = x[rs.permutation(len(x))[:6]].copy()
    a, _, _ = oracle.assign(x, c0)
    assert np.bincount(a, minlength=6).min() > 0              # sklearn relocates empty clusters
    c1, _ = oracle.update(x, a, c0)
    km = KMeans(n_clusters=6, init=c0, n_init=1, max_iter=1, tol=0.0, algorithm="lloyd").fit(x)
    np.testing.assert_allclose(c1, km.cluster_centers_, rtol=1e-10, atol=1e-10)


def test_special_case_k1():
    x = RNG.standard_normal((1, 333, 4)) + 5
    c0 = x[:, :1].copy()
    out = oracle.lloyd_fit(x, c0, iters=2, mode="pure")
    assert (out["labels"] == 0).all()
    np.testing.assert_allclose(out["centroids"][0, 0], x[0].mean(axis=0), rtol=1e-13)


def test_special_case_k_equals_n():
    x = RNG.standard_normal((2, 50, 3))
    out = oracle.lloyd_fit(x, x.copy(), iters=1, mode="pure")
    assert (out["labels"] == np.arange(50)).all()
    assert (out["inertia"] == 0).all()
    assert (out["centroids"] == x).all()


def test_two_blobs_one_step():
    left = np.array([[-10.0], [-11.0], [-12.0]])
    right = np.array([[10.0], [13.0]])
    x = np.concatenate([left, right])[None]
    c0 = np.array([[[-10.0], [10.0]]])
    it = oracle.lloyd_iteration(x, c0, mode="pure")
    assert it["a"][0].tolist() == [0, 0, 0, 1, 1]
    assert it["c_new"][0, :, 0].tolist() == [-11.0, 11.5]
    assert it["counts"][0].tolist() == [3, 2]
    assert it["inertia"][0] == 0 + 1 + 4 + 0 + 9
    # the centroids moved by -1 and +1.5: shift = 1^2 + 1.5^2
    assert it["shift"].tolist() == [3.25]
    assert oracle.shift(it["c_new"], c0).tolist() == [3.25]


# ---------------------------------------------------------------------------------------------
# the shift and the stopping rule (tol semantics: a reading, so the pins below fix the reading's
# arithmetic by hand-computed values; that the pages mean this rule stays unpinned)
# ---------------------------------------------------------------------------------------------
def test_shift_hand_values():
    """sum over clusters of the squared Euclidean move, per problem: (3,4) and (1,0) -> 25 + 1.
    Square roots (sqrt 26), norms (5 + 1), a mean (13) or a max (25) over clusters all differ."""
    c_old = np.array([[[0.0, 0.0], [2.0, 5.0]], [[1.0, 1.0], [0.0, 0.0]]])
    c_new = np.array([[[3.0, 4.0], [3.0, 5.0]], [[1.0, 1.0], [0.0, -2.0]]])
    assert oracle.shift(c_new, c_old).tolist() == [26.0, 4.0]
    assert oracle.shift(c_new[1], c_old[1]) == 4.0          # one problem -> a scalar
    assert oracle.shift(c_old, c_old).tolist() == [0.0, 0.0]


def _two_problem_blobs():
    """Two 1-D problems of five points, K=2.  Problem 0: blobs at means -2 and 6, seeds -3 and 5
    (each seed moves by 1: shift 2.0).  Problem 1: the two-blob example above (shift 3.25).  After
    the first step both problems sit at their blob means: the second step's shift is 0."""
    x = np.array([[[-1.0], [-2.0], [-3.0], [5.0], [7.0]],
                  [[-10.0], [-11.0], [-12.0], [10.0], [13.0]]])
    c0 = np.array([[[-3.0], [5.0]], [[-10.0], [10.0]]])
    return x, c0


def test_shift_per_problem_and_stop_on_max():
    x, c0 = _two_problem_blobs()
    it = oracle.lloyd_iteration(x, c0, mode="pure")
    assert it["shift"].tolist() == [2.0, 3.25]
    assert it["c_new"][:, :, 0].tolist() == [[-2.0, 6.0], [-11.0, 11.5]]
    # the run stops after the first iteration whose max over problems is below tol (strict):
    # tol=4: 3.25 < 4 -> stop after one; tol=3 and tol=3.25: go on, then 0 < tol -> stop after two.
    # A sum over problems (5.25 >= 4), a mean or min over problems (2.625, 2.0 < 3), square roots
    # (1.80 < 3), means or maxima over clusters (1.625, 2.25 < 3) or '<=' (3.25 <= 3.25) each
    # change one of these counts.
    f4 = oracle.lloyd_fit(x, c0, iters=5, tol=4.0, mode="pure")
    assert f4["iters_done"] == 1 and f4["shift"].tolist() == [3.25]
    for tol in (3.0, 3.25):
        f = oracle.lloyd_fit(x, c0, iters=5, tol=tol, mode="pure")
        assert f["iters_done"] == 2 and f["shift"].tolist() == [3.25, 0.0], tol
    assert oracle.lloyd_fit(x, c0, iters=5, tol=0.0, mode="pure")["iters_done"] == 5


# ---------------------------------------------------------------------------------------------
# Lloyd invariants
# ---------------------------------------------------------------------------------------------
def _gmm(B, N, D, M, seed):
    r = np.random.default_rng(seed)
    mu = r.standard_normal((B, M, D)) * 3
    lab = r.integers(0, M, size=(B, N))
    return np.take_along_axis(mu, lab[..., None], axis=1) + r.standard_normal((B, N, D))


def test_inertia_non_increasing_pure():
    x = _gmm(3, 1500, 6, 12, 11)
    c0 = x[:, :12].copy()
    out = oracle.lloyd_fit(x, c0, iters=8, mode="pure")
    J = out["inertia"]
    assert (J[1:] <= J[:-1] * (1 + 1e-12)).all()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_inertia_bound_modelled(dtype):
    """With rounded operands the rise of J is bounded by sum_k n_k ||c~_k - mean_k||^2."""
    x = _gmm(2, 1200, 8, 10, 5)
    c = x[:, :10].copy()
    prev = oracle.lloyd_iteration(x, c, dtype=dtype)
    for _ in range(5):
        exact = np.stack([oracle.update(x[b], prev["a"][b], c[b])[0] for b in range(2)])
        c = prev["c_new"]
        nxt = oracle.lloyd_iteration(x, c, dtype=dtype)
        bound = np.array([(prev["counts"][b][:, None] * (nxt["c_operand"][b] - exact[b]) ** 2).sum()
                          for b in range(2)])
        assert (nxt["inertia"] <= prev["inertia"] + bound + 1e-9 * prev["inertia"]).all()
        prev = nxt


def test_translation_invariance():
    """README, "Centre your data": k-means is translation invariant."""
    x = _gmm(2, 800, 5, 7, 3)
    c0 = x[:, :7].copy()
    t = np.array([64.0, -3.0, 0.5, 0.0, 64.0])
    a = oracle.lloyd_fit(x, c0, iters=5, mode="pure")
    b = oracle.lloyd_fit(x + t, c0 + t, iters=5, mode="pure")
    assert (a["labels"] == b["labels"]).all()
    np.testing.assert_allclose(b["centroids"] - t, a["centroids"], atol=1e-9)


def test_permutation_invariance():
    x = _gmm(1, 900, 4, 5, 9)
    c0 = x[:, :5].copy()
    p = np.random.default_rng(2).permutation(900)
    a = oracle.lloyd_fit(x, c0, iters=4, mode="pure")
    b = oracle.lloyd_fit(x[:, p], c0, iters=4, mode="pure")
    assert (b["labels"][0] == a["labels"][0][p]).all()
    np.testing.assert_allclose(b["centroids"], a["centroids"], rtol=1e-12, atol=1e-12)


def test_tol_rule():
    x = _gmm(2, 500, 3, 4, 8)
    c0 = x[:, :4].copy()
    assert oracle.lloyd_fit(x, c0, iters=6, tol=1e30, mode="pure")["iters_done"] == 1
    assert oracle.lloyd_fit(x, c0, iters=6, tol=0.0, mode="pure")["iters_done"] == 6


# ---------------------------------------------------------------------------------------------
# modelled centroid operand: rounding to the input dtype
# ---------------------------------------------------------------------------------------------
def test_bf16_operand_rounding_values():
    # bfloat16 has 8 significant bits: spacing 2**-7 on [1, 2)
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 3 * 2 ** -8), 2 ** -130])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -(1 + 2 ** -6), 2 ** -130])
    got = oracle.centroid_operand(vals, "bf16")
    assert got.tolist() == want.tolist()


def test_bf16_operand_rounding_matches_torch():
    import torch
    v = (RNG.standard_normal(100000) * np.exp(RNG.uniform(-20, 20, 100000))).astype(np.float32)
    ours = oracle.centroid_operand(v.astype(np.float64), "bf16")
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert (ours == ref).all()


def test_f16_and_f32_operand_rounding():
    vals = np.array([1 + 2 ** -11, 2049.0, 1 + 2 ** -24 + 2 ** -40])
    assert oracle.centroid_operand(vals, "f16").tolist() == [1.0, 2048.0, 1.0]
    assert oracle.centroid_operand(vals, "f32").tolist() == [float(np.float32(1 + 2 ** -11)), 2049.0,
                                                            1 + 2 ** -23]
    assert (oracle.centroid_operand(vals, "bf16", mode="pure") == vals).all()


def test_segment_sums_brute_force_and_blocks():
    """s_k and n_k by explicit loops on a tiny input; sums over disjoint blocks of points add up
    to the sums over all points (the streamed and full-size checks rely on this)."""
    rng = np.random.default_rng(11)
    x = rng.normal(size=(37, 5))
    a = rng.integers(0, 6, size=37)
    a[a == 4] = 5                                     # cluster 4 empty
    sums, counts = oracle.segment_sums(x, a, 6)
    for k in range(6):
        want = np.zeros(5)
        n = 0
        for i in range(37):
            if a[i] == k:
                want += x[i]
                n += 1
        assert counts[k] == n
        assert np.allclose(sums[k], want, rtol=0, atol=1e-12)
    assert counts[4] == 0 and not sums[4].any()
    s1, n1 = oracle.segment_sums(x[:20], a[:20], 6)
    s2, n2 = oracle.segment_sums(x[20:], a[20:], 6)
    assert np.array_equal(n1 + n2, counts)
    assert np.allclose(s1 + s2, sums, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# the blocked composition the full-size GPU tests use (per block of points: the oracle's
# assignment and segment sums; sums added over blocks) against the oracle's own iteration
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_blocked_iteration_equals_oracle_iteration(dtype):
    from concurrent.futures import ThreadPoolExecutor
    from exact_lloyd_means_02_amd import workloads as W
    from helpers import oracle_iteration_blocked
    x64 = _gmm(3, 5000, 8, 9, 21)
    x_store = W.cast_f32(x64.astype(np.float32), dtype)
    xs = W.storage_to_f64(x_store, dtype)
    c = xs[:, 100:107].astype(np.float32).astype(np.float64)
    ref = oracle.lloyd_iteration(xs, c, dtype=dtype, mode="modelled")
    with ThreadPoolExecutor(4) as pool:
        lab, d1, d2, J, cnt, c_new = oracle_iteration_blocked(x_store, dtype, c, [0, 1, 2], pool, block=777)
    assert np.array_equal(lab, ref["a"]) and np.array_equal(cnt, ref["counts"])
    np.testing.assert_allclose(d1, ref["d1"], rtol=1e-13)
    np.testing.assert_allclose(d2, ref["d2"], rtol=1e-13)
    np.testing.assert_allclose(J, ref["inertia"], rtol=1e-12)
    # fp32 master: equal unless an fp64 sum order difference crosses an fp32 rounding boundary
    assert np.max(np.abs(c_new - ref["c_new"]) / np.maximum(np.abs(ref["c_new"]), 1e-30)) <= 2 ** -23
    # a subset of problems runs the same per-problem iteration
    with ThreadPoolExecutor(4) as pool:
        lab1, _, _, J1, _, c1 = oracle_iteration_blocked(x_store, dtype, c[[2]], [2], pool, block=1000)
    assert np.array_equal(lab1[0], ref["a"][2]) and np.allclose(J1[0], ref["inertia"][2], rtol=1e-12)
