"""Parity at the workloads' full sizes, in the launch configuration the benchmark times.

The HIP path runs on the full inputs.  The oracle then checks:
- outputs it can compute one by one: sampled points for the assignment, sampled clusters
  for the centroids;
- outputs that are cheap in full: the arg-sort and the counts of every problem, and the
  inertia as an O(N*D) sum;
- properties that hold at any size: streamed vs device-resident labels.

Stages are teacher forced: each stage takes the GPU's own inputs from the previous stage,
as the parity protocol prescribes.
"""
import os
import sys
import time

import numpy as np
import pytest

import oracle
from exact_lloyd_means_02_amd import workloads as W

from helpers import CENTROID_TOL, INERTIA_TOL, check_argsort, check_assign, check_fit, device, operand

torch = pytest.importorskip("torch")
# each test holds one workload at full size plus its oracle work (up to a few minutes of host time)
pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900, method="thread")]

BLOCK = 1 << 20       # points per host-side conversion block


@pytest.fixture(scope="module")
def fk():
    from exact_lloyd_means_02_amd import flashkm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return flashkm


T0 = time.time()


def _say(msg):
    print("[%6.1fs] %s" % (time.time() - T0, msg), flush=True)
    sys.stdout.flush()


def _rows64(x, w, b, idx):
    return W.storage_to_f64(x[b, idx], w.dtype)


def _inertia_oracle(x, w, ct64, a_np):
    """sum_i ||x_i - c~_{a_i}||^2 per problem, in blocks (oracle.dist_to per block)."""
    B, N = a_np.shape
    J = np.zeros(B)
    for b in range(B):
        for lo in range(0, N, BLOCK):
            xb = W.storage_to_f64(x[b, lo:lo + BLOCK], w.dtype)
            J[b] += float(np.sum(oracle.dist_to(xb, ct64[b], a_np[b, lo:lo + BLOCK])))
    return J


def _check_cluster_sample(x, w, c_old, a_np, counts_gpu, c_new_gpu, ks_per_problem):
    """Counts of every cluster; centroids of the sampled clusters (oracle segment sums over the
    GPU's assignment); empty clusters bit-identical to the old centroids."""
    B, K = counts_gpu.shape
    tol = CENTROID_TOL[w.dtype]
    worst = 0.0
    for b in range(B):
        n_or = np.bincount(a_np[b], minlength=K)
        assert np.array_equal(n_or, counts_gpu[b]), "counts differ in problem %d" % b
        empty = n_or == 0
        assert np.array_equal(c_new_gpu[b][empty], c_old[b][empty]), "empty clusters changed"
        for k in ks_per_problem[b]:
            rows = np.nonzero(a_np[b] == k)[0]
            if rows.size == 0:
                continue
            s = np.zeros(x.shape[2])
            for lo in range(0, rows.size, BLOCK):
                r = rows[lo:lo + BLOCK]
                sk, nk = oracle.segment_sums(_rows64(x, w, b, r), np.zeros(r.size, dtype=np.int64), 1)
                s += sk[0]
            c_or = s / rows.size
            rel = np.linalg.norm(c_new_gpu[b, k].astype(np.float64) - c_or) / max(np.linalg.norm(c_or), 1e-30)
            worst = max(worst, rel)
            assert rel <= tol, "problem %d cluster %d (n=%d): centroid rel err %g > %g" % (b, k, rows.size, rel, tol)
    return worst


def _stage_parity(fk, w, x, c0, xt, ct, n_assign, n_clusters, seed):
    """One teacher-forced iteration at full size; returns the GPU labels (numpy)."""
    B, N, D, K = w.B, w.N, w.D, w.K
    ct64 = operand(c0, w.dtype)
    xn = fk.kmeans_row_norms(xt)
    prep = fk.kmeans_prepare_centroids(ct, xt)
    a, md = fk.kmeans_assign_prepared(xt, prep, x_norms=xn, want_min_dist=True)
    s, i, cnt = fk.kmeans_argsort_ids(a, K)
    cu = ct.clone()
    shift = fk.kmeans_update(xt, s, i, cnt, cu, want_shift=True)
    torch.cuda.synchronize()
    a_np, md_np = a.cpu().numpy(), md.cpu().numpy()
    s_np, i_np, cnt_np = s.cpu().numpy(), i.cpu().numpy(), cnt.cpu().numpy()
    c_new = cu.cpu().numpy()
    shift_np = shift.cpu().numpy()
    _say("GPU stages done")

    rng = np.random.default_rng(seed)
    samp = [np.sort(rng.choice(N, size=min(N, n_assign), replace=False)) for _ in range(B)]
    x64s = np.stack([_rows64(x, w, b, samp[b]) for b in range(B)])
    a_s = np.stack([a_np[b, samp[b]] for b in range(B)])
    md_s = np.stack([md_np[b, samp[b]] for b in range(B)])
    flips = check_assign(x64s, ct64, a_s, md_s)
    _say("assign: %d sampled points per problem, %d near-tie flips" % (n_assign, flips))

    check_argsort(a_np, K, s_np, i_np, cnt_np)
    _say("arg-sort and counts: all %d problems bit-exact" % B)

    ks = []
    for b in range(B):
        hot = np.argsort(-cnt_np[b], kind="stable")[:4]            # the largest segments
        rnd = rng.choice(K, size=min(K, n_clusters), replace=False)
        ks.append(np.unique(np.concatenate([hot, rnd])))
    worst = _check_cluster_sample(x, w, c0, a_np, cnt_np, c_new, ks)
    _say("update: %d sampled clusters per problem, worst rel err %.3g" % (len(ks[0]), worst))

    # shift = sum_k ||c_new - c_old||^2 of the GPU's own centroids (fp64), per problem
    for b in range(B):
        s_or = float(np.sum((c_new[b].astype(np.float64) - c0[b].astype(np.float64)) ** 2))
        assert abs(shift_np[b] - s_or) <= 1e-5 * max(s_or, 1e-30) + 1e-12
    return a_np, ct64


def _fit_inertia_check(fk, w, x, c0, xt, ct, a_stage):
    """kmeans_fit for one iteration: same labels as the stage calls, inertia against the oracle."""
    c = ct.clone()
    a, J, done = fk.kmeans_fit(xt, c, 1, 0.0)
    a_np = a.cpu().numpy()
    assert done == 1
    assert np.array_equal(a_np, a_stage), "kmeans_fit labels differ from the stage calls"
    J_or = _inertia_oracle(x, w, operand(c0, w.dtype), a_np)
    rel = np.abs(J[0] - J_or) / np.abs(J_or)
    _say("fit inertia: max rel diff %.3g" % rel.max())
    assert rel.max() <= INERTIA_TOL


# ---------------------------------------------------------------------------------------------
# headline: B=32, N=65536, D=128, K=1024, bf16 (the benchmark's workload)
# ---------------------------------------------------------------------------------------------
def test_headline_full(fk):
    w = W.WORKLOADS["headline_bf16"]
    _say("headline: generating %s" % (w,))
    x, c0, _ = W.make(w)
    xt = W.to_torch(x, w.dtype).to(device())
    ct = torch.from_numpy(c0).to(device())
    a_np, _ = _stage_parity(fk, w, x, c0, xt, ct, n_assign=512, n_clusters=32, seed=31)
    _fit_inertia_check(fk, w, x, c0, xt, ct, a_np)
    # all 10 iterations free running: the oracle's loop on 4 of the 32 independent problems; the
    # last iteration teacher forced on every point of all 32
    check_fit(fk, w, x, c0, xt, ct, problems=[0, 1, 2, 3], say=_say)


# ---------------------------------------------------------------------------------------------
# batched fp16: B=32, N=75600, D=128, K=1000, tol 1e-4
# ---------------------------------------------------------------------------------------------
def test_batched_f16_full(fk):
    w = W.WORKLOADS["batched_f16"]
    _say("batched f16: generating %s" % (w,))
    x, c0, _ = W.make(w)
    xt = W.to_torch(x, w.dtype).to(device())
    ct = torch.from_numpy(c0).to(device())
    a_np, _ = _stage_parity(fk, w, x, c0, xt, ct, n_assign=384, n_clusters=24, seed=32)
    _fit_inertia_check(fk, w, x, c0, xt, ct, a_np)
    # the whole run with tol = 1e-4: the stopping rule on the fit's own trajectory (the oracle's
    # fp64 shift of its centroids, all 32 problems), the oracle's free-running loop on 2 of the 32
    # problems, the last iteration teacher forced on every point
    check_fit(fk, w, x, c0, xt, ct, problems=[0, 1], say=_say)


# ---------------------------------------------------------------------------------------------
# skewed large N: B=1, N=2^24, D=128, bf16, K in {64, 4096}, Zipf(1.2) clusters, centred
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["skew_bf16_k64", "skew_bf16_k4096"])
def test_skew_full(fk, name):
    w = W.WORKLOADS[name]
    _say("skew: generating %s" % (w,))
    x, c0, mu = W.make(w)
    _say("centring translation, channels 0-3: %s" % np.round(mu[0, :4], 3).tolist())
    xt = W.to_torch(x, w.dtype).to(device())
    ct = torch.from_numpy(c0).to(device())
    a_np, ct64 = _stage_parity(fk, w, x, c0, xt, ct, n_assign=8192, n_clusters=12, seed=33)
    hot = np.bincount(a_np[0], minlength=w.K).max() / w.N
    _say("largest cluster holds %.1f%% of the points" % (100 * hot))
    _fit_inertia_check(fk, w, x, c0, xt, ct, a_np)
    # the whole run: inertia non-increasing up to the bf16 rounding of the centroids
    c = ct.clone()
    _, J, done = fk.kmeans_fit(xt, c, w.iters, 0.0)
    _say("fit %d iterations: inertia %s" % (done, np.round(J[:, 0], 1).tolist()))
    assert done == w.iters and (J[1:, 0] <= J[:-1, 0] * (1 + 1e-3)).all()
    if w.K <= 64:
        # all 5 iterations free running against the oracle's loop (blocked over points), the
        # last one teacher forced on every point
        check_fit(fk, w, x, c0, xt, ct, say=_say)
    else:
        # the oracle's free-running loop at K = 4096 takes minutes per iteration on the host:
        # every iteration of the run teacher forced instead, from the GPU's own centroids
        _check_each_iteration(fk, w, x, xt, ct, n_assign=8192, n_clusters=4, seed=35)


def _check_each_iteration(fk, w, x, xt, ct, n_assign, n_clusters, seed):
    """Every iteration t of a w.iters-iteration kmeans_fit, teacher forced: the fit of t + 1
    iterations returns the labels of iteration t (made from the centroids C_t that the fit of t
    iterations returns) and C_{t+1}.  Sampled labels against the oracle's assignment from C_t
    (near-tie rule), the inertia of iteration t in full, C_{t+1} on the largest and on sampled
    clusters against the oracle's means of the GPU's labels, empty clusters bit-identical; the
    shorter fits follow the longer fit's trajectory bit for bit."""
    B, N, K = w.B, w.N, w.K
    rng = np.random.default_rng(seed)
    c_full = ct.clone()
    _, J_full, done = fk.kmeans_fit(xt, c_full, w.iters, 0.0)
    assert done == w.iters
    c_t = ct.cpu().numpy()
    for t in range(w.iters):
        c = ct.clone()
        a, J, done = fk.kmeans_fit(xt, c, t + 1, 0.0)
        torch.cuda.synchronize()
        assert done == t + 1 and np.array_equal(J, J_full[:t + 1]), "fit of %d iterations left the trajectory" % (t + 1)
        a_np, c_next = a.cpu().numpy(), c.cpu().numpy()
        ct64 = operand(c_t, w.dtype)
        samp = [np.sort(rng.choice(N, size=min(N, n_assign), replace=False)) for _ in range(B)]
        x64s = np.stack([_rows64(x, w, b, samp[b]) for b in range(B)])
        flips = check_assign(x64s, ct64, np.stack([a_np[b, samp[b]] for b in range(B)]))
        J_or = _inertia_oracle(x, w, ct64, a_np)
        rel = float(np.max(np.abs(J[t] - J_or) / np.abs(J_or)))
        assert rel <= INERTIA_TOL, "iteration %d: inertia rel diff %g" % (t, rel)
        cnt = np.stack([np.bincount(a_np[b], minlength=K) for b in range(B)])
        ks = [np.unique(np.concatenate([np.argsort(-cnt[b], kind="stable")[:4],
                                        rng.choice(K, size=n_clusters, replace=False)])) for b in range(B)]
        worst = _check_cluster_sample(x, w, c_t, a_np, cnt, c_next, ks)
        _say("iteration %d: %d sampled labels, %d near-tie flips; inertia rel %.3g; %d clusters, worst rel %.3g"
             % (t, n_assign, flips, rel, len(ks[0]), worst))
        c_t = c_next
    assert np.array_equal(c_t, c_full.cpu().numpy()), "stepwise fits end away from the whole fit"


# ---------------------------------------------------------------------------------------------
# split-D: B=1, N=262144, D=1024, K=512, fp32
# ---------------------------------------------------------------------------------------------
def test_splitd_full(fk):
    w = W.WORKLOADS["splitd_f32"]
    assert fk.kmeans_plan(0, w.B, w.N, w.D, w.K)["path"] == 1
    _say("split-D: generating %s" % (w,))
    x, c0, _ = W.make(w)
    xt = W.to_torch(x, w.dtype).to(device())
    ct = torch.from_numpy(c0).to(device())
    a_np, _ = _stage_parity(fk, w, x, c0, xt, ct, n_assign=2048, n_clusters=48, seed=34)
    _fit_inertia_check(fk, w, x, c0, xt, ct, a_np)
    # all 3 iterations free running against the oracle's loop, the last one teacher forced on
    # every point (labels, every centroid)
    check_fit(fk, w, x, c0, xt, ct, say=_say)


# ---------------------------------------------------------------------------------------------
# streamed: D=64, K=32768, fp16 in pinned host memory, real 2^24-point chunks (two full chunks
# and a ragged one; the full 2^30-point run differs only in the number of chunks)
# ---------------------------------------------------------------------------------------------
def test_streamed_real_chunks(fk):
    w0 = W.WORKLOADS["streamed_f16"]
    N = 2 * w0.chunk + 12345
    w = W.small("streamed_f16", N=N, iters=1)
    assert w.K == 32768 and w.D == 64 and w.chunk == 1 << 24
    _say("streamed: generating %s" % (w,))
    xh = torch.empty((w.B, w.N, w.D), dtype=W.torch_dtype(w.dtype), pin_memory=True)
    x = W.from_torch(xh, w.dtype)                         # numpy view of the pinned buffer
    W.generate_points(w, x)
    c0 = W.init_centroids(w, x)
    ct = torch.from_numpy(c0).to(device())
    c_s = ct.clone()
    a_s, J_s, done = fk.kmeans_fit(xh, c_s, 1, 0.0, chunk_points=w.chunk)
    torch.cuda.synchronize()
    _say("streamed fit done")
    xt = xh.to(device())
    c_d = ct.clone()
    a_d, J_d, _ = fk.kmeans_fit(xt, c_d, 1, 0.0)
    a_np = a_s.cpu().numpy()
    # labels do not depend on the chunking: identical to the device-resident run
    assert np.array_equal(a_np, a_d.cpu().numpy())
    ct64 = operand(c0, w.dtype)
    rng = np.random.default_rng(35)
    samp = np.sort(rng.choice(w.N, size=1 << 12, replace=False))
    flips = check_assign(_rows64(x, w, 0, samp)[None], ct64, a_np[:, samp])
    _say("assign: 4096 sampled points, %d near-tie flips" % flips)
    counts = np.bincount(a_np[0], minlength=w.K)[None].astype(np.int32)
    ks = [np.unique(np.concatenate([np.argsort(-counts[0], kind="stable")[:4],
                                    rng.choice(w.K, size=48, replace=False)]))]
    worst = _check_cluster_sample(x, w, c0, a_np, counts, c_s.cpu().numpy(), ks)
    _say("streamed update: worst rel err over %d clusters %.3g" % (len(ks[0]), worst))
    J_or = _inertia_oracle(x, w, ct64, a_np)
    rel = abs(J_s[0, 0] - J_or[0]) / J_or[0]
    _say("streamed inertia rel diff %.3g (device-resident %.3g)" % (rel, abs(J_d[0, 0] - J_or[0]) / J_or[0]))
    assert rel <= INERTIA_TOL
    # the two runs sum the same points in different orders: centroids agree to fp32 rounding
    cs, cd = c_s.cpu().numpy(), c_d.cpu().numpy()
    num = np.linalg.norm(cs - cd, axis=2)
    den = np.maximum(np.linalg.norm(cd, axis=2), 1e-30)
    assert (num / den).max() <= 1e-5


# ---------------------------------------------------------------------------------------------
# streamed at its full size: N = 2^30, D = 64, K = 32768, fp16 in 8 pinned host blocks of 2^27
# points (128 GiB), 3 iterations.  Needs that much pinned host memory and several minutes of host
# time for the oracle, so it runs only when asked (FLASHKM_FULL_STREAMED=1); FLASHKM_FULL_STREAMED_N
# points (a multiple of 2^27) instead of 2^30 when set.  Up to 64 GiB (the pinned host memory the
# MI355X hosts measured allow one process) the points sit in pinned blocks (kmeans_fit_blocks); above, as at the
# stated 2^30 points (128 GiB), in pageable memory staged through a pinned buffer (kmeans_fit_staged).
# ---------------------------------------------------------------------------------------------
@pytest.mark.skipif(os.environ.get("FLASHKM_FULL_STREAMED") != "1",
                    reason="the 2^30-point streamed workload takes 128 GiB of host memory and minutes of "
                           "oracle time; set FLASHKM_FULL_STREAMED=1 to run it")
def test_streamed_full_size(fk):
    """Per iteration t (a fit of t+1 iterations; the fit is deterministic, so its first t are the
    shorter fit's): the labels of 2^18 sampled points against the oracle's assignment from the
    centroids before t (near-tie rule), the inertia of iteration t against the oracle's in full
    (every point), every cluster's count (through the update: empty clusters keep their centroid)
    and the centroids of sampled clusters against the oracle's means of the GPU's members."""
    import bench
    from concurrent.futures import ThreadPoolExecutor
    w = W.WORKLOADS["streamed_f16"]
    n_env = int(os.environ.get("FLASHKM_FULL_STREAMED_N", "0"))
    if n_env:
        assert n_env % (1 << 27) == 0
        w = W.small("streamed_f16", N=n_env)
    pageable = W.nbytes(w) > bench.PINNED_CAP_BYTES
    _say("streamed full size: generating %s in %s host memory" % (w, "pageable" if pageable else "pinned"))
    if pageable:
        x, c0, _ = W.make(w)
        nb = [x[0]]                                   # one [N, D] block
        xp = W.to_torch(x, w.dtype)
        stage = fk.stage_buffer(fk.dtype_code(xp), 1, w.N, w.D, w.K, w.chunk)
        tb = [xp[0]]
    else:
        try:
            tb, nb = bench.pinned_blocks(w)
        except RuntimeError as e:
            pytest.skip("pinned host allocation refused: %s" % e)
        c0 = W.init_centroids_blocks(w, nb)
    ct = torch.from_numpy(c0).to(device())
    _say("generated; %d blocks" % len(tb))
    rng = np.random.default_rng(36)
    samp = np.sort(rng.choice(w.N, size=1 << 18, replace=False))
    x_s = W.storage_to_f64(W.rows_of_blocks(nb, samp), w.dtype)
    starts = np.cumsum([0] + [t.shape[0] for t in tb])
    c_prev = c0.astype(np.float64)
    tol = CENTROID_TOL[w.dtype]
    for t in range(w.iters):
        c = ct.clone()
        if pageable:
            a, J, done = fk.kmeans_fit_staged(xp, c, t + 1, 0.0, chunk_points=w.chunk, stage=stage)
        else:
            a, J, done = fk.kmeans_fit_blocks(tb, c, t + 1, 0.0, chunk_points=w.chunk)
        torch.cuda.synchronize()
        assert done == t + 1
        a_np = a.cpu().numpy()[0]
        c_next = c.cpu().numpy().astype(np.float64)
        del a
        _say("iteration %d: GPU fit of %d iterations done, inertia %s" % (t, t + 1, J[:, 0].tolist()))
        ct64 = operand(c_prev.astype(np.float32), w.dtype)
        flips = check_assign(x_s[None], ct64, a_np[samp][None])
        _say("  labels: %d sampled points, %d near-tie flips" % (samp.size, flips))

        def block_dist(lo):
            j = int(np.searchsorted(starts, lo, side="right")) - 1
            xb = W.storage_to_f64(nb[j][lo - starts[j]:lo - starts[j] + BLOCK], w.dtype)
            return float(np.sum(oracle.dist_to(xb, ct64[0], a_np[lo:lo + xb.shape[0]])))
        with ThreadPoolExecutor(4) as ex:
            J_or = sum(ex.map(block_dist, range(0, w.N, BLOCK)))
        rel = abs(J[t, 0] - J_or) / J_or
        _say("  inertia in full: rel diff %.3g" % rel)
        assert rel <= INERTIA_TOL
        counts = np.bincount(a_np, minlength=w.K)
        empty = counts == 0
        assert np.array_equal(c_next[0][empty], c_prev[0][empty]), "empty clusters changed"
        ks = np.unique(np.concatenate([np.argsort(-counts, kind="stable")[:4], rng.choice(w.K, 28, replace=False)]))
        ks = ks[counts[ks] > 0]
        members = np.nonzero(np.isin(a_np, ks))[0]
        lab_m = a_np[members]
        worst = 0.0
        for k in ks:
            rows = members[lab_m == k]
            xs = W.storage_to_f64(W.rows_of_blocks(nb, rows), w.dtype)
            sk, nk = oracle.segment_sums(xs, np.zeros(rows.size, dtype=np.int64), 1)
            c_or = sk[0] / rows.size
            r = np.linalg.norm(c_next[0, k] - c_or) / max(np.linalg.norm(c_or), 1e-30)
            worst = max(worst, r)
            assert r <= tol, "cluster %d (n=%d): rel err %g" % (k, rows.size, r)
        _say("  update: %d empty clusters kept, %d sampled clusters (largest n=%d), worst rel err %.3g" % (
            int(empty.sum()), ks.size, int(counts.max()), worst))
        c_prev = c_next
        del a_np


# ---------------------------------------------------------------------------------------------
# dot-product and cosine k-means at the headline size (one iteration, teacher forced)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("metric", ["dot", "cosine"])
def test_headline_metric_full(fk, metric):
    from oracle import similarity as sim
    from helpers import NEAR
    w = W.WORKLOADS["headline_bf16"]
    B, N, D, K = w.B, w.N, w.D, w.K
    _say("headline %s: generating %s" % (metric, w))
    x, c0, _ = W.make(w)
    xt = W.to_torch(x, w.dtype).to(device())
    ct = torch.from_numpy(c0).to(device())
    c = ct.clone()
    a, obj, done = fk.kmeans_fit_metric(xt, c, metric, 1)
    assert done == 1
    if metric == "cosine":
        xa_t = fk.kmeans_normalize_rows(xt)                 # the unit rows the fit used
        c_start = fk.kmeans_normalize_rows(ct).cpu().numpy().astype(np.float64)
        xa = W.from_torch(xa_t, w.dtype)
    else:
        xa, c_start = x, c0.astype(np.float64)
    torch.cuda.synchronize()
    a_np = a.cpu().numpy().astype(np.int64)
    cg = c.cpu().numpy().astype(np.float64)
    ct64 = operand(c_start, w.dtype)
    _say("GPU fit done")
    rng = np.random.default_rng(41)
    flips = 0
    for b in range(B):
        samp = np.sort(rng.choice(N, size=512, replace=False))
        xs = _rows64(xa, w, b, samp)
        a_or, s1, s2, scale = sim.similarity_assign(xs, ct64[b])
        bad = (a_np[b, samp] != a_or) & ~sim.similarity_near_mask(s1, s2, scale, NEAR)
        assert not bad.any(), "problem %d: picks differ outside the near-tie band" % b
        flips += int((a_np[b, samp] != a_or).sum())
    _say("assign: 512 sampled points per problem, %d near-tie flips" % flips)
    tol = CENTROID_TOL[w.dtype]
    worst = 0.0
    for b in range(B):
        counts = np.bincount(a_np[b], minlength=K)
        kept = counts == 0
        assert np.array_equal(cg[b][kept], c_start[b][kept].astype(np.float32).astype(np.float64))
        ks = np.unique(np.concatenate([np.argsort(-counts, kind="stable")[:4], rng.choice(K, 24, replace=False)]))
        for k in ks:
            rows = np.nonzero(a_np[b] == k)[0]
            if rows.size == 0:
                continue
            s = _rows64(xa, w, b, rows).sum(axis=0)
            c_or = s / rows.size if metric == "dot" else s / np.linalg.norm(s)
            rel = np.linalg.norm(cg[b, k] - c_or) / max(np.linalg.norm(c_or), 1e-30)
            worst = max(worst, rel)
            assert rel <= tol, "problem %d cluster %d: rel err %g" % (b, k, rel)
        # the objective in full: sum_i x_i . c~_{a_i}
        j = 0.0
        for lo in range(0, N, BLOCK):
            xb = W.storage_to_f64(xa[b, lo:lo + BLOCK], w.dtype)
            j += float(np.einsum("nd,nd->n", xb, ct64[b][a_np[b, lo:lo + BLOCK]]).sum())
        assert abs(obj[0, b] - j) <= INERTIA_TOL * abs(j)
    _say("update: sampled clusters, worst rel err %.3g; objective matches in full" % worst)
