"""The standard path the benchmark sets beside this one (materialised distances + argmin;
scatter-add update), checked against the oracle like the HIP path: its labels equal the oracle's
except near ties, and its update of those labels is the oracle's means within the dtype's
tolerance.  It is plain PyTorch, context only: the speedups it yields are meaningful only if it
computes the same thing."""
import sys

import numpy as np
import pytest

import oracle

from helpers import CENTROID_TOL, check_assign, make_inputs, operand
from exact_lloyd_means_02_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name,kw", [("headline_bf16", dict(B=2, N=6000, K=300)),
                                     ("batched_f16", dict(B=1, N=5000, K=128)),
                                     ("skew_bf16_k64", dict(N=50000, K=64))])
def test_standard_path_matches_oracle(name, kw):
    import bench
    w = W.small(name, **kw)
    _say(f"standard path, case {w}")
    x, x64, c0, xt, ct = make_inputs(w)
    lab = bench.standard_assign(xt, ct, chunk=2048)
    c_new, cnt = bench.standard_update(xt, lab, ct, chunk=4096)
    torch.cuda.synchronize()
    a = lab.cpu().numpy()
    flips = check_assign(x64, operand(c0, w.dtype), a)
    _say(f"standard assign: {flips} near-tie flips")
    tol = CENTROID_TOL[w.dtype]
    cg = c_new.cpu().numpy().astype(np.float64)
    for b in range(w.B):
        c_or, n_or = oracle.update(x64[b], a[b], c0[b])
        assert np.array_equal(cnt[b].cpu().numpy(), n_or)
        nz = n_or > 0
        rel = np.linalg.norm(cg[b][nz] - c_or[nz], axis=1) / np.maximum(np.linalg.norm(c_or[nz], axis=1), 1e-30)
        assert rel.max() <= tol, rel.max()
        assert np.array_equal(cg[b][~nz], c0[b][~nz].astype(np.float64))
