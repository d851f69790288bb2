"""Concurrent fits on two streams (two host threads) each get their own scratch memory from the
binding and give the same result, bit for bit, as the same fit run alone."""
import sys
import threading

import numpy as np
import pytest

from exact_lloyd_means_02_amd import workloads as W

from helpers import make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_two_streams_two_fits():
    from exact_lloyd_means_02_amd import flashkm as fk
    w = W.small("headline_bf16", B=4, N=20000, K=200)
    print(f"case {w}", flush=True)
    sys.stdout.flush()
    x, x64, c0, xt, ct = make_inputs(w)
    halves = [xt[:2].contiguous(), xt[2:].contiguous()]
    inits = [ct[:2].contiguous(), ct[2:].contiguous()]
    # alone, one after the other on the default stream
    ref = []
    for i in range(2):
        c = inits[i].clone()
        a, J, _ = fk.kmeans_fit(halves[i], c, 5, 0.0)
        torch.cuda.synchronize()
        ref.append((a.cpu().numpy(), c.cpu().numpy(), J))
    # both at once, one stream each
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cs = [inits[0].clone(), inits[1].clone()]
    out = [None, None]
    torch.cuda.synchronize()

    def run(i):
        out[i] = fk.kmeans_fit(halves[i], cs[i], 5, 0.0, stream=streams[i])

    th = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    for i in range(2):
        a, J, done = out[i]
        assert done == 5
        assert np.array_equal(a.cpu().numpy(), ref[i][0])
        assert np.array_equal(cs[i].cpu().numpy(), ref[i][1])
        assert np.array_equal(J, ref[i][2])
