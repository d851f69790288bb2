#!/usr/bin/env python3
"""Benchmark: one batched Lloyd iteration on one MI355X.

A step is one Lloyd iteration of the whole path (centroid preparation, FlashAssign with the
per-point minimum distance, inertia, arg-sort, sort-inverse update with the shift), run by
kmeans_fit on the headline workload (B=32, N=65536, D=128, K=1024, bf16; inputs resident in
HBM).  The timed region is one kmeans_fit call of `--steps` iterations (the point norms are
computed once inside it, as in any fit).  Per-stage times come from HIP events recorded on
the stream the stages run on; the FlashAssign kernel is timed on its own through
kmeans_assign_prepared (one kernel launch per call).  Prints one JSON line.

`--copy-calib` instead runs a plain device copy of known size (the reference for scaling the
FETCH_SIZE / WRITE_SIZE counters into bytes) and prints its size.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms per Lloyd iteration at B=32,N=65536,K=1024,D=128 bf16; % MFMA and % HBM peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50,
                   help="untimed iterations first: the GPU takes a few tens of ms of work to reach its steady clocks")
    p.add_argument("--workload", default="headline_bf16")
    p.add_argument("--stage-reps", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calib", action="store_true", help="run a plain 1 GiB device copy and exit")
    p.add_argument("--metric", default="l2", choices=["l2", "dot", "cosine"],
                   help="k-means variant: Lloyd (l2), dot-product or cosine (spherical) k-means")
    p.add_argument("--context", action="store_true",
                   help="also time the standard path in plain PyTorch (materialised distances + argmin, "
                        "scatter-add update) for the kernel ratios")
    return p.parse_args()


ASSIGN_SRC = os.path.join(ROOT, "exact_lloyd_means_02_amd", "csrc", "k_assign.hip")
BUILD_SCRIPT = os.path.join(ROOT, "exact_lloyd_means_02_amd", "build.py")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "assign_small_d_headline_bf16_traffic.txt")


def assign_source_hash() -> str:
    """Hash of the FlashAssign source and of the build script (which holds its compiler flags)."""
    h = hashlib.sha256(open(ASSIGN_SRC, "rb").read())
    h.update(open(BUILD_SCRIPT, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per FlashAssign launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel factor), or None when the summary is missing, was
    taken on another version of the kernel source, or covers another workload (it covers the
    headline one)."""
    if workload != "headline_bf16" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ": " in line and not line.startswith("#"):
            k, v = line.split(": ", 1)
            kv[k.strip()] = v.strip()
    if kv.get("k_assign.hip + build.py sha256[:16]") != assign_source_hash():
        return None
    try:
        return float(kv["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def copy_calib():
    import torch
    n = 1 << 28                                    # 2^28 float32 = 1 GiB read + 1 GiB written
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib": {"bytes_read": 4 * n, "bytes_written": 4 * n, "launches": 3,
                                     "read_kib": 4 * n / 1024}}), flush=True)


def algorithmic(w):
    """Per-iteration algorithmic work (see the design notes): assign FLOP on MFMA, assign bytes,
    update bytes (arg-sort + segmented reduction + centroid write)."""
    from exact_lloyd_means_02_amd.workloads import ELEM_BYTES
    s = ELEM_BYTES[w.dtype]
    B, N, D, K = w.B, w.N, w.D, w.K
    flops = 2.0 * B * N * K * D
    assign_bytes = B * N * D * s + B * K * D * s + 4 * B * K + 8 * B * N
    update_bytes = 20 * B * N + B * N * D * s + 8 * B * K * (D + 1) + B * K * D * (4 + s) + 4 * B * K
    return flops, assign_bytes, update_bytes


def cpu_baseline(w, x, c0, target_s, metric="l2"):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload: one iteration
    on the first `n` points of the first `p` problems against all K centroids, grown until it
    takes ~0.6 * target_s (or covers everything), then scaled to B*N points."""
    import numpy as np
    import oracle
    from oracle import similarity as sim
    from exact_lloyd_means_02_amd import workloads as W
    n, p = min(w.N, 2048), 1
    while True:
        xs = W.storage_to_f64(x[:p, :n], w.dtype)
        t0 = time.perf_counter()
        if metric == "l2":
            oracle.lloyd_iteration(xs, c0[:p].astype(np.float64), dtype=w.dtype, mode="modelled")
        else:
            if metric == "cosine":
                xs = sim.round_to_dtype(sim.normalize_rows(xs), w.dtype)
            sim.similarity_iteration(xs, c0[:p].astype(np.float64), metric, dtype=w.dtype, mode="modelled")
        dt = time.perf_counter() - t0
        if dt >= 0.6 * target_s or (n >= w.N and p >= w.B):
            break
        grow = max(1.5, min(8.0, 0.7 * target_s / max(dt, 1e-3)))
        if n < w.N:
            n = min(w.N, int(n * grow))
        else:
            p = min(w.B, max(p + 1, int(p * grow)))
    scale = (w.B * w.N) / (p * n)
    return {"value": round(dt * scale * 1e3, 3), "unit": "ms", "cores": oracle.threads(), "kind": "oracle",
            "sample": "one fp64 oracle iteration on %d of %d points (%d problem(s) x %d points, all K=%d "
                      "centroids) took %.2f s; scaled by %.1fx to the full iteration" % (
                          p * n, w.B * w.N, p, n, w.K, dt, scale)}


def standard_path(w, xt, c0t, reps, st):
    """The standard path the method replaces, in plain PyTorch on the same GPU (context only):
    assign materialises the B x N x K distance matrix (hipBLASLt batched product, fp32
    distances, argmin over K); update scatter-adds every row into its cluster's fp32 sum
    with atomics (index_add_) and divides by the bincount.  Returns medians in ms and the
    label agreement with the FlashAssign labels of the same centroids."""
    import numpy as np
    import torch
    from exact_lloyd_means_02_amd import flashkm as fk
    B, N, D, K = w.B, w.N, w.D, w.K
    stream = torch.cuda.current_stream()
    c_lp = c0t.to(xt.dtype)
    c_lp_t = c_lp.transpose(1, 2).contiguous()          # [B, D, K], contiguous right operand
    cn = (c_lp.float() ** 2).sum(-1)                     # ||c~||^2 from the rounded centroids
    xf = xt.view(B * N, D)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ta, tu = [], []
    lab = None
    gemm_out = "fp32"
    for _ in range(reps):
        ev[0].record(stream)
        if gemm_out == "fp32":
            try:
                dots = torch.bmm(xt, c_lp_t, out_dtype=torch.float32)   # [B, N, K], fp32 accumulate and output
            except (RuntimeError, TypeError):
                gemm_out = "input dtype"
        if gemm_out != "fp32":
            dots = torch.bmm(xt, c_lp_t)                 # [B, N, K] in the input dtype
        dist = cn[:, None, :] - 2.0 * dots.float()       # ||x||^2 dropped: constant per point
        lab = torch.argmin(dist, dim=-1)
        del dots, dist
        ev[1].record(stream)
        flat = (lab + torch.arange(B, device=xt.device)[:, None] * K).view(-1)
        sums = torch.zeros(B * K, D, dtype=torch.float32, device=xt.device)
        sums.index_add_(0, flat, xf.float())
        cnt = torch.bincount(flat, minlength=B * K)
        newc = torch.where(cnt[:, None] > 0, sums / cnt.clamp(min=1)[:, None].float(), c0t.view(B * K, D))
        ev[2].record(stream)
        torch.cuda.synchronize()
        ta.append(ev[0].elapsed_time(ev[1]))
        tu.append(ev[1].elapsed_time(ev[2]))
        del sums, cnt, newc, flat
    prep = fk.kmeans_prepare_centroids(c0t, xt)
    a, _ = fk.kmeans_assign_prepared(xt, prep)
    agree = float((a.long() == lab).float().mean().item())
    ma, mu = float(np.median(ta)), float(np.median(tu))
    return {"what": "plain PyTorch on the same GPU: bmm + fp32 distances + argmin; index_add_ scatter + bincount",
            "gemm_output": gemm_out, "materialised_assign_ms": round(ma, 4), "scatter_update_ms": round(mu, 4),
            "assign_speedup": round(ma / st["assign"], 2),
            "update_speedup": round(mu / (st["argsort"] + st["update"]), 2),
            "label_agreement": agree}


def bench_streamed(args, w):
    """Host-resident workload: x in pinned host memory, streamed in chunks by kmeans_fit.  Reports
    ms per Lloyd iteration, the plain host->device copy rate of the same chunks and the GPU time
    of one iteration on one device-resident chunk (the two legs the pipeline overlaps)."""
    import numpy as np
    import torch
    from exact_lloyd_means_02_amd import flashkm as fk
    from exact_lloyd_means_02_amd import workloads as W

    n_override = int(os.environ.get("BENCH_STREAMED_N", "0"))
    if n_override:
        w = W.small(w.name, N=n_override)
    steps = args.steps if args.steps != 20 else w.iters
    print("bench: allocating %.1f GiB of pinned host memory for %s" % (W.nbytes(w) / 2 ** 30, w),
          file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    xh = torch.empty((w.B, w.N, w.D), dtype=W.torch_dtype(w.dtype), pin_memory=True)
    x = W.from_torch(xh, w.dtype)
    print("bench: pinned in %.1f s; generating" % (time.perf_counter() - t0), file=sys.stderr, flush=True)
    W.generate_points(w, x)
    c0 = W.init_centroids(w, x)
    dev = torch.device("cuda:0")
    c0t = torch.from_numpy(c0).to(dev)
    print("bench: generated in %.1f s" % (time.perf_counter() - t0), file=sys.stderr, flush=True)

    # leg 1: plain chunked host->device copies (two staging buffers, one stream)
    chunk = w.chunk
    bufs = [torch.empty((chunk, w.D), dtype=xh.dtype, device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for q, lo in enumerate(range(0, w.N, chunk)):
        n = min(chunk, w.N - lo)
        bufs[q & 1][:n].copy_(xh[0, lo:lo + n], non_blocking=True)
    torch.cuda.synchronize()
    h2d_s = time.perf_counter() - t1
    # leg 2: one iteration on one device-resident chunk
    xc = xh[:, :chunk].to(dev)
    cc = c0t.clone()
    fk.kmeans_fit(xc, cc, 1, 0.0)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    cc.copy_(c0t)
    fk.kmeans_fit(xc, cc, 1, 0.0)
    torch.cuda.synchronize()
    chunk_ms = (time.perf_counter() - t2) * 1e3
    del xc
    print("bench: h2d %.1f GB/s, one-chunk iteration %.1f ms; streaming %d iterations" % (
        W.nbytes(w) / h2d_s / 1e9, chunk_ms, steps), file=sys.stderr, flush=True)

    c = c0t.clone()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    _, inertia, done = fk.kmeans_fit(xh, c, steps, 0.0, chunk_points=chunk, want_assign=False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t3) * 1e3 / steps
    nchunks = -(-w.N // chunk)
    flops = 2.0 * w.B * w.N * w.K * w.D
    out = {
        "metric": "ms per Lloyd iteration (%s, x streamed from pinned host memory)" % w.name,
        "value": round(ms, 2), "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": steps,
        "warmup": 0, "ms_per_step": round(ms, 2), "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "D": w.D, "K": w.K, "chunk_points": chunk,
                   "chunks": nchunks, "iters": steps, "inputs": "pinned host"},
        "assign_tflops_effective": round(flops / (ms * 1e-3) / 1e12, 1),
        "h2d_GBs_plain_copy": round(W.nbytes(w) / h2d_s / 1e9, 1),
        "h2d_ms_per_iteration": round(h2d_s * 1e3, 1),
        "one_chunk_device_iteration_ms": round(chunk_ms, 2),
        "compute_ms_per_iteration_est": round(chunk_ms * nchunks, 1),
        "inertia": [float(v) for v in inertia[:, 0]],
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calib()
        return
    import numpy as np
    import torch
    from exact_lloyd_means_02_amd import flashkm as fk
    from exact_lloyd_means_02_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    if w.host:
        bench_streamed(args, w)
        return
    dev = torch.device("cuda:0")
    print("bench: generating %s" % (w,), file=sys.stderr, flush=True)
    x, c0, _ = W.make(w)
    xt = W.to_torch(x, w.dtype).to(dev)
    c0t = torch.from_numpy(c0).to(dev)
    c = c0t.clone()
    stream = torch.cuda.current_stream(dev)

    def fit(iters):
        if args.metric == "l2":
            return fk.kmeans_fit(xt, c, iters, 0.0)
        return fk.kmeans_fit_metric(xt, c, args.metric, iters, 0.0)

    # ---- warmup (untimed): W iterations
    fit(max(1, args.warmup))
    torch.cuda.synchronize()

    # ---- timed: exactly `steps` iterations in one fit
    c.copy_(c0t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, inertia, done = fit(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert done == args.steps
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    print("bench: %d iterations in %.3f ms" % (args.steps, (t1 - t0) * 1e3), file=sys.stderr, flush=True)

    # ---- per-stage times (HIP events on the stages' stream), teacher forced from c0
    xn = fk.kmeans_row_norms(xt)
    prep = fk.kmeans_prepare_centroids(c0t, xt, metric=args.metric)
    a, md = fk.kmeans_assign_prepared(xt, prep, x_norms=xn, want_min_dist=True)
    s_ids, s_idx, counts = fk.kmeans_argsort_ids(a, w.K)
    cu = c0t.clone()
    torch.cuda.synchronize()
    R = args.stage_reps
    names = ["row_norms", "prepare", "assign", "argsort", "update"]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    times = {k: [] for k in names}
    for _ in range(R):
        cu.copy_(c0t)
        ev[0].record(stream)
        fk.kmeans_row_norms(xt, out=xn)
        ev[1].record(stream)
        fk.kmeans_prepare_centroids(c0t, xt, out=prep.buf, metric=args.metric)
        ev[2].record(stream)
        fk.kmeans_assign_prepared(xt, prep, x_norms=xn, assign=a, min_dist=md)
        ev[3].record(stream)
        fk.kmeans_argsort_ids(a, w.K, sorted_ids=s_ids, sorted_idx=s_idx, counts=counts)
        ev[4].record(stream)
        fk.kmeans_update(xt, s_ids, s_idx, counts, cu)
        ev[5].record(stream)
        torch.cuda.synchronize()
        for i, k in enumerate(names):
            times[k].append(ev[i].elapsed_time(ev[i + 1]))
    st = {k: float(np.median(v)) for k, v in times.items()}
    flops, abytes, ubytes = algorithmic(w)
    peak = PEAK_TFLOPS[w.dtype]
    assign_tflops = flops / (st["assign"] * 1e-3) / 1e12
    upd_ms = st["argsort"] + st["update"]
    upd_gbs = ubytes / (upd_ms * 1e-3) / 1e9

    headline = w.name == "headline_bf16" and args.metric == "l2"
    out = {
        "metric": METRIC if headline else "ms per %s k-means iteration (%s)" % (
            {"l2": "Lloyd", "dot": "dot-product", "cosine": "cosine"}[args.metric], w.name),
        "value": round(ms_per_step, 4),
        "unit": "ms",
        "higher_is_better": False,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "D": w.D, "K": w.K, "iters": args.steps, "tol": 0.0,
                   "inputs": "HBM-resident", "metric": args.metric},
        "roofline": {"bound": "mfma", "achieved": round(assign_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(assign_tflops / peak, 4), "traffic": measured_traffic(w.name),
                     "kernel": "FlashAssign (%s) kernel, one launch per kmeans_assign_prepared call" % (
                         "small-D" if fk.kmeans_plan(fk.dtype_code(xt), w.B, w.N, w.D, w.K)["path"] == 0 else "split-D"),
                     "kernel_ms": round(st["assign"], 4), "flop_per_launch": flops,
                     "algorithmic_bytes_per_launch": abytes},
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "update": {"bound": "hbm", "achieved": round(upd_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(upd_gbs / PEAK_HBM_GBS, 4), "bytes_per_iter": ubytes,
                   "stages": "kmeans_argsort_ids + kmeans_update"},
        ("inertia_last" if args.metric == "l2" else "similarity_last"): [float(v) for v in inertia[-1][:2]],
    }
    if args.context:
        print("bench: timing the standard path", file=sys.stderr, flush=True)
        out["context"] = standard_path(w, xt, c0t, 5, st)
    if not args.no_cpu_baseline:
        print("bench: timing the oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, x, c0, args.cpu_seconds, args.metric)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
