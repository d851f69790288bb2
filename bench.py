#!/usr/bin/env python3
"""Benchmark: one batched Lloyd iteration on one MI355X.

A step is one Lloyd iteration of the whole path (FlashAssign with the per-point minimum
distance and inertia partials, arg-sort, sort-inverse update with the refresh of the next
iteration's centroid operand), run by kmeans_fit on the headline workload (B=32, N=65536,
D=128, K=1024, bf16; inputs resident in HBM).  Every buffer (the fit's workspace included) is
allocated before the first measurement, so the GPU never idles between the measurements.
Order of the run:

  1. per-stage timings, first pass ("stages_ms_first"): `--stage-reps-first` (40) teacher-forced
     repetitions of the stage calls (row norms, centroid preparation, FlashAssign through
     kmeans_assign_prepared -- one kernel launch per call --, arg-sort, update), each bracketed by
     HIP events on the stream the stages run on.  A GPU that was idle during the setup runs its
     first tens of milliseconds of load at lower clocks (FlashAssign up to 30% slower at first,
     settling after 20-40 ms of load; see the design notes).  This pass (about 30 ms) takes that
     load, and its numbers show it; a timed fit after 10 repetitions instead ran 2-3% slower per
     iteration than the same fit repeated right after it.
  2. `--settle-iters` (60) untimed iterations as one fit, about 35 ms of the timed workload's own
     load.  Where the fit runs the batch as two half-batch chains (FlashAssign of one half beside
     the arg-sort and update of the other), its mix of MFMA and memory work settles the clocks at
     another point than the stage calls do: right after the first pass, the first timed fit ran
     2-4% slower per iteration than the fits after it, for 30-40 ms.
  3. `--warmup` untimed iterations as one fit;
  4. the timed region: exactly `--steps` iterations as one kmeans_fit call, bracketed by device
     synchronisations; `value` = its wall time / steps.  `--repeat` more timed fits follow and are
     reported beside it (not in `value`).
  5. per-stage timings, second pass ("stages_ms", the roofline and update figures).
  6. the oracle on a bounded sample on the host (cpu_baseline).

Prints one JSON line.  Other modes: `--copy-calib` (a plain device copy of known size, the
reference for scaling the FETCH_SIZE / WRITE_SIZE counters), `--summarize-trace CSV` (the
per-iteration summary of a rocprofv3 kernel trace of this script), `--context` /
`--context-pages` (the standard path the method replaces, at the headline shape / at the pages'
kernel-ratio shapes), `--plan-regret` (the K split of the plan against every alternative),
`--summarize-counters DIR` (HBM traffic and MFMA counter summaries from rocprofv3 runs), `--clock-probe`
(FlashAssign's shader clock and per-workgroup phase cycles from clock stamps).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import subprocess
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
    p.add_argument("--warmup", type=int, default=5, help="untimed iterations before the timed fit")
    p.add_argument("--repeat", type=int, default=2, help="further timed fits reported beside `value`")
    p.add_argument("--workload", default="headline_bf16")
    p.add_argument("--stage-reps", type=int, default=10, help="repetitions of the second stage pass")
    p.add_argument("--settle-iters", type=int, default=60,
                   help="untimed fit iterations before the warmup (the clocks settle under the fit's own load)")
    p.add_argument("--stage-reps-first", type=int, default=40,
                   help="repetitions of the first stage pass (about 30 ms of load: the clocks settle in it)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--clock-probe", nargs="*", metavar="B N D K [dtype [extra LDS]]",
                   help="run the FlashAssign phase probe (clock stamps per workgroup; headline shape by default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--streamed-source", default="auto", choices=["auto", "pinned", "pageable"],
                   help="streamed workload: x in pinned host blocks (kmeans_fit_blocks) or in pageable host "
                        "memory staged through a pinned buffer (kmeans_fit_staged); auto = pinned up to "
                        "64 GiB (the pinned memory the MI355X hosts measured allow one process), pageable above")
    p.add_argument("--copy-calib", action="store_true", help="run a plain 1 GiB device copy and exit")
    p.add_argument("--metric", default="l2", choices=["l2", "dot", "cosine"],
                   help="k-means variant: Lloyd (l2), dot-product or cosine (spherical) k-means")
    p.add_argument("--context", action="store_true",
                   help="also time the standard path in plain PyTorch (materialised distances + argmin, "
                        "scatter-add update) at the workload's shape")
    p.add_argument("--context-pages", action="store_true",
                   help="time the standard path against this path at the pages' kernel-ratio shapes and exit")
    p.add_argument("--plan-regret", action="store_true",
                   help="time kmeans_assign under the plan's K split and under other splits on a few shapes "
                        "(the regret of the analytic plan) and exit")
    p.add_argument("--summarize-counters", metavar="DIR",
                   help="summarise rocprofv3 --pmc runs of this script kept under DIR (fetch/, write/, cfetch/, "
                        "cwrite/, mfma/) into the HBM-traffic and MFMA summaries and exit")
    p.add_argument("--summarize-trace", metavar="CSV",
                   help="summarise a rocprofv3 kernel trace of this script (same --steps/--warmup/--stage-reps)")
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


# ------------------------------------------------------------------------------------------------
# host description and the oracle baseline
# ------------------------------------------------------------------------------------------------
def host_info():
    """CPU model, sockets, cores and threads (lscpu), and the BLAS numpy is built with."""
    info = {"cpu_count": os.cpu_count(), "machine": platform.machine()}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if ":" not in line:
                continue
            k, v = [t.strip() for t in line.split(":", 1)]
            if k in ("Model name", "Socket(s)", "Core(s) per socket", "Thread(s) per core", "CPU(s)"):
                info[k] = v
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        import numpy as np
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        info["numpy_blas"] = "%s %s" % (blas.get("name", "?"), blas.get("version", ""))
    except Exception:  # an older numpy without mode="dicts"
        info["numpy_blas"] = "unknown"
    return info


def cpu_baseline(w, x, c0, target_s, metric="l2"):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload: one iteration
    on the first `n` points of the first `p` problems against all K centroids, grown until it
    takes ~0.6 * target_s (or covers everything), then scaled to B*N points.  For Lloyd the
    iteration is the oracle's own steps, timed apart: the assignment, then the arg-sort and the
    update."""
    import numpy as np
    import oracle
    from oracle import similarity as sim
    from exact_lloyd_means_02_amd import workloads as W
    n, p = min(w.N, 2048), 1
    per_run = target_s / 3.0   # the sample is grown to about this, then timed three times

    def run_once():
        xs = W.storage_to_f64(x[:p, :n], w.dtype)
        cs = c0[:p].astype(np.float64)
        t0 = time.perf_counter()
        if metric == "l2":
            ct = oracle.centroid_operand(cs, w.dtype)
            a, _, _ = oracle.assign_batched(xs, ct)
            t1 = time.perf_counter()
            for b in range(p):
                oracle.argsort_ids(a[b], w.K)
                oracle.update(xs[b], a[b], cs[b])
        else:
            if metric == "cosine":
                xs = sim.round_to_dtype(sim.normalize_rows(xs), w.dtype)
            sim.similarity_iteration(xs, cs, metric, dtype=w.dtype, mode="modelled")
            t1 = time.perf_counter()
        return time.perf_counter() - t0, t1 - t0

    while True:
        dt, ta = run_once()
        if dt >= 0.6 * per_run or (n >= w.N and p >= w.B):
            break
        grow = max(1.5, min(8.0, 0.7 * per_run / max(dt, 1e-3)))
        if n < w.N:
            n = min(w.N, int(n * grow))
        else:
            p = min(w.B, max(p + 1, int(p * grow)))
    # the grown sample's run and two more: the median of the three
    runs = [(dt, ta), run_once(), run_once()]
    runs.sort()
    dt, ta = runs[1]
    scale = (w.B * w.N) / (p * n)
    out = {"value": round(dt * scale * 1e3, 3), "unit": "ms", "cores": oracle.threads(), "kind": "oracle",
           "sample": "one fp64 oracle iteration on %d of %d points (%d problem(s) x %d points, all K=%d "
                     "centroids), median of 3 runs %.2f s (runs %s s); scaled by %.1fx to the full "
                     "iteration" % (p * n, w.B * w.N, p, n, w.K, dt, ["%.2f" % r[0] for r in runs], scale),
           "runs_s": [round(r[0], 3) for r in runs],
           "host": host_info()}
    if metric == "l2":
        out["assign_ms"] = round(ta * scale * 1e3, 3)
        out["update_ms"] = round((dt - ta) * scale * 1e3, 3)
    return out


# ------------------------------------------------------------------------------------------------
# the standard path the method replaces (plain PyTorch; context only)
# ------------------------------------------------------------------------------------------------
def standard_assign(xt, c_master, chunk=None):
    """Materialised-distance assignment: the [B, N, K] matrix of x.c~ from a batched product with
    fp32 output (hipBLASLt), then ||c~||^2 - 2 x.c~ in fp32 and an argmin over K (the point norm is
    a constant per point).  c~ is the centroid master cast to the points' dtype.  `chunk` splits N
    (the matrix of one chunk is materialised at a time).  Returns int64 labels [B, N]."""
    import torch
    B, N, D = xt.shape
    c_lp = c_master.to(xt.dtype)
    c_lp_t = c_lp.transpose(1, 2).contiguous()          # [B, D, K], contiguous right operand
    cn = (c_lp.float() ** 2).sum(-1)                     # ||c~||^2 from the rounded centroids
    chunk = chunk or N
    out = torch.empty((B, N), dtype=torch.int64, device=xt.device)
    for lo in range(0, N, chunk):
        xs = xt[:, lo:lo + chunk].contiguous()
        try:
            dots = torch.bmm(xs, c_lp_t, out_dtype=torch.float32)
        except (RuntimeError, TypeError):
            dots = torch.bmm(xs, c_lp_t).float()
        dist = cn[:, None, :] - 2.0 * dots
        del dots
        out[:, lo:lo + chunk] = torch.argmin(dist, dim=-1)
        del dist
    return out


def standard_update(xt, labels, c_old, chunk=1 << 22):
    """Scatter-add update: every row added into its cluster's fp32 sum with atomics (index_add_),
    counts by bincount, c = sum / n, empty clusters keep their centroid.  Returns (c_new [B, K, D]
    fp32, counts [B, K])."""
    import torch
    B, N, D = xt.shape
    K = c_old.shape[1]
    flat = (labels + torch.arange(B, device=xt.device)[:, None] * K).reshape(-1)
    xf = xt.reshape(B * N, D)
    sums = torch.zeros(B * K, D, dtype=torch.float32, device=xt.device)
    for lo in range(0, B * N, chunk):
        sums.index_add_(0, flat[lo:lo + chunk], xf[lo:lo + chunk].float())
    cnt = torch.bincount(flat, minlength=B * K)
    newc = torch.where(cnt[:, None] > 0, sums / cnt.clamp(min=1)[:, None].float(), c_old.reshape(B * K, D))
    return newc.view(B, K, D), cnt.view(B, K)


def _event_ms(fn, reps, stream):
    import numpy as np
    import torch
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def standard_path(w, xt, c0t, reps, st):
    """The standard path at the workload's shape, beside this path's stage times `st`."""
    import torch
    from exact_lloyd_means_02_amd import flashkm as fk
    stream = torch.cuda.current_stream()
    lab = standard_assign(xt, c0t)
    ma = _event_ms(lambda: standard_assign(xt, c0t), reps, stream)
    mu = _event_ms(lambda: standard_update(xt, lab, c0t), reps, stream)
    prep = fk.kmeans_prepare_centroids(c0t, xt)
    a, _ = fk.kmeans_assign_prepared(xt, prep)
    agree = float((a.long() == lab).float().mean().item())
    return {"what": "plain PyTorch on the same GPU: bmm (fp32 out) + fp32 distances + argmin; index_add_ "
                    "scatter + bincount", "materialised_assign_ms": round(ma, 4), "scatter_update_ms": round(mu, 4),
            "assign_speedup": round(ma / st["assign"], 2),
            "update_speedup": round(mu / (st["argsort"] + st["update"]), 2), "label_agreement": agree}


def context_pages():
    """The pages' kernel-ratio shapes (paper summary, "Key claims" and "Results"): assignment at
    N = 2^20, K = 8192 (B = 1; D = 128, bf16: the pages state neither) and update at B = 1,
    N = 2^25, K = 4096 (D = 128, bf16, 8.6 GB of points), the standard path against this path on
    the same inputs, and the standard update's effective bandwidth (the pages quote about 50 GB/s
    for the scatter-atomic update under hot-cluster contention on H200)."""
    import numpy as np
    import torch
    from exact_lloyd_means_02_amd import flashkm as fk
    from exact_lloyd_means_02_amd import workloads as W
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    out = {"what": "standard path (plain PyTorch) vs this path at the pages' kernel-ratio shapes, one MI355X"}
    # assignment: B=1, N=2^20, K=8192, D=128 bf16 (GMM points, K seeded point picks)
    wa = W.small("headline_bf16", B=1, N=1 << 20, K=8192, M=8192)
    print("bench: context assign %s" % (wa,), file=sys.stderr, flush=True)
    x, c0, _ = W.make(wa)
    xt = W.to_torch(x, wa.dtype).to(dev)
    ct = torch.from_numpy(c0).to(dev)
    lab = standard_assign(xt, ct, chunk=1 << 18)
    t_std = _event_ms(lambda: standard_assign(xt, ct, chunk=1 << 18), 3, stream)
    prep = fk.kmeans_prepare_centroids(ct, xt)
    a, _ = fk.kmeans_assign_prepared(xt, prep)
    t_fa = _event_ms(lambda: fk.kmeans_assign_prepared(xt, prep, assign=a), 5, stream)
    out["assign"] = {"B": 1, "N": wa.N, "K": wa.K, "D": wa.D, "dtype": wa.dtype,
                     "standard_ms": round(t_std, 3), "flashassign_ms": round(t_fa, 3),
                     "speedup": round(t_std / t_fa, 2),
                     "label_agreement": float((a.long() == lab).float().mean().item()),
                     "pages_H200": "122.5 ms -> 5.8 ms (21.2x)"}
    del x, xt, lab, prep, a
    torch.cuda.empty_cache()
    # update: B=1, N=2^25, K=4096, D=128 bf16, Zipf(1.2) hot clusters (the skewed recipe)
    wu = W.small("skew_bf16_k4096", N=1 << 25)
    print("bench: context update %s" % (wu,), file=sys.stderr, flush=True)
    x, c0, _ = W.make(wu)
    xt = W.to_torch(x, wu.dtype).to(dev)
    del x
    ct = torch.from_numpy(c0).to(dev)
    prep = fk.kmeans_prepare_centroids(ct, xt)
    a, _ = fk.kmeans_assign_prepared(xt, prep)
    t_std_u = _event_ms(lambda: standard_update(xt, a.long(), ct), 3, stream)
    s_ids, s_idx, counts = fk.kmeans_argsort_ids(a, wu.K)
    cu = ct.clone()

    def ours():
        fk.kmeans_argsort_ids(a, wu.K, sorted_ids=s_ids, sorted_idx=s_idx, counts=counts)
        fk.kmeans_update(xt, s_ids, s_idx, counts, cu)
    ours()
    t_ours = _event_ms(ours, 5, stream)
    nbytes = W.nbytes(wu)
    out["update"] = {"B": 1, "N": wu.N, "K": wu.K, "D": wu.D, "dtype": wu.dtype, "points_GB": round(nbytes / 1e9, 2),
                     "largest_cluster_share": round(float(counts.max().item()) / wu.N, 3),
                     "standard_scatter_ms": round(t_std_u, 3), "argsort_plus_update_ms": round(t_ours, 3),
                     "speedup": round(t_std_u / t_ours, 2),
                     "standard_effective_GBs": round(nbytes / (t_std_u * 1e-3) / 1e9, 1),
                     "ours_effective_GBs": round(nbytes / (t_ours * 1e-3) / 1e9, 1),
                     "pages_H200": "up to 6.3x; scatter-atomic update about 50 GB/s"}
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------------------------------------
# the analytic plan against alternatives
# ------------------------------------------------------------------------------------------------
REGRET_SHAPES = [  # (workload recipe, B, N, D, K)
    ("headline_bf16", 1, 65536, 128, 1024), ("headline_bf16", 1, 65536, 128, 4096),
    ("headline_bf16", 4, 32768, 128, 1024), ("headline_bf16", 1, 16384, 128, 8192),
    ("batched_f16", 1, 262144, 64, 1024), ("headline_bf16", 32, 65536, 128, 1024)]
REGRET_SPLITS = [1, 2, 3, 4, 6, 8]


def plan_regret():
    """kmeans_assign (prepare + FlashAssign [+ key merge]) timed with HIP events, median of 10, under
    the plan's K split and under each alternative split (FLASHKM_ASSIGN_SPLIT, read by the plan at
    every call); regret = time of the plan's choice / best time - 1.  Per shape the GPU first runs
    the plan's split for about 30 ms (the clocks settle under load), then the splits are timed in two
    interleaved rounds and each keeps the lower of its two medians, so that no split is timed on a
    colder GPU than the others."""
    import torch
    from exact_lloyd_means_02_amd import flashkm as fk
    from exact_lloyd_means_02_amd import workloads as W
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []
    for name, B, N, D, K in REGRET_SHAPES:
        w = W.small(name, B=B, N=N, D=D, K=K)
        x, c0, _ = W.make(w)
        xt = W.to_torch(x, w.dtype).to(dev)
        ct = torch.from_numpy(c0).to(dev)
        os.environ.pop("FLASHKM_ASSIGN_SPLIT", None)
        plan = fk.kmeans_plan(fk.DT_CODES[w.dtype], B, N, D, K)
        ref = None
        times = {}
        a, _ = fk.kmeans_assign(xt, ct)
        t_one = _event_ms(lambda: fk.kmeans_assign(xt, ct, assign=a), 3, stream)
        _event_ms(lambda: fk.kmeans_assign(xt, ct, assign=a), max(3, int(30.0 / max(t_one, 1e-3))), stream)
        for _round in range(2):
            for sp in REGRET_SPLITS:
                os.environ["FLASHKM_ASSIGN_SPLIT"] = str(sp)
                got = fk.kmeans_plan(fk.DT_CODES[w.dtype], B, N, D, K)["assign_splits"]
                if got != sp:
                    continue                               # more shares than stages
                for _ in range(3):
                    fk.kmeans_assign(xt, ct, assign=a)
                t = _event_ms(lambda: fk.kmeans_assign(xt, ct, assign=a), 10, stream)
                times[sp] = min(t, times.get(sp, t))
                lab = a.cpu()
                if ref is None:
                    ref = lab
                assert torch.equal(lab, ref), "labels depend on the split"
        os.environ.pop("FLASHKM_ASSIGN_SPLIT", None)
        best = min(times, key=times.get)
        chosen = plan["assign_splits"]
        row = {"B": B, "N": N, "D": D, "K": K, "dtype": w.dtype, "point_tiles": plan["assign_wgs"],
               "plan_splits": chosen, "ms": {str(k): round(v, 4) for k, v in times.items()}, "best_splits": best,
               "regret": round(times[chosen] / times[best] - 1.0, 4)}
        print(json.dumps(row), flush=True)
        rows.append(row)
        del xt, ct
        torch.cuda.empty_cache()
    print(json.dumps({"plan_regret_max": max(r["regret"] for r in rows),
                      "plan_regret_mean": round(sum(r["regret"] for r in rows) / len(rows), 4)}), flush=True)


# ------------------------------------------------------------------------------------------------
# rocprofv3 counter summaries
# ------------------------------------------------------------------------------------------------
COUNTER_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc %s --output-format csv -d <out>/%s -o run -- "
               "python3 /root/repo/bench.py %s")
BENCH_ARGS_COUNTERS = "--steps 1 --warmup 1 --settle-iters 0 --stage-reps-first 2 --stage-reps 2 --repeat 0 --no-cpu-baseline"


def _counter_means(path):
    """{kernel name: {counter: mean value per dispatch}} from a rocprofv3 counter_collection CSV,
    over each kernel's dispatches of its largest grid: the whole-batch launches of the stage calls
    (a fit that runs two half-batch chains launches the same kernels over half the problems)."""
    import csv
    per, grid = {}, {}
    for r in csv.DictReader(open(path)):
        g = int(r.get("Grid_Size", 0) or 0)
        k = r["Kernel_Name"]
        if g < grid.get(k, 0):
            continue
        if g > grid.get(k, 0):
            grid[k] = g
            per = {key: v for key, v in per.items() if key[0] != k}
        key = (k, r["Counter_Name"])
        per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
        per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    out = {}
    for (k, c), d in per.items():
        out.setdefault(k, {})[c] = (sum(d.values()) / len(d), len(d))
    return out


def _short(name):
    return name.split("(")[0].replace("void ", "").replace("fkm::", "")


def summarize_counters(root):
    """HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE (each its own run), scaled by what the
    same counters read for a plain 1 GiB device copy, against the algorithmic bytes of the
    headline shape; MFMA counters of FlashAssign.  Prints the markdown summary, then writes the
    FlashAssign traffic file bench.py reads (profiles/assign_small_d_headline_bf16_traffic.txt)."""
    import glob
    import numpy as np

    def load(sub):
        f = glob.glob(os.path.join(root, sub, "**", "*counter_collection.csv"), recursive=True)
        return _counter_means(f[0]) if f else {}
    fetch, write, cfetch, cwrite, mfma = (load(s) for s in ("fetch", "write", "cfetch", "cwrite", "mfma"))
    copy = [k for k in cfetch if "copyBuffer" in k][0]
    fscale = (1 << 30) / 1024 / cfetch[copy]["FETCH_SIZE"][0]
    wscale = (1 << 30) / 1024 / cwrite[[k for k in cwrite if "copyBuffer" in k][0]]["WRITE_SIZE"][0]
    B, N, D, K, s = 32, 65536, 128, 1024, 2
    KT = 32
    algo = {"assign_small_d_kernel": B * N * D * s + B * KT * 32 * D * s + 4 * B * KT * 32 + 8 * B * N,
            "sort_hist_kernel": 4 * B * N, "sort_scatter_kernel": 16 * B * N,
            "upd_segsum_kernel": B * N * D * s + 8 * B * N + B * K * D * (4 + 4 + s) + 4 * B * K}
    lines = ["# HBM traffic per dispatch and FlashAssign MFMA counters: headline workload "
             "(B=32, N=65536, D=128, K=1024, bf16)", "",
             "Each counter set is its own run (the commands below; `<out>` = a scratch directory).  Values are",
             "per dispatch, averaged over each kernel's dispatches of its largest grid: the whole-batch stage",
             "calls (the fit's half-batch launches, which share the chip with the other half, are left out).", ""]
    for c, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        lines.append("    " + COUNTER_CMD % (c, sub, BENCH_ARGS_COUNTERS))
    for c, sub in (("FETCH_SIZE", "cfetch"), ("WRITE_SIZE", "cwrite")):
        lines.append("    " + COUNTER_CMD % (c, sub, "--copy-calib"))
    lines.append("    " + COUNTER_CMD % ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU "
                                       "GRBM_GUI_ACTIVE", "mfma", BENCH_ARGS_COUNTERS))
    lines += ["", "Scale (a plain 1 GiB device copy): FETCH_SIZE x %.4f, WRITE_SIZE x %.4f give bytes." % (fscale, wscale),
              "", "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes | algorithmic bytes | ratio |",
              "|---|---:|---:|---:|---:|---:|---:|"]
    assign_traffic = None
    for k in sorted(fetch, key=lambda n: -fetch[n]["FETCH_SIZE"][0]):
        f, n = fetch[k]["FETCH_SIZE"]
        wv = write.get(k, {}).get("WRITE_SIZE", (float("nan"), 0))[0]
        scaled = (f * fscale + wv * wscale) * 1024
        a = next((v for key, v in algo.items() if key in k), None)
        lines.append("| `%s` | %d | %.1f | %.1f | %.4g | %s | %s |" % (
            _short(k), n, f, wv, scaled, "%.4g" % a if a else "-", "%.3f" % (scaled / a) if a else "-"))
        if "assign_small_d_kernel" in k:
            assign_traffic = (f, wv, scaled, n)
    lines += ["", "Algorithmic bytes: assign = x (B N D 2) + prepared centroids (B KT 32 D 2) + their half-norms "
              "(4 B KT 32) + labels and point norms (8 B N); hist = labels; scatter = labels and indices read, sorted "
              "ids and indices written (16 B N); segsum = gathered rows + sorted ids and indices (8 B N) + old and new "
              "centroids (f32) + refreshed operand (2 bytes) + half-norms."]
    for k, v in mfma.items():
        if "assign_small_d_kernel" not in k:
            continue
        mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", (0, 0))[0]
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", (0, 0))[0]
        gui = v.get("GRBM_GUI_ACTIVE", (0, 0))[0]
        valu = v.get("SQ_INSTS_VALU", (0, 0))[0]
        flops = 2.0 * B * N * K * D
        lines += ["", "FlashAssign MFMA counters (%d dispatches): SQ_INSTS_VALU_MFMA_MOPS_BF16 %.4g (x 512 = %.4g FLOP; "
                  "2 B N K D = %.4g), SQ_VALU_MFMA_BUSY_CYCLES %.4g, GRBM_GUI_ACTIVE %.4g, SQ_INSTS_VALU %.4g "
                  "(%.1f per 32-centroid tile and wave; the MFMA count per tile and wave is 16)." % (
                      v["SQ_INSTS_VALU_MFMA_MOPS_BF16"][1], mops, mops * 512, flops, busy, gui, valu,
                      valu / (B * N / 64 * KT) if valu else 0.0),
                  "SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE = %.1f (both summed over their counting units; the "
                  "MFMA fraction of peak is taken from time instead: 2 B N K D / kernel time / 2.5 PFLOP/s)." % (
                      busy / gui if gui else 0.0)]
    print("\n".join(lines))
    if assign_traffic:
        f, wv, scaled, n = assign_traffic
        txt = ["# FlashAssign (small-D kernel) HBM traffic, headline workload B=32 N=65536 D=128 K=1024 bf16",
               "# read by bench.py for roofline.traffic; valid only for the kernel source whose hash is below",
               "k_assign.hip + build.py sha256[:16]: %s" % assign_source_hash(),
               "fetch command: " + COUNTER_CMD % ("FETCH_SIZE", "fetch", BENCH_ARGS_COUNTERS),
               "write command: " + COUNTER_CMD % ("WRITE_SIZE", "write", BENCH_ARGS_COUNTERS),
               "copy fetch command: " + COUNTER_CMD % ("FETCH_SIZE", "cfetch", "--copy-calib"),
               "copy write command: " + COUNTER_CMD % ("WRITE_SIZE", "cwrite", "--copy-calib"),
               "summary command: python3 bench.py --summarize-counters <out>",
               "FETCH_SIZE KiB per dispatch: %.1f (%d dispatches)" % (f, n),
               "WRITE_SIZE KiB per dispatch: %.1f" % wv,
               "fetch scale (1 GiB copy): %.4f" % fscale, "write scale (1 GiB copy): %.4f" % wscale,
               "traffic bytes per launch: %d" % round(scaled),
               "algorithmic bytes per launch: %d" % algo["assign_small_d_kernel"]]
        open(TRAFFIC_FILE, "w").write("\n".join(txt) + "\n")


# ------------------------------------------------------------------------------------------------
# rocprofv3 kernel-trace summary
# ------------------------------------------------------------------------------------------------
KERNEL_TAGS = [("assign_small_d", "assign"), ("assign_split_d", "assign"), ("sort_hist", "hist"),
               ("sort_scatter", "scatter"), ("sort_rowscan", "rowscan"), ("segment_counts", "segcounts"),
               ("upd_segsum", "segsum"), ("upd_prologue", "prologue"), ("prep_centroids", "prep"),
               ("rows_short", "rownorm"), ("row_norms", "rownorm"), ("fill_i32", "fill"),
               ("sum_f64_rows", "sumrows"), ("copyBuffer", "copy"), ("upd_finalize", "finalize")]


def summarize_trace(path, args):
    """Per-iteration summary of a `rocprofv3 --kernel-trace` CSV of this script: the FlashAssign
    launches of the per-stage timings (the launches `roofline` averages) and the timed fit's
    iterations.  A fit that runs two half-batch chains has two hardware queues (the FlashAssign
    launches of both chains on one, their arg-sorts and updates on the other); an iteration runs
    from one FlashAssign launch of the first chain to its next, and its kernel times add both
    chains' kernels (which overlap, so they may exceed the iteration's span)."""
    import csv
    import numpy as np
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))

    def tag(n):
        for k, t in KERNEL_TAGS:
            if k in n:
                return t
        return n[:24]
    seq = [(tag(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r.get("Queue_Id", "0"))
           for r in rows]
    names = [s[0] for s in seq]
    # stage calls: row norms, prep, assign, in two passes of 1 + R triples (the first triple of a
    # pass is its untimed priming call); `roofline` averages the second pass
    triples = [(seq[i + 2][2] - seq[i + 2][1]) / 1e3 for i in range(len(seq) - 2)
               if names[i] == "rownorm" and names[i + 1] == "prep" and names[i + 2] == "assign"]
    R1, R = args.stage_reps_first, args.stage_reps
    first_pass = triples[1:1 + R1]
    stage_assign = triples[2 + R1:2 + R1 + R] if len(triples) >= 2 + R1 + R else first_pass
    # fits: each chain starts with prep then fill on its queue (two chains: two such starts within
    # a millisecond); a fit's kernels run to the next fit or stage call (prep or row norms).  Its
    # inertia sums, fills and copies to the host are not counted in the iterations.
    starts = []
    for i in range(len(seq)):
        if names[i] != "prep":
            continue
        nxt = next((j for j in range(i + 1, len(seq)) if seq[j][3] == seq[i][3]), None)
        if nxt is not None and names[nxt] == "fill":
            if starts and seq[i][1] - seq[starts[-1]][1] < 1000000:
                continue  # the second chain's start of the same fit
            starts.append(i)
    fits = []
    for fi, i in enumerate(starts):
        end = starts[fi + 1] if fi + 1 < len(starts) else len(seq)
        ks = []
        for j in range(i, end):
            if names[j] == "rownorm" or (names[j] == "prep" and j > i + 4 and not ks == []
                                         and names[j - 1] not in ("fill", "prep")):
                break
            if names[j] not in ("sumrows", "fill", "copy", "prep"):
                ks.append(seq[j])
        if not ks:
            continue
        # chains: the prep launches before the first FlashAssign; an iteration has one FlashAssign
        # per chain, on one queue or on one queue per chain
        first_a = next(j for j in range(i, end) if names[j] == "assign")
        nch = max(1, sum(1 for j in range(i, first_a) if names[j] == "prep"))
        qa = set(k[3] for k in ks if k[0] == "assign")
        per_it = max(1, nch // len(qa))
        q0 = next(k[3] for k in ks if k[0] == "assign")
        its, cur, na = [], [], 0
        for k in ks:
            if k[0] == "assign" and k[3] == q0:
                if cur and na % per_it == 0:
                    its.append(cur)
                    cur = []
                na += 1
            cur.append(k)
        if cur:
            its.append(cur)
        fits.append((its, nch))
    lines = ["# rocprofv3 kernel trace summary (bench.py --summarize-trace)", "source: %s" % os.path.basename(path)]
    lines.append("FlashAssign launches of the first stage pass: %d, mean %.2f us" % (
        len(first_pass), np.mean(first_pass)))
    lines.append("FlashAssign launches of the second stage pass (the roofline's): %d, mean %.2f us, median %.2f us, "
                 "min %.2f us" % (len(stage_assign), np.mean(stage_assign), np.median(stage_assign),
                                  np.min(stage_assign)))
    flops = 2.0 * 32 * 65536 * 1024 * 128
    lines.append("  2*B*N*K*D / mean / 2.5 PFLOP/s = %.4f (headline shape)" % (flops / (np.mean(stage_assign) * 1e-6)
                                                                              / 2.5e15))
    lines.append("fits found: %d (iterations: %s; chains: %s)" % (
        len(fits), [len(f[0]) for f in fits], [f[1] for f in fits]))
    ti = (1 if getattr(args, "settle_iters", 0) > 0 else 0) + (1 if args.warmup > 0 else 0)
    if len(fits) > ti:
        timed, nchains = fits[ti]
        lines.append("timed fit (fit %d): %d iterations, %d chain(s)" % (ti + 1, len(timed), nchains))
        lines.append("  it  assign   hist  scatter  segsum | kernels   span (us)")
        tot_k, tot_span = 0.0, 0.0
        per = {}
        for t, it in enumerate(timed):
            d = {}
            for n, s0, e0, _ in it:
                d[n] = d.get(n, 0.0) + (e0 - s0) / 1e3
                per.setdefault(n, []).append((e0 - s0) / 1e3)
            k = sum(d.values())
            end = timed[t + 1][0][1] if t + 1 < len(timed) else max(e0 for _, _, e0, _ in it)
            span = (end - it[0][1]) / 1e3
            tot_k += k
            tot_span += span
            lines.append("  %2d %7.1f %6.1f %7.1f %7.1f | %7.1f %7.1f" % (
                t, d.get("assign", 0), d.get("hist", 0), d.get("scatter", 0), d.get("segsum", 0), k, span))
        n = len(timed)
        lines.append("  per iteration: kernels %.1f us (both chains added), span %.1f us" % (tot_k / n, tot_span / n))
        lines.append("  per kernel launch mean: " + ", ".join("%s %.1f" % (k, np.mean(v)) for k, v in per.items()))
    print("\n".join(lines))


# ------------------------------------------------------------------------------------------------
# the streamed (pinned host) workload
# ------------------------------------------------------------------------------------------------
def pinned_blocks(w, block_points=1 << 27):
    """The workload's points in pinned host blocks of `block_points` rows (the last one shorter),
    generated in place (B = 1).  Returns (torch tensors, numpy views)."""
    import torch
    from exact_lloyd_means_02_amd import workloads as W
    sizes = [min(block_points, w.N - lo) for lo in range(0, w.N, block_points)]
    tb = [torch.empty((n, w.D), dtype=W.torch_dtype(w.dtype), pin_memory=True) for n in sizes]
    # numpy views sharing the pinned memory (bf16 as its uint16 bit patterns)
    nb = [t.view(torch.int16).numpy().view("uint16") if w.dtype == "bf16" else t.numpy() for t in tb]
    W.generate_points(w, out_blocks=nb)
    return tb, nb


PINNED_CAP_BYTES = 64 << 30   # pinned host memory the MI355X hosts measured allow one process


def bench_streamed(args, w):
    """Host-resident workload, streamed in chunks: x in pinned host memory (blocks of 2^27
    points, so no single allocation exceeds 16 GiB at D = 64 fp16) through kmeans_fit_blocks, or
    (above the pinned cap, e.g. the stated N = 2^30, 128 GiB) in pageable host memory through
    kmeans_fit_staged and its pinned staging buffer.  Reports ms per Lloyd iteration, the plain
    host->device copy rate of the same chunks and the GPU time of one iteration on one
    device-resident chunk (the legs the pipeline overlaps)."""
    import torch
    from exact_lloyd_means_02_amd import flashkm as fk
    from exact_lloyd_means_02_amd import workloads as W

    n_override = int(os.environ.get("BENCH_STREAMED_N", "0"))
    if n_override:
        w = W.small(w.name, N=n_override)
    steps = args.steps if args.steps != 20 else w.iters
    pageable = args.streamed_source == "pageable" or (args.streamed_source == "auto"
                                                      and W.nbytes(w) > PINNED_CAP_BYTES)
    t0 = time.perf_counter()
    dev = torch.device("cuda:0")
    if pageable:
        print("bench: generating %.1f GiB of points in pageable host memory for %s" % (
            W.nbytes(w) / 2 ** 30, w), file=sys.stderr, flush=True)
        x, c0, _ = W.make(w)
        tb = [W.to_torch(x, w.dtype)[0]]          # one pageable [N, D] view
        xp = W.to_torch(x, w.dtype)
    else:
        print("bench: allocating %.1f GiB of pinned host memory (blocks of 2^27 points) for %s" % (
            W.nbytes(w) / 2 ** 30, w), file=sys.stderr, flush=True)
        tb, nb = pinned_blocks(w)
        c0 = W.init_centroids_blocks(w, nb)
    c0t = torch.from_numpy(c0).to(dev)
    print("bench: generated in %.1f s (%s)" % (time.perf_counter() - t0,
                                               "pageable" if pageable else "%d pinned blocks" % len(tb)),
          file=sys.stderr, flush=True)

    # leg 1: plain chunked host->device copies (two staging buffers, one stream)
    chunk = w.chunk
    bufs = [torch.empty((chunk, w.D), dtype=tb[0].dtype, device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    q = 0
    for t in tb:
        for lo in range(0, t.shape[0], chunk):
            n = min(chunk, t.shape[0] - lo)
            bufs[q & 1][:n].copy_(t[lo:lo + n], non_blocking=True)
            q += 1
    torch.cuda.synchronize()
    h2d_s = time.perf_counter() - t1
    # leg 2: one iteration on one device-resident chunk
    xc = tb[0][:chunk].to(dev)[None]
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
    stage = fk.stage_buffer(fk.dtype_code(tb[0]), w.B, w.N, w.D, w.K, chunk) if pageable else None
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    if pageable:
        _, inertia, done = fk.kmeans_fit_staged(xp, c, steps, 0.0, chunk_points=chunk, stage=stage,
                                                want_assign=False)
    else:
        _, inertia, done = fk.kmeans_fit_blocks(tb, c, steps, 0.0, chunk_points=chunk, want_assign=False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t3) * 1e3 / steps
    nchunks = -(-w.N // chunk)
    flops = 2.0 * w.B * w.N * w.K * w.D
    out = {
        "metric": "ms per Lloyd iteration (%s, x streamed from %s host memory)" % (
            w.name, "pageable (staged through pinned buffers)" if pageable else "pinned"),
        "value": round(ms, 2), "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": steps,
        "warmup": 0, "ms_per_step": round(ms, 2), "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "D": w.D, "K": w.K, "chunk_points": chunk,
                   "chunks": nchunks, "host_blocks": len(tb), "iters": steps,
                   "inputs": "pageable host, pinned staging" if pageable else "pinned host"},
        "assign_tflops_effective": round(flops / (ms * 1e-3) / 1e12, 1),
        "h2d_GBs_plain_copy": round(W.nbytes(w) / h2d_s / 1e9, 1),
        "h2d_ms_per_iteration": round(h2d_s * 1e3, 1),
        "one_chunk_device_iteration_ms": round(chunk_ms, 2),
        "compute_ms_per_iteration_est": round(chunk_ms * nchunks, 1),
        "inertia": [float(v) for v in inertia[:, 0]],
    }
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------------------------------------
# the device-resident workloads
# ------------------------------------------------------------------------------------------------
def stage_times(fk, w, xt, c0t, reps, metric, stream):
    """Teacher-forced stage calls from c0, each bracketed by HIP events on `stream`; returns the
    medians (ms) and the FlashAssign launches' individual times."""
    import numpy as np
    import torch
    xn = fk.kmeans_row_norms(xt)
    prep = fk.kmeans_prepare_centroids(c0t, xt, metric=metric)
    a, md = fk.kmeans_assign_prepared(xt, prep, x_norms=xn, want_min_dist=True)
    s_ids, s_idx, counts = fk.kmeans_argsort_ids(a, w.K)
    cu = c0t.clone()
    torch.cuda.synchronize()
    names = ["row_norms", "prepare", "assign", "argsort", "update"]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    times = {k: [] for k in names}
    for _ in range(reps):
        cu.copy_(c0t)
        ev[0].record(stream)
        fk.kmeans_row_norms(xt, out=xn)
        ev[1].record(stream)
        fk.kmeans_prepare_centroids(c0t, xt, out=prep.buf, metric=metric)
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
    # plain-Python medians: a first np.median call spends tens of milliseconds of host time, which
    # would leave the GPU idle between the measurements
    return {k: float(statistics.median(v)) for k, v in times.items()}, times["assign"]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.copy_calib:
        copy_calib()
        return
    if args.context_pages:
        context_pages()
        return
    if args.plan_regret:
        plan_regret()
        return
    if args.clock_probe is not None:
        # the probe executable built beside the library (its own compilation of the assign source
        # with clock stamps); it prints its own summary
        exe = os.path.join(ROOT, "exact_lloyd_means_02_amd", "probe_assign_clock")
        if not os.path.exists(exe):
            print("bench.py: %s is not built (build the package first)" % exe, file=sys.stderr)
            sys.exit(2)
        sys.exit(subprocess.call([exe] + list(args.clock_probe)))
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
    # the fit's workspace and label buffer, allocated now (the binding caches the workspace)
    dt = fk.dtype_code(xt)
    op = {"l2": fk.KM_OP_FIT, "dot": fk.KM_OP_FIT_DOT, "cosine": fk.KM_OP_FIT_COSINE}[args.metric]
    fk.workspace(op, dt, w.B, w.N, w.D, w.K, dev, stream=fk._stream(c, None))
    labels = torch.empty((w.B, w.N), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def fit(iters):
        if args.metric == "l2":
            return fk.kmeans_fit(xt, c, iters, 0.0, assign=labels)
        return fk.kmeans_fit_metric(xt, c, args.metric, iters, 0.0, assign=labels)

    # ---- 1. per-stage times, first pass (HIP events on the stages' stream), teacher forced from c0
    st_first, _ = stage_times(fk, w, xt, c0t, args.stage_reps_first, args.metric, stream)

    # ---- 2. settle (untimed): the fit's own load for about 35 ms
    if args.settle_iters > 0:
        fit(args.settle_iters)
        c.copy_(c0t)
    # ---- 3. warmup (untimed): W iterations
    if args.warmup > 0:
        fit(args.warmup)
    torch.cuda.synchronize()

    # ---- 4. timed: exactly `steps` iterations in one fit (then `repeat` more, reported apart)
    runs = []
    for r in range(1 + max(0, args.repeat)):
        c.copy_(c0t)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, inertia, done = fit(args.steps)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        assert done == args.steps
        runs.append((t1 - t0) * 1e3 / args.steps)
        if r == 0:
            inertia_first = inertia.copy()
            # every squared distance is positive on these inputs; a zero is a value never written
            assert args.metric != "l2" or bool(np.all(inertia > 0)), "fit returned a non-positive inertia"
        else:  # the same start, the same fixed-order sums: the same values to the bit
            assert np.array_equal(inertia, inertia_first), "repeat fit's inertia differs from the first"
    ms_per_step = runs[0]
    print("bench: %d iterations in %.3f ms (repeats: %s ms per iteration)" % (
        args.steps, ms_per_step * args.steps, ["%.4f" % v for v in runs[1:]]), file=sys.stderr, flush=True)

    # ---- 5. per-stage times, second pass
    st, assign_launches = stage_times(fk, w, xt, c0t, args.stage_reps, args.metric, stream)

    flops, abytes, ubytes = algorithmic(w)
    peak = PEAK_TFLOPS[w.dtype]
    assign_ms = float(np.mean(assign_launches))      # the mean the kernel trace reproduces
    assign_tflops = flops / (assign_ms * 1e-3) / 1e12
    upd_ms = st["argsort"] + st["update"]
    upd_gbs = ubytes / (upd_ms * 1e-3) / 1e9

    # the assign's bound: the MFMA floor (flops / peak) or the HBM floor (algorithmic bytes / peak
    # bandwidth), whichever is longer; K below about 300 makes it HBM-bound
    if abytes / (PEAK_HBM_GBS * 1e9) > flops / (peak * 1e12):
        assign_gbs = abytes / (assign_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(assign_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(assign_gbs / PEAK_HBM_GBS, 4),
                "mfma": {"achieved": round(assign_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(assign_tflops / peak, 4)}}
    else:
        roof = {"bound": "mfma", "achieved": round(assign_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(assign_tflops / peak, 4)}
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
        "repeat_ms_per_step": [round(v, 4) for v in runs[1:]],
        "roofline": dict(roof, **{
                     "traffic": measured_traffic(w.name),
                     "kernel": "FlashAssign (%s) kernel, one launch per kmeans_assign_prepared call" % (
                         "small-D" if fk.kmeans_plan(fk.dtype_code(xt), w.B, w.N, w.D, w.K)["path"] == 0 else "split-D"),
                     "kernel_ms": round(assign_ms, 4), "kernel_ms_median": round(st["assign"], 4),
                     "launches": len(assign_launches), "flop_per_launch": flops,
                     "algorithmic_bytes_per_launch": abytes}),
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "stages_ms_first": {k: round(v, 4) for k, v in st_first.items()},
        "update": {"bound": "hbm", "achieved": round(upd_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(upd_gbs / PEAK_HBM_GBS, 4), "bytes_per_iter": ubytes,
                   "stages": "kmeans_argsort_ids + kmeans_update"},
        ("inertia_last" if args.metric == "l2" else "similarity_last"): [float(v) for v in inertia_first[-1][:2]],
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
