#!/usr/bin/env python3
"""Bench: batch-one N:M sparse matrix-vector product on one MI355X.

Metric: effective HBM GB/s of nm_spmv (bytes the method must move: values + masks + x
+ y), its fraction of the 8 TB/s HBM3E peak, and the speedup over the hand-written
dense fp16 GEMV on the same GPU, on seeded synthetic layers with the shapes of the
evaluated models' projections.

A step is one pass of the sparse product over every layer of the workload (each N:M
pattern of each projection shape), with the weights already packed and resident in
HBM. Each step reads the next copy of every layer from a rotating pool of distinct
copies (>= 1 GiB of other data between two reads of the same bytes), so the weights
come from HBM and not from the last-level cache.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "N:M SpMV effective HBM GB/s (% of peak) + speedup vs dense GEMV, batch 1"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak, 8 TB/s
SPMV_SRC = os.path.join(ROOT, "semi_structured_sparse_amd", "csrc", "nm_spmv.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "nm_spmv_counters.txt")
WORKLOAD_BY_NAME = {"llama8b": 2, "qwen3": 3, "llama70b": 4}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", choices=sorted(WORKLOAD_BY_NAME), default="llama8b")
    ap.add_argument("--pool-gib", type=float, default=1.0,
                    help="minimum bytes read between two reads of the same copy")
    ap.add_argument("--cpu-rows-frac", type=float, default=0.125,
                    help="fraction of each layer's rows the CPU oracle baseline processes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--patterns", default="", help="restrict to patterns, e.g. 2:4,16:32")
    return ap.parse_args()


def alg_bytes_sparse(R, C, N, M):
    return 2 * R * C * N // M + 4 * R * C // 32 + 2 * C + 2 * R


def alg_bytes_dense(R, C):
    return 2 * R * C + 2 * C + 2 * R


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_traffic(kernel_name: str):
    """HBM bytes per launch of `kernel_name` from the committed counter summary, or None
    when there is none or the kernel source changed since the counters were taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != source_sha(SPMV_SRC):
        return None
    if kv.get("kernel") != kernel_name or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the sparse product of one layer is measured on one GPU; sharding is design-only)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import semi_structured_sparse_amd as nm
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nm.lib()  # fail loudly if the HIP library is missing

    cfg = WORKLOAD_BY_NAME[args.workload]
    wl = synth.WORKLOADS[cfg]
    pats = [tuple(p) for p in wl["patterns"]]
    if args.patterns:
        want = {tuple(int(v) for v in p.split(":")) for p in args.patterns.split(",")}
        pats = [p for p in pats if p in want]

    # ------------------------------------------------------------------ inputs (untimed)
    layers = []   # sparse layers: dict(name, R, C, N, M, values[], masks[], x, y, bytes, cpu rows)
    dense = {}    # shape -> dict(W[], x, y, bytes)
    t_gen = time.time()
    for li, (name, R, C) in enumerate(wl["layers"]):
        for pat in pats:
            N, M = pat
            ws, xs = synth.weight_seed(cfg, li, pat), synth.x_seed(cfg, li, pat)
            W = synth.weight(R, C, ws)
            x = synth.activation(C, xs)
            Wd = torch.from_numpy(W).to(dev)
            xd = torch.from_numpy(x).to(dev)
            values, masks = nm.nm_pack(Wd, N, M)
            ncpu = max(1, int(math.ceil(R * args.cpu_rows_frac)))
            layers.append(dict(name=name, R=R, C=C, N=N, M=M, seed_w=ws, seed_x=xs,
                               values=[values], masks=[masks], x=xd, x_host=x,
                               W_cpu=W[:ncpu].copy(), y=torch.empty(R, dtype=torch.float16, device=dev),
                               bytes=alg_bytes_sparse(R, C, N, M)))
            if (R, C) not in dense:
                dense[(R, C)] = dict(name=name, R=R, C=C, W=[Wd], x=xd,
                                     y=torch.empty(R, dtype=torch.float16, device=dev),
                                     bytes=alg_bytes_dense(R, C))
            else:
                del Wd
            del W
    torch.cuda.synchronize()
    log(f"generated and packed {len(layers)} layers in {time.time() - t_gen:.1f}s")

    pool_bytes = args.pool_gib * (1 << 30)
    step_sparse = sum(L["bytes"] for L in layers)
    step_dense = sum(D["bytes"] for D in dense.values())
    P_s = max(2, math.ceil(pool_bytes / step_sparse))
    P_d = max(2, math.ceil(pool_bytes / step_dense))
    for L in layers:
        for _ in range(P_s - 1):
            L["values"].append(L["values"][0].clone())
            L["masks"].append(L["masks"][0].clone())
    for D in dense.values():
        for _ in range(P_d - 1):
            D["W"].append(D["W"][0].clone())
    torch.cuda.synchronize()
    log(f"pools: sparse {P_s} copies x {step_sparse / 1e6:.1f} MB, dense {P_d} copies x {step_dense / 1e6:.1f} MB")

    lib = nm.lib()
    main_stream = torch.cuda.current_stream(dev)

    # Raw C-ABI calls with pre-built arguments: the Python binding's checks already ran
    # during packing and warm-up; in the timed regions only the library call remains.
    sp_args = [[(L["values"][c].data_ptr(), L["masks"][c].data_ptr(), L["x"].data_ptr(), L["y"].data_ptr(),
                 L["R"], L["C"], L["N"], L["M"]) for c in range(P_s)] for L in layers]
    dense_list = list(dense.values())
    dn_args = [[(D["W"][c].data_ptr(), D["x"].data_ptr(), D["y"].data_ptr(), D["R"], D["C"])
                for c in range(P_d)] for D in dense_list]

    def sparse_step(k, sp, evs=None):
        c = k % P_s
        for i in range(len(layers)):
            if evs is not None:
                evs[i][0].record()
            st = lib.nm_spmv(*sp_args[i][c], sp)
            if st:
                raise RuntimeError(f"nm_spmv: {nm.status_string(st)}")
            if evs is not None:
                evs[i][1].record()

    def dense_step(k, sp, evs=None):
        c = k % P_d
        for i in range(len(dense_list)):
            if evs is not None:
                evs[i][0].record()
            st = lib.nm_gemv_dense(*dn_args[i][c], sp)
            if st:
                raise RuntimeError(f"nm_gemv_dense: {nm.status_string(st)}")
            if evs is not None:
                evs[i][1].record()

    # ------------------------------------------------------------------ read ceiling probe
    probe_buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(3):
        nm.nm_probe_read(probe_buf, sink)
    torch.cuda.synchronize()
    pt = []
    for _ in range(10):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        nm.nm_probe_read(probe_buf, sink)
        b_.record()
        torch.cuda.synchronize()
        pt.append(a_.elapsed_time(b_))
    probe_ms = statistics.median(pt)
    read_ceiling = probe_buf.numel() / (probe_ms * 1e-3) / 1e9
    log(f"read ceiling {read_ceiling:.0f} GB/s")

    def head_start(ms):
        """Queue about `ms` of untimed GPU work so that the launches that follow are all
        enqueued before the GPU reaches them: their timing is then the GPU's, never the
        host's launch overhead."""
        for _ in range(max(1, int(math.ceil(ms / probe_ms)))):
            nm.nm_probe_read(probe_buf, sink)

    def timed_graph(step_fn, K, W_):
        """Warm-up, then K steps captured in one HIP graph and replayed between events."""
        sp = main_stream.cuda_stream
        for k in range(W_):
            step_fn(k, sp)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for k in range(K):
                step_fn(W_ + k, cs)
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del g
        return start.elapsed_time(end), wall

    def timed_events(step_fn, K, n_launch, per_launch):
        """K eager steps after a GPU head start; with per_launch, an event pair around
        every launch (launch durations as the GPU sees them)."""
        sp = main_stream.cuda_stream
        evs = None
        if per_launch:
            evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                    for _ in range(n_launch)] for _ in range(K)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        head_start(25.0)
        start.record()
        for k in range(K):
            step_fn(k, sp, evs[k] if per_launch else None)
        end.record()
        torch.cuda.synchronize()
        per = None
        if per_launch:
            per = [[evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(K)] for i in range(n_launch)]
        return start.elapsed_time(end), per

    # ------------------------------------------------------------------ timed regions
    K, Wm = args.steps, args.warmup
    ms_s, wall_s = timed_graph(sparse_step, K, Wm)
    ms_d, wall_d = timed_graph(dense_step, K, Wm)
    ms_s_eager, _ = timed_events(sparse_step, K, len(layers), False)
    ms_s_ev, per_s = timed_events(sparse_step, K, len(layers), True)
    ms_d_ev, per_d = timed_events(dense_step, K, len(dense_list), True)
    torch.cuda.synchronize()
    del probe_buf

    value = step_sparse * K / (ms_s * 1e-3) / 1e9
    dense_gbps = step_dense * K / (ms_d * 1e-3) / 1e9
    # speedup over the same (shape, pattern) launches: each dense shape stands for the
    # patterns measured at that shape
    pats_per_shape = len(layers) / len(dense_list)
    speedup = (ms_d * pats_per_shape) / ms_s
    log(f"sparse {value:.0f} GB/s ({value / HBM_PEAK_GBPS:.1%}), dense {dense_gbps:.0f} GB/s, "
        f"speedup {speedup:.3f}x, {ms_s / K * 1e3:.1f} us/step (graph); eager {ms_s_eager / K * 1e3:.1f}, "
        f"with launch events {ms_s_ev / K * 1e3:.1f} us/step")

    per_layer = []
    dense_med = {}
    for i, D in enumerate(dense_list):
        dense_med[(D["R"], D["C"])] = statistics.median(per_d[i])
    kern_bytes, kern_ms = {}, {}
    for i, L in enumerate(layers):
        med = statistics.median(per_s[i])
        mean = statistics.fmean(per_s[i])
        kname = f"nm_spmv_kernel<{L['N']},{L['M']}>"
        kern_bytes[kname] = kern_bytes.get(kname, 0) + L["bytes"] * K
        kern_ms[kname] = kern_ms.get(kname, 0.0) + mean * K
        dm = dense_med[(L["R"], L["C"])]
        per_layer.append({"layer": L["name"], "shape": f"{L['R']}x{L['C']}", "pattern": f"{L['N']}:{L['M']}",
                          "us": round(med * 1e3, 2), "GBps": round(L["bytes"] / (med * 1e-3) / 1e9, 1),
                          "pct_peak": round(L["bytes"] / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "dense_us": round(dm * 1e3, 2), "speedup": round(dm / med, 3)})
    dominant = max(kern_ms, key=lambda k: kern_ms[k])
    achieved = kern_bytes[dominant] / (kern_ms[dominant] * 1e-3) / 1e9
    n_launch_dom = sum(1 for L in layers if f"nm_spmv_kernel<{L['N']},{L['M']}>" == dominant)
    traffic = read_traffic(dominant)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": dominant,
                "bytes_per_launch": kern_bytes[dominant] / (K * n_launch_dom),
                "avg_launch_us": round(kern_ms[dominant] / (K * n_launch_dom) * 1e3, 3)}

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, args.cpu_rows_frac)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_s / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl['name']}: {len(wl['layers'])} projection shapes x patterns "
                        f"{','.join(f'{n}:{m}' for n, m in pats)}, batch 1, fp16 W ~N(0,0.02^2) "
                        f"magnitude-pruned, x ~N(0,1)",
            "layers": [f"{L['R']}x{L['C']} {L['N']}:{L['M']}" for L in layers],
            "bytes_per_step": step_sparse,
            "pool_copies_sparse": P_s,
            "pool_copies_dense": P_d,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(value / HBM_PEAK_GBPS, 4),
        "speedup_vs_dense": round(speedup, 3),
        "dense_GBps": round(dense_gbps, 1),
        "dense_ms_per_step": round(ms_d / K, 5),
        "read_ceiling_GBps": round(read_ceiling, 1),
        "wall_s_sparse": round(wall_s, 4),
        "timing": "value: K steps in one HIP graph replay between events; per_layer: median of "
                  "event pairs around each eager launch",
        "ms_per_step_eager": round(ms_s_eager / K, 5),
        "ms_per_step_with_launch_events": round(ms_s_ev / K, 5),
        "per_layer": per_layer,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(layers, frac):
    """Time the oracle (as it is) on the first `frac` of every layer's rows, on the host
    cores; also compare its y with the GPU's for those rows."""
    import numpy as np
    import oracle

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    t_total, b_total, worst, rel = 0.0, 0, 0.0, 0.0
    rows_total = 0
    t_start = time.time()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = None
    for L in layers:
        W = L["W_cpu"]
        nrow = W.shape[0]
        rv, rm = oracle.pack_ref(W, L["N"], L["M"])          # untimed: oracle input from W only
        t0 = time.perf_counter()
        y = oracle.spmv_ref(rv, rm, L["x_host"], L["C"], L["N"], L["M"])
        t_total += time.perf_counter() - t0
        b_total += alg_bytes_sparse(nrow, L["C"], L["N"], L["M"])
        rows_total += nrow
        gpu_y = L["y"][:nrow].cpu().numpy()
        rep = oracle.y_tolerance_report(gpu_y, y)
        worst = max(worst, rep["max_err_over_bound"])
        rel = max(rel, rep["rel_l2"])
    if limiter is not None:
        limiter.restore_original_limits()
    log(f"cpu baseline: {b_total / t_total / 1e9:.4f} GB/s over {rows_total} rows in {t_total:.1f}s "
        f"(leg {time.time() - t_start:.1f}s)")
    return {"value": round(b_total / t_total / 1e9, 5), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"first {frac:g} of the rows of each of the {len(layers)} layers ({rows_total} rows), "
                      f"densify + fp64 matvec, numpy/BLAS on {cores} threads",
            "seconds": round(t_total, 2), "cpu_model": cpu_info(),
            "parity_vs_gpu": {"max_err_over_bound": worst, "rel_l2": rel, "ok": worst <= 1.0 and rel <= 1e-3}}


if __name__ == "__main__":
    main()
