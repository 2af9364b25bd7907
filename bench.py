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
import ctypes
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
CPU_LEG_SECONDS = 10.0  # oracle work the CPU baseline leg repeats its sample for
COUNTERS_FILE = os.path.join(ROOT, "profiles", "nm_spmv_counters.txt")
WORKLOAD_BY_NAME = {"llama8b": 2, "qwen3": 3, "llama70b": 4, "decode": 5, "prefill": 6}
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix-core peak (no sparsity credit)
PREFILL_COUNTERS_FILE = os.path.join(ROOT, "profiles", "nm_prefill_counters.txt")
COPY_CAL_BYTES = 256 << 20  # size of the counter-calibration copy


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
    ap.add_argument("--cpu-rows-frac", type=float, default=1.0,
                    help="fraction of each layer's rows the CPU oracle baseline processes")
    ap.add_argument("--tokens", type=int, default=20,
                    help="decode workload: tokens (passes over the 32 blocks) timed per graph")
    ap.add_argument("--prompt", type=int, default=2048,
                    help="prefill workload: prompt tokens per product (rows of X)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="default workload: skip the Llama-3.3-70B 2:4 layers and the decode sweep")
    ap.add_argument("--patterns", default="", help="patterns to run instead of the workload's, e.g. 2:4,16:32 "
                                                  "or the 25%% ones 1:4,2:8,4:16,8:32")
    ap.add_argument("--batch", type=int, default=1,
                    help="activation vectors per product (1: nm_spmv / nm_gemv_dense; 2..31: "
                         "nm_spmm_ws with a workspace per layer / nm_gemm_dense)")
    return ap.parse_args()


def alg_bytes_sparse(R, C, N, M, B=1):
    """values + masks + B activation vectors (x) + B outputs (y)."""
    return 2 * R * C * N // M + 4 * R * C // 32 + B * (2 * C + 2 * R)


def alg_bytes_dense(R, C, B=1):
    return 2 * R * C + B * (2 * C + 2 * R)


# the sources of the kernels and launch rules whose counters are committed (the shared
# internal header holds declarations only and is left out)
KERNEL_SOURCES = [os.path.join(ROOT, "semi_structured_sparse_amd", "csrc", f)
                  for f in ("nm_spmv_impl.h", "nm_spmv.hip")]
PREFILL_SOURCES = [os.path.join(ROOT, "semi_structured_sparse_amd", "csrc", f)
                   for f in ("nm_prefill_impl.h", "nm_prefill.hip")]


def kernel_source_sha(sources=None):
    """Hash of the kernel sources with comments and blank space removed, so that only a
    change of code (not of its comments) voids the committed counter figures."""
    import re
    h = hashlib.sha256()
    for path in sources or KERNEL_SOURCES:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def read_traffic(kernel_name: str, counters_file=COUNTERS_FILE, sources=None):
    """HBM bytes per launch of `kernel_name` (averaged over the shapes it serves in one
    step) from the committed counter summary, or None when there is none or the kernel
    sources changed since the counters were taken."""
    if not os.path.exists(counters_file):
        return None
    sha, traffic = None, {}
    with open(counters_file) as f:
        for line in f:
            line = line.strip()
            if line.startswith("kernel_source_sha256:"):
                sha = line.split(":", 1)[1].strip()
            elif line.startswith("traffic "):
                name, val = line[len("traffic "):].rsplit(":", 1)
                traffic[name.strip()] = float(val)
    if sha != kernel_source_sha(sources):
        return None
    return traffic.get(kernel_name)


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


def graph_us_per_launch(torch, launch, launches, reps=5):
    """Median time per launch of `launch(k, stream)` for k = 0..launches-1, captured in one
    HIP graph and replayed `reps` times between events."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for k in range(launches):
            launch(k, cs)
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        g.replay()
        b_.record()
        torch.cuda.synchronize()
        ts.append(a_.elapsed_time(b_) * 1e3 / launches)
    del g
    return statistics.median(ts)


def pool_copies(nbytes, pool_bytes):
    """Copies of an operand of `nbytes` such that >= pool_bytes of distinct data rotate."""
    return max(2, math.ceil(pool_bytes / nbytes))


# Launch shapes of the shaped read probe (workgroups per CU, lanes per workgroup, loads in
# flight per lane, blocked slices) tried at each layer's byte count; the fastest is the
# attainable time of a single launch that only reads those bytes. They are the fastest
# shapes of a sweep on MI355X over 1..16 workgroups per CU, 256..1024 lanes, 1..8 loads in
# flight and both layouts at 4.7..264 MB: many resident waves with one or two 16-byte loads
# in flight each, sweeping the buffer grid-stride, read fastest at every size.
PROBE_SHAPES = ((4, 512, 1, 0), (8, 256, 1, 0), (3, 512, 2, 0), (2, 1024, 1, 0), (16, 256, 2, 0),
                (8, 512, 1, 0), (16, 512, 4, 0), (16, 1024, 2, 0), (1, 512, 4, 0))


class ReadCeiling:
    """Attainable single-launch read times (the shaped read probe, fastest of PROBE_SHAPES,
    each launch on the next region of a >= 2 GiB buffer) and the whole-chip read rate."""

    def __init__(self, torch, nm, dev, buf_bytes=4 << 30):
        self.torch, self.nm, self.dev = torch, nm, dev
        self.lib = nm.lib()
        self.buf = torch.empty(buf_bytes, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)
        props = torch.cuda.get_device_properties(dev)
        self.cus = int(getattr(props, "multi_processor_count", 256) or 256)
        self.cache = {}

    def chip_rate_gbps(self):
        """Whole-chip read rate of nm_probe_read over 2 GiB (median of 10)."""
        torch, nm = self.torch, self.nm
        part = self.buf[:2 << 30]
        for _ in range(3):
            nm.nm_probe_read(part, self.sink)
        torch.cuda.synchronize()
        pt = []
        for _ in range(10):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            nm.nm_probe_read(part, self.sink)
            b_.record()
            torch.cuda.synchronize()
            pt.append(a_.elapsed_time(b_))
        return part.numel() / (statistics.median(pt) * 1e-3) / 1e9

    def attainable_us(self, nbytes, launches=40):
        """(time, shape) of the fastest probe shape reading `nbytes` in one launch."""
        nbytes = nbytes - nbytes % 16
        if nbytes in self.cache:
            return self.cache[nbytes]
        step = (nbytes + 4095) // 4096 * 4096
        nreg = self.buf.numel() // step
        base = self.buf.data_ptr()
        sink = self.sink.data_ptr()
        best = None
        for wpc, threads, unroll, blocked in PROBE_SHAPES:
            blocks = wpc * self.cus

            def launch(k, s_, b=blocks, t=threads, u=unroll, bl=blocked):
                st = self.lib.nm_probe_read_shaped(base + (k % nreg) * step, nbytes, sink, 0x9E3779B9, b, t, u, bl, s_)
                if st:
                    raise RuntimeError(f"nm_probe_read_shaped: {self.nm.status_string(st)}")
            us = graph_us_per_launch(self.torch, launch, launches, reps=3)
            if best is None or us < best[0]:
                best = (us, {"workgroups": blocks, "threads": threads, "loads_in_flight": unroll,
                             "layout": "blocked" if blocked else "grid-stride"})
        self.cache[nbytes] = best
        return best

    def release(self):
        del self.buf
        self.torch.cuda.empty_cache()


def parity_failures(obj, path="", under=False) -> list:
    """Paths of every parity record whose "ok" is false, anywhere in the bench's output: a
    dict with an "ok" key that sits under a key starting with "parity" (directly or deeper)."""
    bad = []
    if isinstance(obj, dict):
        if under and obj.get("ok") is False:
            bad.append(path)
        for k, v in obj.items():
            p = f"{path}.{k}" if path else str(k)
            bad += parity_failures(v, p, under or str(k).startswith("parity"))
    elif isinstance(obj, list):
        for i, v in enumerate(obj):
            bad += parity_failures(v, f"{path}[{i}]", under)
    return bad


def emit(out) -> int:
    """Print the JSON line; the exit status is 3 when any parity record failed."""
    bad = parity_failures(out)
    out["parity_ok"] = not bad
    print(json.dumps(out), flush=True)
    if bad:
        log(f"PARITY FAILED: {', '.join(bad)}")
        return 3
    return 0


def make_layers(torch, nm, synth, dev, cfg, specs, pats, B, cpu_rows_frac, keep_cpu=True):
    """Seeded W and x of every (layer, pattern), packed on the GPU; the dense W once per shape."""
    import numpy as np
    layers, dense = [], {}
    for li, (name, R, C) in specs:
        for pat in pats:
            N, M = pat
            ws, xs = synth.weight_seed(cfg, li, pat), synth.x_seed(cfg, li, pat)
            W = synth.weight(R, C, ws)
            x = synth.activation(C, xs)
            if B > 1:  # B activation vectors, one per row; the first is the layer's x
                x = np.stack([x] + [synth.activation(C, xs + 7919 * b) for b in range(1, B)])
            Wd = torch.from_numpy(W).to(dev)
            xd = torch.from_numpy(x).to(dev)
            values, masks = nm.nm_pack(Wd, N, M)
            ncpu = max(1, int(math.ceil(R * cpu_rows_frac)))
            yshape = (R,) if B == 1 else (B, R)
            layers.append(dict(name=name, R=R, C=C, N=N, M=M, seed_w=ws, seed_x=xs,
                               values=[values], masks=[masks], x=xd, x_host=x,
                               W_cpu=W[:ncpu].copy() if keep_cpu else None,
                               y=torch.empty(yshape, dtype=torch.float16, device=dev),
                               bytes=alg_bytes_sparse(R, C, N, M, B)))
            if (R, C) not in dense:
                dense[(R, C)] = dict(name=name, R=R, C=C, W=[Wd], x=xd,
                                     y=torch.empty(yshape, dtype=torch.float16, device=dev),
                                     bytes=alg_bytes_dense(R, C, B))
            else:
                del Wd
            del W
    torch.cuda.synchronize()
    return layers, dense


def ws_args(L, B):
    """The workspace arguments of nm_spmm_ws for layer L (none at batch one; NULL where the
    shape takes no column split)."""
    if B == 1:
        return ()
    ws = L.get("ws")
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel())


def batch_kernel_name(nm, L, B):
    """Kernel of nm_spmm_ws for layer L: a column-split kernel where it has a workspace,
    nm_spmm's kernel otherwise (for several launches, the first one's)."""
    if L.get("ws") is not None:
        return nm.spmm_ws_variant(L["R"], L["C"], B, L["N"], L["M"])
    return nm.spmm_variant(L["R"], L["C"], B, L["N"], L["M"])


def per_layer_times(torch, nm, layers, dense, B, pool_bytes, launches, ceiling=None, tag=None):
    """Each layer alone: `launches` launches cycling over its own >= pool_bytes rotation, in a
    graph (median of 5 replays), for the sparse product and for the dense one of its shape."""
    lib = nm.lib()
    sp_fn = lib.nm_spmv if B == 1 else lib.nm_spmm_ws
    dn_fn = lib.nm_gemv_dense if B == 1 else lib.nm_gemm_dense
    bx = () if B == 1 else (B,)

    def rotation(tensors, nbytes):
        return [tensors] + [[t.clone() for t in tensors] for _ in range(pool_copies(nbytes, pool_bytes) - 1)]

    def checked(fn, name):
        def call(*a):
            st = fn(*a)
            if st:
                raise RuntimeError(f"{name}: {nm.status_string(st)}")
        return call
    sp_call, dn_call = checked(sp_fn, "sparse product"), checked(dn_fn, "dense product")
    per_s = []
    for L in layers:
        pool = rotation([L["values"][0], L["masks"][0]], L["bytes"])
        argsets = [(p[0].data_ptr(), p[1].data_ptr(), L["x"].data_ptr(), L["y"].data_ptr(),
                    L["R"], L["C"]) + bx + (L["N"], L["M"]) + ws_args(L, B) for p in pool]
        per_s.append(graph_us_per_launch(torch, lambda c, sp, A=argsets: sp_call(*A[c % len(A)], sp), launches))
        del pool
    per_d = {}
    for D in dense.values():
        pool = rotation([D["W"][0]], D["bytes"])
        argsets = [(p[0].data_ptr(), D["x"].data_ptr(), D["y"].data_ptr(), D["R"], D["C"]) + bx for p in pool]
        per_d[(D["R"], D["C"])] = graph_us_per_launch(
            torch, lambda c, sp, A=argsets: dn_call(*A[c % len(A)], sp), launches)
        del pool
    # batches: the vendor BLAS on the same dense product too (torch.mm on a transposed copy of
    # W, rotated the same way), so that each layer's speedup can be quoted against the faster
    # dense product
    per_t = {}
    if B > 1:
        for D in dense.values():
            Xb = D["x"].view(B, D["C"])
            pool = rotation([D["W"][0].t().contiguous()], D["bytes"])
            try:
                for P in pool:   # eager first calls: the BLAS sets itself up outside the capture
                    torch.mm(Xb, P[0])
                torch.cuda.synchronize()
                per_t[(D["R"], D["C"])] = graph_us_per_launch(
                    torch, lambda c, sp, P=pool, Xb=Xb: torch.mm(Xb, P[c % len(P)][0]), launches)
            except Exception as e:  # pragma: no cover
                log(f"torch.mm timing unavailable: {e}")
            del pool
    torch.cuda.synchronize()
    rows = []
    for L, us in zip(layers, per_s):
        kname = nm.spmv_variant(L["R"], L["C"], L["N"], L["M"]) if B == 1 else batch_kernel_name(nm, L, B)
        dus = per_d[(L["R"], L["C"])]
        gbps = L["bytes"] / (us * 1e-6) / 1e9
        rec = {"layer": L["name"], "shape": f"{L['R']}x{L['C']}", "pattern": f"{L['N']}:{L['M']}", "kernel": kname}
        if tag:
            rec["workload"] = tag
            rec["in_step"] = False
        if B == 1:
            ls = nm.spmv_launch_shape(L["R"], L["C"], L["N"], L["M"])
            rec["workgroups"] = ls["workgroups"]
            rec["workgroup"] = f"{ls['rows_per_workgroup']} rows, {ls['row_groups']}x{ls['waves_per_row_group']} waves"
        rec.update({"us": round(us, 2), "GBps": round(gbps, 1), "pct_peak": round(gbps / HBM_PEAK_GBPS, 4),
                    "dense_us": round(dus, 2), "speedup": round(dus / us, 3)})
        tus = per_t.get((L["R"], L["C"]))
        if tus is not None:
            rec.update({"torch_mm_us": round(tus, 2), "best_dense_us": round(best_dense_us(dus, tus), 2),
                        "speedup_vs_best_dense": round(best_dense_us(dus, tus) / us, 3)})
        if ceiling is not None:
            att, shape = ceiling.attainable_us(L["bytes"])
            rec["attainable_us"] = round(att, 2)
            rec["frac_of_attainable"] = round(att / us, 4)
            rec["attainable_probe"] = shape
        rows.append(rec)
    return rows, per_s


def pattern_spread(per_layer) -> dict:
    """Per shape: (slowest - fastest) / fastest time over the patterns measured at it."""
    by = {}
    for r in per_layer:
        if r.get("in_step", True):
            by.setdefault(r["shape"], {})[r["pattern"]] = r["us"]
    out = {}
    for shape, t in by.items():
        if len(t) > 1:
            lo, hi = min(t.values()), max(t.values())
            out[shape] = {"spread": round((hi - lo) / lo, 4), "fastest": min(t, key=t.get),
                          "slowest": max(t, key=t.get)}
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the sparse product of one layer is measured on one GPU; sharding is design-only)",
              file=sys.stderr, flush=True)
        sys.exit(2)

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
    if cfg == 5:
        sys.exit(decode_main(args, torch, nm, synth, dev))
    if cfg == 6:
        sys.exit(prefill_main(args, torch, nm, synth, dev))
    wl = synth.WORKLOADS[cfg]
    pats = [tuple(p) for p in wl["patterns"]]
    B = args.batch
    if not 1 <= B <= 31:
        print("--batch must be in 1..31", file=sys.stderr)
        sys.exit(2)
    if args.patterns:  # any supported patterns, in the order given
        pats = [tuple(int(v) for v in p.split(":")) for p in args.patterns.split(",")]
        bad = [p for p in pats if p not in nm.ALL_PATTERNS]
        if bad:
            print(f"unsupported patterns {bad}", file=sys.stderr)
            sys.exit(2)
    # the default run also covers the Llama-3.3-70B 2:4 layers and the decode sweep
    extra = cfg == 2 and B == 1 and not args.patterns and not args.no_extra

    # ------------------------------------------------------------------ inputs (untimed)
    t_gen = time.time()
    layers, dense = make_layers(torch, nm, synth, dev, cfg, list(enumerate(wl["layers"])), pats, B,
                                args.cpu_rows_frac)
    log(f"generated and packed {len(layers)} layers in {time.time() - t_gen:.1f}s")

    pool_bytes = args.pool_gib * (1 << 30)
    step_sparse = sum(L["bytes"] for L in layers)
    step_dense = sum(D["bytes"] for D in dense.values())
    P_s = pool_copies(step_sparse, pool_bytes)
    P_d = pool_copies(step_dense, pool_bytes)
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
    bx = () if B == 1 else (B,)   # the batch argument of nm_spmm_ws / nm_gemm_dense
    sp_fn = lib.nm_spmv if B == 1 else lib.nm_spmm_ws
    dn_fn = lib.nm_gemv_dense if B == 1 else lib.nm_gemm_dense
    if B > 1:   # one zeroed workspace per layer (launches are stream-ordered), where it splits
        for L in layers:
            L["ws"] = nm.spmm_workspace(L["R"], L["C"], B, L["N"], L["M"], device=dev)
    sp_args = [[(L["values"][c].data_ptr(), L["masks"][c].data_ptr(), L["x"].data_ptr(), L["y"].data_ptr(),
                 L["R"], L["C"]) + bx + (L["N"], L["M"]) + ws_args(L, B) for c in range(P_s)] for L in layers]
    dense_list = list(dense.values())
    dn_args = [[(D["W"][c].data_ptr(), D["x"].data_ptr(), D["y"].data_ptr(), D["R"], D["C"]) + bx
                for c in range(P_d)] for D in dense_list]

    def sparse_step(k, sp):
        c = k % P_s
        for i in range(len(layers)):
            st = sp_fn(*sp_args[i][c], sp)
            if st:
                raise RuntimeError(f"sparse product: {nm.status_string(st)}")

    def dense_step(k, sp):
        c = k % P_d
        for i in range(len(dense_list)):
            st = dn_fn(*dn_args[i][c], sp)
            if st:
                raise RuntimeError(f"dense product: {nm.status_string(st)}")

    # ------------------------------------------------------------------ read ceiling probe
    ceiling = ReadCeiling(torch, nm, dev)
    read_ceiling = ceiling.chip_rate_gbps()
    log(f"read ceiling {read_ceiling:.0f} GB/s")
    # one plain copy of known size: under a counter profile its FETCH_SIZE / WRITE_SIZE
    # calibrate the counters against real bytes
    nm.nm_probe_copy(ceiling.buf[COPY_CAL_BYTES:2 * COPY_CAL_BYTES], ceiling.buf[:COPY_CAL_BYTES])
    torch.cuda.synchronize()

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

    # Every layer gets the same number of per-layer launches (enough to cycle through the
    # largest pool), so that each shape weighs the same in a kernel's average duration as
    # it does in a step, in these timings and in a profiler's per-kernel statistics.
    L_PL = max(40, max(pool_copies(L["bytes"], pool_bytes) for L in layers),
               max(pool_copies(D["bytes"], pool_bytes) for D in dense.values()))

    # ------------------------------------------------------------------ timed regions
    K, Wm = args.steps, args.warmup
    ms_s, wall_s = timed_graph(sparse_step, K, Wm)
    ms_d, wall_d = timed_graph(dense_step, K, Wm)

    # per-layer durations (each layer alone, its own >= pool_bytes rotation)
    per_layer, per_s = per_layer_times(torch, nm, layers, dense, B, pool_bytes, L_PL,
                                       ceiling=ceiling if B == 1 else None)

    value = step_sparse * K / (ms_s * 1e-3) / 1e9
    dense_gbps = step_dense * K / (ms_d * 1e-3) / 1e9
    # speedup over the same (shape, pattern) launches: each dense shape stands for the
    # patterns measured at that shape
    pats_per_shape = len(layers) / len(dense_list)
    speedup = (ms_d * pats_per_shape) / ms_s
    log(f"sparse {value:.0f} GB/s ({value / HBM_PEAK_GBPS:.1%}), dense {dense_gbps:.0f} GB/s, "
        f"speedup {speedup:.3f}x, {ms_s / K * 1e3:.1f} us/step")

    kern_bytes, kern_us, kern_n = {}, {}, {}
    for L, us, rec in zip(layers, per_s, per_layer):
        kname = rec["kernel"]
        kern_bytes[kname] = kern_bytes.get(kname, 0) + L["bytes"]
        kern_us[kname] = kern_us.get(kname, 0.0) + us
        kern_n[kname] = kern_n.get(kname, 0) + 1
    dominant = max(kern_us, key=lambda k: kern_us[k])
    achieved = kern_bytes[dominant] / (kern_us[dominant] * 1e-6) / 1e9
    traffic = read_traffic(dominant)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": dominant, "launches_per_step": kern_n[dominant],
                "bytes_per_launch": kern_bytes[dominant] / kern_n[dominant],
                "avg_launch_us": round(kern_us[dominant] / kern_n[dominant], 3)}
    if B == 1:
        att = sum(r["attainable_us"] for r in per_layer if r["kernel"] == dominant)
        roofline["frac_of_attainable"] = round(att / kern_us[dominant], 4)

    # ------------------------------------------------------------------ the other 2:4 layers
    more = []
    if extra:
        for L in layers:   # the step's pools are no longer needed
            del L["values"][1:], L["masks"][1:]
        for D in dense.values():
            del D["W"][1:]
        torch.cuda.empty_cache()
        t_gen = time.time()
        wl70 = synth.WORKLOADS[4]
        l70, d70 = make_layers(torch, nm, synth, dev, 4, list(enumerate(wl70["layers"])), [(2, 4)], 1,
                               args.cpu_rows_frac, keep_cpu=False)
        log(f"llama3.3-70b 2:4 layers generated and packed in {time.time() - t_gen:.1f}s")
        L70 = max(40, max(pool_copies(L["bytes"], pool_bytes) for L in l70))
        more, _ = per_layer_times(torch, nm, l70, d70, 1, pool_bytes, L70, ceiling=ceiling, tag=wl70["name"])
        del l70, d70
        # one GPU's share of the 70B MLP split over 8 GPUs (rows of gate/up, columns of down)
        shards = list(enumerate(synth.LLAMA33_70B_TP8_SHARDS, start=len(wl70["layers"])))
        lsh, dsh = make_layers(torch, nm, synth, dev, 4, shards, [(2, 4)], 1, args.cpu_rows_frac, keep_cpu=False)
        Lsh = max(40, max(pool_copies(L["bytes"], pool_bytes) for L in lsh))
        more += per_layer_times(torch, nm, lsh, dsh, 1, pool_bytes, Lsh, ceiling=ceiling,
                                tag="llama3.3-70b-mlp-8-way-shard")[0]
        del lsh, dsh
        torch.cuda.empty_cache()
    ceiling.release()

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, args.cpu_rows_frac, B)
    decode = None
    if extra:
        for L in layers:
            L["values"], L["masks"], L["W_cpu"] = None, None, None
        dense.clear()
        torch.cuda.empty_cache()
        decode = decode_sweep(args, torch, nm, synth, dev, args.tokens, max(1, min(args.warmup, 5)),
                              with_cpu=not args.no_cpu_baseline)
        torch.cuda.empty_cache()
        # the batch products and the prefill product (2048 and 512 tokens), summarised (their
        # own workloads give the full lines: --batch B, --workload prefill --prompt T)
        batches = [batch_summary(args, torch, nm, synth, dev, b) for b in EXTRA_BATCHES]
        torch.cuda.empty_cache()
        prefill = prefill_summary(prefill_run(args, torch, nm, synth, dev, EXTRA_PROMPT, (2, 4), 5, 2,
                                              None if args.no_cpu_baseline else EXTRA_PREFILL_CPU_FRAC))
        torch.cuda.empty_cache()
        prefill_mid = prefill_summary(prefill_run(args, torch, nm, synth, dev, EXTRA_MID_PROMPT, (2, 4), 10, 3,
                                                  None if args.no_cpu_baseline else EXTRA_PREFILL_CPU_FRAC))

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
                        f"{','.join(f'{n}:{m}' for n, m in pats)}, batch {B}, fp16 W ~N(0,0.02^2) "
                        f"magnitude-pruned, x ~N(0,1)",
            "batch": B,
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
        "timing": "value: K steps in one HIP graph replayed between events; per_layer: each layer "
                  "alone, the same number of launches for every layer cycling over its own >= 1 GiB "
                  "rotation, in a graph, median of 5 replays; attainable_us: the fastest shape of the "
                  "read probe reading the layer's bytes in one launch, timed the same way",
        "per_layer": per_layer + more,
        "speedup_vs_best_dense_per_layer_sum": (
            round(sum(r["best_dense_us"] for r in per_layer) / sum(r["us"] for r in per_layer), 3)
            if per_layer and all("best_dense_us" in r for r in per_layer) else None),
        "pattern_spread": pattern_spread(per_layer),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if decode is not None:
        out["decode"] = decode
        out["batch_products"] = batches
        out["prefill"] = prefill
        out["prefill_mid"] = prefill_mid
    sys.exit(emit(out))


EXTRA_BATCHES = (8, 24)        # batch products summarised in the default line
EXTRA_PROMPT = 2048            # prompt of the prefill summary
EXTRA_MID_PROMPT = 512         # prompt of the mid-size prefill summary (column splits of taller tiles)
EXTRA_PREFILL_CPU_FRAC = 1 / 64  # rows of each prefill layer the oracle checks (all tokens)


def batch_summary(args, torch, nm, synth, dev, B):
    """The Llama-3.1-8B projections (4 shapes x 4 patterns) at B activation vectors through
    nm_spmm_ws (a workspace per layer), each layer alone as in --batch B: time per layer for
    the sparse product, our dense batch product and torch.mm, the step's effective GB/s (the
    sum of the layers' bytes over the sum of their times), and the oracle's Y against the
    GPU's on each layer's first rows (all B vectors)."""
    import oracle
    wl = synth.WORKLOADS[2]
    pats = [tuple(p) for p in wl["patterns"]]
    t0 = time.time()
    layers, dense = make_layers(torch, nm, synth, dev, 2, list(enumerate(wl["layers"])), pats, B, 1 / 64)
    for L in layers:
        L["ws"] = nm.spmm_workspace(L["R"], L["C"], B, L["N"], L["M"], device=dev)
    pool_bytes = args.pool_gib * (1 << 30)
    launches = max(40, max(pool_copies(L["bytes"], pool_bytes) for L in layers),
                   max(pool_copies(D["bytes"], pool_bytes) for D in dense.values()))
    per_layer, per_s = per_layer_times(torch, nm, layers, dense, B, pool_bytes, launches)
    worst, rel = 0.0, 0.0
    for L in layers:
        rv, rm = oracle.pack_ref(L["W_cpu"], L["N"], L["M"])
        ref = oracle.spmm_ref(rv, rm, L["x_host"], L["C"], L["N"], L["M"])
        rep = oracle.y_tolerance_report(L["y"][:, :ref.shape[-1]].cpu().numpy(), ref)
        worst, rel = max(worst, rep["max_err_over_bound"]), max(rel, rep["rel_l2"])
    us = sum(per_s)
    nbytes = sum(L["bytes"] for L in layers)
    best = [r.get("best_dense_us", r["dense_us"]) for r in per_layer]
    log(f"batch {B}: {nbytes / (us * 1e-6) / 1e9:.0f} GB/s, {sum(r['dense_us'] for r in per_layer) / us:.3f}x "
        f"over the dense kernel, {sum(best) / us:.3f}x over the faster dense ({time.time() - t0:.1f}s)")
    out = {"batch": B, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "us_per_step": round(us, 2),
           "speedup_vs_dense": round(sum(r["dense_us"] for r in per_layer) / us, 3),
           "speedup_vs_best_dense": round(sum(best) / us, 3),
           "slowest_layer_vs_best_dense": min(r.get("speedup_vs_best_dense", r["speedup"]) for r in per_layer),
           "per_layer": [{k: r[k] for k in ("shape", "pattern", "kernel", "us", "dense_us", "torch_mm_us",
                                            "speedup_vs_best_dense") if k in r} for r in per_layer],
           "timing": "each layer alone as in --batch B (sum of the layers' times, no step graph)",
           "parity_vs_gpu": {"rows": "first 1/64 of each layer's rows, all vectors", "max_err_over_bound": worst,
                             "rel_l2": rel, "ok": worst <= 1.0 and rel <= 1e-3}}
    del layers, dense
    return out


def prefill_summary(full):
    """The fields of a prefill line (prefill_run) that the default line carries."""
    keep = ("value", "unit", "ms_per_step", "speedup_vs_dense", "speedup_vs_best_dense_per_layer_sum",
            "dense_equiv_TFLOPs")
    out = {k: full[k] for k in keep}
    out["config"] = full["config"]["workload"]
    out["roofline"] = {k: full["roofline"][k] for k in ("kernel", "achieved", "peak", "frac", "traffic")}
    out["per_layer"] = [{k: r[k] for k in ("layer", "kernel", "us", "useful_TFLOPs", "dense_us", "torch_mm_us",
                                           "speedup_vs_best_dense")} for r in full["per_layer"]]
    if full.get("cpu_baseline"):
        out["parity_vs_gpu"] = dict(full["cpu_baseline"]["parity_vs_gpu"],
                                    rows=full["cpu_baseline"]["sample"])
    return out


def decode_sweep(args, torch, nm, synth, dev, K, Wm, with_cpu=True):
    """The Llama-3.1-8B decode sweep: 32 transformer blocks x 7 projections (q, k, v, o,
    gate, up, down), 2:4, every projection with its own seeded W and x; a step is one
    token, i.e. one in-order pass over the 224 products. Also timed: the dense GEMV over
    the same 224 weights, and two sweeps in which q/k/v and gate/up read one x, as they do
    in the model (the x of q, resp. gate): fused into one product over their concatenated
    rows (against the dense GEMV fused the same way), and grouped from their separate
    matrices (nm_spmv_group). Each sweep writes its own outputs, and each is checked against
    the oracle on the x it used, in the first and the last block."""
    wl = synth.WORKLOADS[5]
    NB, (N, M) = wl["n_layers"], tuple(wl["patterns"][0])
    lib = nm.lib()
    t_gen = time.time()
    check_blocks = (0, NB - 1)
    sp, dn, host = [], [], {}
    for b in range(NB):
        for p, (name, R, C) in enumerate(wl["layers"]):
            W = synth.weight(R, C, synth.decode_seed(b, p))
            x = synth.activation(C, synth.decode_x_seed(b, p))
            Wd = torch.from_numpy(W).to(dev)
            xd = torch.from_numpy(x).to(dev)
            values, masks = nm.nm_pack(Wd, N, M)
            sp.append(dict(name=name, block=b, R=R, C=C, values=values, masks=masks, x=xd,
                           y=torch.empty(R, dtype=torch.float16, device=dev),    # plain sweep
                           yg=torch.empty(R, dtype=torch.float16, device=dev),   # grouped sweep
                           bytes=alg_bytes_sparse(R, C, N, M)))
            dn.append(dict(R=R, C=C, W=Wd, x=xd, y=torch.empty(R, dtype=torch.float16, device=dev),
                           bytes=alg_bytes_dense(R, C)))
            if b in check_blocks:
                host[(b, p)] = (W, x)
            del W
    # which projection's x each projection reads when q/k/v and gate/up share theirs
    shared_x = {0: 0, 1: 0, 2: 0, 3: 3, 4: 4, 5: 4, 6: 6}
    groups = ((0, 1, 2), (3,), (4, 5), (6,))
    fused, fused_dn = [], []
    for b in range(NB):
        blk = sp[7 * b:7 * b + 7]
        for idx in groups:
            parts = [blk[i] for i in idx]
            R = sum(q["R"] for q in parts)
            C = parts[0]["C"]
            v = torch.cat([q["values"] for q in parts]) if len(parts) > 1 else parts[0]["values"]
            m = torch.cat([q["masks"] for q in parts]) if len(parts) > 1 else parts[0]["masks"]
            fused.append(dict(block=b, idx=idx, R=R, C=C, values=v, masks=m, x=blk[idx[0]]["x"],
                              y=torch.empty(R, dtype=torch.float16, device=dev),
                              bytes=alg_bytes_sparse(R, C, N, M)))
            dparts = [dn[7 * b + i] for i in idx]
            Wf = torch.cat([q["W"] for q in dparts]) if len(dparts) > 1 else dparts[0]["W"]
            fused_dn.append(dict(R=R, C=C, W=Wf, x=blk[idx[0]]["x"],
                                 y=torch.empty(R, dtype=torch.float16, device=dev),
                                 bytes=alg_bytes_dense(R, C)))
    torch.cuda.synchronize()
    log(f"decode sweep: generated and packed {len(sp)} projections in {time.time() - t_gen:.1f}s")

    def sp_launches(items):
        return [(q["values"].data_ptr(), q["masks"].data_ptr(), q["x"].data_ptr(), q["y"].data_ptr(),
                 q["R"], q["C"], N, M) for q in items]
    sp_a, fu_a = sp_launches(sp), sp_launches(fused)

    def dn_launches(items):
        return [(q["W"].data_ptr(), q["x"].data_ptr(), q["y"].data_ptr(), q["R"], q["C"]) for q in items]
    dn_a, fdn_a = dn_launches(dn), dn_launches(fused_dn)

    def token_sparse(A):
        def run(sp_):
            for a in A:
                st = lib.nm_spmv(*a, sp_)
                if st:
                    raise RuntimeError(f"nm_spmv: {nm.status_string(st)}")
        return run

    def token_dense(A):
        def run(sp_):
            for a in A:
                st = lib.nm_gemv_dense(*a, sp_)
                if st:
                    raise RuntimeError(f"nm_gemv_dense: {nm.status_string(st)}")
        return run

    def timed_tokens(fn, K_, W_):
        s_ = torch.cuda.current_stream(dev).cuda_stream
        for _ in range(W_):
            fn(s_)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for _ in range(K_):
                fn(cs)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            g.replay()
            b_.record()
            torch.cuda.synchronize()
            ts.append(a_.elapsed_time(b_) / K_)
        del g
        return statistics.median(ts)

    # q/k/v and gate/up as groups of their separate matrices (nm_spmv_group, one launch each),
    # writing the grouped outputs
    gr_a = []
    for b in range(NB):
        blk = sp[7 * b:7 * b + 7]
        for idx in groups:
            parts = [blk[i] for i in idx]
            n = len(parts)
            gr_a.append((n, (ctypes.c_void_p * n)(*[q["values"].data_ptr() for q in parts]),
                         (ctypes.c_void_p * n)(*[q["masks"].data_ptr() for q in parts]),
                         parts[0]["x"].data_ptr(), (ctypes.c_void_p * n)(*[q["yg"].data_ptr() for q in parts]),
                         (ctypes.c_int64 * n)(*[q["R"] for q in parts]), parts[0]["C"]))

    def token_group(sp_):
        for n, v, m, x, y, r, c in gr_a:
            st = lib.nm_spmv_group(n, v, m, x, y, r, c, N, M, sp_)
            if st:
                raise RuntimeError(f"nm_spmv_group: {nm.status_string(st)}")

    ms_sp = timed_tokens(token_sparse(sp_a), K, Wm)
    ms_dn = timed_tokens(token_dense(dn_a), K, Wm)
    ms_fu = timed_tokens(token_sparse(fu_a), K, Wm)
    ms_fu_dn = timed_tokens(token_dense(fdn_a), K, Wm)
    ms_gr = timed_tokens(token_group, K, Wm)
    torch.cuda.synchronize()
    bytes_tok = sum(q["bytes"] for q in sp)
    bytes_dn = sum(q["bytes"] for q in dn)
    gbps = bytes_tok / (ms_sp * 1e-3) / 1e9
    log(f"decode: sparse {ms_sp * 1e3:.1f} us/token ({gbps:.0f} GB/s), dense {ms_dn * 1e3:.1f} us/token, "
        f"speedup {ms_dn / ms_sp:.3f}x; fused q/k/v and gate/up: sparse {ms_fu * 1e3:.1f} us/token, "
        f"dense {ms_fu_dn * 1e3:.1f} us/token, speedup {ms_fu_dn / ms_fu:.3f}x; grouped (separate matrices): "
        f"sparse {ms_gr * 1e3:.1f} us/token")

    # ---------------------------------------------------------------- parity (untimed)
    # outputs of the checked blocks as the three sweeps left them
    outs = {"plain": {}, "grouped": {}, "fused": {}}
    for b in check_blocks:
        for p in range(7):
            q = sp[7 * b + p]
            outs["plain"][(b, p)] = q["y"].cpu().numpy()
            outs["grouped"][(b, p)] = q["yg"].cpu().numpy()
        for f in fused[4 * b:4 * b + 4]:
            yf = f["y"].cpu().numpy()
            r0 = 0
            for p in f["idx"]:
                R = sp[7 * b + p]["R"]
                outs["fused"][(b, p)] = yf[r0:r0 + R]
                r0 += R
    own = {k: host[k][1] for k in host}
    shared = {(b, p): host[(b, shared_x[p])][1] for (b, p) in host}
    parity = {"plain": oracle_parity(host, own, outs["plain"], N, M),
              "grouped": oracle_parity(host, shared, outs["grouped"], N, M),
              "fused": oracle_parity(host, shared, outs["fused"], N, M)}
    for k, v in parity.items():
        v["blocks"] = list(check_blocks)
    log("decode parity: " + ", ".join(f"{k} max_err/bound {v['max_err_over_bound']:.3f} ok={v['ok']}"
                                      for k, v in parity.items()))
    cpu = None
    if with_cpu:
        cpu_layers = [dict(name=wl["layers"][p][0], R=wl["layers"][p][1], C=wl["layers"][p][2], N=N, M=M,
                           x_host=host[(0, p)][1], y=sp[p]["y"], W_cpu=host[(0, p)][0]) for p in range(7)]
        cpu = cpu_baseline(cpu_layers, 1.0)
    return {
        "workload": f"{wl['name']}: {NB} blocks x 7 Llama-3.1-8B projections, 2:4, batch 1, a fresh seeded W "
                    f"and x per projection; a step is one token (224 products in order)",
        "us_per_token": round(ms_sp * 1e3, 2),
        "GBps": round(gbps, 1),
        "pct_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_token": bytes_tok,
        "dense_us_per_token": round(ms_dn * 1e3, 2),
        "dense_GBps": round(bytes_dn / (ms_dn * 1e-3) / 1e9, 1),
        "speedup_vs_dense": round(ms_dn / ms_sp, 3),
        "fused_qkv_gateup": {"us_per_token": round(ms_fu * 1e3, 2), "launches_per_token": len(fused) // NB,
                             "GBps": round(sum(q["bytes"] for q in fused) / (ms_fu * 1e-3) / 1e9, 1),
                             "dense_us_per_token": round(ms_fu_dn * 1e3, 2),
                             "dense_GBps": round(sum(q["bytes"] for q in fused_dn) / (ms_fu_dn * 1e-3) / 1e9, 1),
                             "speedup_vs_fused_dense": round(ms_fu_dn / ms_fu, 3),
                             "x": "q, k, v read the x of q; gate, up the x of gate (concatenated rows)"},
        "grouped_qkv_gateup": {"us_per_token": round(ms_gr * 1e3, 2), "launches_per_token": len(gr_a) // NB,
                               "GBps": round(bytes_tok / (ms_gr * 1e-3) / 1e9, 1),
                               "speedup_vs_fused_dense": round(ms_fu_dn / ms_gr, 3),
                               "x": "q, k, v read the x of q; gate, up the x of gate (nm_spmv_group over the "
                                    "separate matrices)"},
        "byte_floor_us_per_token_at_8TBps": round(bytes_tok / 8e12 * 1e6, 1),
        "timing": "K tokens in one HIP graph replayed between events, median of 3 replays",
        "parity": parity,
        "roofline": decode_roofline(nm, sp, ms_sp, N, M),
        "cpu_baseline": cpu,
    }


def oracle_parity(host, xs, ys, N, M) -> dict:
    """Each GPU output ys[k] against the oracle (pack, then densify + fp64 matvec) of the
    weights host[k][0] on the x it used, xs[k]; rows in chunks over the host cores."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(16, cores))

    def one(k):
        W = host[k][0]
        x = xs[k]
        refs = []
        for a in range(0, W.shape[0], 512):
            rv, rm = oracle.pack_ref(W[a:a + 512], N, M)
            refs.append(oracle.spmv_ref(rv, rm, x, W.shape[1], N, M))
        return k, np.concatenate(refs)

    worst, rel, rows = 0.0, 0.0, 0
    finite = True
    with ThreadPoolExecutor(cores) as ex:
        for k, ref in ex.map(one, sorted(ys)):
            rep = oracle.y_tolerance_report(ys[k], ref)
            worst = max(worst, rep["max_err_over_bound"])
            rel = max(rel, rep["rel_l2"])
            finite = finite and rep["finite"]
            rows += ref.shape[0]
    return {"max_err_over_bound": worst, "rel_l2": rel, "rows": rows,
            "ok": bool(finite and worst <= 1.0 and rel <= 1e-3)}


def decode_main(args, torch, nm, synth, dev) -> int:
    """--workload decode: the decode sweep as the line's own workload."""
    K, Wm = args.tokens, max(1, min(args.warmup, 5))
    d = decode_sweep(args, torch, nm, synth, dev, K, Wm, with_cpu=not args.no_cpu_baseline)
    out = {
        "metric": METRIC,
        "value": d["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(d["us_per_token"] * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": d["workload"], "bytes_per_step": d["bytes_per_token"], "parallelism": "single GPU"},
        "roofline": d["roofline"],
        "cpu_baseline": d["cpu_baseline"],
        "decode": {k: v for k, v in d.items() if k not in ("roofline", "cpu_baseline", "workload")},
    }
    return emit(out)


def decode_roofline(nm, items, ms_token, N, M):
    """Roofline of the decode sweep: every product of the token runs one kernel variant (2:4:
    the pair table), so its average launch is the token time over the launches, and its achieved
    rate is the token's algorithmic bytes over the token time (gaps between launches
    included, as in the per-layer figures of the projection workloads)."""
    names = {nm.spmv_variant(q["R"], q["C"], N, M) for q in items}
    if len(names) != 1:
        return None
    n = len(items)
    b = sum(q["bytes"] for q in items) / n
    us = ms_token * 1e3 / n
    achieved = b / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": names.pop(),
            "launches_per_step": n, "bytes_per_launch": round(b), "avg_launch_us": round(us, 3)}


def prefill_main(args, torch, nm, synth, dev):
    """The prefill workload (prefill_run) at --prompt tokens, 2:4 or the first of --patterns."""
    pat = (2, 4)
    if args.patterns:   # one of the patterns with a matrix-core product
        pat = tuple(int(v) for v in args.patterns.split(",")[0].split(":"))
        if pat not in ((2, 4), (4, 8), (8, 16), (16, 32)):
            print(f"prefill: pattern {pat} has no matrix-core product (2:4, 4:8, 8:16, 16:32)", file=sys.stderr)
            sys.exit(2)
    return emit(prefill_run(args, torch, nm, synth, dev, args.prompt, pat, args.steps, args.warmup,
                            None if args.no_cpu_baseline else args.cpu_rows_frac))


def prefill_run(args, torch, nm, synth, dev, T, pat, K, Wm, cpu_frac):
    """Prefill: the Llama-3.1-8B projection shapes (q, kv, gate_up, down) as packed weights of
    pattern `pat` (4:8 and 8:16 as two 2:4 operands, 16:32 expanded) times a prompt of
    --prompt tokens (X [tokens][cols], seeded N(0,1)), on the sparse matrix cores (nm_spmm_ws
    with a workspace per layer: the prefill kernel, whose output tiles' columns are split
    over several workgroups where the prompt is too short for the tiles to fill the GPU); a
    step is one pass over the four products. Also
    timed: the dense matrix-core product over the same dense weights (nm_gemm_dense_prefill)
    and, as context only, torch.mm (the vendor BLAS) on the same shapes.

    Useful flops of a sparse product: 2 * rows * (cols / 2) * tokens (kept weights only);
    the roofline prices them against the dense fp16 matrix-core peak (the sparse
    instruction's doubled rate is not counted as peak)."""
    import numpy as np
    lib = nm.lib()
    cfg = 6
    shapes = synth.LLAMA31_8B
    N, M = pat
    t_gen = time.time()
    items = []
    for li, (name, R, C) in enumerate(shapes):
        W = synth.weight(R, C, synth.weight_seed(cfg, li, pat))
        X = synth.activations(T, C, synth.x_seed(cfg, li, pat))
        Wd = torch.from_numpy(W).to(dev)
        Xd = torch.from_numpy(X).to(dev)
        values, masks = nm.nm_pack(Wd, N, M)
        items.append(dict(name=name, R=R, C=C, W=Wd, Wt=Wd.t().contiguous(), X=Xd, X_host=X, values=values,
                          masks=masks, ws=nm.spmm_workspace(R, C, T, N, M, device=dev),
                          Y=torch.empty((T, R), dtype=torch.float16, device=dev),
                          Yd=torch.empty((T, R), dtype=torch.float16, device=dev),
                          W_cpu=W, flops_useful=R * C * T, flops_dense=2 * R * C * T))
        del W
    torch.cuda.synchronize()
    log(f"prefill: generated and packed {len(items)} layers x {T} tokens in {time.time() - t_gen:.1f}s")
    sp_a = [(q["values"].data_ptr(), q["masks"].data_ptr(), q["X"].data_ptr(), q["Y"].data_ptr(), q["R"], q["C"],
             T, N, M) + ((None, 0) if q["ws"] is None else (q["ws"].data_ptr(), q["ws"].numel())) for q in items]
    dn_a = [(q["W"].data_ptr(), q["X"].data_ptr(), q["Yd"].data_ptr(), q["R"], q["C"], T) for q in items]

    def sp_step(s_):
        for a in sp_a:
            st = lib.nm_spmm_ws(*a, s_)
            if st:
                raise RuntimeError(f"nm_spmm_ws: {nm.status_string(st)}")

    def dn_step(s_):
        for a in dn_a:
            st = lib.nm_gemm_dense_prefill(*a, s_)
            if st:
                raise RuntimeError(f"nm_gemm_dense_prefill: {nm.status_string(st)}")

    def graph_ms(fn, K, W_, reps=3):
        s_ = torch.cuda.current_stream(dev).cuda_stream
        for _ in range(W_):
            fn(s_)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for _ in range(K):
                fn(cs)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            g.replay()
            b_.record()
            torch.cuda.synchronize()
            ts.append(a_.elapsed_time(b_) / K)
        del g
        return statistics.median(ts)

    # one plain copy of known size: under a counter profile its FETCH_SIZE / WRITE_SIZE
    # calibrate the counters against real bytes
    cal = torch.empty(2 * COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
    nm.nm_probe_copy(cal[COPY_CAL_BYTES:], cal[:COPY_CAL_BYTES])
    torch.cuda.synchronize()
    del cal

    ms_sp = graph_ms(sp_step, K, Wm)
    ms_dn = graph_ms(dn_step, K, Wm)
    # per layer: each product alone, 20 launches in a graph, median of 3 replays
    per_layer = []
    for i, q in enumerate(items):
        us_s = graph_ms(lambda s_, a=sp_a[i]: lib.nm_spmm_ws(*a, s_), 20, 3) * 1e3
        us_d = graph_ms(lambda s_, a=dn_a[i]: lib.nm_gemm_dense_prefill(*a, s_), 20, 3) * 1e3
        Wt, Xd = q["Wt"], q["X"]
        try:   # context only: the vendor BLAS on the same dense product
            us_t = graph_ms(lambda s_, Wt=Wt, Xd=Xd: torch.mm(Xd, Wt), 20, 3) * 1e3
        except Exception as e:  # pragma: no cover
            log(f"torch.mm timing unavailable: {e}")
            us_t = float("nan")
        per_layer.append({"layer": q["name"], "shape": f"{q['R']}x{q['C']}", "tokens": T,
                          "kernel": nm.spmm_ws_variant(q["R"], q["C"], T, N, M),
                          "us": round(us_s, 2), "useful_TFLOPs": round(q["flops_useful"] / us_s / 1e6, 1),
                          "alg_GBs": round(alg_bytes_sparse(q["R"], q["C"], N, M, T) / us_s / 1e3, 1),
                          "dense_equiv_TFLOPs": round(q["flops_dense"] / us_s / 1e6, 1),
                          "dense_kernel": nm.prefill_variant(q["R"], q["C"], T, False),
                          "dense_us": round(us_d, 2), "dense_TFLOPs": round(q["flops_dense"] / us_d / 1e6, 1),
                          "speedup": round(us_d / us_s, 3),
                          "torch_mm_us": None if us_t != us_t else round(us_t, 2),
                          "torch_mm_TFLOPs": None if us_t != us_t else round(q["flops_dense"] / us_t / 1e6, 1),
                          "best_dense_us": round(best_dense_us(us_d, us_t), 2),
                          "speedup_vs_best_dense": round(best_dense_us(us_d, us_t) / us_s, 3)})
    torch.cuda.synchronize()
    useful = sum(q["flops_useful"] for q in items)
    dense_f = sum(q["flops_dense"] for q in items)
    value = useful / (ms_sp * 1e-3) / 1e12
    log(f"prefill: sparse {ms_sp * 1e3:.1f} us/step ({value:.0f} useful TFLOP/s, "
        f"{dense_f / (ms_sp * 1e-3) / 1e12:.0f} dense-equivalent), dense {ms_dn * 1e3:.1f} us/step, "
        f"speedup {ms_dn / ms_sp:.3f}x")
    # dominant kernel: the one with the most time per step
    kern_us, kern_f, kern_n = {}, {}, {}
    for pl, q in zip(per_layer, items):
        k = pl["kernel"]
        kern_us[k] = kern_us.get(k, 0.0) + pl["us"]
        kern_f[k] = kern_f.get(k, 0) + q["flops_useful"]
        kern_n[k] = kern_n.get(k, 0) + 1
    dom = max(kern_us, key=lambda k: kern_us[k])
    achieved = kern_f[dom] / (kern_us[dom] * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": read_traffic(dom, PREFILL_COUNTERS_FILE, PREFILL_SOURCES),
                "kernel": dom, "launches_per_step": kern_n[dom], "flops_per_launch": kern_f[dom] / kern_n[dom],
                "avg_launch_us": round(kern_us[dom] / kern_n[dom], 3),
                "flops_counted": "useful: 2 x rows x cols/2 x tokens (kept weights)"}
    cpu = None
    if cpu_frac is not None:
        cpu = prefill_cpu_baseline(items, T, cpu_frac, N, M)
    out = {
        "metric": f"{N}:{M} prefill SpMM useful TFLOP/s on the "
                  f"{'dense matrix cores (expanded fragments)' if N == 16 else 'sparse matrix cores'} "
                  f"+ speedup vs dense matrix-core GEMM",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_sp, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": f"llama3.1-8b prefill: {len(items)} projection shapes (q, kv, gate_up, down) x "
                               f"{T}-token prompt, {N}:{M}, fp16 W ~N(0,0.02^2) magnitude-pruned, X ~N(0,1)",
                   "tokens": T, "flops_useful_per_step": useful, "parallelism": "single GPU"},
        "dense_equiv_TFLOPs": round(dense_f / (ms_sp * 1e-3) / 1e12, 1),
        "dense_ms_per_step": round(ms_dn, 5),
        "dense_TFLOPs": round(dense_f / (ms_dn * 1e-3) / 1e12, 1),
        "speedup_vs_dense": round(ms_dn / ms_sp, 3),
        "speedup_vs_best_dense_per_layer_sum": round(
            sum(pl["best_dense_us"] for pl in per_layer) / sum(pl["us"] for pl in per_layer), 3),
        "timing": "K steps in one HIP graph replayed between events, median of 3 replays; per_layer: 20 launches "
                  "of one product in a graph, median of 3 replays; best dense per layer: the faster of the dense "
                  "matrix-core kernel and torch.mm on the same dense product",
        "per_layer": per_layer,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    return out


def best_dense_us(ours_us, torch_mm_us):
    """The faster dense product of a layer: our dense matrix-core kernel or torch.mm (the vendor
    BLAS), whichever took less time (torch.mm may be unavailable: NaN)."""
    if torch_mm_us != torch_mm_us:
        return ours_us
    return min(ours_us, torch_mm_us)


def _rows_phrase(frac):
    return "all rows" if frac >= 1.0 else f"the first {frac:g} of the rows"


def prefill_cpu_baseline(items, T, frac, N=2, M=4):
    """Time the oracle (as it is: densify, fp64 matrix product through numpy's BLAS) on the
    first rows of every prefill layer with all tokens, and compare its Y with the GPU's."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    t_start = time.time()
    flops, secs, worst, rel, rows_total = 0, 0.0, 0.0, 0.0, 0
    for q in items:
        n = max(16, int(q["R"] * frac) // 16 * 16)
        n = min(n, q["R"])
        rv, rm = oracle.pack_ref(q["W_cpu"][:n], N, M)
        t0 = time.perf_counter()
        ref = oracle.spmm_ref(rv, rm, q["X_host"], q["C"], N, M)
        secs += time.perf_counter() - t0
        flops += n * q["C"] * T
        rows_total += n
        rep = oracle.y_tolerance_report(q["Y"][:, :n].cpu().numpy(), ref)
        worst = max(worst, rep["max_err_over_bound"])
        rel = max(rel, rep["rel_l2"])
    log(f"prefill cpu baseline: {flops / secs / 1e12:.5f} useful TFLOP/s over {rows_total} rows x {T} tokens "
        f"in {secs:.1f}s (leg {time.time() - t_start:.1f}s)")
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{_rows_phrase(frac)} of each of the {len(items)} layers ({rows_total} rows) x {T} "
                      f"tokens; densify + fp64 matrix product (numpy BLAS, {cores} threads)",
            "seconds": round(secs, 2), "cpu_model": cpu_info(),
            "parity_vs_gpu": {"max_err_over_bound": worst, "rel_l2": rel, "ok": worst <= 1.0 and rel <= 1e-3}}


def cpu_baseline(layers, frac, B=1):
    """Time the oracle (as it is) on the first `frac` of every layer's rows on the host
    cores: the rows are cut into chunks that a pool of threads (one per core) hands to
    oracle.spmv_ref (oracle.spmm_ref for B > 1 vectors; numpy releases the interpreter lock
    inside its array operations), with BLAS held to one thread per call. Also: the same
    oracle on one thread, and the oracle's y compared with the GPU's for those rows."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_limits
        blas_one = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        blas_one = None
    t_start = time.time()
    chunks = []
    for li, L in enumerate(layers):
        n = L["W_cpu"].shape[0]
        step = max(1, min(256, -(-n // cores)))
        chunks += [(li, a, min(n, a + step)) for a in range(0, n, step)]

    def prep(ch):          # oracle input from W only (untimed)
        li, a, b = ch
        L = layers[li]
        return oracle.pack_ref(L["W_cpu"][a:b], L["N"], L["M"])

    with ThreadPoolExecutor(cores) as ex:
        packed = list(ex.map(prep, chunks))

    def run(i):
        li = chunks[i][0]
        L = layers[li]
        rv, rm = packed[i]
        if B > 1:
            return oracle.spmm_ref(rv, rm, L["x_host"], L["C"], L["N"], L["M"])
        return oracle.spmv_ref(rv, rm, L["x_host"], L["C"], L["N"], L["M"])

    passes = []
    with ThreadPoolExecutor(cores) as ex:
        # timed passes over the sample until about CPU_LEG_SECONDS of oracle work (at least 3,
        # at most 50); the median pass is reported
        while len(passes) < 3 or (sum(passes) < CPU_LEG_SECONDS and len(passes) < 50):
            t0 = time.perf_counter()
            ys = list(ex.map(run, range(len(chunks))))
            passes.append(time.perf_counter() - t0)
    t_total = statistics.median(passes)
    b_total = sum(alg_bytes_sparse(b - a, layers[li]["C"], layers[li]["N"], layers[li]["M"], B)
                  for li, a, b in chunks)
    rows_total = sum(L["W_cpu"].shape[0] for L in layers)
    worst, rel = 0.0, 0.0
    for li, L in enumerate(layers):
        y = np.concatenate([ys[i] for i, ch in enumerate(chunks) if ch[0] == li], axis=-1)
        rep = oracle.y_tolerance_report(L["y"][..., :y.shape[-1]].cpu().numpy(), y)
        worst = max(worst, rep["max_err_over_bound"])
        rel = max(rel, rep["rel_l2"])
    # the same oracle on one thread, over every 16th chunk
    t1, b1 = 0.0, 0
    for i in range(0, len(chunks), 16):
        li, a, b = chunks[i]
        t0 = time.perf_counter()
        run(i)
        t1 += time.perf_counter() - t0
        b1 += alg_bytes_sparse(b - a, layers[li]["C"], layers[li]["N"], layers[li]["M"], B)
    if blas_one is not None:
        blas_one.restore_original_limits()
    del packed
    log(f"cpu baseline: {b_total / t_total / 1e9:.4f} GB/s over {rows_total} rows in {t_total:.1f}s on "
        f"{cores} threads, {b1 / t1 / 1e9:.4f} GB/s on 1 thread (leg {time.time() - t_start:.1f}s)")
    return {"value": round(b_total / t_total / 1e9, 5), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{_rows_phrase(frac)} of each of the {len(layers)} layers ({rows_total} rows) in "
                      f"{len(chunks)} chunks over {cores} threads; densify + fp64 "
                      f"{'matvec' if B == 1 else f'product with the {B} vectors'} (numpy); median of "
                      f"{len(passes)} passes ({sum(passes):.1f} s of oracle work)",
            "seconds": round(t_total, 2), "cpu_model": cpu_info(),
            "single_thread": {"value": round(b1 / t1 / 1e9, 5), "unit": "GB/s", "seconds": round(t1, 2),
                              "sample": "every 16th chunk, one thread"},
            "parity_vs_gpu": {"max_err_over_bound": worst, "rel_l2": rel, "ok": worst <= 1.0 and rel <= 1e-3}}


if __name__ == "__main__":
    main()
