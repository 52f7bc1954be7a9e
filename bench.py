"""Throughput of the truly sparse COO layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--warm]

One step is one training pass of the layer over one batch: spmm_fwd, then
spmm_bwd (input gradient and value gradient in one launch sequence).  The
default workload is the single sparse linear layer 4096 x 4096 at 95%
unstructured sparsity (838,861 stored fp32 entries), batch 16.

Inputs are resident in HBM before timing starts.  Unless --warm is given,
steps cycle through enough replicas of the layer and its dense operands
(together more than twice the 256 MiB last-level cache) that each step reads
its data from HBM rather than from cache.

Printed: one JSON line.  `value` is the effective bandwidth of the step:
algorithmic bytes of forward + input gradient + value gradient (byte models
below) over the measured step time.  `roofline` covers the dominant kernel,
timed with HIP events that the library records immediately around it, in a
second pass with the same work.  `cpu_baseline` times the CPU oracle (plain C
loops, fp64 accumulation, one core) on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCE = os.path.join(ROOT, "coo_spmm_fwd_amd", "csrc", "spmm.hip")


# ------------------------------------------------------------------ byte models
def bytes_fwd(nnz, out, in_, B, sv=4, sx=4):
    """Forward: column index + value per entry, row offsets, X read once, Y written once."""
    return nnz * (sv + 4) + 4 * (out + 1) + sx * B * (in_ + out)


def bytes_dx(nnz, out, in_, B):
    """Input gradient: gathered value + permutation + row index per entry, column offsets, dY, dX."""
    return nnz * (4 + 4 + 4) + 4 * (in_ + 1) + 4 * B * (in_ + out)


def bytes_dw(nnz, out, in_, B):
    """Value gradient: column index read + dW written per entry, row offsets, X and dY."""
    return nnz * (4 + 4) + 4 * (out + 1) + 4 * B * (in_ + out)


def bytes_gradients(nnz, out, in_, B):
    """Both gradients in one launch: input gradient over the transposed view (row index and
    column-ordered value per entry) and value gradient over rows (column index read, dW written
    per entry); both offset arrays; X and dY read once; dX written once."""
    return nnz * 16 + 4 * (in_ + 1) + 4 * (out + 1) + 4 * B * (2 * in_ + out)


def source_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel: str, launch_args: dict):
    """HBM bytes per launch from committed counter runs, if taken on the current kernel source."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(kernel)
    if not e or e.get("source_sha") != source_sha() or e.get("args") != launch_args:
        return None
    return e.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ HBM counters
COPY_KERNEL_KEY = "copyBuffer"   # the runtime's device-to-device copy kernel (torch copy_ of a tensor)


def _counter_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter, match):
    """Average counter value (KiB) per dispatch of kernels whose name satisfies match()."""
    per = {}
    for r in rows:
        name = r.get("Kernel_Name", "").replace("csp::(anonymous namespace)::", "")
        if r.get("Counter_Name") != counter or not match(name):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        return None, 0
    return sum(per.values()) / len(per), len(per)


def ingest_counters(fetch_dir, write_dir, workload, batch, copy_mib=256):
    """Scale each counter by what it reads for a plain copy of known size, then store bytes per launch."""
    from coo_spmm_fwd_amd import workloads as W
    w = W.WORKLOADS[workload]
    B = batch or w.batches[0]
    ld = 1
    while ld < min(B, 64):
        ld *= 2
    fetch, write = _counter_rows(fetch_dir), _counter_rows(write_dir)
    copy_bytes = copy_mib << 20
    # the calibration copy is the only copy dispatch of that size (grid of copy_bytes / 2048 work-items)
    big = [r for r in fetch + write if COPY_KERNEL_KEY in r.get("Kernel_Name", "")]
    gmax = max((int(r["Grid_Size"]) for r in big), default=0)
    is_copy = lambda n: COPY_KERNEL_KEY in n
    fetch_c = [r for r in fetch if is_copy(r.get("Kernel_Name", "")) and int(r["Grid_Size"]) == gmax]
    write_c = [r for r in write if is_copy(r.get("Kernel_Name", "")) and int(r["Grid_Size"]) == gmax]
    cf, _ = _per_dispatch(fetch_c, "FETCH_SIZE", lambda n: True)
    cw, _ = _per_dispatch(write_c, "WRITE_SIZE", lambda n: True)
    f_scale = copy_bytes / (cf * 1024) if cf else None
    w_scale = copy_bytes / (cw * 1024) if cw else None
    rec = {}
    for name in (f"k_gradients<{ld}, false>", f"k_segment_spmm<{ld}, F32, false>"):
        m = lambda n, name=name: name in n
        kf, nf = _per_dispatch(fetch, "FETCH_SIZE", m)
        kw, nw = _per_dispatch(write, "WRITE_SIZE", m)
        if kf is None or kw is None or f_scale is None or w_scale is None:
            continue
        fb, wb = kf * 1024 * f_scale, kw * 1024 * w_scale
        rec[name] = {"source_sha": source_sha(), "args": {"workload": workload, "batch": B},
                     "fetch_kib_raw": kf, "write_kib_raw": kw, "dispatches": [nf, nw],
                     "copy_scale": {"fetch": f_scale, "write": w_scale, "copy_bytes": copy_bytes},
                     "hbm_bytes_per_launch": round(fb + wb)}
    os.makedirs(os.path.dirname(PROFILE_TRAFFIC), exist_ok=True)
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(w, L, acts, B, budget_s=12.0):
    """The oracle as written (fp64 loops, one core) on the same step: forward, dX, dW."""
    import numpy as np
    import oracle
    orc = oracle.default()
    X, dY = acts[B]["X"], acts[B]["dY"]
    canon = orc.canonicalize(L.out, L.in_, L.rows, L.cols, L.vals)
    reps, t_all = 0, 0.0
    while True:
        t0 = time.perf_counter()
        orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, X)
        orc.spmm_bwd_input(L.out, L.in_, L.rows, L.cols, L.vals, dY)
        orc.spmm_bwd_values(L.out, L.in_, canon["rows"], canon["cols"], dY, X)
        t_all += time.perf_counter() - t0
        reps += 1
        if t_all >= budget_s or reps >= 100:
            break
    step_s = t_all / reps
    nbytes = bytes_fwd(L.nnz, L.out, L.in_, B) + bytes_dx(L.nnz, L.out, L.in_, B) + bytes_dw(L.nnz, L.out, L.in_, B)
    return {"value": round(nbytes / step_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full step(s) (forward, input gradient, value gradient) of the same layer and batch, "
                      f"{step_s * 1e3:.1f} ms per step"}


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="linear4096_b16_s95")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--warm", action="store_true", help="reuse one replica (cache-resident data)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--eager", action="store_true", help="launch each call from Python instead of graph replay")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic_counters.json")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, workload=args.workload, batch=args.batch)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each MI355X runs its own layer; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from coo_spmm_fwd_amd import binding as csp
    from coo_spmm_fwd_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    w, layers, acts = W.build(args.workload)
    if w.dtype != "f32" or len(layers) != 1:
        print(f"workload {args.workload} is not a single fp32 training layer", file=sys.stderr)
        sys.exit(2)
    L = layers[0]
    B = args.batch or w.batches[0]
    if B not in acts:
        acts[B] = dict(X=W.random_dense((B, L.in_), 11), dY=W.random_dense((B, L.out), 12))
    nnz, out, in_ = L.nnz, L.out, L.in_

    b_fwd, b_dx, b_dw = bytes_fwd(nnz, out, in_, B), bytes_dx(nnz, out, in_, B), bytes_dw(nnz, out, in_, B)
    b_bwd = bytes_gradients(nnz, out, in_, B)
    step_bytes = b_fwd + b_dx + b_dw
    # bytes one step touches in one replica: structure of both orders, values, dW, dense operands
    touched = nnz * (4 * 5 + 4) + 4 * B * (3 * in_ + 2 * out)
    R = 1 if args.warm else max(2, -(-2 * MALL_BYTES // touched) + 1)

    t = lambda a: torch.from_numpy(a).to(dev)
    rows, cols, vals = t(L.rows), t(L.cols), t(L.vals)
    handles = [csp.sparse_layer_create(out, in_, rows, cols, vals) for _ in range(R)]
    Xs = [t(acts[B]["X"]) for _ in range(R)]
    dYs = [t(acts[B]["dY"]) for _ in range(R)]
    Ys = [torch.empty((B, out), device=dev) for _ in range(R)]
    dXs = [torch.empty((B, in_), device=dev) for _ in range(R)]
    dWs = [torch.empty((nnz,), device=dev) for _ in range(R)]
    stream = torch.cuda.current_stream()

    def step(i):
        j = i % R
        csp.spmm_fwd(handles[j], Xs[j], Ys[j], stream=stream)
        csp.spmm_bwd(handles[j], dYs[j], Xs[j], dXs[j], dWs[j], stream=stream)

    for i in range(max(args.warmup, R)):  # eager warm-up; also sizes every layer's operand workspace
        step(i)
    torch.cuda.synchronize()

    # One HIP graph per replica holds one step (two library calls, five kernels),
    # so the timed loop is K graph launches and host-side Python costs stay out.
    graphs = []
    if not args.eager:
        for j in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                s_cap = torch.cuda.current_stream()
                csp.spmm_fwd(handles[j], Xs[j], Ys[j], stream=s_cap)
                csp.spmm_bwd(handles[j], dYs[j], Xs[j], dXs[j], dWs[j], stream=s_cap)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()

    # timed region: exactly K steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        if graphs:
            graphs[i % R].replay()
        else:
            step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # second pass, same work: events around each op and around the main kernels
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for evs in ev:  # instantiate the events
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(K):
        j = i % R
        a = ev[i]
        a[0].record(stream)
        csp.sparse_layer_time_next(handles[j], a[1], a[2])
        csp.spmm_fwd(handles[j], Xs[j], Ys[j], stream=stream)
        a[3].record(stream)
        csp.sparse_layer_time_next(handles[j], a[4], a[5])
        csp.spmm_bwd(handles[j], dYs[j], Xs[j], dXs[j], dWs[j], stream=stream)
    torch.cuda.synchronize()
    fwd_op = sum(a[0].elapsed_time(a[3]) for a in ev) / K
    fwd_k = sum(a[1].elapsed_time(a[2]) for a in ev) / K
    bwd_k = sum(a[4].elapsed_time(a[5]) for a in ev) / K
    ld = 1
    while ld < min(B, 64):
        ld *= 2
    kernels = {
        "forward": {"name": f"k_segment_spmm<{ld}, F32, false>", "us": fwd_k * 1e3, "bytes": b_fwd},
        "backward": {"name": f"k_gradients<{ld}, false>", "us": bwd_k * 1e3, "bytes": b_bwd},
    }
    dom_key = max(kernels, key=lambda k: kernels[k]["us"])
    dom = kernels[dom_key]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    traffic = traffic_for(dom["name"], {"workload": args.workload, "batch": B})

    # restructure on the same layer (10% of entries), timed separately
    n_prune = nnz // 10
    torch.cuda.synchronize()
    r0 = time.perf_counter()
    csp.restructure(handles[0], n_prune, seed=w.seed, step=1)
    restructure_ms = (time.perf_counter() - r0) * 1e3

    if args.calibrate_copy:
        n = (args.calibrate_copy << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    del graphs
    torch.cuda.synchronize()
    for h in handles:
        csp.sparse_layer_destroy(h)

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    flops = 3 * 2 * nnz * B
    rec = {
        "metric": "SpMM fwd+bwd effective GB/s and GFLOP/s (2*nnz*B); % of HBM roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "out": out, "in": in_, "nnz": nnz, "batch": B,
                   "sparsity": round(1 - nnz / (out * in_), 4), "step": "spmm_fwd + spmm_bwd (dX and dW)",
                   "replicas": R, "cache": "warm" if args.warm else "cold",
                   "launch": "eager" if args.eager else "hip_graph_per_step"},
        "gflops": round(flops / (ms_per_step * 1e-3) / 1e9, 2),
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": dom["name"], "avg_launch_us": round(dom["us"], 3),
                     "bytes_per_launch": dom["bytes"]},
        "ops_us": {"forward_call": round(fwd_op * 1e3, 3), "forward_kernel": round(fwd_k * 1e3, 3),
                   "backward_kernel": round(bwd_k * 1e3, 3)},
        "restructure_ms": round(restructure_ms, 3),
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, L, acts, B)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
