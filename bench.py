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
timed with a pair of HIP events that the library attaches to that kernel's
dispatch (so they carry its own start and end), in a second pass with the
same work; its `ceiling` holds a same-byte device copy and the launch floor
measured on the same stream.  `cpu_baseline` times the CPU oracle (plain C
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
    for name in (f"k_gradients<{ld}, csp::F32, false, 0, 1>", f"k_segment_spmm<{ld}, csp::F32, false, 0, 1>"):
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
def cpu_baseline(kind, layers, acts, B, n_prune=0, seed=0, budget_s=12.0):
    """The oracle as written (fp64 loops, one core) on the same step, repeated until ~budget_s."""
    import numpy as np
    import oracle
    orc = oracle.default()
    X, dY = acts[B]["X"], acts[B]["dY"]
    canon = [orc.canonicalize(L.out, L.in_, L.rows, L.cols, L.vals) for L in layers]

    def one_step():
        if kind == "inference":
            L = layers[0]
            orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, X)
            return
        if kind == "stack":
            from coo_spmm_fwd_amd.workloads import f32_to_bf16_bits
            A = X
            for li, L in enumerate(layers):
                H, _ = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, A)
                if li + 1 < len(layers):
                    A = f32_to_bf16_bits(orc.gelu(H).astype(np.float32))
            return
        if kind == "mlp":
            L1, L2 = layers
            H, _ = orc.spmm_fwd(L1.out, L1.in_, L1.rows, L1.cols, L1.vals, X)
            A = orc.gelu(H).astype(np.float32)
            orc.spmm_fwd(L2.out, L2.in_, L2.rows, L2.cols, L2.vals, A)
            dA, _ = orc.spmm_bwd_input(L2.out, L2.in_, L2.rows, L2.cols, L2.vals, dY)
            orc.spmm_bwd_values(L2.out, L2.in_, canon[1]["rows"], canon[1]["cols"], dY, A)
            dH = (dA * orc.gelu_grad(H)).astype(np.float32)
            orc.spmm_bwd_input(L1.out, L1.in_, L1.rows, L1.cols, L1.vals, dH)
            orc.spmm_bwd_values(L1.out, L1.in_, canon[0]["rows"], canon[0]["cols"], dH, X)
            return
        L = layers[0]
        orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, X)
        orc.spmm_bwd_input(L.out, L.in_, L.rows, L.cols, L.vals, dY)
        orc.spmm_bwd_values(L.out, L.in_, canon[0]["rows"], canon[0]["cols"], dY, X)
        if kind == "dst":
            c = canon[0]
            orc.restructure(L.out, L.in_, c["rows"], c["cols"], c["vals"], n_prune, seed, 1)

    reps, t_all = 0, 0.0
    while True:
        t0 = time.perf_counter()
        one_step()
        t_all += time.perf_counter() - t0
        reps += 1
        if t_all >= budget_s or reps >= 100:
            break
    step_s = t_all / reps
    nbytes = step_bytes(kind, layers, B, n_prune)
    return {"value": round(nbytes / step_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full step(s) of the same workload and batch on one core, {step_s * 1e3:.1f} ms per step"}


# ------------------------------------------------------------------ steps
def dense_baselines(kind, layers, uploaded, X, dY, B, ours_ms, steps=20):
    """The same step with torch's dense matmul (hipBLASLt) on the same shapes: a dense layer, and
    Dense+Mask (the weight multiplied by its 0/1 mask before use, the weight gradient masked after).
    Warm (one copy).  A restructure has no dense counterpart here, so a DST step is compared on its
    products only.  Also checks that the dense forward agrees with the layer's."""
    import torch
    dev = X.device
    dt = X.dtype
    Ws, Ms = [], []
    for L, (r, c, v) in zip(layers, uploaded):
        Wd = torch.zeros((L.out, L.in_), dtype=dt, device=dev)
        Wd[r.long(), c.long()] = v
        Ws.append(Wd)
        Ms.append((Wd != 0).to(dt))

    def gelu_parts(H):
        cdf = 0.5 * (1.0 + torch.erf(H * 0.7071067811865476))
        return H * cdf, cdf + H * torch.exp(-0.5 * H * H) * 0.3989422804014327

    def step(masked):
        W = [w * m for w, m in zip(Ws, Ms)] if masked else Ws
        if kind == "inference":
            return X @ W[0].t()
        if kind == "stack":
            A = X
            for li, w in enumerate(W):
                A = A @ w.t()
                if li + 1 < len(W):
                    A = torch.nn.functional.gelu(A)
            return A
        if kind == "mlp":
            H = X @ W[0].t()
            A, G = gelu_parts(H)
            Y = A @ W[1].t()
            dA = dY @ W[1]
            dW2 = dY.t() @ A
            dH = dA * G
            dX = dH @ W[0]
            dW1 = dH.t() @ X
            if masked:
                dW1, dW2 = dW1 * Ms[0], dW2 * Ms[1]
            return Y
        Y = X @ W[0].t()
        dX = dY @ W[0]
        dWd = dY.t() @ X
        if masked:
            dWd = dWd * Ms[0]
        return Y

    res = {}
    for name, masked in (("dense", False), ("dense_mask", True)):
        for _ in range(3):
            step(masked)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            step(masked)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"ms_per_step": round(ms, 5), "ratio": round(ms / ours_ms, 2)}
    res["note"] = ("torch dense matmul (hipBLASLt) on the same shapes and dtype, warm; ratio = their step "
                   "time / ours" + (" (products only: no restructure on the dense side)" if kind == "dst" else ""))
    return res, Ws


def practical_ceiling(nbytes, stream, launches=100):
    """Same-stream references for the dominant kernel, each as the average over `launches` back-to-back
    launches captured in one HIP graph (so the host's launch rate does not enter): a device copy moving
    the same number of bytes (half read, half written) through buffers cycled past the last-level cache,
    and a one-element torch add (the launch floor)."""
    import torch
    half = max(4, (nbytes // 2) // 4 * 4)
    nbuf = max(2, -(-(600 << 20) // half))  # > 2 x 256 MiB of buffers, so copies read HBM
    bufs = [torch.empty(half // 4, dtype=torch.float32, device="cuda") for _ in range(nbuf)]
    tiny = torch.zeros(1, device="cuda")
    for b in bufs:
        b.fill_(1.0)
    torch.cuda.synchronize()

    def timed(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):  # captured on torch's side stream, replayed on the bench stream
            body()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()  # warm
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / launches

    def copies():
        for i in range(launches):
            bufs[(2 * i + 1) % nbuf].copy_(bufs[(2 * i) % nbuf])

    def adds():
        for _ in range(launches):
            tiny.add_(1.0)

    copy_us = timed(copies)
    empty_us = timed(adds)
    del bufs
    moved = 2 * half
    return {"copy_bytes": moved, "copy_us": round(copy_us, 3), "copy_gbs": round(moved / (copy_us * 1e-6) / 1e9, 1),
            "copy_frac": round(moved / (copy_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4), "empty_kernel_us": round(empty_us, 3),
            "note": "torch device copy of the dominant kernel's algorithmic bytes (half read, half written), cold "
                    "buffers, and a one-element torch add; each averaged over 100 launches replayed from one HIP graph"}


def workload_kind(w) -> str:
    if w.dtype == "bf16":
        return "stack" if len(w.layers) > 1 else "inference"
    if len(w.layers) == 2:
        return "mlp"
    if w.prune_frac > 0:
        return "dst"
    return "linear"


def step_bytes(kind, layers, B, n_prune=0):
    """Algorithmic bytes of one step: forward + input gradient + value gradient of every layer
    (forward only for inference), plus 36 B per entry for a restructure."""
    tot = 0
    for L in layers:
        sv = 2 if L.dtype == "bf16" else 4
        tot += bytes_fwd(L.nnz, L.out, L.in_, B, sv=sv, sx=sv)
        if kind not in ("inference", "stack"):
            tot += bytes_dx(L.nnz, L.out, L.in_, B) + bytes_dw(L.nnz, L.out, L.in_, B)
    if kind == "dst":
        tot += 36 * layers[0].nnz
    return tot


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
    ap.add_argument("--no-baselines", action="store_true", help="skip the dense and Dense+Mask torch baselines")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic_counters.json")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, workload=args.workload, batch=args.batch)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each MI355X runs its own layer). Run with --gpus 1.", file=sys.stderr)
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
    kind = workload_kind(w)
    B = args.batch or (max(w.batches) if kind == "mlp" else w.batches[0])
    if B not in acts:
        acts[B] = dict(X=W.random_dense((B, layers[0].in_), 11, dtype=w.dtype),
                       dY=W.random_dense((B, layers[-1].out), 12, dtype=w.dtype))
    n_prune = int(w.prune_frac * layers[0].nnz) if kind == "dst" else 0
    sbytes = step_bytes(kind, layers, B, n_prune)
    # bytes one step touches in one replica: both index orders, both value orders, dW, dense operands
    if kind in ("inference", "stack"):  # forward only: column index, value, task list, X and Y
        sv = 2 if w.dtype == "bf16" else 4
        touched = sum(L.nnz * (4 + sv) + 16 * (L.out + L.nnz // 512) + sv * B * (L.in_ + L.out) for L in layers)
    else:
        touched = sum(L.nnz * 28 + 4 * B * (3 * L.in_ + 2 * L.out) for L in layers)
    R = 1 if args.warm else max(2, -(-2 * MALL_BYTES // touched) + 1)
    # Steps per captured graph: a graph launch costs ~18 us of host time and ~7 us on the GPU, more
    # than a small step itself, so several consecutive steps (over consecutive replicas) share one
    # graph, as a launch-bound training or serving loop would capture them.  Exactly K steps are timed.
    S = next(d for d in (10, 8, 5, 4, 2, 1) if args.steps % d == 0)
    if args.eager or workload_kind(w) == "dst":
        S = 1
    if not args.warm:
        R = -(-R // S) * S

    def t(a):
        if a.dtype.name == "uint16":
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    uploaded = [(t(L.rows), t(L.cols), t(L.vals)) for L in layers]
    reps = []
    for j in range(R):
        st = {"h": [csp.sparse_layer_create(L.out, L.in_, *u) for L, u in zip(layers, uploaded)],
              "X": t(acts[B]["X"]), "dY": t(acts[B]["dY"])}
        if kind == "stack":
            st.update(acts=[torch.empty((B, L.out), device=dev, dtype=torch.bfloat16) for L in layers])
        elif kind == "mlp":
            L1, L2 = layers
            st.update(H=torch.empty((B, L1.out), device=dev), A=torch.empty((B, L1.out), device=dev),
                      Y=torch.empty((B, L2.out), device=dev), dA=torch.empty((B, L1.out), device=dev),
                      dH=torch.empty((B, L1.out), device=dev), dX=torch.empty((B, L1.in_), device=dev),
                      dW1=torch.empty((L1.nnz,), device=dev), dW2=torch.empty((L2.nnz,), device=dev))
        else:
            L = layers[0]
            st.update(Y=torch.empty((B, L.out), device=dev, dtype=st["X"].dtype))
            if kind != "inference":
                st.update(dX=torch.empty((B, L.in_), device=dev), dW=torch.empty((L.nnz,), device=dev))
        reps.append(st)

    ld = 1
    while ld < min(B, 64):
        ld *= 2
    # kernel names as the profiler prints them (template arguments: batch width, element type,
    # 64-bit offsets, epilogue 0 none / 1 forward bias+activation / 2 input gradient times act')
    dt_name = "csp::BF16" if w.dtype == "bf16" else "csp::F32"

    esz = 2 if w.dtype == "bf16" else 4
    lds_on = os.environ.get("COOSPMM_LDS_TABLES", "1")[:1] != "0"

    def lds_fits(n, segment=False):
        """The library gathers from an LDS copy of an operand of n columns (2 <= B <= 64,
        <= 64 KiB; the segment passes also need every segment to be at most 64 tasks)."""
        if segment and -(-n // 512) > 64:
            return False
        return lds_on and 2 <= B <= 64 and n * ld * esz <= (64 << 10)

    grouped_on = os.environ.get("COOSPMM_GROUPED_SPLITS", "1")[:1] != "0"
    import numpy as np

    # longest row and column of each layer (segments over 512 entries are split into tasks);
    # computed once here, outside every timed loop
    seg_max = {}
    for L in layers:
        seg_max[id(L)] = tuple(int(np.bincount(a, minlength=n).max()) if L.nnz else 0
                               for a, n in ((L.rows, L.out), (L.cols, L.in_)))

    def longest(L, rows):
        return seg_max[id(L)][0 if rows else 1]

    # The last template argument of the segment kernels is 1 when the pass's task list has no
    # split segment (every task stores its output), else 0.
    def fwd_name(L, epi=0):
        ks = int(longest(L, True) <= 512)
        if lds_fits(L.in_, segment=True):
            return f"k_segment_lds<{ld}, {dt_name}, {epi}>"
        # split rows finish inside the pass when no row can exceed 64 tasks
        if grouped_on and B <= 8 and not ks and L.in_ <= 64 * 512:
            return f"k_segment_grouped<{ld}, {dt_name}, false, {epi}>"
        return f"k_segment_spmm<{ld}, {dt_name}, false, {epi}, {ks}>"

    def grad_name(L, epi=0):
        ks = int(longest(L, False) <= 512)
        if lds_fits(max(L.in_, L.out)):
            return f"k_gradients_lds<{ld}, {dt_name}, {epi}, {ks}>"
        # spmm_bwd runs both gradient passes in one launch unless their two batch-minor
        # operand tables exceed 2 MiB together (then the two kernels run back to back)
        if esz * ld * (L.in_ + L.out) > (2 << 20):
            return f"k_segment_spmm<{ld}, {dt_name}, false, {epi}, {ks}> + k_values_rows<{ld}, {dt_name}, false>"
        return f"k_gradients<{ld}, {dt_name}, false, {epi}, {ks}>"

    def calls(st, stream):
        """The library calls of one step as (label, layer handle, thunk, main kernel name, algorithmic bytes)."""
        out = []
        if kind == "stack":
            for li, (h, L) in enumerate(zip(st["h"], layers)):
                src = st["X"] if li == 0 else st["acts"][li - 1]

                def f(h=h, src=src, dst=st["acts"][li], last=li + 1 == len(layers)):
                    # GELU fused into the producing layer's epilogue
                    csp.spmm_fwd_act(h, src, act="none" if last else "gelu", Y=dst, stream=stream)

                out.append((f"forward {li + 1}", h, f, fwd_name(L, 1), bytes_fwd(L.nnz, L.out, L.in_, B, sv=2, sx=2)))
            return out
        if kind == "mlp":
            (h1, h2), (L1, L2) = st["h"], layers

            # GELU in the first layer's forward epilogue (A = GELU(H), H kept), GELU' in the
            # second layer's input-gradient epilogue (dH = (dY W2) * GELU'(H))
            def f1():
                csp.spmm_fwd_act(h1, st["X"], act="gelu", Y=st["A"], H=st["H"], stream=stream)

            def b2():
                csp.spmm_bwd_act(h2, st["dY"], st["A"], st["H"], act="gelu", dX=st["dH"], dW=st["dW2"],
                                 stream=stream)

            out.append(("forward 1", h1, f1, fwd_name(L1, 1), bytes_fwd(L1.nnz, L1.out, L1.in_, B)))
            out.append(("forward 2", h2, lambda: csp.spmm_fwd(h2, st["A"], st["Y"], stream=stream), fwd_name(L2),
                        bytes_fwd(L2.nnz, L2.out, L2.in_, B)))
            out.append(("backward 2", h2, b2, grad_name(L2, 2), bytes_gradients(L2.nnz, L2.out, L2.in_, B)))
            out.append(("backward 1", h1, lambda: csp.spmm_bwd(h1, st["dH"], st["X"], st["dX"], st["dW1"],
                                                               stream=stream), grad_name(L1),
                        bytes_gradients(L1.nnz, L1.out, L1.in_, B)))
            return out
        h, L = st["h"][0], layers[0]
        sv = 2 if w.dtype == "bf16" else 4
        out.append(("forward", h, lambda: csp.spmm_fwd(h, st["X"], st["Y"], stream=stream), fwd_name(L),
                    bytes_fwd(L.nnz, L.out, L.in_, B, sv=sv, sx=sv)))
        if kind != "inference":
            out.append(("backward", h, lambda: csp.spmm_bwd(h, st["dY"], st["X"], st["dX"], st["dW"], stream=stream),
                        grad_name(L), bytes_gradients(L.nnz, L.out, L.in_, B)))
        return out

    stream = torch.cuda.current_stream()

    def run_calls(st, s):
        for _, _, fn, _, _ in calls(st, s):
            fn()

    step_no = [0]

    def after(st):  # the part of a step that cannot be captured (restructure reads back and syncs)
        if kind == "dst":
            csp.restructure(st["h"][0], n_prune, seed=w.seed, step=step_no[0], stream=stream)
            step_no[0] += 1

    for i in range(max(args.warmup, R)):  # eager warm-up; also sizes every layer's operand workspace
        run_calls(reps[i % R], stream)
        after(reps[i % R])
    torch.cuda.synchronize()

    graphs = []
    # A restructure rebuilds the task lists (their sizes set launch grids), so a
    # step that restructures is launched eagerly rather than from a captured graph.
    use_graphs = not args.eager and kind != "dst"
    if use_graphs:  # graph j runs steps over replicas jS .. jS + S - 1
        for j in range(max(1, R // S)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for t in range(S):
                    run_calls(reps[(j * S + t) % R], torch.cuda.current_stream())
            graphs.append(g)
        for i in range(-(-args.warmup // S)):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()

    # timed region: exactly K steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    if graphs:
        for i in range(args.steps // S):
            graphs[i % len(graphs)].replay()
    else:
        for i in range(args.steps):
            run_calls(reps[i % R], stream)
            after(reps[i % R])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # second pass, same work, eager: the library attaches a pair of HIP events to each call's main
    # kernel dispatch (sparse_layer_time_next), so each pair carries that kernel's own start and end
    K = args.steps
    labels = [c[0] for c in calls(reps[0], stream)]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in labels]
          for _ in range(K)]
    for row in ev:
        for a, b in row:
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()
    # Hold the GPU with a spin kernel while the K steps are queued, so that they run back to back
    # as in the timed region instead of each waiting for its launch from the host.
    if kind != "dst" and hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(2.0e9 * min(0.2, 1e-4 * K * len(labels))))
    for i in range(K):
        for (label, h, fn, _, _), (a, b) in zip(calls(reps[i % R], stream), ev[i]):
            csp.sparse_layer_time_next(h, a, b)
            fn()
        after(reps[i % R])
    torch.cuda.synchronize()
    per_call = {}
    for ci, (label, _, _, kname, kbytes) in enumerate(calls(reps[0], stream)):
        ts = sorted(ev[i][ci][0].elapsed_time(ev[i][ci][1]) * 1e3 for i in range(K))
        us = sum(ts) / K
        med = ts[K // 2] if K % 2 else 0.5 * (ts[K // 2 - 1] + ts[K // 2])
        per_call[label] = {"kernel": kname, "us": us, "median_us": med, "bytes": kbytes}
    dom_label = max(per_call, key=lambda k: per_call[k]["us"])
    dom = per_call[dom_label]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    traffic = traffic_for(dom["kernel"], {"workload": args.workload, "batch": B})

    restructure_ms = restructure_grad_ms = None
    if kind in ("linear", "dst"):  # one restructure of 10% of the entries (second call: steady state)
        for k in range(2):
            torch.cuda.synchronize()
            r0 = time.perf_counter()
            csp.restructure(reps[0]["h"][0], layers[0].nnz // 10, seed=w.seed, step=12345 + k, stream=stream)
            restructure_ms = (time.perf_counter() - r0) * 1e3
        for k in range(2):  # the gradient-informed variant, scored with this batch's dY and X
            torch.cuda.synchronize()
            r0 = time.perf_counter()
            csp.restructure_grad(reps[0]["h"][0], layers[0].nnz // 10, reps[0]["dY"], reps[0]["X"], stream=stream)
            restructure_grad_ms = (time.perf_counter() - r0) * 1e3

    baselines = None
    if not args.no_baselines:
        ours_ms = ms_per_step
        if kind == "dst":  # products only, eager like the timed steps
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.steps):
                run_calls(reps[i % R], stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ours_ms = e0.elapsed_time(e1) / args.steps
        X0, dY0 = reps[0]["X"], reps[0]["dY"]
        current = [csp.sparse_layer_export(h) for h in reps[0]["h"]]  # after any restructures
        baselines, Ws = dense_baselines(kind, layers, current, X0, dY0, B, ours_ms)
        if kind not in ("mlp", "stack"):  # the dense forward must agree with the layer's
            Yd = (X0.float() @ Ws[0].float().t())
            Ys = csp.spmm_fwd(reps[0]["h"][0], X0).float()
            baselines["forward_max_abs_diff"] = float((Yd - Ys).abs().max())
        baselines["ours_ms_per_step"] = round(ours_ms, 5)
        del Ws

    # not in counter runs: the calibration copy must be the run's only large copy
    ceiling = None if args.calibrate_copy else practical_ceiling(dom["bytes"], stream)

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
    for st in reps:
        for h in st["h"]:
            csp.sparse_layer_destroy(h)

    value = sbytes / (ms_per_step * 1e-3) / 1e9
    flops = sum(2 * L.nnz * B * (1 if kind in ("inference", "stack") else 3) for L in layers)
    steps_desc = {"stack": f"{len(layers)} x spmm_fwd with GELU between (one token batch through the stack)",
                  "linear": "spmm_fwd + spmm_bwd (dX and dW)",
                  "dst": f"spmm_fwd + spmm_bwd + restructure({n_prune} of {layers[0].nnz})",
                  "inference": "spmm_fwd",
                  "mlp": "fwd1 with GELU epilogue, fwd2, bwd2 (dA * GELU'(H) epilogue, dW2), bwd1 (dX, dW1)"}[kind]
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
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "layers": [{"out": L.out, "in": L.in_, "nnz": L.nnz} for L in layers], "batch": B,
                   "sparsity": round(1 - layers[0].nnz / (layers[0].out * layers[0].in_), 4), "step": steps_desc,
                   "replicas": R, "cache": "warm" if args.warm else "cold",
                   "launch": f"hip_graph, {S} steps per graph" if use_graphs else "eager"},
        "gflops": round(flops / (ms_per_step * 1e-3) / 1e9, 2),
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": dom["kernel"], "call": dom_label, "avg_launch_us": round(dom["us"], 3),
                     "median_launch_us": round(dom["median_us"], 3),
                     "bytes_per_launch": dom["bytes"], "ceiling": ceiling},
        "kernels_us": {k: round(v["us"], 3) for k, v in per_call.items()},
        "restructure_ms": None if restructure_ms is None else round(restructure_ms, 3),
        "restructure_grad_ms": None if restructure_grad_ms is None else round(restructure_grad_ms, 3),
        "wall_s": round(wall, 3),
    }
    if baselines is not None:
        rec["dense_baselines"] = baselines
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(kind, layers, acts, B, n_prune, w.seed)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
