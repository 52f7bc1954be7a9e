"""Throughput of the truly sparse COO layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--batch B] [--warm]

One step is one training pass of the layer over one batch: spmm_fwd, then
spmm_bwd (input gradient and value gradient).  The default workload is the
dynamic-sparse-training layer 8192 x 8192 at 95% unstructured sparsity
(3,355,443 stored fp32 entries), batch 64; its full training step (products,
an SGD update of the stored values, the refresh of their column-ordered copy
and a prune-and-regrow restructure of 10% of the entries) is timed beside the
products step.

Inputs are resident in HBM before timing starts.  Unless --warm is given,
every step, from the first warm-up step to the last step of the per-kernel
timing pass, runs on replica g mod R of the layer and its dense operands (g
counts steps), with R chosen so that the other R - 1 replicas between two uses
of one replica touch more than twice the 256 MiB last-level cache: each step
reads its data from HBM.

Printed: one JSON line.  `value` is the effective bandwidth of the products
step: algorithmic bytes of forward + input gradient + value gradient (byte
models below; the input gradient reads the layer's column-ordered value copy,
so it is charged 8 bytes per entry, and the copy's refresh belongs to the
training step that changes the values) over the measured step time.
`roofline` covers the dominant kernel, timed with a pair of HIP events that
the library attaches to that kernel's dispatch, in a second pass over the
same replicas; its `ceiling` holds a same-byte device copy and the launch
floor measured on the same stream.  `cpu_baseline` times the CPU oracle (plain
C loops, fp64 accumulation, one core) and, beside it, the same loops in fp32
on every host core.  `page_ratios` holds the pages' three ratio metrics
(kernel at 95%, training and inference at 90%) against torch's dense and
Dense+Mask layers on the same GPU, under the same cold protocol.
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
DEFAULT_WORKLOAD = "dst8192_b64_s95"
RATIO_WORKLOAD_90 = "linear4096_b16_s90"
SGD_LR = 1e-3


# ------------------------------------------------------------------ byte models
def bytes_fwd(nnz, out, in_, B, sv=4, sx=4):
    """Forward: column index + value per entry, row offsets, X read once, Y written once."""
    return nnz * (sv + 4) + 4 * (out + 1) + sx * B * (in_ + out)


def bytes_dx(nnz, out, in_, B):
    """Input gradient, permuted-read model: gathered value + permutation + row index per entry,
    column offsets, dY read once, dX written once."""
    return nnz * (4 + 4 + 4) + 4 * (in_ + 1) + 4 * B * (in_ + out)


def bytes_dx_mirror(nnz, out, in_, B, sv=4, sx=4):
    """Input gradient over the column-ordered value copy: row index + copied value per entry,
    column offsets, dY read once, dX written once."""
    return nnz * (4 + sv) + 4 * (in_ + 1) + sx * B * (in_ + out)


def bytes_dw(nnz, out, in_, B):
    """Value gradient: column index read + dW written per entry, row offsets, X and dY."""
    return nnz * (4 + 4) + 4 * (out + 1) + 4 * B * (in_ + out)


def bytes_gradients(nnz, out, in_, B):
    """Both gradients in one launch: input gradient over the transposed view (row index and
    column-ordered value per entry) and value gradient over rows (column index read, dW written
    per entry); both offset arrays; X and dY read once; dX written once."""
    return nnz * 16 + 4 * (in_ + 1) + 4 * (out + 1) + 4 * B * (2 * in_ + out)


def bytes_restructure(nnz):
    """Prune-and-regrow with re-sort: read the 12-byte triples, write canonical and transposed arrays."""
    return 36 * nnz


def bytes_sgd_refresh(nnz):
    """SGD on the stored values (read value and dW, write value) and the column-ordered copy's refresh
    (read the permutation, gather the value, write the copy)."""
    return 12 * nnz + 12 * nnz


def source_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(label: str, launch_args: dict):
    """HBM bytes per launch from committed counter runs, if taken on the current kernel source."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{launch_args['workload']}/B={launch_args['batch']}/{label}"
    e = rec.get(key)
    if not e or e.get("source_sha") != source_sha():
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


def ingest_counters(fetch_dir, write_dir, workload, batch, label, kernel, copy_mib=256):
    """Scale each counter by what it reads for a plain copy of known size, then store the bytes per
    launch of `kernel` (a run made with --only, so one op's kernel) under workload/B/label."""
    fetch, write = _counter_rows(fetch_dir), _counter_rows(write_dir)
    copy_bytes = copy_mib << 20
    # the calibration copy is the only copy dispatch of that size (the largest copy grid of the run)
    big = [r for r in fetch + write if COPY_KERNEL_KEY in r.get("Kernel_Name", "")]
    gmax = max((int(r["Grid_Size"]) for r in big), default=0)
    is_copy = lambda n: COPY_KERNEL_KEY in n
    fetch_c = [r for r in fetch if is_copy(r.get("Kernel_Name", "")) and int(r["Grid_Size"]) == gmax]
    write_c = [r for r in write if is_copy(r.get("Kernel_Name", "")) and int(r["Grid_Size"]) == gmax]
    cf, _ = _per_dispatch(fetch_c, "FETCH_SIZE", lambda n: True)
    cw, _ = _per_dispatch(write_c, "WRITE_SIZE", lambda n: True)
    if not cf or not cw:
        raise SystemExit("no calibration copy in the counter runs (run them with --calibrate-copy)")
    f_scale, w_scale = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    # a call of several launches ("a + b") moves the sum of its kernels' bytes
    kf = kw = 0.0
    nf, nw = [], []
    for name in (k.strip() for k in kernel.split(" + ")):
        f1, n1 = _per_dispatch(fetch, "FETCH_SIZE", lambda n, k=name: k in n)
        w1, n2 = _per_dispatch(write, "WRITE_SIZE", lambda n, k=name: k in n)
        if f1 is None or w1 is None:
            raise SystemExit(f"kernel {name!r} not in the counter runs")
        kf, kw = kf + f1, kw + w1
        nf.append(n1)
        nw.append(n2)
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[f"{workload}/B={batch}/{label}"] = {
        "kernel": kernel, "source_sha": source_sha(), "fetch_kib_raw": kf, "write_kib_raw": kw,
        "dispatches": [nf, nw], "copy_scale": {"fetch": f_scale, "write": w_scale, "copy_bytes": copy_bytes},
        "hbm_bytes_per_launch": round(kf * 1024 * f_scale + kw * 1024 * w_scale)}
    os.makedirs(os.path.dirname(PROFILE_TRAFFIC), exist_ok=True)
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1))


# ------------------------------------------------------------------ CPU baselines
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(kind, layers, acts, B, sbytes, n_prune=0, seed=0, budget_s=10.0):
    """The oracle as written (fp64 loops, one core) on the products step of the same workload and
    batch, repeated until ~budget_s; beside it the same loops in fp32 over every host core
    (oracle/parallel.c, median of 5 after one warm-up) and, for a training workload, the oracle's
    restructure once."""
    import numpy as np
    import oracle
    from oracle import parallel
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

    reps, t_all = 0, 0.0
    while True:
        t0 = time.perf_counter()
        one_step()
        t_all += time.perf_counter() - t0
        reps += 1
        if t_all >= budget_s or reps >= 100:
            break
    step_s = t_all / reps
    rec = {"value": round(sbytes / step_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{reps} full products step(s) of the same workload and batch on one core, "
                     f"{step_s * 1e3:.1f} ms per step", "cpu_model": cpu_model()}
    if kind == "dst":
        c = canon[0]
        t0 = time.perf_counter()
        orc.restructure(layers[0].out, layers[0].in_, c["rows"], c["cols"], c["vals"], n_prune, seed, 1)
        rec["restructure_ms"] = round((time.perf_counter() - t0) * 1e3, 1)
    if kind in ("linear", "dst", "inference") and layers[0].dtype == "f32":
        par = parallel.Parallel()
        L, c = layers[0], canon[0]

        def par_step():
            par.spmm_fwd(c, L.out, L.in_, X)
            if kind != "inference":
                par.spmm_bwd_input(c, L.out, L.in_, dY)
                par.spmm_bwd_values(c, L.out, L.in_, dY, X)

        par_step()
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            par_step()
            ts.append(time.perf_counter() - t0)
        med = sorted(ts)[2]
        rec["all_cores"] = {"value": round(sbytes / med / 1e9, 3), "unit": "GB/s", "cores": par.threads,
                            "affinity_cores": len(os.sched_getaffinity(0)), "kind": "fp32 loops, OpenMP",
                            "sample": f"median of 5 products steps after one warm-up, {med * 1e3:.2f} ms per step"}
    return rec


# ------------------------------------------------------------------ cold replica cycle
class Cycle:
    """Step g runs on replica g mod R, through warm-up, graph uploads, timed steps and the timing
    pass, so a step's previous use of its replica lies R - 1 steps back."""

    def __init__(self, R):
        self.R, self.g = R, 0

    def next(self):
        r = self.g % self.R
        self.g += 1
        return r


def replicas_for(touched, warm):
    return 1 if warm else max(2, -(-2 * MALL_BYTES // touched) + 1)


# ------------------------------------------------------------------ dense references
def dense_layers(layers, uploaded, dt, dev):
    import torch
    Ws, Ms = [], []
    for L, (r, c, v) in zip(layers, uploaded):
        Wd = torch.zeros((L.out, L.in_), dtype=dt, device=dev)
        Wd[r.long(), c.long()] = v.to(dt)
        Ws.append(Wd)
        Ms.append((Wd != 0).to(dt))
    return Ws, Ms


def dense_step_fn(kind, masked, forward_only=False):
    """The step with torch's dense matmul (hipBLASLt): a dense layer, or Dense+Mask (the weight
    multiplied by its 0/1 mask before use, the weight gradient masked after)."""
    import torch

    def gelu_parts(H):
        cdf = 0.5 * (1.0 + torch.erf(H * 0.7071067811865476))
        return H * cdf, cdf + H * torch.exp(-0.5 * H * H) * 0.3989422804014327

    def step(Ws, Ms, X, dY):
        W = [w * m for w, m in zip(Ws, Ms)] if masked else Ws
        if kind in ("inference",) or forward_only:
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
    return step


def time_dense(kind, layers, uploaded, X, dY, steps, warm, forward_only=False):
    """ms per step of the dense and Dense+Mask steps, each cycling through enough copies of its
    weights (and masks) that a copy's reuse distance passes twice the last-level cache."""
    import torch
    dt, dev = X.dtype, X.device
    W0, M0 = dense_layers(layers, uploaded, dt, dev)
    res = {}
    esz = X.element_size()
    for name, masked in (("dense", False), ("dense_mask", True)):
        per = sum(w.numel() for w in W0) * esz * (2 if masked else 1)
        R = replicas_for(per, warm)
        copies = [([w.clone() for w in W0], [m.clone() for m in M0] if masked else M0) for _ in range(R)]
        fn = dense_step_fn(kind, masked, forward_only)
        cyc = Cycle(R)
        for _ in range(max(3, R)):
            Ws, Ms = copies[cyc.next()]
            fn(Ws, Ms, X, dY)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            Ws, Ms = copies[cyc.next()]
            fn(Ws, Ms, X, dY)
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"ms_per_step": round(e0.elapsed_time(e1) / steps, 5), "copies": R}
        del copies
    Yd = (X.float() @ W0[0].float().t()) if kind not in ("mlp", "stack") else None
    del W0, M0
    torch.cuda.empty_cache()
    return res, Yd


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
    if w.ops == "fwd":
        return "inference"
    return "linear"


def step_bytes(kind, layers, B):
    """Algorithmic bytes of one products step: forward + input gradient (over the column-ordered value
    copy) + value gradient of every layer, forward only for inference."""
    tot = 0
    for L in layers:
        sv = 2 if L.dtype == "bf16" else 4
        tot += bytes_fwd(L.nnz, L.out, L.in_, B, sv=sv, sx=sv)
        if kind not in ("inference", "stack"):
            tot += bytes_dx_mirror(L.nnz, L.out, L.in_, B, sv=sv, sx=sv) + bytes_dw(L.nnz, L.out, L.in_, B)
    return tot


# ------------------------------------------------------------------ one workload, measured
class Bench:
    """A workload's replicas on the GPU, its step as library calls, the cold replica cycle, graph
    replay of the timed steps and the per-kernel timing pass."""

    def __init__(self, name, B=None, warm=False, only=None, steps=100, eager=False):
        import numpy as np
        import torch
        from coo_spmm_fwd_amd import binding as csp
        from coo_spmm_fwd_amd import workloads as W
        self.csp, self.torch = csp, torch
        self.name, self.only = name, only
        w, layers, acts = W.build(name)
        self.w, self.layers, self.acts = w, layers, acts
        self.kind = kind = workload_kind(w)
        self.B = B = B or (max(w.batches) if kind == "mlp" else w.batches[0])
        if B not in acts:
            acts[B] = dict(X=W.random_dense((B, layers[0].in_), 11, dtype=w.dtype),
                           dY=W.random_dense((B, layers[-1].out), 12, dtype=w.dtype))
        self.dev = dev = torch.device("cuda", 0)
        self.esz = esz = 2 if w.dtype == "bf16" else 4
        # bytes one step touches in one replica
        if kind in ("inference", "stack"):  # forward only: column index, value, task list, X and Y
            touched = sum(L.nnz * (4 + esz) + 16 * (L.out + L.nnz // 512) + esz * B * (L.in_ + L.out)
                          for L in layers)
        else:  # both index orders, both value orders, dW, dense operands and their batch-minor copies
            touched = sum(L.nnz * 28 + 4 * B * (3 * L.in_ + 2 * L.out) for L in layers)
        self.touched = touched
        # S consecutive steps per captured graph (S divides the timed steps); the cycle's length is a
        # multiple of S, so the graphs partition it
        self.S = 1 if eager else next(d for d in (10, 8, 5, 4, 2, 1) if steps % d == 0)
        self.R = replicas_for(touched, warm)
        if self.R > 1:
            self.R = -(-self.R // self.S) * self.S
        self.uploaded = [(self.t(L.rows), self.t(L.cols), self.t(L.vals)) for L in layers]
        self.reps = [self.make_replica() for _ in range(self.R)]
        self.ld = 1
        while self.ld < min(B, 64):
            self.ld *= 2
        # longest row and column of each layer (segments over 512 entries are split into tasks)
        self.seg_max = {id(L): tuple(int(np.bincount(a, minlength=n).max()) if L.nnz else 0
                                     for a, n in ((L.rows, L.out), (L.cols, L.in_))) for L in layers}
        self.cycle = Cycle(self.R)

    def t(self, a):
        torch = self.torch
        if a.dtype.name == "uint16":
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(self.dev)
        return torch.from_numpy(a).to(self.dev)

    def make_replica(self):
        torch, csp, B, kind, dev = self.torch, self.csp, self.B, self.kind, self.dev
        layers = self.layers
        st = {"h": [csp.sparse_layer_create(L.out, L.in_, *u) for L, u in zip(layers, self.uploaded)],
              "X": self.t(self.acts[B]["X"]), "dY": self.t(self.acts[B]["dY"])}
        ld = csp.batch_minor_ld(B)
        if kind == "stack":
            st.update(acts=[torch.empty((B, L.out), device=dev, dtype=torch.bfloat16) for L in layers])
            if B >= 2:  # batch-minor copies handed from layer to layer (pad slots stay zero)
                st.update(XT=torch.zeros((layers[0].in_, ld), device=dev, dtype=torch.bfloat16),
                          actsT=[torch.zeros((L.out, ld), device=dev, dtype=torch.bfloat16) for L in layers[:-1]])
        elif kind == "mlp":
            L1, L2 = layers
            st.update(H=torch.empty((B, L1.out), device=dev), A=torch.empty((B, L1.out), device=dev),
                      Y=torch.empty((B, L2.out), device=dev), dA=torch.empty((B, L1.out), device=dev),
                      dH=torch.empty((B, L1.out), device=dev), dX=torch.empty((B, L1.in_), device=dev),
                      dW1=torch.empty((L1.nnz,), device=dev), dW2=torch.empty((L2.nnz,), device=dev))
            if B >= 2:
                st.update(XT=torch.zeros((L1.in_, ld), device=dev), AT=torch.zeros((L1.out, ld), device=dev),
                          dHT=torch.zeros((L1.out, ld), device=dev), dYT=torch.zeros((L2.out, ld), device=dev))
        else:
            L = layers[0]
            st.update(Y=torch.empty((B, L.out), device=dev, dtype=st["X"].dtype))
            if kind != "inference":
                st.update(dX=torch.empty((B, L.in_), device=dev), dW=torch.empty((L.nnz,), device=dev))
        return st

    # kernel names as the profiler prints them (template arguments: batch width, element type,
    # 64-bit offsets, epilogue 0 none / 1 forward bias+activation / 2 input gradient times act',
    # and 1 when the pass's task list has no split segment)
    def lds_fits(self, n, segment=False):
        lds_on = os.environ.get("COOSPMM_LDS_TABLES", "1")[:1] != "0"
        if segment and -(-n // 512) > 64:
            return False
        return lds_on and 2 <= self.B <= 64 and n * self.ld * self.esz <= (64 << 10)

    def dt_name(self):
        return "csp::BF16" if self.w.dtype == "bf16" else "csp::F32"

    def tiled(self, L, which):
        """The library's LDS-tile path for this layer and call (fp32, a 64-wide batch chunk, at least one
        512 x 512 tile per compute unit; the environment switches turn it off)."""
        import torch
        env = "COOSPMM_VALUE_TILES" if which == "values" else "COOSPMM_SEGMENT_TILES"
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        return (self.esz == 4 and self.ld == 64 and os.environ.get(env, "1")[:1] != "0"
                and -(-L.out // 512) * -(-L.in_ // 512) >= cus)

    def fwd_name(self, L, epi=0):
        ld, dt, B = self.ld, self.dt_name(), self.B
        if self.tiled(L, "segments"):
            return f"k_segment_tiles + k_tile_reduce<{epi}>"
        ks = int(self.seg_max[id(L)][0] <= 512)
        grouped_on = os.environ.get("COOSPMM_GROUPED_SPLITS", "1")[:1] != "0"
        if self.lds_fits(L.in_, segment=True):
            return f"k_segment_lds<{ld}, {dt}, {epi}>"
        if grouped_on and B <= 8 and not ks and L.in_ <= 64 * 512:
            return f"k_segment_grouped<{ld}, {dt}, false, {epi}>"
        return f"k_segment_spmm<{ld}, {dt}, false, {epi}, {ks}>"

    def dx_name(self, L, epi=0):
        if self.tiled(L, "segments"):
            return f"k_segment_tiles + k_tile_reduce<{epi}>"
        ks = int(self.seg_max[id(L)][1] <= 512)
        return f"k_segment_spmm<{self.ld}, {self.dt_name()}, false, {epi}, {ks}>"

    def dw_name(self, L):
        if self.tiled(L, "values"):
            return "k_values_tiles"
        return f"k_values_rows<{self.ld}, {self.dt_name()}, false>"

    def grad_fused(self, L):
        """spmm_bwd runs both gradient passes in one launch (k_gradients / k_gradients_lds) unless their
        two batch-minor operand tables exceed 2 MiB together (then two kernels back to back)."""
        return self.lds_fits(max(L.in_, L.out)) or self.esz * self.ld * (L.in_ + L.out) <= (2 << 20)

    def grad_name(self, L, epi=0):
        ks = int(self.seg_max[id(L)][1] <= 512)
        if self.lds_fits(max(L.in_, L.out)):
            return f"k_gradients_lds<{self.ld}, {self.dt_name()}, {epi}, {ks}>"
        return f"k_gradients<{self.ld}, {self.dt_name()}, false, {epi}, {ks}>"

    def hands_copies(self):
        """Whether the step hands batch-minor copies from call to call: B >= 2 and the first layer's
        operand table too large for the LDS-table path (which reads row-major operands and copies
        nothing; a one-row operand is its own copy)."""
        return self.kind in ("mlp", "stack") and self.B >= 2 and not self.lds_fits(self.layers[0].in_, segment=True)

    def calls(self, st, stream, split=False):
        """The library calls of one step as (label, layer handle, thunk, main kernel name, algorithmic
        bytes).  split: time the two gradients of a single layer as separate calls when spmm_bwd would
        run them as two kernels anyway (one main kernel per call)."""
        csp, kind, B = self.csp, self.kind, self.B
        out = []
        ld = csp.batch_minor_ld(B)
        copy_bytes = lambda n, s: s * n * (B + ld)  # a batch-minor copy: read [B, n], write [n, ld]
        copies = self.hands_copies()
        if kind == "stack":
            if not copies:
                for li, (h, L) in enumerate(zip(st["h"], self.layers)):
                    src = st["X"] if li == 0 else st["acts"][li - 1]

                    def f(h=h, src=src, dst=st["acts"][li], last=li + 1 == len(self.layers)):
                        # GELU fused into the producing layer's epilogue
                        csp.spmm_fwd_act(h, src, act="none" if last else "gelu", Y=dst, stream=stream)

                    out.append((f"forward {li + 1}", h, f, self.fwd_name(L, 1),
                                bytes_fwd(L.nnz, L.out, L.in_, B, 2, 2)))
                return out
            # B >= 2: the input's copy once, then each layer writes its output's copy for the next
            out.append(("copy of X", None, lambda: csp.spmm_batch_minor(st["X"], st["XT"], stream=stream),
                        "k_batch_minor", copy_bytes(self.layers[0].in_, 2)))
            n = len(self.layers)
            for li, (h, L) in enumerate(zip(st["h"], self.layers)):
                src, srcT = (st["X"], st["XT"]) if li == 0 else (st["acts"][li - 1], st["actsT"][li - 1])
                last = li + 1 == n
                dstT = None if last else st["actsT"][li]

                def f(h=h, src=src, srcT=srcT, dst=st["acts"][li], dstT=dstT, last=last):
                    csp.spmm_fwd_bm(h, src, XT=srcT, act="none" if last else "gelu", Y=dst, YT=dstT, stream=stream)

                out.append((f"forward {li + 1}", h, f, self.fwd_name(L, 0 if last else 1),
                            bytes_fwd(L.nnz, L.out, L.in_, B, 2, 2) + (0 if last else 2 * ld * L.out)))
            return out
        if kind == "mlp" and copies:
            (h1, h2), (L1, L2) = st["h"], self.layers

            # the copies handed along: X's and dY's made by explicit copy calls (each charged with its
            # own bytes and time); A's written by the first forward (read by the second forward and the
            # second backward); dH's written by the second backward (read by the first)
            def c0():
                csp.spmm_batch_minor(st["X"], st["XT"], stream=stream)

            def c1():
                csp.spmm_batch_minor(st["dY"], st["dYT"], stream=stream)

            def f1():
                csp.spmm_fwd_bm(h1, st["X"], XT=st["XT"], act="gelu", Y=st["A"], H=st["H"], YT=st["AT"],
                                stream=stream)

            def f2():
                csp.spmm_fwd_bm(h2, st["A"], XT=st["AT"], Y=st["Y"], stream=stream)

            def b2():
                csp.spmm_bwd_bm(h2, st["dY"], st["A"], dYT=st["dYT"], XT=st["AT"], H_in=st["H"], act="gelu",
                                dX=st["dH"], dXT=st["dHT"], dW=st["dW2"], stream=stream)

            def b1():
                csp.spmm_bwd_bm(h1, st["dH"], st["X"], dYT=st["dHT"], XT=st["XT"], dX=st["dX"], dW=st["dW1"],
                                stream=stream)

            out.append(("copy of X", None, c0, "k_batch_minor", copy_bytes(L1.in_, 4)))
            out.append(("forward 1", h1, f1, self.fwd_name(L1, 1),
                        bytes_fwd(L1.nnz, L1.out, L1.in_, B) + 4 * ld * L1.out))
            out.append(("forward 2", h2, f2, self.fwd_name(L2), bytes_fwd(L2.nnz, L2.out, L2.in_, B)))
            out.append(("copy of dY", None, c1, "k_batch_minor", copy_bytes(L2.out, 4)))
            out.append(("backward 2", h2, b2, self.grad_name(L2, 2),
                        bytes_gradients(L2.nnz, L2.out, L2.in_, B) + 4 * ld * L2.in_))
            out.append(("backward 1", h1, b1, self.grad_name(L1), bytes_gradients(L1.nnz, L1.out, L1.in_, B)))
            return out
        if kind == "mlp":
            (h1, h2), (L1, L2) = st["h"], self.layers

            # GELU in the first layer's forward epilogue (A = GELU(H), H kept), GELU' in the
            # second layer's input-gradient epilogue (dH = (dY W2) * GELU'(H))
            def f1():
                csp.spmm_fwd_act(h1, st["X"], act="gelu", Y=st["A"], H=st["H"], stream=stream)

            def b2():
                csp.spmm_bwd_act(h2, st["dY"], st["A"], st["H"], act="gelu", dX=st["dH"], dW=st["dW2"],
                                 stream=stream)

            out.append(("forward 1", h1, f1, self.fwd_name(L1, 1), bytes_fwd(L1.nnz, L1.out, L1.in_, B)))
            out.append(("forward 2", h2, lambda: csp.spmm_fwd(h2, st["A"], st["Y"], stream=stream),
                        self.fwd_name(L2), bytes_fwd(L2.nnz, L2.out, L2.in_, B)))
            out.append(("backward 2", h2, b2, self.grad_name(L2, 2), bytes_gradients(L2.nnz, L2.out, L2.in_, B)))
            out.append(("backward 1", h1, lambda: csp.spmm_bwd(h1, st["dH"], st["X"], st["dX"], st["dW1"],
                                                               stream=stream), self.grad_name(L1),
                        bytes_gradients(L1.nnz, L1.out, L1.in_, B)))
            return out
        h, L = st["h"][0], self.layers[0]
        sv = self.esz
        ops = {
            "fwd": ("forward", h, lambda: csp.spmm_fwd(h, st["X"], st["Y"], stream=stream), self.fwd_name(L),
                    bytes_fwd(L.nnz, L.out, L.in_, B, sv=sv, sx=sv)),
            "dx": ("input gradient", h, lambda: csp.spmm_bwd_input(h, st["dY"], st["dX"], stream=stream),
                   self.dx_name(L), bytes_dx_mirror(L.nnz, L.out, L.in_, B)),
            "dw": ("value gradient", h, lambda: csp.spmm_bwd_values(h, st["dY"], st["X"], st["dW"], stream=stream),
                   self.dw_name(L), bytes_dw(L.nnz, L.out, L.in_, B)),
        }
        if self.only:
            return [ops[self.only]]
        out.append(ops["fwd"])
        if kind == "inference":
            return out
        if split and not self.grad_fused(L):
            return out + [ops["dx"], ops["dw"]]
        bw = ("backward", h, lambda: csp.spmm_bwd(h, st["dY"], st["X"], st["dX"], st["dW"], stream=stream),
              self.grad_name(L) if self.grad_fused(L) else f"{self.dx_name(L)} + {self.dw_name(L)}",
              bytes_gradients(L.nnz, L.out, L.in_, B) if self.grad_fused(L)
              else bytes_dx_mirror(L.nnz, L.out, L.in_, B) + bytes_dw(L.nnz, L.out, L.in_, B))
        return out + [bw]

    def run_step(self, st, stream):
        for _, _, fn, _, _ in self.calls(st, stream):
            fn()

    def measure(self, steps, warmup, eager=False):
        """Warm-up, graph capture (S consecutive steps per graph), one upload replay of every graph,
        then exactly `steps` timed steps; all on the replica cycle.  Returns ms per step."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        for _ in range(max(warmup, 1)):
            self.run_step(self.reps[self.cycle.next()], stream)
        torch.cuda.synchronize()
        S = self.S
        graphs = []
        if not eager:
            o = self.cycle.g % self.R
            for j in range(max(1, self.R // S)):  # graph j: the next S steps of the cycle
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for t in range(S):
                        self.run_step(self.reps[(o + j * S + t) % self.R], torch.cuda.current_stream())
                graphs.append(g)
            for g in graphs:  # upload replay of every graph, continuing the cycle
                g.replay()
                self.cycle.g += S
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        e0.record(stream)
        if graphs:
            for i in range(steps // S):
                graphs[i % len(graphs)].replay()
                self.cycle.g += S
        else:
            for _ in range(steps):
                self.run_step(self.reps[self.cycle.next()], stream)
        e1.record(stream)
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - wall0
        del graphs
        return e0.elapsed_time(e1) / steps

    def kernel_pass(self, K):
        """Same work, eager, continuing the cycle: the library attaches a pair of HIP events to each
        call's main kernel dispatch (sparse_layer_time_next), so each pair carries that kernel's own
        start and end.  The steps are queued behind a spin kernel so they run back to back."""
        torch, csp = self.torch, self.csp
        stream = torch.cuda.current_stream()
        labels = [c[0] for c in self.calls(self.reps[0], stream, split=True)]
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in labels]
              for _ in range(K)]
        for row in ev:
            for a, b in row:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(2.0e9 * min(0.2, 1e-4 * K * len(labels))))
        for i in range(K):
            st = self.reps[self.cycle.next()]
            for (label, h, fn, _, _), (a, b) in zip(self.calls(st, stream, split=True), ev[i]):
                if h is None:  # a layer-free call (the batch-minor copy): events around it
                    a.record(stream)
                    fn()
                    b.record(stream)
                else:
                    csp.sparse_layer_time_next(h, a, b)
                    fn()
        torch.cuda.synchronize()
        per = {}
        for ci, (label, _, _, kname, kbytes) in enumerate(self.calls(self.reps[0], stream, split=True)):
            # (kernel names and byte models do not depend on the replica)
            ts = sorted(ev[i][ci][0].elapsed_time(ev[i][ci][1]) * 1e3 for i in range(K))
            med = ts[K // 2] if K % 2 else 0.5 * (ts[K // 2 - 1] + ts[K // 2])
            per[label] = {"kernel": kname, "us": sum(ts) / K, "median_us": med, "bytes": kbytes}
        return per

    def dst_steps(self, n, n_prune):
        """The full training step of the DST workload, eager, on the replica cycle: forward, both
        gradients, SGD on the stored values (harness), refresh of the column-ordered copy, restructure
        (which reads back once).  Events bracket the step and the restructure call on the stream."""
        torch, csp = self.torch, self.csp
        stream = torch.cuda.current_stream()
        t_step, t_rs = [], []
        for k in range(-1, n):  # step -1 is an untimed warm-up (first calls of the harness's torch kernels)
            st = self.reps[self.cycle.next()]
            h = st["h"][0]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            csp.spmm_fwd(h, st["X"], st["Y"], stream=stream)
            csp.spmm_bwd(h, st["dY"], st["X"], st["dX"], st["dW"], stream=stream)
            v = csp.sparse_layer_values_tensor(h)
            v.sub_(SGD_LR * st["dW"])
            csp.sparse_layer_set_values(h, None, stream=stream)
            e[1].record(stream)
            csp.restructure(h, n_prune, seed=self.w.seed, step=1000 + k, stream=stream)
            e[2].record(stream)
            torch.cuda.synchronize()
            if k >= 0:
                t_step.append(e[0].elapsed_time(e[2]))
                t_rs.append(e[1].elapsed_time(e[2]))
        # the gradient-informed regrow, scored with each replica's dY and X: one untimed call (the
        # first launches of its kernels in the process), then the mean of three on the next replicas
        t_grad = []
        for k in range(4):
            st = self.reps[self.cycle.next()]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            csp.restructure_grad(st["h"][0], n_prune, st["dY"], st["X"], stream=stream)
            e[1].record(stream)
            torch.cuda.synchronize()
            if k > 0:
                t_grad.append(e[0].elapsed_time(e[1]))
        return sum(t_step) / n, sum(t_rs) / n, sum(t_grad) / len(t_grad)

    def dst_graph_steps(self, n, n_prune):
        """The same full training step with restructure_async in place of restructure, captured per
        replica in two HIP graphs (products + SGD + refresh of the column-ordered copy; the restructure)
        and replayed on the replica cycle.  Events between the two replays time the restructure on its
        own: no launch gaps, no host round trip.  Each replica draws its candidates from its own device
        step counter.  The first pass over the replicas uploads the graphs (untimed); afterwards every
        replica is synchronized (sparse_layer_sync), which would report a short regrow."""
        torch, csp = self.torch, self.csp
        stream = torch.cuda.current_stream()
        caps = []
        for r, st in enumerate(self.reps):
            h = st["h"][0]
            csp.sparse_layer_sync(h)
            v = csp.sparse_layer_values_tensor(h)  # stays the layer's buffer under restructure_async
            step = torch.tensor([5000 + 100 * r], dtype=torch.int64, device=self.dev)
            torch.cuda.synchronize()
            ga, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(ga):
                s = torch.cuda.current_stream()
                csp.spmm_fwd(h, st["X"], st["Y"], stream=s)
                csp.spmm_bwd(h, st["dY"], st["X"], st["dX"], st["dW"], stream=s)
                v.sub_(SGD_LR * st["dW"])
                csp.sparse_layer_set_values(h, None, stream=s)
            with torch.cuda.graph(gb):
                csp.restructure_async(h, n_prune, seed=self.w.seed, step_dev=step, stream=torch.cuda.current_stream())
            caps.append((ga, gb, step, v))
        t_step, t_rs = [], []
        for k in range(len(caps) + n):
            ga, gb = caps[self.cycle.next()][:2]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            ga.replay()
            e[1].record(stream)
            gb.replay()
            e[2].record(stream)
            torch.cuda.synchronize()
            if k >= len(caps):
                t_step.append(e[0].elapsed_time(e[2]))
                t_rs.append(e[1].elapsed_time(e[2]))
        for st in self.reps:
            csp.sparse_layer_sync(st["h"][0])
        del caps
        torch.cuda.synchronize()
        return sum(t_step) / n, sum(t_rs) / n

    def destroy(self):
        self.torch.cuda.synchronize()
        for st in self.reps:
            for h in st["h"]:
                self.csp.sparse_layer_destroy(h)
        self.reps = []


def page_ratios(main, per_call, steps, warm):
    """The pages' ratio metrics on this GPU (their own figures are context, on unnamed hardware):
    the SpMM kernel at 95% sparsity against Dense+Mask (forward of this run's 95% layer), and one
    sparse layer at 90% sparsity, training step and inference (forward), against dense and
    Dense+Mask.  Ours and theirs run under the same cold protocol."""
    import torch
    out = {}
    if main.kind in ("linear", "dst") and abs(main.w.density - 0.05) < 1e-9:
        st = main.reps[0]
        cur = [main.csp.sparse_layer_export(h) for h in st["h"]]
        dn, Yd = time_dense(main.kind, main.layers, cur, st["X"], st["dY"], steps, warm, forward_only=True)
        fwd_us = per_call["forward"]["us"]
        Ys = main.csp.spmm_fwd(st["h"][0], st["X"]).float()
        diff = float((Yd - Ys).abs().max())
        out["kernel_95"] = {"workload": main.name, "ours_forward_kernel_us": round(fwd_us, 3),
                            "dense_forward_us": round(dn["dense"]["ms_per_step"] * 1e3, 3),
                            "dense_mask_forward_us": round(dn["dense_mask"]["ms_per_step"] * 1e3, 3),
                            "vs_dense": round(dn["dense"]["ms_per_step"] * 1e3 / fwd_us, 2),
                            "vs_dense_mask": round(dn["dense_mask"]["ms_per_step"] * 1e3 / fwd_us, 2),
                            "forward_max_abs_diff": diff, "pages": "up to 7x vs Dense+Mask"}
    for label, forward_only in (("training_90", False), ("inference_90", True)):
        b = Bench(RATIO_WORKLOAD_90, warm=warm, only="fwd" if forward_only else None, steps=steps)
        ms = b.measure(steps, 5)
        st = b.reps[0]
        cur = [b.csp.sparse_layer_export(h) for h in st["h"]]
        dn, _ = time_dense(b.kind, b.layers, cur, st["X"], st["dY"], steps, warm, forward_only=forward_only)
        out[label] = {"workload": RATIO_WORKLOAD_90, "batch": b.B, "ours_ms_per_step": round(ms, 5),
                      "dense_ms_per_step": dn["dense"]["ms_per_step"],
                      "dense_mask_ms_per_step": dn["dense_mask"]["ms_per_step"],
                      "vs_dense": round(dn["dense"]["ms_per_step"] / ms, 2),
                      "vs_dense_mask": round(dn["dense_mask"]["ms_per_step"] / ms, 2),
                      "pages": "training 8x / 3.7x, inference 4x / 2x vs Dense+Mask / dense"}
        b.destroy()
        del b
        torch.cuda.empty_cache()
    out["note"] = ("torch dense matmul (hipBLASLt) on the same shapes and dtype; Dense+Mask multiplies the "
                   "weight by its 0/1 mask before use and the weight gradient after; each side cycles through "
                   "enough copies to read HBM; ratio = their time / ours")
    return out


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--warm", action="store_true", help="reuse one replica (cache-resident data)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baselines")
    ap.add_argument("--eager", action="store_true", help="launch each call from Python instead of graph replay")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense baselines, page ratios, DST step, ceiling and CPU baselines")
    ap.add_argument("--only", choices=("fwd", "dx", "dw"), default=None,
                    help="run only this product call of a single-layer workload (for per-kernel counter runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "LABEL", "KERNEL"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of one --only op into "
                         "profiles/traffic_counters.json under workload/B/LABEL")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each MI355X runs its own layer). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.ingest_counters:
        from coo_spmm_fwd_amd import workloads as W
        w = W.WORKLOADS[args.workload]
        ingest_counters(*args.ingest_counters[:2], workload=args.workload, batch=args.batch or w.batches[0],
                        label=args.ingest_counters[2], kernel=args.ingest_counters[3])
        return

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    extras = not (args.no_extras or args.only)

    main_b = Bench(args.workload, args.batch, args.warm, args.only, args.steps, args.eager)
    kind, layers, B = main_b.kind, main_b.layers, main_b.B
    sbytes = step_bytes(kind, layers, B)
    if args.only:
        sbytes = main_b.calls(main_b.reps[0], None)[0][4]
    ms_per_step = main_b.measure(args.steps, args.warmup, eager=args.eager)
    reuse_bytes = (main_b.R - 1) * main_b.touched
    per_call = main_b.kernel_pass(args.steps)
    dom_label = max(per_call, key=lambda k: per_call[k]["us"])
    dom = per_call[dom_label]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    traffic = traffic_for(dom_label, {"workload": args.workload, "batch": B})
    stream = torch.cuda.current_stream()

    dst = None
    if kind == "dst" and extras:
        n_prune = int(main_b.w.prune_frac * layers[0].nnz)
        step_ms, rs_ms, rsg_ms = main_b.dst_steps(5, n_prune)
        gstep_ms, grs_ms = main_b.dst_graph_steps(10, n_prune)
        nnz = layers[0].nnz
        rbytes = bytes_restructure(nnz)
        dbytes = sbytes + bytes_sgd_refresh(nnz) + rbytes
        dst = {"step": f"spmm_fwd + spmm_bwd + SGD on the values (harness, lr {SGD_LR}) + refresh of the "
                       f"column-ordered copy + restructure({n_prune} of {nnz}), eager, on the replica cycle",
               "ms_per_step": round(step_ms, 4), "bytes_per_step": dbytes,
               "gbs": round(dbytes / (step_ms * 1e-3) / 1e9, 2),
               "restructure_ms": round(rs_ms, 4), "restructure_bytes": rbytes,
               "restructure_gbs": round(rbytes / (rs_ms * 1e-3) / 1e9, 2),
               "restructure_frac": round(rbytes / (rs_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
               "restructure_grad_ms": round(rsg_ms, 4),
               "graph": {"step": "the same step with restructure_async (no host read-back), captured per replica "
                                 "in two HIP graphs and replayed on the replica cycle",
                         "ms_per_step": round(gstep_ms, 4), "gbs": round(dbytes / (gstep_ms * 1e-3) / 1e9, 2),
                         "restructure_ms": round(grs_ms, 4),
                         "restructure_gbs": round(rbytes / (grs_ms * 1e-3) / 1e9, 2),
                         "restructure_frac": round(rbytes / (grs_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
               "note": "GPU time between events on the stream; the restructure reads back its accepted count "
                       "once, so its bracket includes that round trip"}

    ratios = page_ratios(main_b, per_call, min(args.steps, 20), args.warm) if extras else None
    ceiling = practical_ceiling(dom["bytes"], stream) if extras and not args.calibrate_copy else None

    if args.calibrate_copy:
        n = (args.calibrate_copy << 20) // 4
        src = torch.randn(n, device="cuda")
        dst_t = torch.empty_like(src)
        for _ in range(3):
            dst_t.copy_(src)
        torch.cuda.synchronize()
        del src, dst_t

    wall = main_b.wall
    R, S = main_b.R, main_b.S
    main_b.destroy()

    value = sbytes / (ms_per_step * 1e-3) / 1e9
    n_ops = 1 if (kind in ("inference", "stack") or args.only) else 3
    flops = sum(2 * L.nnz * B * n_ops for L in layers)
    copies = " (batch-minor copies handed from call to call: the inputs' copies made by explicit copy calls, each " \
             "later operand's copy written by the call that produced it; all charged in the byte model)" \
        if main_b.hands_copies() else ""
    steps_desc = {"stack": f"{len(layers)} x spmm_fwd with GELU between (one token batch through the stack)" + copies,
                  "linear": "spmm_fwd + spmm_bwd (dX and dW)",
                  "dst": "spmm_fwd + spmm_bwd (dX and dW); the full training step is under dst_step",
                  "inference": "spmm_fwd",
                  "mlp": "fwd1 with GELU epilogue, fwd2, bwd2 (dA * GELU'(H) epilogue, dW2), bwd1 (dX, dW1)"
                         + copies}[kind]
    if args.only:
        steps_desc = {"fwd": "spmm_fwd", "dx": "spmm_bwd_input", "dw": "spmm_bwd_values"}[args.only] + " only"
    w = main_b.w
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
                   "reuse_distance_bytes": reuse_bytes,
                   "launch": f"hip_graph, {S} steps per graph" if not args.eager else "eager",
                   "bytes_per_step": sbytes},
        "gflops": round(flops / (ms_per_step * 1e-3) / 1e9, 2),
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": dom["kernel"], "call": dom_label, "avg_launch_us": round(dom["us"], 3),
                     "median_launch_us": round(dom["median_us"], 3),
                     "bytes_per_launch": dom["bytes"], "ceiling": ceiling},
        "kernels_us": {k: round(v["us"], 3) for k, v in per_call.items()},
        "wall_s": round(wall, 3),
    }
    if dst is not None:
        rec["dst_step"] = dst
    if ratios is not None:
        rec["page_ratios"] = ratios
    if extras and not args.no_cpu:
        n_prune = int(w.prune_frac * layers[0].nnz) if kind == "dst" else 0
        rec["cpu_baseline"] = cpu_baseline(kind, layers, main_b.acts, B, sbytes, n_prune, w.seed)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
