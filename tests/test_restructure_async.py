"""restructure_async: the restructure step enqueued without host synchronization, for graph capture.

It must leave exactly the layer restructure leaves for the same seed and step values (every canonical
and index array bit for bit, every product after it), with its step read from and advanced on the
device; one step is also pinned to the oracle directly.  A whole dynamic-sparse-training step
(products, SGD on the values, refresh of the column-ordered copy, restructure_async) captured in one
graph and replayed must track an eager twin layer step by step.  Calls that need the task lists
while their counts are pending refuse to run under capture (an error, not a stale launch).
"""
import numpy as np
import pytest
import torch

import oracle
from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import FP32_REL, assert_within, bits, dev, host

pytestmark = pytest.mark.gpu

SMALL = (900, 700, 40000)
TILED = (8192 + 37, 8192 + 100, int(0.05 * (8192 + 37) * (8192 + 100)))   # fp32 with LDS tiles


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def twins(shape, seed):
    out, in_, nnz = shape
    L = W.random_layer(out, in_, nnz, seed=seed)
    mk = lambda: csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    return L, mk(), mk()


def same_layer(h1, h2, what):
    a = [host(t) for t in csp.sparse_layer_export(h1) + csp.sparse_layer_export_index(h1)]
    b = [host(t) for t in csp.sparse_layer_export(h2) + csp.sparse_layer_export_index(h2)]
    names = ("rows", "cols", "vals", "row_ptr", "perm_c", "rows_by_col", "col_ptr")
    for n, x, y in zip(names, a, b):
        assert np.array_equal(bits(x) if x.dtype == np.float32 else x, bits(y) if y.dtype == np.float32 else y), \
            f"{what}: {n} differs"


@pytest.mark.parametrize("shape", [SMALL, TILED], ids=["small", "tiled"])
def test_async_matches_eager(shape):
    out, in_, nnz = shape
    L, h1, h2 = twins(shape, 11)
    try:
        n_prune, seed, s0 = nnz // 10, 12, 40
        step = torch.tensor([s0], dtype=torch.int64, device="cuda")
        for k in range(3):
            csp.restructure(h1, n_prune, seed, s0 + k, regrow_value=0.5)
            csp.restructure_async(h2, n_prune, seed, step, regrow_value=0.5)
            torch.cuda.synchronize()
            same_layer(h1, h2, f"step {k}")
        assert int(step.item()) == s0 + 3, "the device step counter did not advance once per call"
        # products before the pending task counts are read back (tile path at B = 64 on the tiled
        # layer), then calls that need them (B = 8), which read them back first
        for B in (64, 8):
            X = dev(W.random_dense((B, in_), 13 + B))
            dY = dev(W.random_dense((B, out), 14 + B))
            for name, fn in (("forward", lambda h: csp.spmm_fwd(h, X)),
                             ("input gradient", lambda h: csp.spmm_bwd_input(h, dY)),
                             ("both gradients", lambda h: torch.cat([t.flatten() for t in csp.spmm_bwd(h, dY, X)]))):
                assert np.array_equal(bits(host(fn(h1))), bits(host(fn(h2)))), f"{name} at B={B}"
        csp.sparse_layer_sync(h2)
        csp.restructure(h2, n_prune, seed, s0 + 3)   # eager after async
        csp.restructure(h1, n_prune, seed, s0 + 3)
        same_layer(h1, h2, "eager step after the async ones")
    finally:
        csp.sparse_layer_destroy(h1)
        csp.sparse_layer_destroy(h2)


def test_async_step_against_oracle(orc):
    out, in_, nnz = SMALL
    L = W.random_layer(out, in_, nnz, seed=21)
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        c = orc.canonicalize(out, in_, L.rows, L.cols, L.vals)
        step = torch.tensor([7], dtype=torch.int64, device="cuda")
        csp.restructure_async(h, nnz // 10, 22, step, regrow_value=0.25)
        csp.sparse_layer_sync(h)
        rr, rc, rv, _ = orc.restructure(out, in_, c["rows"], c["cols"], c["vals"], nnz // 10, 22, 7, regrow_value=0.25)
        r, cc, v = (host(t) for t in csp.sparse_layer_export(h))
        assert np.array_equal(r, rr) and np.array_equal(cc, rc)
        assert np.array_equal(bits(v), bits(rv))
    finally:
        csp.sparse_layer_destroy(h)


def test_captured_dst_step_tracks_eager_twin():
    """Forward, both gradients, SGD on the values, refresh of the column-ordered copy and
    restructure_async, captured once on the tiled layer at B = 64 and replayed: after every replay the
    layer and the step's outputs equal those of an eager twin run with the same step values."""
    out, in_, nnz = TILED
    L, h1, h2 = twins(TILED, 31)
    try:
        B, lr, n_prune, seed, s0 = 64, 0.01, nnz // 10, 32, 100
        X = dev(W.random_dense((B, in_), 33))
        dY = dev(W.random_dense((B, out), 34))
        Y2 = torch.empty((B, out), device="cuda")
        dX2 = torch.empty((B, in_), device="cuda")
        dW2 = torch.empty(nnz, device="cuda")
        step = torch.tensor([s0], dtype=torch.int64, device="cuda")
        v2 = csp.sparse_layer_values_tensor(h2)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s = torch.cuda.current_stream()
            csp.spmm_fwd(h2, X, Y2, stream=s)
            csp.spmm_bwd(h2, dY, X, dX2, dW2, stream=s)
            v2.sub_(lr * dW2)
            csp.sparse_layer_set_values(h2, None, stream=s)
            csp.restructure_async(h2, n_prune, seed, step, stream=s)
        for k in range(3):
            Y1 = csp.spmm_fwd(h1, X)
            dX1, dW1 = csp.spmm_bwd(h1, dY, X)
            v1 = csp.sparse_layer_values_tensor(h1)
            v1.sub_(lr * dW1)
            csp.sparse_layer_set_values(h1, None)
            csp.restructure(h1, n_prune, seed, s0 + k)
            g.replay()
            torch.cuda.synchronize()
            for name, a, b in (("Y", Y1, Y2), ("dX", dX1, dX2), ("dW", dW1, dW2)):
                assert torch.equal(a, b), f"replay {k}: {name}"
            same_layer(h1, h2, f"replay {k}")
        assert int(step.item()) == s0 + 3
        csp.sparse_layer_sync(h2)
        del g
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h1)
        csp.sparse_layer_destroy(h2)


def test_pending_counts_refused_under_capture():
    out, in_, nnz = SMALL
    L = W.random_layer(out, in_, nnz, seed=41)
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        step = torch.tensor([0], dtype=torch.int64, device="cuda")
        csp.restructure_async(h, nnz // 10, 42, step)
        X = dev(W.random_dense((8, in_), 43))
        Y = torch.empty((8, out), device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with pytest.raises(csp.CspError, match="sparse_layer_sync"):
            with torch.cuda.graph(g):
                csp.spmm_fwd(h, X, Y, stream=torch.cuda.current_stream())
        del g
        torch.cuda.synchronize()
        csp.sparse_layer_sync(h)   # then the call works, eagerly or captured
        csp.spmm_fwd(h, X, Y)
        torch.cuda.synchronize()
    finally:
        csp.sparse_layer_destroy(h)


def test_async_refusals(monkeypatch):
    out, in_, nnz = SMALL
    L = W.random_layer(out, in_, nnz, seed=51)
    step = torch.tensor([0], dtype=torch.int64, device="cuda")
    monkeypatch.setenv("COOSPMM_RESTRUCTURE", "sorted")   # a layer without position bitmaps
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        with pytest.raises(csp.CspError, match="bitmaps"):
            csp.restructure_async(h, nnz // 10, 1, step)
    finally:
        csp.sparse_layer_destroy(h)
    monkeypatch.delenv("COOSPMM_RESTRUCTURE")
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        with pytest.raises(csp.CspError):
            csp.restructure_async(h, nnz + 1, 1, step)
        with pytest.raises((TypeError, ValueError)):
            csp.restructure_async(h, 10, 1, torch.zeros(2, dtype=torch.int64, device="cuda"))
        csp.restructure_async(h, 0, 1, step)   # nothing to do: the step stays
        torch.cuda.synchronize()
        assert int(step.item()) == 0
    finally:
        csp.sparse_layer_destroy(h)


def products_equal(h1, h2, X, dY, what):
    for name, fn in (("forward", lambda h: csp.spmm_fwd(h, X)),
                     ("input gradient", lambda h: csp.spmm_bwd_input(h, dY)),
                     ("both gradients", lambda h: torch.cat([t.flatten() for t in csp.spmm_bwd(h, dY, X)]))):
        assert np.array_equal(bits(host(fn(h1))), bits(host(fn(h2)))), f"{what}: {name}"


def test_task_lists_left_to_first_reader():
    """On a layer with LDS tiles restructure_async leaves the task lists to the first call that reads
    them: an eager restructure straight after it rebuilds them itself, a call that needs them is
    refused under capture, and sparse_layer_sync builds them.  Products at a batch off the tile
    path (B = 8) then equal an eager twin's bit for bit."""
    out, in_, nnz = TILED
    L, h1, h2 = twins(TILED, 61)
    try:
        n_prune, seed, B = nnz // 10, 62, 8
        X = dev(W.random_dense((B, in_), 63))
        dY = dev(W.random_dense((B, out), 64))
        Y = torch.empty((B, out), device="cuda")
        step = torch.tensor([5], dtype=torch.int64, device="cuda")
        csp.restructure(h1, n_prune, seed, 5)
        csp.restructure_async(h2, n_prune, seed, step)
        csp.restructure(h1, n_prune, seed, 6)
        csp.restructure(h2, n_prune, seed, 6)   # straight after the async step
        same_layer(h1, h2, "eager step after an async one")
        products_equal(h1, h2, X, dY, "after the eager step")
        step.fill_(7)
        csp.restructure(h1, n_prune, seed, 7)
        csp.restructure_async(h2, n_prune, seed, step)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with pytest.raises(csp.CspError, match="sparse_layer_sync"):
            with torch.cuda.graph(g):
                csp.spmm_fwd(h2, X, Y, stream=torch.cuda.current_stream())
        del g
        torch.cuda.synchronize()
        csp.sparse_layer_sync(h2)
        same_layer(h1, h2, "async step, then sync")
        products_equal(h1, h2, X, dY, "after sync")
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h1)
        csp.sparse_layer_destroy(h2)


@pytest.mark.parametrize("shape", [SMALL, TILED], ids=["small", "tiled"])
def test_replayed_async_then_task_readers(shape):
    """A captured restructure_async changes the layer at every replay, which host state cannot
    follow: each later call that needs the task lists rebuilds (tiled layer) and reads them back
    first, so products at B = 8 equal an eager twin's after every replay; such a call cannot itself
    be captured."""
    out, in_, nnz = shape
    L, h1, h2 = twins(shape, 71)
    try:
        n_prune, seed, s0, B = nnz // 10, 72, 300, 8
        X = dev(W.random_dense((B, in_), 73))
        dY = dev(W.random_dense((B, out), 74))
        Y = torch.empty((B, out), device="cuda")
        step = torch.tensor([s0], dtype=torch.int64, device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            csp.restructure_async(h2, n_prune, seed, step, stream=torch.cuda.current_stream())
        for k in range(2):
            g.replay()
            csp.restructure(h1, n_prune, seed, s0 + k)
            torch.cuda.synchronize()
            same_layer(h1, h2, f"replay {k}")
            products_equal(h1, h2, X, dY, f"replay {k}")
        g2 = torch.cuda.CUDAGraph()
        with pytest.raises(csp.CspError, match="captured restructure_async"):
            with torch.cuda.graph(g2):
                csp.spmm_fwd(h2, X, Y, stream=torch.cuda.current_stream())
        del g2
        torch.cuda.synchronize()
        csp.sparse_layer_sync(h2)
        del g
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h1)
        csp.sparse_layer_destroy(h2)


def test_async_capture_refused_after_task_reader_captured():
    """A captured product that reads the task lists has its launch sizes fixed at capture; a
    captured restructure_async on the same layer would make them stale, so its capture is refused
    (and the layer stays usable: the same call runs eagerly)."""
    out, in_, nnz = SMALL
    L = W.random_layer(out, in_, nnz, seed=81)
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        X = dev(W.random_dense((8, in_), 82))
        Y = torch.empty((8, out), device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            csp.spmm_fwd(h, X, Y, stream=torch.cuda.current_stream())
        g.replay()
        torch.cuda.synchronize()
        step = torch.tensor([0], dtype=torch.int64, device="cuda")
        g2 = torch.cuda.CUDAGraph()
        with pytest.raises(csp.CspError, match="captured calls that read"):
            with torch.cuda.graph(g2):
                csp.restructure_async(h, nnz // 10, 83, step, stream=torch.cuda.current_stream())
        del g2
        torch.cuda.synchronize()
        assert int(step.item()) == 0
        csp.restructure_async(h, nnz // 10, 83, step)
        csp.sparse_layer_sync(h)
        assert int(step.item()) == 1
        del g
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h)


def test_short_async_batch_refuses_layer(monkeypatch):
    """A batch with fewer empty, first-seen positions than were pruned (forced here with a batch of
    64 candidates) sets the device flag: the step counter still advances, the next synchronizing call
    reports the short regrow, and the layer is refused from then on."""
    out, in_, nnz = SMALL
    L = W.random_layer(out, in_, nnz, seed=91)
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        monkeypatch.setenv("COOSPMM_REGROW_BATCH", "64")
        step = torch.tensor([3], dtype=torch.int64, device="cuda")
        csp.restructure_async(h, nnz // 10, 92, step)
        torch.cuda.synchronize()
        assert int(step.item()) == 4
        with pytest.raises(csp.CspError, match="fewer empty positions"):
            csp.sparse_layer_sync(h)
        X = dev(W.random_dense((8, in_), 93))
        with pytest.raises(csp.CspError):
            csp.spmm_fwd(h, X)
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h)


def test_pending_task_lists_with_packed_rows(orc):
    """The packed row list (forward at B <= 4) through the pending task lists: after the first narrow
    forward a restructure rebuilds it, so the lists restructure_async left pending on the tiled layer
    are built with it by the next narrow forward.  Twice, each time against an eager twin bit for
    bit (the first time both on the plain list, then both on the packed one), and once against the
    oracle."""
    out, in_, nnz = TILED
    L, h1, h2 = twins(TILED, 111)
    try:
        n_prune, seed = nnz // 10, 112
        step = torch.tensor([50], dtype=torch.int64, device="cuda")
        for k in range(2):
            csp.restructure(h1, n_prune, seed, 50 + k)
            csp.restructure_async(h2, n_prune, seed, step)
            torch.cuda.synchronize()
            same_layer(h1, h2, f"step {k}")
            for B in (2, 4):
                X = dev(W.random_dense((B, in_), 113 + B))
                assert np.array_equal(bits(host(csp.spmm_fwd(h1, X))), bits(host(csp.spmm_fwd(h2, X)))), \
                    f"step {k}, B = {B}"
        X = dev(W.random_dense((2, in_), 117))
        r, c, v = (host(t) for t in csp.sparse_layer_export(h2))
        ref, S = orc.spmm_fwd(out, in_, r, c, v, host(X))
        assert_within(host(csp.spmm_fwd(h2, X)), ref, S, FP32_REL, "forward at B = 2 after the async steps")
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h1)
        csp.sparse_layer_destroy(h2)
