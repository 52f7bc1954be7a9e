"""The product calls can be captured in a HIP graph: every replay equals the eager result bit for bit.

Replays are interleaved with the program's own eager work and synchronizations.
"""
import pytest
import torch

from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B", [1, 16, 64])
def test_graph_replay_matches_eager(B):
    L = W.random_layer(2000, 1500, 120000, seed=31 + B)
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        X = dev(W.random_dense((B, L.in_), 1))
        dY = dev(W.random_dense((B, L.out), 2))
        Y_ref = csp.spmm_fwd(h, X)
        dX_ref, dW_ref = csp.spmm_bwd(h, dY, X)
        torch.cuda.synchronize()
        Y = torch.full_like(Y_ref, float("nan"))
        dX = torch.full_like(dX_ref, float("nan"))
        dW = torch.full_like(dW_ref, float("nan"))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s = torch.cuda.current_stream()
            csp.spmm_fwd(h, X, Y, stream=s)
            csp.spmm_bwd(h, dY, X, dX, dW, stream=s)
        for rep in range(4):
            Y.fill_(float("nan"))
            dX.fill_(float("nan"))
            dW.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y, Y_ref), rep
            assert torch.equal(dX, dX_ref), rep
            assert torch.equal(dW, dW_ref), rep
            # eager work between replays, on other buffers
            csp.spmm_fwd(h, dev(W.random_dense((B, L.in_), 10 + rep)))
            torch.cuda.synchronize()
        del g
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h)


@pytest.mark.parametrize("B", [16, 130])
def test_first_calls_captured(orc, B):
    """A fresh layer's very first product calls are captured: nothing in them allocates (the workspace is
    sized at create; B = 130 runs as three slices of at most 64 rows).  Replays match the oracle, and a
    layer used eagerly afterwards gives the same bits."""
    import numpy as np

    from tests.gpu_util import FP32_REL, assert_within, host
    L = W.random_layer(900, 700, 40000, seed=77 + B)
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        Xh, dYh = W.random_dense((B, L.in_), 3), W.random_dense((B, L.out), 4)
        X, dY = dev(Xh), dev(dYh)
        Y = torch.empty((B, L.out), device="cuda")
        dX = torch.empty((B, L.in_), device="cuda")
        dW = torch.empty((L.nnz,), device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s = torch.cuda.current_stream()
            csp.spmm_fwd(h, X, Y, stream=s)
            csp.spmm_bwd(h, dY, X, dX, dW, stream=s)
        for rep in range(3):
            g.replay()
            torch.cuda.synchronize()
            c = orc.canonicalize(L.out, L.in_, L.rows, L.cols, L.vals)
            ref, S = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, Xh)
            assert_within(host(Y), ref, S, FP32_REL, f"captured forward, replay {rep}")
            refx, Sx = orc.spmm_bwd_input(L.out, L.in_, L.rows, L.cols, L.vals, dYh)
            assert_within(host(dX), refx, Sx, FP32_REL, f"captured dX, replay {rep}")
            refw, Sw = orc.spmm_bwd_values(L.out, L.in_, c["rows"], c["cols"], dYh, Xh)
            assert_within(host(dW), refw, Sw, FP32_REL, f"captured dW, replay {rep}")
        Ye = host(csp.spmm_fwd(h, X))
        dXe, dWe = (host(t) for t in csp.spmm_bwd(h, dY, X))
        assert np.array_equal(Ye, host(Y)) and np.array_equal(dXe, host(dX)) and np.array_equal(dWe, host(dW))
        del g
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h)


@pytest.mark.parametrize("B", [64, 100])
def test_graph_replay_tiled_layer(B):
    """An 8192-square fp32 layer takes the LDS tiles at batch chunks of 33..64 (forward and input
    gradient: a tile pass and the reduce of its partial sums; value gradient: the tile pass): every
    replay of the captured calls equals the eager result bit for bit (B = 100: two slices)."""
    L = W.random_layer(8192, 8192, 8192 * 8192 // 100, seed=41 + B)
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        X = dev(W.random_dense((B, L.in_), 3))
        dY = dev(W.random_dense((B, L.out), 4))
        Y_ref = csp.spmm_fwd(h, X)
        dX_ref, dW_ref = csp.spmm_bwd(h, dY, X)
        torch.cuda.synchronize()
        Y = torch.full_like(Y_ref, float("nan"))
        dX = torch.full_like(dX_ref, float("nan"))
        dW = torch.full_like(dW_ref, float("nan"))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s = torch.cuda.current_stream()
            csp.spmm_fwd(h, X, Y, stream=s)
            csp.spmm_bwd(h, dY, X, dX, dW, stream=s)
        for rep in range(3):
            Y.fill_(float("nan"))
            dX.fill_(float("nan"))
            dW.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y, Y_ref), rep
            assert torch.equal(dX, dX_ref), rep
            assert torch.equal(dW, dW_ref), rep
            csp.spmm_bwd(h, dev(W.random_dense((B, L.out), 20 + rep)), X)   # eager work between replays
            torch.cuda.synchronize()
        del g
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h)
