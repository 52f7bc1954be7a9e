"""spmm_fwd_static -- the forward for callers that cannot allocate -- through the C ABI: its output
equals spmm_fwd's bit for bit (same task-list kernels, its workspace in the library's static per-GPU
array) and the oracle's within 1e-5 * S, over two calls in a row (the second with a smaller input)
and a third on another layer; on a layer where spmm_fwd takes the LDS-tile path it equals the
task-list path bit for bit and the tile path to rounding; a layer and batch whose workspace exceeds
the array are refused on the host before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import FP32_REL, assert_within, dev, host

pytestmark = pytest.mark.gpu


def long_row_layer(out, in_, nnz, seed):
    """Uniform entries plus rows 0 and out - 1 full (longer than one 512-entry task: split rows)."""
    rng = W.streams(seed, 1)[0]
    flat = rng.choice((out - 2) * in_, size=nnz, replace=False) + in_
    rows = np.concatenate([np.zeros(in_, np.int64), np.full(in_, out - 1), flat // in_]).astype(np.int32)
    cols = np.concatenate([np.arange(in_), np.arange(in_), flat % in_]).astype(np.int32)
    v = rng.standard_normal(rows.size).astype(np.float32)
    return W.CooWeights(out, in_, rows, cols, v, "f32")


def call_static(h, X, B, Y):
    lib = csp.load()
    return lib.spmm_fwd_static(ctypes.c_void_p(h), ctypes.c_void_p(X.data_ptr()), B, ctypes.c_void_p(Y.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def check(orc, L, h, B, seed):
    Xh = W.random_dense((B, L.in_), seed)
    X = dev(Xh)
    Y = torch.full((B, L.out), float("nan"), device="cuda")
    assert call_static(h, X, B, Y) == 0, csp.sparse_layer_last_error()
    got = host(Y)
    want = host(csp.spmm_fwd(h, X))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"B={B}: differs from spmm_fwd"
    ref, S = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, Xh)
    assert_within(got, ref, S, FP32_REL, f"spmm_fwd_static B={B}")


def test_static_forward_matches_spmm_fwd(orc):
    big = long_row_layer(3000, 2500, 200_000, seed=41)     # split rows; B = 64 and 16 gather a copy of X
    small = W.random_layer(700, 900, 20_000, seed=42)
    hb = csp.sparse_layer_create(big.out, big.in_, dev(big.rows), dev(big.cols), dev(big.vals))
    hs = csp.sparse_layer_create(small.out, small.in_, dev(small.rows), dev(small.cols), dev(small.vals))
    try:
        check(orc, big, hb, 64, 1)   # first call on the device: largest workspace
        check(orc, big, hb, 16, 2)   # second call in a row, smaller input (split rows, partial sums)
        check(orc, small, hs, 5, 3)  # another layer, smaller again
        check(orc, big, hb, 70, 4)   # two slices (64 + 6 rows)
    finally:
        csp.sparse_layer_destroy(hb)
        csp.sparse_layer_destroy(hs)


def test_static_forward_refuses_oversized_workspace():
    """in = 70000 fp32 columns at B = 64 needs a 17.9 MB copy of X: refused before any launch."""
    r = torch.tensor([0, 5], dtype=torch.int32, device="cuda")
    c = torch.tensor([3, 69999], dtype=torch.int32, device="cuda")
    h = csp.sparse_layer_create(10, 70000, r, c, torch.ones(2, device="cuda"))
    try:
        X = torch.randn(64, 70000, device="cuda")
        Y = torch.full((64, 10), 7.0, device="cuda")
        st = call_static(h, X, 64, Y)
        assert st == -1 and "static" in csp.sparse_layer_last_error()
        torch.cuda.synchronize()
        assert torch.all(Y == 7.0)   # nothing ran
        Y2 = torch.empty(1, 10, device="cuda")
        assert call_static(h, X[:1].contiguous(), 1, Y2) == 0   # one row needs no copy
        assert torch.equal(Y2, csp.spmm_fwd(h, X[:1].contiguous()))
    finally:
        csp.sparse_layer_destroy(h)


def test_static_forward_on_a_tiled_layer(orc, monkeypatch):
    """8192 x 8192 at 5%, B = 64: spmm_fwd runs the LDS tiles there (their partial sums do not fit the
    static array), the static variant the task list.  It must equal spmm_fwd with the tiles switched
    off bit for bit, and the tiled output within twice the fp32 bound."""
    L = W.random_layer(8192, 8192, 3_355_443, seed=44)
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        Xh = W.random_dense((64, L.in_), 45)
        X = dev(Xh)
        Y = torch.full((64, L.out), float("nan"), device="cuda")
        assert call_static(h, X, 64, Y) == 0, csp.sparse_layer_last_error()
        got = host(Y)
        monkeypatch.setenv("COOSPMM_SEGMENT_TILES", "0")
        plain = host(csp.spmm_fwd(h, X))
        monkeypatch.delenv("COOSPMM_SEGMENT_TILES")
        tiled = host(csp.spmm_fwd(h, X))
        assert np.array_equal(got.view(np.uint32), plain.view(np.uint32)), "differs from the task-list forward"
        _, S = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, Xh)
        assert_within(got, tiled.astype(np.float64), S, 2 * FP32_REL, "static against the tiled forward")
    finally:
        csp.sparse_layer_destroy(h)
