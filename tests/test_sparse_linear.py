"""SparseLinear (torch module + autograd) against the oracle: forward, both gradients through
autograd, an optimizer step through the zero-copy values parameter, and a restructure."""
import gc
import weakref

import numpy as np
import pytest
import torch

import oracle
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import FP32_REL, assert_within, bits, dev, host


def test_module_imports_without_gpu():
    from coo_spmm_fwd_amd.sparse_linear import SparseLinear
    assert "truly sparse" in SparseLinear.__doc__ or "COO" in SparseLinear.__doc__


def test_layer_owner_outlives_its_views():
    """The owner destroys its layer exactly once, only after the last view that holds it is gone
    (a stand-in destroy callback: no library call)."""
    from coo_spmm_fwd_amd import binding as csp
    destroyed = []
    owner = csp.LayerOwner(1234, destroy=destroyed.append)
    views = [csp._DeviceArray(0x1000, 4, "<f4", owner), csp._DeviceArray(0x1000, 4, "<f4", owner)]
    del owner
    gc.collect()
    assert destroyed == []
    views.pop()
    assert destroyed == []
    views.pop()
    gc.collect()
    assert destroyed == [1234]


@pytest.mark.gpu
def test_values_parameter_outlives_module():
    """An optimizer may hold the values parameter after the module is gone: the view keeps the
    layer alive, still reads and writes its buffer, and the layer goes with the last view."""
    from coo_spmm_fwd_amd.sparse_linear import SparseLinear
    L = W.random_layer(300, 200, 9000, seed=57)
    m = SparseLinear(dev(L.rows), dev(L.cols), dev(L.vals), 300, 200)
    m.restructure(900, 2, 0)                      # the parameter now views a buffer made by the restructure
    v = m.values
    want = host(v.detach()).copy()
    owner = weakref.ref(m._owner)
    del m
    gc.collect()
    assert owner() is not None
    torch.cuda.synchronize()
    assert np.array_equal(bits(host(v.detach())), bits(want))
    with torch.no_grad():
        v.mul_(2.0)
    assert np.array_equal(bits(host(v.detach())), bits(want * np.float32(2.0)))
    del v
    gc.collect()
    assert owner() is None


@pytest.mark.gpu
def test_sparse_linear_autograd_step_and_restructure():
    from coo_spmm_fwd_amd.sparse_linear import SparseLinear
    orc = oracle.default()
    out, in_, nnz, B = 600, 450, 27000, 12
    L = W.random_layer(out, in_, nnz, seed=51)
    m = SparseLinear(dev(L.rows), dev(L.cols), dev(L.vals), out, in_)
    c = orc.canonicalize(out, in_, L.rows, L.cols, L.vals)
    rows, cols, vals = c["rows"], c["cols"], c["vals"]
    assert np.array_equal(bits(host(m.values.detach())), bits(vals))

    X_h = W.random_dense((B, in_), 5)
    dY_h = W.random_dense((B, out), 6)
    X = dev(X_h).requires_grad_(True)
    Y = m(X)
    ref, S = orc.spmm_fwd(out, in_, rows, cols, vals, X_h)
    assert_within(host(Y.detach()), ref, S, FP32_REL, "module forward")
    Y.backward(dev(dY_h))
    ref, S = orc.spmm_bwd_input(out, in_, rows, cols, vals, dY_h)
    assert_within(host(X.grad), ref, S, FP32_REL, "autograd dX")
    ref, S = orc.spmm_bwd_values(out, in_, rows, cols, dY_h, X_h)
    assert_within(host(m.values.grad), ref, S, FP32_REL, "autograd dW")

    # An optimizer step writes the layer in place; the next forward and backward see it.
    opt = torch.optim.SGD(m.parameters(), lr=0.5)
    opt.step()
    new_vals = host(m.values.detach().clone())
    assert not np.array_equal(new_vals, vals)
    X2 = dev(X_h).requires_grad_(True)
    Y2 = m(X2)
    ref, S = orc.spmm_fwd(out, in_, rows, cols, new_vals, X_h)
    assert_within(host(Y2.detach()), ref, S, FP32_REL, "forward after the optimizer step")
    Y2.backward(dev(dY_h))
    ref, S = orc.spmm_bwd_input(out, in_, rows, cols, new_vals, dY_h)
    assert_within(host(X2.grad), ref, S, FP32_REL, "dX after the optimizer step")

    # Restructure through the module: the layer and the re-pointed parameter hold the oracle's result.
    r0 = orc.restructure(out, in_, rows, cols, new_vals, 2700, 9, 4, 0.0)
    m.restructure(2700, 9, 4)
    r, c_, v = (host(t) for t in m.coo())
    assert np.array_equal(r, r0[0]) and np.array_equal(c_, r0[1]) and np.array_equal(bits(v), bits(r0[2]))
    assert np.array_equal(bits(host(m.values.detach())), bits(r0[2]))
    dense = host(m.to_dense())
    assert np.count_nonzero(dense) <= nnz and dense[r0[0][5], r0[1][5]] == r0[2][5]
    del m
