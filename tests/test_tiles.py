"""Value gradient through LDS tiles (fp32 layers, batch chunks 33..64 wide) against the task-list
kernel it replaces and against fp64 sums.

The two kernels run the same fused multiply-add chains and add the same pairs, so their results
must be bitwise equal.  Covered here: tiles cut by the layer's edges (out and in not multiples of
the tile), rows longer than the windows loaded ahead (up to 1400 entries, 512 in one tile), empty
rows, batches of one and two chunks (the second chunk accumulates), spmm_bwd_values and spmm_bwd,
and a restructure (the tiles are rebuilt).  Parity with the oracle at the 8192-square full size is
in test_parity; here sampled entries are checked against fp64 sums computed in the test.
"""
import numpy as np
import pytest
import torch

from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import FP32_REL, assert_within, bits, dev, host

pytestmark = pytest.mark.gpu

OUT, IN = 8192 + 37, 8192 + 100   # 17 x 17 tiles of 512 x 512, the last ones partial


def tiled_layer(seed):
    """5% uniform over rows 16.., long dense runs in rows 0..7, rows 8..15 empty."""
    rng = np.random.default_rng(seed)
    L = W.random_layer(OUT - 16, IN, int(0.05 * (OUT - 16) * IN), seed=seed)
    rows, cols, vals = [L.rows + 16], [L.cols], [L.vals]
    for r in range(8):
        span = 700 + 100 * r
        c0 = int(rng.integers(0, IN - span))
        rows.append(np.full(span, r, np.int32))
        cols.append(np.arange(c0, c0 + span, dtype=np.int32))
        vals.append(rng.standard_normal(span).astype(np.float32))
    return (np.concatenate(rows).astype(np.int32), np.concatenate(cols).astype(np.int32),
            np.concatenate(vals).astype(np.float32))


def both(monkeypatch, fn):
    monkeypatch.setenv("COOSPMM_VALUE_TILES", "0")
    a = fn()
    torch.cuda.synchronize()
    monkeypatch.setenv("COOSPMM_VALUE_TILES", "1")
    b = fn()
    torch.cuda.synchronize()
    return a, b


def check_sample(h, dW, X, dY, seed):
    """dW at sampled canonical entries (every long-row entry of row 0 and 3000 others) against fp64."""
    r, c, _ = (host(t) for t in csp.sparse_layer_export(h))
    rng = np.random.default_rng(seed)
    pick = np.unique(np.concatenate([np.nonzero(r == 0)[0], rng.integers(0, len(r), 3000)]))
    Xh, dYh = host(X).astype(np.float64), host(dY).astype(np.float64)
    terms = dYh[:, r[pick]] * Xh[:, c[pick]]
    assert_within(host(dW)[pick], terms.sum(0), np.abs(terms).sum(0), FP32_REL, "tiled value gradient")


@pytest.mark.parametrize("B", [33, 64, 100, 128])
def test_value_tiles_match_task_kernel(monkeypatch, B):
    rows, cols, vals = tiled_layer(61)
    h = csp.sparse_layer_create(OUT, IN, dev(rows), dev(cols), dev(vals))
    try:
        X = dev(W.random_dense((B, IN), 62 + B))
        dY = dev(W.random_dense((B, OUT), 63 + B))
        a, b = both(monkeypatch, lambda: csp.spmm_bwd_values(h, dY, X))
        assert np.array_equal(bits(host(a)), bits(host(b))), "spmm_bwd_values differs between the kernels"
        (ax, aw), (bx, bw) = both(monkeypatch, lambda: csp.spmm_bwd(h, dY, X))
        assert np.array_equal(bits(host(aw)), bits(host(bw))), "spmm_bwd value gradient differs"
        assert np.array_equal(bits(host(ax)), bits(host(bx))), "spmm_bwd input gradient differs"
        assert np.array_equal(bits(host(aw)), bits(host(a)))
        check_sample(h, b, X, dY, B)
    finally:
        csp.sparse_layer_destroy(h)


def test_value_tiles_after_restructure(monkeypatch):
    rows, cols, vals = tiled_layer(67)
    h = csp.sparse_layer_create(OUT, IN, dev(rows), dev(cols), dev(vals))
    try:
        X = dev(W.random_dense((64, IN), 68))
        dY = dev(W.random_dense((64, OUT), 69))
        for step in range(2):
            csp.restructure(h, csp.sparse_layer_nnz(h) // 10, seed=70, step=step, regrow_value=0.5)
            a, b = both(monkeypatch, lambda: csp.spmm_bwd_values(h, dY, X))
            assert np.array_equal(bits(host(a)), bits(host(b))), f"differs after restructure {step}"
            check_sample(h, b, X, dY, 71 + step)
    finally:
        csp.sparse_layer_destroy(h)
