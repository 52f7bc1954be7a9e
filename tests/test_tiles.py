"""The LDS-tile kernels of fp32 layers at batch chunks 33..64 wide, against the oracle and against
the task-list kernels they replace.

Value gradient: the tile kernel runs the task kernel's fused multiply-add chains and adds the same
pairs, so the two must agree bitwise.  Forward and input gradient: the tiles add a segment's
entries per column block and then the blocks in order, so they agree with the oracle within the
fp32 bound (and the fused epilogues within theirs), not bitwise with the task kernel.

The layer has tiles cut by its edges (out and in not multiples of 512), rows longer than the
windows loaded ahead (up to 1400 entries, 512 in one tile), empty rows, and batches of one and two
chunks (the second chunk of the value gradient accumulates).  A restructure rebuilds the tiles of
both views.  An infinite operand value in the first column of a block must not reach the sums of
rows that do not hold that column.
"""
import numpy as np
import pytest
import torch

import oracle
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


ACT_REL = 1.3e-5   # fused GELU / GELU' outputs (derivation in tests/test_epilogue.py)


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


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


@pytest.mark.parametrize("B", [64, 100])
def test_gradient_tiles_one_launch_match_two(orc, monkeypatch, B):
    """spmm_bwd on a tiled layer runs both gradients' tile passes in one launch, one tile of each
    view per workgroup (17 x 17 = 289 of each here, partial ones at the edges).  Its outputs must be
    the bits of the two separate launches, also with the GELU' epilogue and over two batch chunks
    (the second accumulates dW), and dX must match the oracle."""
    rows, cols, vals = tiled_layer(65)
    h = csp.sparse_layer_create(OUT, IN, dev(rows), dev(cols), dev(vals))
    try:
        X = dev(W.random_dense((B, IN), 66 + B))
        dY = W.random_dense((B, OUT), 67 + B)
        Hin = dev(W.random_dense((B, IN), 68 + B))
        out = {}
        for flag in ("0", "1"):
            monkeypatch.setenv("COOSPMM_FUSED_TILES", flag)
            dX, dW = csp.spmm_bwd(h, dev(dY), X)
            dXa, dWa = csp.spmm_bwd_act(h, dev(dY), X, Hin, act="gelu")
            torch.cuda.synchronize()
            out[flag] = [host(t) for t in (dX, dW, dXa, dWa)]
        for k, name in enumerate(("dX", "dW", "dX with GELU'", "dW beside it")):
            assert np.array_equal(bits(out["0"][k]), bits(out["1"][k])), f"{name}: one launch differs from two"
        refx, Sx = orc.spmm_bwd_input(OUT, IN, rows, cols, vals, dY)
        assert_within(out["1"][0], refx, Sx, FP32_REL, f"input gradient of the one-launch tiles B={B}")
        check_sample(h, dev(out["1"][1]), X, dev(dY), 69 + B)
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


@pytest.mark.parametrize("B", [33, 64, 100])
def test_segment_tiles_against_oracle(orc, B):
    """Forward (plain and with bias + GELU), input gradient (plain, times GELU', and inside
    spmm_bwd) through the tiles, each against the oracle on the same inputs."""
    rows, cols, vals = tiled_layer(73)
    h = csp.sparse_layer_create(OUT, IN, dev(rows), dev(cols), dev(vals))
    try:
        X = W.random_dense((B, IN), 74 + B)
        dY = W.random_dense((B, OUT), 75 + B)
        bias = W.random_dense((OUT,), 76)
        ref, S = orc.spmm_fwd(OUT, IN, rows, cols, vals, X)
        assert_within(host(csp.spmm_fwd(h, dev(X))), ref, S, FP32_REL, f"tiled forward B={B}")
        Hd = torch.empty((B, OUT), device="cuda")
        A = host(csp.spmm_fwd_act(h, dev(X), bias=dev(bias), act="gelu", H=Hd))
        pre, Sp = ref + bias.astype(np.float64), S + np.abs(bias.astype(np.float64))
        assert_within(host(Hd), pre, Sp, FP32_REL, f"tiled forward pre-activation B={B}")
        assert_within(A, orc.gelu(pre), Sp, ACT_REL, f"tiled forward GELU B={B}")
        refx, Sx = orc.spmm_bwd_input(OUT, IN, rows, cols, vals, dY)
        assert_within(host(csp.spmm_bwd_input(h, dev(dY))), refx, Sx, FP32_REL, f"tiled input gradient B={B}")
        dX, _ = csp.spmm_bwd(h, dev(dY), dev(X))
        assert_within(host(dX), refx, Sx, FP32_REL, f"tiled input gradient in spmm_bwd B={B}")
        Hin = W.random_dense((B, IN), 77 + B)
        g = orc.gelu_grad(Hin.astype(np.float64))
        dXa = host(csp.spmm_bwd_input_act(h, dev(dY), dev(Hin), act="gelu"))
        assert_within(dXa, refx * g, Sx, ACT_REL, f"tiled input gradient times GELU' B={B}")
    finally:
        csp.sparse_layer_destroy(h)


def test_segment_tiles_close_to_task_kernels(orc, monkeypatch):
    """The tiled sums and the task-list sums of the same call differ only by rounding: each is
    within the fp32 bound of the exact sum, so they are within twice that bound of each other."""
    rows, cols, vals = tiled_layer(79)
    h = csp.sparse_layer_create(OUT, IN, dev(rows), dev(cols), dev(vals))
    try:
        X = W.random_dense((64, IN), 80)
        dY = W.random_dense((64, OUT), 81)
        out = {}
        for flag in ("0", "1"):
            monkeypatch.setenv("COOSPMM_SEGMENT_TILES", flag)
            out[flag] = (host(csp.spmm_fwd(h, dev(X))), host(csp.spmm_bwd_input(h, dev(dY))))
        _, Sf = orc.spmm_fwd(OUT, IN, rows, cols, vals, X)
        _, Sx = orc.spmm_bwd_input(OUT, IN, rows, cols, vals, dY)
        for k, S in enumerate((Sf, Sx)):
            assert_within(out["1"][k], out["0"][k].astype(np.float64), S, 2 * FP32_REL,
                          f"output {k}: tiled against task-list sums")
    finally:
        csp.sparse_layer_destroy(h)


def test_segment_tiles_after_restructure(orc):
    rows, cols, vals = tiled_layer(83)
    h = csp.sparse_layer_create(OUT, IN, dev(rows), dev(cols), dev(vals))
    try:
        X = W.random_dense((64, IN), 84)
        dY = W.random_dense((64, OUT), 85)
        for step in range(2):
            csp.restructure(h, csp.sparse_layer_nnz(h) // 10, seed=86, step=step, regrow_value=0.25)
            r, c, v = (host(t) for t in csp.sparse_layer_export(h))
            ref, S = orc.spmm_fwd(OUT, IN, r, c, v, X)
            assert_within(host(csp.spmm_fwd(h, dev(X))), ref, S, FP32_REL, f"forward after restructure {step}")
            ref, S = orc.spmm_bwd_input(OUT, IN, r, c, v, dY)
            assert_within(host(csp.spmm_bwd_input(h, dev(dY))), ref, S, FP32_REL,
                          f"input gradient after restructure {step}")
    finally:
        csp.sparse_layer_destroy(h)


def test_segment_tiles_keep_infinity_out_of_other_rows(orc):
    """An inf in X at the first column of a column block: rows without that column stay finite and
    match the oracle; the steps past a row's entries read a zero row, not the block's first one."""
    rows, cols, vals = tiled_layer(87)
    h = csp.sparse_layer_create(OUT, IN, dev(rows), dev(cols), dev(vals))
    try:
        X = W.random_dense((64, IN), 88)
        X[:, 512] = np.inf
        Y = host(csp.spmm_fwd(h, dev(X)))
        has = np.zeros(OUT, bool)
        has[rows[cols == 512]] = True
        assert np.all(np.isfinite(Y[:, ~has])), "an inf reached rows that do not hold its column"
        Xf = X.copy()
        Xf[:, 512] = 0.0
        ref, S = orc.spmm_fwd(OUT, IN, rows, cols, vals, Xf)
        assert_within(Y[:, ~has], ref[:, ~has], S[:, ~has], FP32_REL, "rows without the inf column")
    finally:
        csp.sparse_layer_destroy(h)


def test_restructured_tiles_match_a_fresh_layer():
    """After a bitmap restructure (random and gradient-informed regrow) the tiles' offsets come from
    the rebuild's ranks, not from a pass over the new entries.  The forward, input gradient and value
    gradient must then equal, bit for bit, those of a fresh layer created from the restructured
    layer's entries (whose tile offsets come from that pass): a wrong offset would move or drop
    entries of a tile."""
    rows, cols, vals = tiled_layer(99)
    h = csp.sparse_layer_create(OUT, IN, dev(rows), dev(cols), dev(vals))
    try:
        X = dev(W.random_dense((64, IN), 100))
        dY = dev(W.random_dense((64, OUT), 101))
        for kind in ("random", "gradient"):
            n_prune = csp.sparse_layer_nnz(h) // 10
            if kind == "random":
                csp.restructure(h, n_prune, seed=102, step=0, regrow_value=0.5)
            else:
                csp.restructure_grad(h, n_prune, dY, X, 0.25)
            r, c, v = csp.sparse_layer_export(h)
            h2 = csp.sparse_layer_create(OUT, IN, r, c, v)
            try:
                for name, fn in (("forward", lambda k: csp.spmm_fwd(k, X)),
                                 ("input gradient", lambda k: csp.spmm_bwd_input(k, dY)),
                                 ("value gradient", lambda k: csp.spmm_bwd_values(k, dY, X))):
                    a, b = host(fn(h)), host(fn(h2))
                    assert np.array_equal(bits(a), bits(b)), f"{name} after {kind} restructure"
            finally:
                csp.sparse_layer_destroy(h2)
    finally:
        csp.sparse_layer_destroy(h)


NS_OUT, NS_IN = 6000 + 11, 12000 + 5   # row view 12 x 24 tiles, column view 24 x 12


def test_nonsquare_tiles_against_oracle(orc):
    """A layer whose two views cut into different tile grids (12 x 24 and 24 x 12 blocks of 512),
    so every per-view tile count and block stride is exercised: forward, input gradient and sampled
    value gradient at B = 64 against the oracle, at create and after a restructure, and the
    asynchronous restructure's layer equal to the eager one bit for bit."""
    B, nnz = 64, int(0.04 * NS_OUT * NS_IN)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert -(-NS_OUT // 512) * -(-NS_IN // 512) >= cus, "the layer must have a tile per compute unit"
    L = W.random_layer(NS_OUT, NS_IN, nnz, seed=301)
    mk = lambda: csp.sparse_layer_create(NS_OUT, NS_IN, dev(L.rows), dev(L.cols), dev(L.vals))
    h, h2 = mk(), mk()
    try:
        X = dev(W.random_dense((B, NS_IN), 302))
        dY = dev(W.random_dense((B, NS_OUT), 303))

        def check(hh, what):
            r, c, v = (host(t) for t in csp.sparse_layer_export(hh))
            ref, S = orc.spmm_fwd(NS_OUT, NS_IN, r, c, v, host(X))
            assert_within(host(csp.spmm_fwd(hh, X)), ref, S, FP32_REL, f"{what}: forward")
            dX, dW = csp.spmm_bwd(hh, dY, X)
            refx, Sx = orc.spmm_bwd_input(NS_OUT, NS_IN, r, c, v, host(dY))
            assert_within(host(dX), refx, Sx, FP32_REL, f"{what}: input gradient")
            check_sample(hh, dW, X, dY, 304)

        check(h, "created")
        step = torch.tensor([9], dtype=torch.int64, device="cuda")
        csp.restructure(h, nnz // 10, 305, 9)
        csp.restructure_async(h2, nnz // 10, 305, step)
        torch.cuda.synchronize()
        a = [host(t) for t in csp.sparse_layer_export(h) + csp.sparse_layer_export_index(h)]
        b = [host(t) for t in csp.sparse_layer_export(h2) + csp.sparse_layer_export_index(h2)]
        for x, y in zip(a, b):
            assert np.array_equal(bits(x) if x.dtype == np.float32 else x, bits(y) if y.dtype == np.float32 else y)
        check(h, "restructured")
        check(h2, "restructured asynchronously")
    finally:
        torch.cuda.synchronize()
        csp.sparse_layer_destroy(h)
        csp.sparse_layer_destroy(h2)
