"""GPU parity of restructure (prune + regrow + re-sort): bit-exact against the oracle, step by step."""
import numpy as np
import pytest
import torch

import oracle
from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import FP32_REL, assert_within, bits, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.fixture(params=["bitmap", "sorted"])
def path(request, monkeypatch):
    """Both restructure implementations: position bitmaps (the default when they
    fit) and the sorted fallback, chosen when the layer is created."""
    if request.param == "sorted":
        monkeypatch.setenv("COOSPMM_RESTRUCTURE", "sorted")
    else:
        monkeypatch.delenv("COOSPMM_RESTRUCTURE", raising=False)
    return request.param


def export(h):
    return tuple(host(t) for t in csp.sparse_layer_export(h))


def check_state(orc, h, out, in_, rows, cols, vals):
    """GPU layer holds exactly (rows, cols, vals) and its index arrays match the oracle's."""
    r, c, v = export(h)
    assert np.array_equal(r, rows) and np.array_equal(c, cols)
    assert np.array_equal(bits(v), bits(vals))
    ref = orc.canonicalize(out, in_, rows, cols, vals)
    assert ref["status"] == 0 and np.array_equal(ref["rows"], rows)     # still canonical, no duplicates
    row_ptr, perm_c, rbc, col_ptr = (host(t) for t in csp.sparse_layer_export_index(h))
    assert np.array_equal(row_ptr, ref["row_ptr"]) and np.array_equal(col_ptr, ref["col_ptr"])
    assert np.array_equal(perm_c, ref["perm_c"]) and np.array_equal(rbc, ref["rows_by_col"])


def run_steps(orc, L: W.CooWeights, n_prune, seed, steps, regrow=0.0):
    """Create the layer and run `steps` restructures, checking every step against the oracle."""
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        c = orc.canonicalize(L.out, L.in_, L.rows, L.cols, L.vals)
        rows, cols, vals = c["rows"], c["cols"], c["vals"]
        for step in range(steps):
            r0 = orc.restructure(L.out, L.in_, rows, cols, vals, n_prune, seed, step, regrow)
            csp.restructure(h, n_prune, seed, step, regrow)
            rows, cols, vals = r0[0], r0[1], r0[2]
            check_state(orc, h, L.out, L.in_, rows, cols, vals)
        return h, rows, cols, vals
    except Exception:
        csp.sparse_layer_destroy(h)
        raise


@pytest.mark.parametrize("out,in_,nnz,n_prune,seed", [
    (6, 7, 12, 3, 1), (6, 7, 42, 5, 2), (6, 7, 40, 40, 3), (20, 30, 200, 20, 5), (1, 50, 10, 4, 6),
    (50, 1, 10, 4, 7), (1000, 700, 35000, 3500, 11), (333, 777, 50000, 1, 12), (30, 30, 900, 5, 13)])
def test_restructure_matches_oracle(orc, path, out, in_, nnz, n_prune, seed):
    L = W.random_layer(out, in_, nnz, seed=seed)
    if nnz >= 6:   # plant magnitude ties and signed zeros
        L.vals[1] = -L.vals[0]
        L.vals[2] = 0.0
        L.vals[3] = -0.0
    h, *_ = run_steps(orc, L, n_prune, seed, steps=3, regrow=0.5)
    csp.sparse_layer_destroy(h)


def test_restructure_zero_prune_is_identity(orc, path):
    L = W.random_layer(100, 90, 900, seed=3)
    h, rows, cols, vals = run_steps(orc, L, 0, 1, steps=1)
    csp.sparse_layer_destroy(h)


def test_restructure_multi_batch_path(orc, path, monkeypatch):
    """Tiny candidate batches force several regrow rounds; the result must not change."""
    monkeypatch.setenv("COOSPMM_REGROW_BATCH", "37")
    L = W.random_layer(200, 150, 15000, seed=17)
    h, *_ = run_steps(orc, L, 1500, 4, steps=2)
    csp.sparse_layer_destroy(h)


def test_restructure_bf16(orc, path):
    L = W.random_layer(300, 200, 6000, seed=19, dtype="bf16")
    h = csp.sparse_layer_create(300, 200, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        c = orc.canonicalize(300, 200, L.rows, L.cols, L.vals)
        regrow_bits = W.f32_to_bf16_bits(np.array([0.125], np.float32))[0]
        rr, cr, vr, _ = orc.restructure(300, 200, c["rows"], c["cols"], c["vals"], 600, 9, 2, regrow_bits)
        csp.restructure(h, 600, 9, 2, 0.125)
        check_state(orc, h, 300, 200, rr, cr, vr)
    finally:
        csp.sparse_layer_destroy(h)


def test_restructure_wide_layer_sorted_path(orc):
    """out*in >= 2^32: positions need 64 bits, so the layer takes the sorted path by itself."""
    L = W.random_layer(70000, 70000, 30000, seed=41)
    h, *_ = run_steps(orc, L, 3000, 5, steps=2, regrow=-1.0)
    csp.sparse_layer_destroy(h)


def test_restructure_multi_batch_bf16(orc, path, monkeypatch):
    """Short batches on a bf16 layer: several rounds, each rebuilding the view until all are taken."""
    monkeypatch.setenv("COOSPMM_REGROW_BATCH", "300")
    L = W.random_layer(64, 96, 5000, seed=43, dtype="bf16")
    h = csp.sparse_layer_create(64, 96, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        c = orc.canonicalize(64, 96, L.rows, L.cols, L.vals)
        rows, cols, vals = c["rows"], c["cols"], c["vals"]
        regrow_bits = W.f32_to_bf16_bits(np.array([2.0], np.float32))[0]
        for step in range(3):
            rows, cols, vals, _ = orc.restructure(64, 96, rows, cols, vals, 900, 21, step, regrow_bits)
            csp.restructure(h, 900, 21, step, 2.0)
            check_state(orc, h, 64, 96, rows, cols, vals)
    finally:
        csp.sparse_layer_destroy(h)


def test_values_view_after_restructure(orc, path):
    """A values view taken after a restructure sees the new values, and in-place
    updates through it reach every pass."""
    L = W.random_layer(400, 300, 12000, seed=47)
    h, rows, cols, vals = run_steps(orc, L, 1200, 3, steps=1, regrow=0.25)
    try:
        v = csp.sparse_layer_values_tensor(h)
        assert np.array_equal(bits(host(v.clone())), bits(vals))
        v.mul_(3.0)
        csp.sparse_layer_set_values(h, None)
        newv = host(v.clone())
        dY = W.random_dense((5, 400), 8)
        dX = host(csp.spmm_bwd_input(h, dev(dY)))
        ref, S = orc.spmm_bwd_input(400, 300, rows, cols, newv, dY)
        assert_within(dX, ref, S, FP32_REL, "dX after restructure and in-place update")
    finally:
        csp.sparse_layer_destroy(h)


@pytest.mark.parametrize("out,in_,nnz,n_prune,B,dtype,integer", [
    (6, 7, 12, 3, 2, "f32", True), (40, 30, 300, 40, 3, "f32", True), (1000, 700, 35000, 3500, 16, "f32", False),
    (333, 777, 50000, 700, 70, "f32", False), (300, 200, 6000, 600, 4, "bf16", False),
    (1, 3000, 500, 50, 5, "f32", False), (3000, 1, 500, 50, 5, "f32", False)])
def test_restructure_grad_matches_oracle(orc, out, in_, nnz, n_prune, B, dtype, integer):
    """Gradient-informed regrow, bit-exact against the oracle over three steps (integer operands give
    exact scores with many ties, so the tie rule is exercised)."""
    L = W.random_layer(out, in_, nnz, seed=out + 7 * in_, dtype=dtype)
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        c = orc.canonicalize(out, in_, L.rows, L.cols, L.vals)
        rows, cols, vals = c["rows"], c["cols"], c["vals"]
        regrow = W.f32_to_bf16_bits(np.array([0.5], np.float32))[0] if dtype == "bf16" else 0.5
        for step in range(3):
            dY = W.random_dense((B, out), 100 + step, dtype=dtype, integer=integer)
            X = W.random_dense((B, in_), 200 + step, dtype=dtype, integer=integer)
            rows, cols, vals = orc.restructure_grad(out, in_, rows, cols, vals, n_prune, dY, X, regrow)
            csp.restructure_grad(h, n_prune, dev(dY), dev(X), 0.5)
            check_state(orc, h, out, in_, rows, cols, vals)
    finally:
        csp.sparse_layer_destroy(h)


def test_restructure_grad_full_size(orc):
    """4096 x 4096 at 95%, B = 16: one gradient-informed step of 10%, bit-exact."""
    w, layers, acts = W.build("linear4096_b16_s95")
    L = layers[0]
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        c = orc.canonicalize(L.out, L.in_, L.rows, L.cols, L.vals)
        X, dY = acts[16]["X"], acts[16]["dY"]
        n_prune = L.nnz // 10
        r0 = orc.restructure_grad(L.out, L.in_, c["rows"], c["cols"], c["vals"], n_prune, dY, X, 0.0)
        csp.restructure_grad(h, n_prune, dev(dY), dev(X), 0.0)
        check_state(orc, h, L.out, L.in_, *r0)
    finally:
        csp.sparse_layer_destroy(h)


def test_restructure_grad_needs_bitmaps(monkeypatch):
    monkeypatch.setenv("COOSPMM_RESTRUCTURE", "sorted")
    L = W.random_layer(50, 40, 300, seed=3)
    h = csp.sparse_layer_create(50, 40, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        with pytest.raises(csp.CspError) as e:
            csp.restructure_grad(h, 10, dev(W.random_dense((2, 50), 1)), dev(W.random_dense((2, 40), 2)))
        assert e.value.status == -1 and "bitmap" in str(e.value)
    finally:
        csp.sparse_layer_destroy(h)


def test_restructure_rejects_bad_count():
    L = W.random_layer(10, 10, 20, seed=1)
    h = csp.sparse_layer_create(10, 10, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        for bad in (-1, 21):
            with pytest.raises(csp.CspError) as e:
                csp.restructure(h, bad, 1, 1)
            assert e.value.status == -1
    finally:
        csp.sparse_layer_destroy(h)


def test_products_after_restructure(orc, path):
    """After restructure the products use the new structure (offsets and transposed view rebuilt)."""
    L = W.random_layer(700, 500, 20000, seed=23)
    h, rows, cols, vals = run_steps(orc, L, 2000, 8, steps=2)
    try:
        X = W.random_dense((16, 500), 1)
        dY = W.random_dense((16, 700), 2)
        Y = host(csp.spmm_fwd(h, dev(X)))
        ref, S = orc.spmm_fwd(700, 500, rows, cols, vals, X)
        assert_within(Y, ref, S, FP32_REL, "fwd after restructure")
        dX = host(csp.spmm_bwd_input(h, dev(dY)))
        ref, S = orc.spmm_bwd_input(700, 500, rows, cols, vals, dY)
        assert_within(dX, ref, S, FP32_REL, "dX after restructure")
        dW = host(csp.spmm_bwd_values(h, dev(dY), dev(X)))
        ref, S = orc.spmm_bwd_values(700, 500, rows, cols, dY, X)
        assert_within(dW, ref, S, FP32_REL, "dW after restructure")
    finally:
        csp.sparse_layer_destroy(h)


def test_in_place_value_update_then_refresh(orc):
    """Values changed through the zero-copy view are seen by every pass once the copy is refreshed."""
    L = W.random_layer(500, 400, 20000, seed=29)
    h = csp.sparse_layer_create(500, 400, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        c = orc.canonicalize(500, 400, L.rows, L.cols, L.vals)
        v = csp.sparse_layer_values_tensor(h)
        v.mul_(-2.0)
        v[:7] = 0.5
        csp.sparse_layer_set_values(h, None)
        newv = host(v.clone())
        rows, cols = c["rows"], c["cols"]
        X = W.random_dense((8, 400), 3)
        dY = W.random_dense((8, 500), 4)
        Y = host(csp.spmm_fwd(h, dev(X)))
        ref, S = orc.spmm_fwd(500, 400, rows, cols, newv, X)
        assert_within(Y, ref, S, FP32_REL, "fwd after in-place update")
        for dX in (host(csp.spmm_bwd_input(h, dev(dY))), host(csp.spmm_bwd(h, dev(dY), dev(X))[0])):
            ref, S = orc.spmm_bwd_input(500, 400, rows, cols, newv, dY)
            assert_within(dX, ref, S, FP32_REL, "dX after in-place update")
    finally:
        csp.sparse_layer_destroy(h)


def test_dst_loop_full_size(orc):
    """8192x8192 at 95% sparsity, B=64: 10 steps of value gradient, SGD (harness), restructure of 10%."""
    w, layers, acts = W.build("dst8192_b64_s95")
    L = layers[0]
    n_prune = int(np.floor(w.prune_frac * L.nnz))
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        c = orc.canonicalize(L.out, L.in_, L.rows, L.cols, L.vals)
        X, dY = dev(acts[64]["X"]), dev(acts[64]["dY"])
        for step in range(w.steps):
            dW = csp.spmm_bwd_values(h, dY, X)
            _, _, v = csp.sparse_layer_export(h)
            csp.sparse_layer_set_values(h, (v - 1e-3 * dW).contiguous())
            rows, cols, vals = export(h)
            r0 = orc.restructure(L.out, L.in_, rows, cols, vals, n_prune, w.seed, step, 0.0)
            csp.restructure(h, n_prune, w.seed, step, 0.0)
            r, c_, v_ = export(h)
            assert np.array_equal(r, r0[0]) and np.array_equal(c_, r0[1])
            assert np.array_equal(bits(v_), bits(r0[2])), f"step {step}"
        check_state(orc, h, L.out, L.in_, r0[0], r0[1], r0[2])
    finally:
        csp.sparse_layer_destroy(h)


def test_failed_restructure_marks_layer_unusable(path, monkeypatch):
    """A regrow that cannot place every pruned entry within its batch limit (forced from the host
    with four-draw batches: about 4096 * 4 * 0.85 < 30000 candidates land on empty positions)
    returns an error; the layer is then half rebuilt, so every call but destroy refuses it."""
    monkeypatch.setenv("COOSPMM_REGROW_BATCH", "4")
    L = W.random_layer(200, 200, 36000, seed=53)
    h = csp.sparse_layer_create(200, 200, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        with pytest.raises(csp.CspError, match="regrow found only"):
            csp.restructure(h, 30000, 3, 0)
        X = dev(W.random_dense((2, 200), 1))
        refused = [lambda: csp.spmm_fwd(h, X), lambda: csp.spmm_fwd_static(h, X),
                   lambda: csp.spmm_bwd_input(h, X), lambda: csp.spmm_bwd(h, X, X),
                   lambda: csp.sparse_layer_export(h), lambda: csp.sparse_layer_export_index(h),
                   lambda: csp.sparse_layer_set_values(h, None), lambda: csp.restructure(h, 10, 3, 1),
                   lambda: csp.restructure_grad(h, 10, X, X)]
        for call in refused:
            with pytest.raises(csp.CspError, match="failed restructure"):
                call()
    finally:
        csp.sparse_layer_destroy(h)
