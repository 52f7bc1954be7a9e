"""Hand-worked examples (tests/golden/worked_examples.json) against the oracle
(CPU) and against the HIP path through the C-ABI (GPU).

Every expected value in the fixture was derived by hand from the definitions
of the truly sparse COO layer ("Beyond Masked Sparsity: SNACK Enables Truly
Sparse Neural Networks on GPU", Abstract) and the restructure readings, not
computed by either implementation.  The values are short binary fractions,
so both sides must match them exactly.
"""
import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
    GOLD = json.load(f)


def f32(a):
    return np.asarray(a, dtype=np.float32)


def i32(a):
    return np.asarray(a, dtype=np.int32)


def triples(ex):
    t = ex["triples_any_order"]
    return i32([x[0] for x in t]), i32([x[1] for x in t]), f32([x[2] for x in t])


def canon(ex):
    c = ex["canonical"]
    return i32(c["rows"]), i32(c["cols"]), f32(c["vals"])


def assert_exact(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want, dtype=got.dtype)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.array_equal(got, want), f"{what}: {got.tolist()} != {want.tolist()}"


def test_fixture_is_self_consistent():
    """The hand-worked products satisfy the adjoint identity the fixture states."""
    ex = GOLD["products"][0]
    _, _, v = canon(ex)
    lhs = float(np.sum(f32(ex["dY"]) * f32(ex["Y"])))
    mid = float(np.sum(f32(ex["dX"]) * f32(ex["X"])))
    rhs = float(np.dot(f32(ex["dW"]), v))
    assert lhs == mid == rhs == ex["adjoint"]


@pytest.mark.parametrize("ex", GOLD["products"], ids=lambda e: e["name"])
def test_oracle_products(orc, ex):
    out, in_ = ex["out"], ex["in"]
    r, c, v = triples(ex)
    cz = orc.canonicalize(out, in_, r, c, v)
    assert cz["status"] == 0
    for k in ("rows", "cols", "vals"):
        assert_exact(cz[k], ex["canonical"][k], k)
    for k in ("row_ptr", "perm_c", "rows_by_col", "col_ptr"):
        assert_exact(cz[k], ex[k], k)
    Y, _ = orc.spmm_fwd(out, in_, r, c, v, f32(ex["X"]))
    assert_exact(Y, ex["Y"], "Y")
    dX, _ = orc.spmm_bwd_input(out, in_, r, c, v, f32(ex["dY"]))
    assert_exact(dX, ex["dX"], "dX")
    rc, cc, _ = canon(ex)
    dW, _ = orc.spmm_bwd_values(out, in_, rc, cc, f32(ex["dY"]), f32(ex["X"]))
    assert_exact(dW, ex["dW"], "dW")


@pytest.mark.parametrize("ex", GOLD["restructure"], ids=lambda e: e["name"])
def test_oracle_restructure(orc, ex):
    r, c, v = canon(ex)
    rr, cr, vr, _ = orc.restructure(ex["out"], ex["in"], r, c, v, ex["n_prune"], ex["seed"], ex["step"],
                                    ex["regrow_value"])
    for k, got in zip(("rows", "cols", "vals"), (rr, cr, vr)):
        assert_exact(got, ex["expected"][k], k)


@pytest.mark.parametrize("ex", GOLD["restructure_grad"], ids=lambda e: e["name"])
def test_oracle_restructure_grad(orc, ex):
    r, c, v = canon(ex)
    rr, cr, vr = orc.restructure_grad(ex["out"], ex["in"], r, c, v, ex["n_prune"], f32(ex["dY"]), f32(ex["X"]),
                                      ex["regrow_value"])[:3]
    for k, got in zip(("rows", "cols", "vals"), (rr, cr, vr)):
        assert_exact(got, ex["expected"][k], k)


@pytest.mark.gpu
@pytest.mark.parametrize("ex", GOLD["products"], ids=lambda e: e["name"])
def test_gpu_products(ex):
    from coo_spmm_fwd_amd import binding as csp
    from tests.gpu_util import dev, host
    out, in_ = ex["out"], ex["in"]
    r, c, v = triples(ex)
    h = csp.sparse_layer_create(out, in_, dev(r), dev(c), dev(v))
    try:
        rows, cols, vals = (host(t) for t in csp.sparse_layer_export(h))
        for k, got in zip(("rows", "cols", "vals"), (rows, cols, vals)):
            assert_exact(got, ex["canonical"][k], k)
        for k, got in zip(("row_ptr", "perm_c", "rows_by_col", "col_ptr"), csp.sparse_layer_export_index(h)):
            assert_exact(host(got), ex[k], k)
        X, dY = dev(f32(ex["X"])), dev(f32(ex["dY"]))
        assert_exact(host(csp.spmm_fwd(h, X)), ex["Y"], "Y")
        assert_exact(host(csp.spmm_bwd_input(h, dY)), ex["dX"], "dX")
        assert_exact(host(csp.spmm_bwd_values(h, dY, X)), ex["dW"], "dW")
        dX, dW = csp.spmm_bwd(h, dY, X)
        assert_exact(host(dX), ex["dX"], "fused dX")
        assert_exact(host(dW), ex["dW"], "fused dW")
    finally:
        csp.sparse_layer_destroy(h)


RESTRUCTURE_CASES = [("random", e) for e in GOLD["restructure"]] + [("grad", e) for e in GOLD["restructure_grad"]]


@pytest.mark.gpu
@pytest.mark.parametrize("kind,ex", RESTRUCTURE_CASES, ids=[f"{k}-{e['name']}" for k, e in RESTRUCTURE_CASES])
def test_gpu_restructure(kind, ex):
    from coo_spmm_fwd_amd import binding as csp
    from tests.gpu_util import dev, host
    r, c, v = canon(ex)
    h = csp.sparse_layer_create(ex["out"], ex["in"], dev(r), dev(c), dev(v))
    try:
        if kind == "random":
            csp.restructure(h, ex["n_prune"], ex["seed"], ex["step"], ex["regrow_value"])
        else:
            csp.restructure_grad(h, ex["n_prune"], dev(f32(ex["dY"])), dev(f32(ex["X"])), ex["regrow_value"])
        rows, cols, vals = (host(t) for t in csp.sparse_layer_export(h))
        for k, got in zip(("rows", "cols", "vals"), (rows, cols, vals)):
            assert_exact(got, ex["expected"][k], k)
    finally:
        csp.sparse_layer_destroy(h)
