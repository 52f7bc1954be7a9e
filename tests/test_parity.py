"""GPU parity: the HIP library against the CPU oracle, element by element, through the C ABI.

Sizes span many wavefront tiles with ragged tails; the full workload sizes are
checked on every output element (the C oracle finishes them in seconds).
"""
import numpy as np
import pytest
import torch

import oracle
from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import BF16_REL, FP32_REL, as_f64, assert_within, bits, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


class Layer:
    """A layer on the GPU plus the oracle's canonical view of the same triples."""

    def __init__(self, orc, L: W.CooWeights):
        self.L = L
        self.h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
        self.canon = orc.canonicalize(L.out, L.in_, L.rows, L.cols, L.vals)
        assert self.canon["status"] == 0

    def close(self):
        csp.sparse_layer_destroy(self.h)


def check_canonical(layer: Layer):
    c = layer.canon
    rows, cols, vals = (host(t) for t in csp.sparse_layer_export(layer.h))
    assert np.array_equal(rows, c["rows"]) and np.array_equal(cols, c["cols"])
    assert np.array_equal(bits(vals), bits(c["vals"]))
    row_ptr, perm_c, rbc, col_ptr = (host(t) for t in csp.sparse_layer_export_index(layer.h))
    assert np.array_equal(row_ptr, c["row_ptr"])
    assert np.array_equal(perm_c, c["perm_c"])
    assert np.array_equal(rbc, c["rows_by_col"])
    assert np.array_equal(col_ptr, c["col_ptr"])


def check_ops(orc, layer: Layer, B: int, seed: int, rel=FP32_REL, ops=("fwd", "dX", "dW", "bwd"), integer=False):
    L = layer.L
    X = W.random_dense((B, L.in_), seed, dtype=L.dtype, integer=integer)
    dY = W.random_dense((B, L.out), seed + 1, dtype=L.dtype, integer=integer)
    if "fwd" in ops:
        Y = host(csp.spmm_fwd(layer.h, dev(X)))
        ref, S = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, X)
        if integer:
            assert np.array_equal(as_f64(Y), ref)
        assert_within(Y, ref, S, rel, f"fwd B={B}")
    if "dX" in ops:
        dX = host(csp.spmm_bwd_input(layer.h, dev(dY)))
        ref, S = orc.spmm_bwd_input(L.out, L.in_, L.rows, L.cols, L.vals, dY)
        if integer:
            assert np.array_equal(as_f64(dX), ref)
        assert_within(dX, ref, S, rel, f"dX B={B}")
    if "dW" in ops:
        dW = host(csp.spmm_bwd_values(layer.h, dev(dY), dev(X)))
        c = layer.canon
        ref, S = orc.spmm_bwd_values(L.out, L.in_, c["rows"], c["cols"], dY, X)
        if integer:
            assert np.array_equal(dW.astype(np.float64), ref)
        assert_within(dW, ref, S, rel, f"dW B={B}")
    if "bwd" in ops:
        dX, dW = (host(t) for t in csp.spmm_bwd(layer.h, dev(dY), dev(X)))
        ref, S = orc.spmm_bwd_input(L.out, L.in_, L.rows, L.cols, L.vals, dY)
        assert_within(dX, ref, S, rel, f"fused dX B={B}")
        c = layer.canon
        ref, S = orc.spmm_bwd_values(L.out, L.in_, c["rows"], c["cols"], dY, X)
        if integer:
            assert np.array_equal(dW.astype(np.float64), ref)
        assert_within(dW, ref, S, rel, f"fused dW B={B}")


# ------------------------------------------------------------------ small and ragged
@pytest.mark.parametrize("B", [1, 2, 3, 5, 8, 16, 17, 32, 64, 65, 130])
def test_ops_ragged_batches(orc, B):
    layer = Layer(orc, W.random_layer(1000, 700, 35000, seed=100 + B))
    try:
        if B == 1:
            check_canonical(layer)
        check_ops(orc, layer, B, seed=200 + B)
    finally:
        layer.close()


@pytest.mark.parametrize("shape,nnz", [((1, 1), 1), ((1, 1), 0), ((1, 300), 77), ((300, 1), 77), ((50, 80), 30),
                                       ((257, 129), 257 * 129), ((4100, 3), 5000)])
def test_shapes_and_edge_densities(orc, shape, nnz):
    out, in_ = shape
    layer = Layer(orc, W.random_layer(out, in_, nnz, seed=nnz + out))
    try:
        check_canonical(layer)
        for B in (1, 4, 16):
            check_ops(orc, layer, B, seed=7 * B + out)
    finally:
        layer.close()


def test_integer_inputs_bit_exact(orc):
    """Integer-valued inputs are exact in fp32 under any summation order: GPU == oracle bit for bit."""
    layer = Layer(orc, W.random_layer(600, 500, 30000, seed=5, integer=True))
    try:
        for B in (1, 3, 16, 64):
            check_ops(orc, layer, B, seed=40 + B, integer=True)
    finally:
        layer.close()


def test_long_rows_and_columns(orc):
    """A few full rows and full columns among short ones (segments far longer than a wavefront)."""
    out, in_ = 300, 5000
    rng = np.random.default_rng(3)
    full_rows = [0, 17, 299]
    pos = set()
    for r in full_rows:
        pos.update(r * in_ + c for c in range(in_))
    for c in (4, 4999):
        pos.update(r * in_ + c for c in range(out))
    pos.update(int(p) for p in rng.choice(out * in_, 20000, replace=False))
    flat = rng.permutation(np.array(sorted(pos), np.int64))
    L = W.CooWeights(out, in_, (flat // in_).astype(np.int32), (flat % in_).astype(np.int32),
                     rng.standard_normal(flat.size).astype(np.float32), "f32")
    layer = Layer(orc, L)
    try:
        check_canonical(layer)
        for B in (1, 4, 16, 64):
            check_ops(orc, layer, B, seed=B)
    finally:
        layer.close()


def test_bf16_forward(orc):
    layer = Layer(orc, W.random_layer(900, 1100, 20000, seed=8, dtype="bf16"))
    try:
        check_canonical(layer)
        for B in (1, 2, 4, 7, 64, 70):
            check_ops(orc, layer, B, seed=60 + B, rel=BF16_REL, ops=("fwd",))
    finally:
        layer.close()


def test_bf16_training(orc):
    """bf16 backward: dX in bf16 (1e-2 * S), dW in fp32 from exact bf16 products (fp32 bound)."""
    layer = Layer(orc, W.random_layer(700, 900, 30000, seed=18, dtype="bf16"))
    L, c = layer.L, layer.canon
    try:
        for B in (1, 3, 16, 64, 70):
            X = W.random_dense((B, L.in_), 80 + B, dtype="bf16")
            dY = W.random_dense((B, L.out), 90 + B, dtype="bf16")
            refx, Sx = orc.spmm_bwd_input(L.out, L.in_, L.rows, L.cols, L.vals, dY)
            refw, Sw = orc.spmm_bwd_values(L.out, L.in_, c["rows"], c["cols"], dY, X)
            dX = host(csp.spmm_bwd_input(layer.h, dev(dY)))
            assert dX.dtype == np.uint16
            assert_within(dX, refx, Sx, BF16_REL, f"bf16 dX B={B}")
            dW = host(csp.spmm_bwd_values(layer.h, dev(dY), dev(X)))
            assert dW.dtype == np.float32
            assert_within(dW, refw, Sw, FP32_REL, f"bf16 dW B={B}")
            dX2, dW2 = (host(t) for t in csp.spmm_bwd(layer.h, dev(dY), dev(X)))
            assert_within(dX2, refx, Sx, BF16_REL, f"bf16 fused dX B={B}")
            assert_within(dW2, refw, Sw, FP32_REL, f"bf16 fused dW B={B}")
    finally:
        layer.close()


def test_empty_layer_outputs_zero(orc):
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    h = csp.sparse_layer_create(40, 30, e, e, torch.zeros(0, device="cuda"))
    try:
        Y = csp.spmm_fwd(h, torch.randn(5, 30, device="cuda"))
        dX = csp.spmm_bwd_input(h, torch.randn(5, 40, device="cuda"))
        dW = csp.spmm_bwd_values(h, torch.randn(5, 40, device="cuda"), torch.randn(5, 30, device="cuda"))
        assert torch.all(Y == 0) and torch.all(dX == 0) and dW.numel() == 0
        row_ptr, _, _, col_ptr = csp.sparse_layer_export_index(h)
        assert torch.all(row_ptr == 0) and torch.all(col_ptr == 0)
    finally:
        csp.sparse_layer_destroy(h)


def test_create_reports_bad_triples():
    r = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    c = torch.tensor([0, 5, 1], dtype=torch.int32, device="cuda")
    v = torch.ones(3, device="cuda")
    with pytest.raises(csp.CspError) as e:
        csp.sparse_layer_create(3, 5, r, c, v)          # column 5 out of range
    assert e.value.status == -2
    with pytest.raises(csp.CspError) as e:
        csp.sparse_layer_create(3, 6, torch.tensor([2, 0, 2], dtype=torch.int32, device="cuda"),
                                torch.tensor([1, 0, 1], dtype=torch.int32, device="cuda"), v)
    assert e.value.status == -3
    with pytest.raises(csp.CspError) as e:
        csp.sparse_layer_create(3, 6, torch.tensor([-1, 0, 2], dtype=torch.int32, device="cuda"), c, v)
    assert e.value.status == -2


def test_outputs_overwrite_and_repeat_bitwise(orc):
    """Outputs are overwritten (not accumulated) and repeated calls give identical bits."""
    layer = Layer(orc, W.random_layer(800, 900, 40000, seed=21))
    try:
        X = dev(W.random_dense((16, 900), 22))
        Y = torch.full((16, 800), float("nan"), device="cuda")
        csp.spmm_fwd(layer.h, X, Y)
        Y1 = Y.clone()
        csp.spmm_fwd(layer.h, X, Y)
        assert torch.equal(Y, Y1)
        dY = dev(W.random_dense((16, 800), 23))
        dX = torch.full((16, 900), float("nan"), device="cuda")
        csp.spmm_bwd_input(layer.h, dY, dX)
        assert torch.isfinite(dX).all()
        dW = torch.full((40000,), float("nan"), device="cuda")
        csp.spmm_bwd_values(layer.h, dY, X, dW)
        assert torch.isfinite(dW).all()
    finally:
        layer.close()


# ------------------------------------------------------------------ full workload sizes
@pytest.mark.parametrize("name", ["linear1024_b8_s90", "linear4096_b16_s95", "dst8192_b64_s95"])
def test_full_size_linear(orc, name):
    w, layers, acts = W.build(name)
    layer = Layer(orc, layers[0])
    try:
        check_canonical(layer)
        for B in w.batches:
            X, dY = acts[B]["X"], acts[B]["dY"]
            L = layer.L
            Y = host(csp.spmm_fwd(layer.h, dev(X)))
            ref, S = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, X)
            assert_within(Y, ref, S, FP32_REL, f"{name} fwd")
            dX = host(csp.spmm_bwd_input(layer.h, dev(dY)))
            ref, S = orc.spmm_bwd_input(L.out, L.in_, L.rows, L.cols, L.vals, dY)
            assert_within(dX, ref, S, FP32_REL, f"{name} dX")
            dW = host(csp.spmm_bwd_values(layer.h, dev(dY), dev(X)))
            refw, Sw = orc.spmm_bwd_values(L.out, L.in_, layer.canon["rows"], layer.canon["cols"], dY, X)
            assert_within(dW, refw, Sw, FP32_REL, f"{name} dW")
            dX2, dW2 = (host(t) for t in csp.spmm_bwd(layer.h, dev(dY), dev(X)))
            assert_within(dX2, ref, S, FP32_REL, f"{name} fused dX")
            assert_within(dW2, refw, Sw, FP32_REL, f"{name} fused dW")
    finally:
        layer.close()


def test_full_size_zipf_bf16_inference(orc):
    w, layers, acts = W.build("inference16384_zipf_s99_bf16")
    layer = Layer(orc, layers[0])
    try:
        check_canonical(layer)
        L = layer.L
        for B in w.batches:
            X = acts[B]["X"]
            Y = host(csp.spmm_fwd(layer.h, dev(X)))
            ref, S = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, X)
            assert_within(Y, ref, S, BF16_REL, f"zipf bf16 fwd B={B}")
    finally:
        layer.close()


def test_full_size_mlp_pair_plain(orc):
    """768 -> 3072 (GELU) -> 768 through the plain calls (GELU in the harness): every op compared on
    the GPU's own inputs to that op."""
    from scipy.special import erf
    w, layers, acts = W.build("mlp768x3072_s90")
    l1, l2 = Layer(orc, layers[0]), Layer(orc, layers[1])
    try:
        check_canonical(l1)
        check_canonical(l2)
        for B in w.batches:
            X, dY = acts[B]["X"], acts[B]["dY"]
            H = host(csp.spmm_fwd(l1.h, dev(X)))
            ref, S = orc.spmm_fwd(3072, 768, l1.L.rows, l1.L.cols, l1.L.vals, X)
            assert_within(H, ref, S, FP32_REL, f"mlp fwd1 B={B}")
            Hd = H.astype(np.float64)
            A = (0.5 * Hd * (1 + erf(Hd / np.sqrt(2)))).astype(np.float32)   # harness GELU
            Y = host(csp.spmm_fwd(l2.h, dev(A)))
            ref, S = orc.spmm_fwd(768, 3072, l2.L.rows, l2.L.cols, l2.L.vals, A)
            assert_within(Y, ref, S, FP32_REL, f"mlp fwd2 B={B}")
            dA = host(csp.spmm_bwd_input(l2.h, dev(dY)))
            ref, S = orc.spmm_bwd_input(768, 3072, l2.L.rows, l2.L.cols, l2.L.vals, dY)
            assert_within(dA, ref, S, FP32_REL, f"mlp dX2 B={B}")
            dW2 = host(csp.spmm_bwd_values(l2.h, dev(dY), dev(A)))
            ref, S = orc.spmm_bwd_values(768, 3072, l2.canon["rows"], l2.canon["cols"], dY, A)
            assert_within(dW2, ref, S, FP32_REL, f"mlp dW2 B={B}")
            g = orc.gelu_grad(Hd)
            dH = (dA.astype(np.float64) * g).astype(np.float32)
            dW1 = host(csp.spmm_bwd_values(l1.h, dev(dH), dev(X)))
            ref, S = orc.spmm_bwd_values(3072, 768, l1.canon["rows"], l1.canon["cols"], dH, X)
            assert_within(dW1, ref, S, FP32_REL, f"mlp dW1 B={B}")
            dX = host(csp.spmm_bwd_input(l1.h, dev(dH)))
            ref, S = orc.spmm_bwd_input(3072, 768, l1.L.rows, l1.L.cols, l1.L.vals, dH)
            assert_within(dX, ref, S, FP32_REL, f"mlp dX1 B={B}")
    finally:
        l1.close()
        l2.close()


ACT_REL = 1.3e-5   # fused GELU / GELU' outputs (derivation in tests/test_epilogue.py)


def test_full_size_mlp_pair_fused(orc):
    """The MLP pair exactly as the training step runs it, at the full 768 -> 3072 -> 768 size and
    B in {1, 4, 32}: spmm_fwd_act (GELU epilogue, pre-activation H kept), spmm_fwd,
    spmm_bwd_act (dH = (dY W2) * GELU'(H) and dW2 in one call), spmm_bwd (dX, dW1).  Each output
    is compared with the oracle on the GPU's own inputs to that call; the activations go through
    the oracle's fp64 GELU and GELU'."""
    w, layers, acts = W.build("mlp768x3072_s90")
    l1, l2 = Layer(orc, layers[0]), Layer(orc, layers[1])
    L1, L2 = l1.L, l2.L
    try:
        for B in w.batches:
            X, dY = acts[B]["X"], acts[B]["dY"]
            Hd = torch.empty((B, L1.out), device="cuda")
            A = host(csp.spmm_fwd_act(l1.h, dev(X), act="gelu", H=Hd))
            H = host(Hd)
            ref, S = orc.spmm_fwd(L1.out, L1.in_, L1.rows, L1.cols, L1.vals, X)
            assert_within(H, ref, S, FP32_REL, f"mlp fused fwd1 pre-activation B={B}")
            assert_within(A, orc.gelu(ref), S, ACT_REL, f"mlp fused fwd1 GELU B={B}")
            Y = host(csp.spmm_fwd(l2.h, dev(A)))
            ref, S = orc.spmm_fwd(L2.out, L2.in_, L2.rows, L2.cols, L2.vals, A)
            assert_within(Y, ref, S, FP32_REL, f"mlp fused fwd2 B={B}")
            dH, dW2 = (host(t) for t in csp.spmm_bwd_act(l2.h, dev(dY), dev(A), dev(H), act="gelu"))
            refa, Sa = orc.spmm_bwd_input(L2.out, L2.in_, L2.rows, L2.cols, L2.vals, dY)
            assert_within(dH, refa * orc.gelu_grad(H.astype(np.float64)), Sa, ACT_REL, f"mlp fused dH B={B}")
            refw, Sw = orc.spmm_bwd_values(L2.out, L2.in_, l2.canon["rows"], l2.canon["cols"], dY, A)
            assert_within(dW2, refw, Sw, FP32_REL, f"mlp fused dW2 B={B}")
            dX, dW1 = (host(t) for t in csp.spmm_bwd(l1.h, dev(dH), dev(X)))
            ref, S = orc.spmm_bwd_input(L1.out, L1.in_, L1.rows, L1.cols, L1.vals, dH)
            assert_within(dX, ref, S, FP32_REL, f"mlp fused dX1 B={B}")
            ref, S = orc.spmm_bwd_values(L1.out, L1.in_, l1.canon["rows"], l1.canon["cols"], dH, X)
            assert_within(dW1, ref, S, FP32_REL, f"mlp fused dW1 B={B}")
    finally:
        l1.close()
        l2.close()
