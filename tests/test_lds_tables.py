"""Small operand tables in LDS against the global-table path and the oracle.

When the operand a pass gathers from is small in its batch-minor layout
(2 <= B <= 64 and n * ld * element size <= 64 KiB, ld = B rounded up to a
power of two), the library copies it into LDS inside the product kernel
instead of launching the batch-minor copy and gathering from L2 (for the
segment passes, forward and input gradient, in a persistent grid of about
two workgroups per CU, split segments finished in the same launch).  The task code and its
arithmetic order are those of the global-table path, so every output must be
bitwise the same as with COOSPMM_LDS_TABLES=0 (which forces the global
tables).  Parity with the oracle uses the usual bounds (fp32 1e-5 * S, bf16
outputs 1e-2 * S, fp32 value gradients of bf16 operands 1e-5 * S since their
products are exact).

Cases cover the size edges (a table of exactly 64 KiB and one column more;
B = 64 and 65; B = 1, which keeps the global path), pad slots (B = 3), bf16
at B = 2 with 16384 columns and B = 4 with 8192,
rows and columns long enough to be split across tasks (their sums finish in
the fixup launch), a layer with mostly empty rows and columns, and an empty
layer.
"""
import os
from contextlib import contextmanager

import numpy as np
import pytest
import torch

import oracle
from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import BF16_REL, FP32_REL, as_f64, assert_within, dev, host

pytestmark = pytest.mark.gpu


@contextmanager
def lds_tables(on: bool):
    old = os.environ.get("COOSPMM_LDS_TABLES")
    os.environ["COOSPMM_LDS_TABLES"] = "1" if on else "0"
    try:
        yield
    finally:
        if old is None:
            del os.environ["COOSPMM_LDS_TABLES"]
        else:
            os.environ["COOSPMM_LDS_TABLES"] = old


def table_fits(n, B, dtype):
    ld = 1
    while ld < min(B, 64):
        ld *= 2
    return 2 <= B <= 64 and n * ld * (2 if dtype == "bf16" else 4) <= (64 << 10)


def zipf_layer(out, in_, nnz, seed, dtype, transpose=False):
    """Capped power-law rows (long rows split into several tasks); transposed for long columns."""
    r_pos, r_val = W.streams(seed, 2)
    if transpose:
        cols, rows = W.zipf_positions(in_, out, nnz, 1.1, r_pos)
    else:
        rows, cols = W.zipf_positions(out, in_, nnz, 1.1, r_pos)
    v = r_val.standard_normal(nnz).astype(np.float32)
    vals = W.f32_to_bf16_bits(v) if dtype == "bf16" else v
    return W.CooWeights(out, in_, rows, cols, vals, dtype)


def run_all(h, X, dY, Hin, bias):
    """Every product entry point once, as host arrays."""
    r = {"fwd": host(csp.spmm_fwd(h, X))}
    H = torch.empty((X.shape[0], csp.sparse_layer_shape(h)[0]), dtype=X.dtype, device="cuda")
    r["fwd_act"] = host(csp.spmm_fwd_act(h, X, bias=bias, act="gelu", H=H))
    r["fwd_pre"] = host(H)
    r["dx"] = host(csp.spmm_bwd_input(h, dY))
    r["dx_act"] = host(csp.spmm_bwd_input_act(h, dY, Hin, act="gelu"))
    r["dw"] = host(csp.spmm_bwd_values(h, dY, X))
    dX, dW = csp.spmm_bwd(h, dY, X)
    r["bwd_dx"], r["bwd_dw"] = host(dX), host(dW)
    dX, dW = csp.spmm_bwd_act(h, dY, X, Hin, act="gelu")
    r["bwd_act_dx"], r["bwd_act_dw"] = host(dX), host(dW)
    return r


CASES = [
    # (name, out, in, nnz, B, dtype, structure)
    ("tiny_b1_global", 300, 200, 9000, 1, "f32", "uniform"),
    ("tiny_b2", 300, 200, 9000, 2, "f32", "uniform"),
    ("x_table_64k", 1000, 1024, 40000, 16, "f32", "uniform"),
    ("x_table_64k_plus_1", 1000, 1025, 40000, 16, "f32", "uniform"),
    ("dy_table_64k", 1024, 900, 40000, 16, "f32", "uniform"),
    ("b64", 500, 256, 30000, 64, "f32", "uniform"),
    ("b65_two_chunks", 500, 256, 30000, 65, "f32", "uniform"),
    ("pad_b3_bf16", 500, 400, 30000, 3, "bf16", "uniform"),
    ("wide_b2_bf16", 700, 16384, 100000, 2, "bf16", "uniform"),
    ("wide_b4_bf16", 700, 8192, 100000, 4, "bf16", "uniform"),
    ("long_rows", 64, 3000, 150000, 4, "f32", "zipf"),
    ("long_cols", 3000, 64, 150000, 4, "f32", "zipf_t"),
    ("long_rows_bf16_b2", 64, 3000, 150000, 2, "bf16", "zipf"),
    ("sparse_rows_cols", 400, 300, 50, 4, "f32", "uniform"),
    # X table fits, dY table does not: forward and value gradient alone on LDS, the rest global
    ("x_fits_dy_not", 5000, 64, 20000, 16, "f32", "uniform"),
]


@pytest.mark.parametrize("name,out,in_,nnz,B,dtype,structure", CASES, ids=[c[0] for c in CASES])
def test_lds_tables_match_global_tables_and_oracle(orc, name, out, in_, nnz, B, dtype, structure):
    seed = out * 7 + in_ + B
    if structure == "uniform":
        L = W.random_layer(out, in_, nnz, seed=seed, dtype=dtype)
    else:
        L = zipf_layer(out, in_, nnz, seed, dtype, transpose=structure == "zipf_t")
    c = orc.canonicalize(out, in_, L.rows, L.cols, L.vals)
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        Xh = W.random_dense((B, in_), seed + 1, dtype=dtype)
        dYh = W.random_dense((B, out), seed + 2, dtype=dtype)
        Hh = W.random_dense((B, in_), seed + 3, dtype=dtype)
        bh = W.random_dense((out,), seed + 4, dtype=dtype)
        X, dY, Hin, bias = dev(Xh), dev(dYh), dev(Hh), dev(bh)
        with lds_tables(True):
            on = run_all(h, X, dY, Hin, bias)
        with lds_tables(False):
            off = run_all(h, X, dY, Hin, bias)
        for k in on:
            assert on[k].dtype == off[k].dtype and on[k].shape == off[k].shape, k
            diff = np.flatnonzero(on[k].view(np.uint8) != off[k].view(np.uint8))
            assert diff.size == 0, f"{k}: LDS-table result differs bitwise from the global-table result"
        rel = BF16_REL if dtype == "bf16" else FP32_REL
        ref, S = orc.spmm_fwd(out, in_, L.rows, L.cols, L.vals, Xh)
        assert_within(on["fwd"], ref, S, rel, f"{name} forward")
        refx, Sx = orc.spmm_bwd_input(out, in_, L.rows, L.cols, L.vals, dYh)
        assert_within(on["dx"], refx, Sx, rel, f"{name} input gradient")
        assert_within(on["bwd_dx"], refx, Sx, rel, f"{name} fused input gradient")
        g = orc.gelu_grad(as_f64(Hh))
        assert_within(on["dx_act"], refx * g, Sx, 1.3e-5 if dtype == "f32" else 1.2e-2, f"{name} dX * GELU'")
        refw, Sw = orc.spmm_bwd_values(out, in_, c["rows"], c["cols"], dYh, Xh)
        for k in ("dw", "bwd_dw", "bwd_act_dw"):
            assert_within(on[k], refw, Sw, FP32_REL, f"{name} {k}")
    finally:
        csp.sparse_layer_destroy(h)


def test_lds_table_size_rule():
    """The cases above straddle the rule as intended."""
    assert table_fits(1024, 16, "f32") and not table_fits(1025, 16, "f32")
    assert table_fits(16384, 2, "bf16") and table_fits(8192, 4, "bf16") and not table_fits(16384, 4, "bf16")
    assert table_fits(256, 64, "f32") and not table_fits(256, 65, "f32") and not table_fits(200, 1, "f32")
    assert table_fits(64, 16, "f32") and not table_fits(5000, 16, "f32")


def test_empty_layer_lds_path():
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    h = csp.sparse_layer_create(40, 30, e, e, torch.zeros(0, device="cuda"))
    try:
        with lds_tables(True):
            Y = csp.spmm_fwd(h, torch.randn(5, 30, device="cuda"))
            dX, dW = csp.spmm_bwd(h, torch.randn(5, 40, device="cuda"), torch.randn(5, 30, device="cuda"))
            dW2 = csp.spmm_bwd_values(h, torch.randn(5, 40, device="cuda"), torch.randn(5, 30, device="cuda"))
        assert torch.all(Y == 0) and torch.all(dX == 0) and dW.numel() == 0 and dW2.numel() == 0
    finally:
        csp.sparse_layer_destroy(h)
