"""Split segments finished inside the segment pass.

A row (forward) or column (input gradient) longer than 512 entries is cut
into tasks.  Three paths add up the tasks of such a segment, all in task
order:
- the split-plus-fixup path: tasks store partial sums, a fixup launch adds
  them (global tables, COOSPMM_GROUPED_SPLITS=0);
- k_segment_grouped: with global tables, B <= 8 and at most 64 tasks per
  segment (the other dimension is at most 32768), one 16-wave workgroup
  runs all tasks of a split segment and adds their sums in LDS;
- k_segment_lds: when the gathered operand fits an LDS table (2 <= B <= 64,
  at most 64 KiB), the persistent small-table kernel does the same for its
  split segments.
Results must be bitwise equal across the three, and within the oracle's
bounds.

Cases: power-law rows and columns (many split segments of different task
counts next to unsplit ones and empty ones), B = 1, 3 (pad slots), 8, and 16
and 64 (above the limit: both settings take the split-plus-fixup path),
fp32 and bf16, the epilogues (bias + GELU forward, input gradient times
GELU'), a row of 32768 entries (exactly 64 tasks) and a layer with 32769
columns (more than 64 tasks possible: the fixup path stays), and layers
whose operand tables fit LDS exactly (64 KiB) with split rows or columns.
"""
import os
from contextlib import contextmanager

import numpy as np
import pytest
import torch

from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import BF16_REL, FP32_REL, as_f64, assert_within, dev, host

pytestmark = pytest.mark.gpu


@contextmanager
def env(**kv):
    old = {k: os.environ.get(k) for k in kv}
    os.environ.update(kv)
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def zipf_layer(out, in_, nnz, seed, dtype, transpose=False):
    r_pos, r_val = W.streams(seed, 2)
    if transpose:
        cols, rows = W.zipf_positions(in_, out, nnz, 1.1, r_pos)
    else:
        rows, cols = W.zipf_positions(out, in_, nnz, 1.1, r_pos)
    v = r_val.standard_normal(nnz).astype(np.float32)
    return W.CooWeights(out, in_, rows, cols, W.f32_to_bf16_bits(v) if dtype == "bf16" else v, dtype)


def full_row_layer(out, in_, extra, seed, dtype):
    """Row 0 holds every column (in_ entries); `extra` more entries scattered over the other rows."""
    rng = W.streams(seed, 1)[0]
    flat = rng.choice((out - 1) * in_, size=extra, replace=False) + in_
    rows = np.concatenate([np.zeros(in_, np.int64), flat // in_]).astype(np.int32)
    cols = np.concatenate([np.arange(in_), flat % in_]).astype(np.int32)
    v = rng.standard_normal(rows.size).astype(np.float32)
    return W.CooWeights(out, in_, rows, cols, W.f32_to_bf16_bits(v) if dtype == "bf16" else v, dtype)


CASES = [
    # (name, builder, B, dtype)
    ("zipf_rows_b1_bf16", lambda d: zipf_layer(4096, 16384, 300000, 11, d), 1, "bf16"),
    ("zipf_rows_b3", lambda d: zipf_layer(4096, 16384, 300000, 12, d), 3, "f32"),
    ("zipf_rows_b8", lambda d: zipf_layer(2048, 8192, 200000, 19, d), 8, "f32"),
    ("zipf_rows_b16", lambda d: zipf_layer(2048, 8192, 200000, 13, d), 16, "f32"),
    ("zipf_rows_b64", lambda d: zipf_layer(1024, 4096, 100000, 14, d), 64, "f32"),
    ("zipf_cols_b1", lambda d: zipf_layer(16384, 4096, 300000, 15, d, transpose=True), 1, "f32"),
    ("zipf_cols_b4_bf16", lambda d: zipf_layer(16384, 4096, 300000, 16, d, transpose=True), 4, "bf16"),
    ("row_of_64_tasks", lambda d: full_row_layer(8, 32768, 5000, 17, d), 1, "f32"),
    # LDS tables: X of 16384 bf16 columns at B = 2 is exactly 64 KiB (a 32-task row); X of 4096
    # fp32 columns at B = 4 is 64 KiB; dY of 16384 bf16 columns at B = 2 is 64 KiB (long columns)
    ("row_of_32_tasks_lds_b2_bf16", lambda d: full_row_layer(8, 16384, 5000, 20, d), 2, "bf16"),
    ("zipf_rows_lds_b4", lambda d: zipf_layer(1024, 4096, 150000, 21, d), 4, "f32"),
    ("zipf_cols_lds_b2_bf16", lambda d: zipf_layer(16384, 2048, 200000, 22, d, transpose=True), 2, "bf16"),
    ("over_64_tasks_fixup", lambda d: full_row_layer(8, 32769, 5000, 18, d), 2, "f32"),
]


@pytest.mark.parametrize("name,builder,B,dtype", CASES, ids=[c[0] for c in CASES])
def test_grouped_splits_bitwise_and_oracle(orc, name, builder, B, dtype):
    L = builder(dtype)
    out, in_ = L.out, L.in_
    h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        seed = out + in_ + B
        Xh = W.random_dense((B, in_), seed + 1, dtype=dtype)
        dYh = W.random_dense((B, out), seed + 2, dtype=dtype)
        Hh = W.random_dense((B, in_), seed + 3, dtype=dtype)
        bh = W.random_dense((out,), seed + 4, dtype=dtype)
        X, dY, Hin, bias = dev(Xh), dev(dYh), dev(Hh), dev(bh)

        def run():
            H = torch.empty((B, out), dtype=X.dtype, device="cuda")
            r = {"fwd": host(csp.spmm_fwd(h, X)), "fwd_act": host(csp.spmm_fwd_act(h, X, bias=bias, act="gelu", H=H))}
            r["pre"] = host(H)
            r["dx"] = host(csp.spmm_bwd_input(h, dY))
            r["dx_act"] = host(csp.spmm_bwd_input_act(h, dY, Hin, act="gelu"))
            return r

        with env(COOSPMM_GROUPED_SPLITS="1", COOSPMM_LDS_TABLES="0"):
            on = run()
        with env(COOSPMM_GROUPED_SPLITS="0", COOSPMM_LDS_TABLES="0"):
            off = run()
        with env(COOSPMM_GROUPED_SPLITS="1", COOSPMM_LDS_TABLES="1"):
            lds = run()
        for k in on:
            assert np.array_equal(on[k].view(np.uint8), off[k].view(np.uint8)), f"{k}: grouped result differs"
            assert np.array_equal(lds[k].view(np.uint8), off[k].view(np.uint8)), f"{k}: LDS-table result differs"
        rel = BF16_REL if dtype == "bf16" else FP32_REL
        ref, S = orc.spmm_fwd(out, in_, L.rows, L.cols, L.vals, Xh)
        assert_within(on["fwd"], ref, S, rel, f"{name} forward")
        refx, Sx = orc.spmm_bwd_input(out, in_, L.rows, L.cols, L.vals, dYh)
        assert_within(on["dx"], refx, Sx, rel, f"{name} input gradient")
        # the fused forward: pre-activation y = X W^T + bias and GELU(y), bias counted in S
        yb = ref + as_f64(bh)[None, :]
        Sb = S + np.abs(as_f64(bh))[None, :]
        assert_within(on["pre"], yb, Sb, rel, f"{name} pre-activation")
        assert_within(on["fwd_act"], orc.gelu(yb), Sb, 1.3e-5 if dtype == "f32" else 1.2e-2, f"{name} GELU")
        g = orc.gelu_grad(as_f64(Hh))
        assert_within(on["dx_act"], refx * g, Sx, 1.3e-5 if dtype == "f32" else 1.2e-2, f"{name} dX * GELU'")
    finally:
        csp.sparse_layer_destroy(h)
