"""Packed row tasks of the forward pass at narrow batches (B <= 4).

At B <= 4 a lane holds one stored entry, so a task of one short row leaves
most of the wave idle.  The forward then runs from the packed row list:
consecutive whole rows of at most 512 entries each share a task of at most
505 entries and 64 rows (rows past 512 entries are split as in the plain
list); the entry limit shrinks with the layer, so that small layers keep
about one task per wave slot, and the tests set it to 505 (widest packing).
A task's rows are summed by each lane over its eight consecutive entries and
a segmented scan over the lanes.

Checks, on layouts made to hit the packing rule's edges (runs of empty rows,
single-entry rows, rows of 504..513 and 1024/1025 entries, a lone non-empty
row, an empty layer, 70000 short rows (over 1024 packing windows), power-law
rows):
- integer-valued inputs (every sum exact in fp32): the packed result equals
  the oracle exactly, and the plain list's result bit for bit, also through
  the bias + GELU epilogue and its pre-activation output;
- the three packed paths (global operand, LDS table, split rows by fixup
  launch instead of in the pass) agree bit for bit;
- normal inputs: within the oracle's bound.
"""
import os
from contextlib import contextmanager

import numpy as np
import pytest
import torch

from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import BF16_REL, FP32_REL, as_f64, assert_within, dev, host


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


def lengths_for(name: str) -> tuple[np.ndarray, int]:
    """Row lengths and the column count of a named layout."""
    rng = np.random.default_rng(sum(map(ord, name)))
    if name == "mixed_short":
        n = rng.choice(np.r_[0, 0, 0, np.arange(1, 41)], size=3000)
        n[[100, 101, 102, 103, 500, 501, 502]] = [505, 506, 512, 513, 1100, 0, 1]
        return n, 1200
    if name == "single_entry":
        n = np.ones(5000, np.int64)
        n[::7] = 0
        return n, 300
    if name == "empty_runs":
        n = rng.integers(1, 21, size=4000)
        n[:300] = 0
        n[3700:] = 0
        return n, 500
    if name == "edge_lengths":
        cyc = [8, 8, 7, 9, 505, 0, 506, 3, 511, 512, 513, 1, 1024, 1025, 2, 64, 63, 65, 504, 0, 0]
        return np.resize(np.array(cyc), 600), 1100
    if name == "one_row":
        n = np.zeros(9000, np.int64)
        n[-1] = 300
        return n, 400
    if name == "empty_layer":
        return np.zeros(1000, np.int64), 100
    if name == "tall":  # more than 1024 packing windows: the task-list build takes its separate scan launch
        return rng.integers(0, 6, size=70000), 64
    raise KeyError(name)


def layer_from_lengths(lengths, in_, seed, dtype, integer):
    rng = np.random.default_rng(seed)
    rows = np.repeat(np.arange(len(lengths)), lengths).astype(np.int32)
    cols = np.concatenate([rng.choice(in_, int(k), replace=False) for k in lengths] + [np.zeros(0, np.int64)])
    cols = cols.astype(np.int32)
    perm = rng.permutation(rows.size)  # creation takes any order
    rows, cols = rows[perm], cols[perm]
    if integer:
        v = rng.integers(-3, 4, size=rows.size).astype(np.float32)
    else:
        v = (rng.standard_normal(rows.size) * 0.05).astype(np.float32)
    return W.CooWeights(len(lengths), in_, rows, cols, W.f32_to_bf16_bits(v) if dtype == "bf16" else v, dtype)


def zipf_layer(dtype, integer, seed=31):
    r_pos, r_val = W.streams(seed, 2)
    rows, cols = W.zipf_positions(2048, 16384, 150000, 1.1, r_pos)
    if integer:
        v = r_val.integers(-3, 4, size=rows.size).astype(np.float32)
    else:
        v = (r_val.standard_normal(rows.size) * 0.02).astype(np.float32)
    return W.CooWeights(2048, 16384, rows, cols, W.f32_to_bf16_bits(v) if dtype == "bf16" else v, dtype)


LAYOUTS = ["mixed_short", "single_entry", "empty_runs", "edge_lengths", "one_row", "empty_layer", "tall", "zipf"]
CASES = [(lay, B, dt) for lay in LAYOUTS for B in (1, 2, 3, 4) for dt in ("f32", "bf16")
         if not (dt == "bf16" and B in (2, 3))]


def build(layout, dtype, integer):
    if layout == "zipf":
        return zipf_layer(dtype, integer)
    n, in_ = lengths_for(layout)
    return layer_from_lengths(n, in_, 7 + len(layout), dtype, integer)


def test_layouts_hit_the_packing_edges():
    """The layouts contain what the cases are meant to cover (CPU check)."""
    n, _ = lengths_for("edge_lengths")
    assert {504, 505, 506, 511, 512, 513, 1024, 1025, 0, 1} <= set(n.tolist())
    n, _ = lengths_for("empty_runs")
    assert n[:300].sum() == 0 and n[-300:].sum() == 0 and n[300:3700].min() >= 1
    n, _ = lengths_for("single_entry")
    assert set(n.tolist()) == {0, 1}
    n, _ = lengths_for("mixed_short")
    assert (n > 512).sum() == 2 and (n == 0).sum() > 100
    n, _ = lengths_for("tall")
    assert -(-len(n) // 64) > 1024


@pytest.mark.gpu
@pytest.mark.parametrize("layout,B,dtype", CASES, ids=[f"{c[0]}-b{c[1]}-{c[2]}" for c in CASES])
def test_packed_forward(orc, layout, B, dtype):
    rel = BF16_REL if dtype == "bf16" else FP32_REL
    for integer in (True, False):
        L = build(layout, dtype, integer)
        out, in_ = L.out, L.in_
        # the widest packing (a layer this small would otherwise hardly pack)
        with env(COOSPMM_PACK_LIMIT="505"):
            h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
        try:
            seed = out + in_ + B
            Xh = W.random_dense((B, in_), seed + 1, dtype=dtype, integer=integer)
            bh = W.random_dense((out,), seed + 2, dtype=dtype, integer=integer)
            X, bias = dev(Xh), dev(bh)

            def run():
                H = torch.empty((B, out), dtype=X.dtype, device="cuda")
                r = {"fwd": host(csp.spmm_fwd(h, X)),
                     "act": host(csp.spmm_fwd_act(h, X, bias=bias, act="gelu", H=H))}
                r["pre"] = host(H)
                return r

            with env(COOSPMM_PACKED="1"):
                packed = run()
                with env(COOSPMM_LDS_TABLES="0"):
                    glob = run()
                with env(COOSPMM_LDS_TABLES="0", COOSPMM_GROUPED_SPLITS="0"):
                    fixup = run()
            for k in packed:
                assert np.array_equal(glob[k].view(np.uint8), packed[k].view(np.uint8)), f"{k}: global vs LDS"
                assert np.array_equal(fixup[k].view(np.uint8), packed[k].view(np.uint8)), f"{k}: fixup vs in-pass"
            ref, S = orc.spmm_fwd(out, in_, L.rows, L.cols, L.vals, Xh)
            if integer:
                want = ref.astype(np.float32)
                if dtype == "bf16":
                    want = W.f32_to_bf16_bits(want)
                assert np.array_equal(packed["fwd"].view(np.uint8), want.view(np.uint8)), "exact sums"
                with env(COOSPMM_PACKED="0"):
                    plain = run()
                for k in packed:
                    assert np.array_equal(plain[k].view(np.uint8), packed[k].view(np.uint8)), f"{k}: plain list"
            else:
                assert_within(packed["fwd"], ref, S, rel, f"{layout} B={B} forward")
                yb = ref + as_f64(bh)[None, :]
                Sb = S + np.abs(as_f64(bh))[None, :]
                assert_within(packed["pre"], yb, Sb, rel, f"{layout} B={B} pre-activation")
                assert_within(packed["act"], orc.gelu(yb), Sb, 1.3e-5 if dtype == "f32" else 1.2e-2,
                              f"{layout} B={B} GELU")
        finally:
            csp.sparse_layer_destroy(h)


@pytest.mark.gpu
def test_packed_list_across_restructures(orc):
    """The packed list is rebuilt by a restructure only after a narrow forward was asked for; in
    between the forward uses the plain list.  Every state must give the oracle's exact sums."""
    n, in_ = lengths_for("mixed_short")
    L = layer_from_lengths(n, in_, 5, "f32", integer=True)
    out = L.out
    with env(COOSPMM_PACK_LIMIT="505"):
        h = csp.sparse_layer_create(out, in_, dev(L.rows), dev(L.cols), dev(L.vals))
        try:
            Xh = W.random_dense((1, in_), 77, integer=True)
            X = dev(Xh)

            def check(tag):
                r, c, v = (host(t) for t in csp.sparse_layer_export(h))
                ref, _ = orc.spmm_fwd(out, in_, r, c, v, Xh)
                got = host(csp.spmm_fwd(h, X))
                assert np.array_equal(got, ref.astype(np.float32)), tag
                with env(COOSPMM_PACKED="0"):
                    plain = host(csp.spmm_fwd(h, X))
                assert np.array_equal(plain.view(np.uint32), got.view(np.uint32)), tag

            csp.restructure(h, 5000, seed=9, step=1)   # no narrow forward yet: packed list not rebuilt
            check("after a restructure that skipped the packed list")
            csp.restructure(h, 5000, seed=9, step=2)   # narrow forward seen: rebuilt
            check("after a restructure that rebuilt it")
        finally:
            csp.sparse_layer_destroy(h)
