"""Seeded synthetic inputs for the truly sparse COO layer.

This module only draws inputs: COO positions, weight values and dense
activations.  It holds none of the layer's arithmetic and imports neither the
HIP binding nor the CPU oracle, so both sides can consume the same arrays.

The page this layer comes from ("Beyond Masked Sparsity: SNACK Enables Truly
Sparse Neural Networks on GPU", Abstract) reports results for single sparse
layers at 90-99% sparsity in the small-batch regime of training and of
single-stream inference, and for GPT-2 training; it publishes no data set or
layer shape.  The workloads below are synthetic stand-ins with those
properties: unstructured uniform positions, a power-law (Zipf) row-degree
variant for inference, and GPT-2-small MLP shapes (768 -> 3072 -> 768) without
any GPT-2 weights or data.

Conventions (each is a stated reading, not something the page fixes):
  * nnz = round(density * out * in) distinct positions, drawn uniformly
    without replacement (not Bernoulli per position);
  * "N(0, s)" means standard deviation s;
  * bf16 inputs are drawn in fp32 and rounded to nearest-even bf16;
  * triples are returned in random order, so the layer builder must sort.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass
class CooWeights:
    out: int
    in_: int
    rows: np.ndarray  # int32 [nnz], random order
    cols: np.ndarray  # int32 [nnz]
    vals: np.ndarray  # float32 [nnz], or uint16 bf16 bit patterns
    dtype: str        # "f32" or "bf16"

    @property
    def nnz(self) -> int:
        return int(self.rows.shape[0])


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: tuple          # ((out, in), ...)
    density: float
    batches: tuple         # batch sizes B
    w_std: object          # float, or "inv_sqrt_row" for 1/sqrt(nnz per row)
    dtype: str             # "f32" | "bf16"
    structure: str         # "uniform" | "zipf"
    seed: int
    ops: str               # which layer calls one step runs
    zipf_s: float = 1.1
    steps: int = 1
    prune_frac: float = 0.0
    gelu: bool = False


WORKLOADS = {
    w.name: w
    for w in (
        Workload("linear1024_b8_s90", ((1024, 1024),), 0.10, (8,), "inv_sqrt_row", "f32", "uniform", 1,
                 "fwd+dX+dW"),
        Workload("linear4096_b16_s95", ((4096, 4096),), 0.05, (16,), 0.02, "f32", "uniform", 2, "fwd+dX+dW"),
        Workload("mlp768x3072_s90", ((3072, 768), (768, 3072)), 0.10, (1, 4, 32), 0.02, "f32", "uniform", 3,
                 "fwd+bwd of both layers, GELU between", gelu=True),
        Workload("inference16384_zipf_s99_bf16", ((16384, 16384),), 0.01, (1, 4), 0.02, "bf16", "zipf", 4,
                 "fwd"),
        Workload("dst8192_b64_s95", ((8192, 8192),), 0.05, (64,), 0.02, "f32", "uniform", 5,
                 "fwd+dX+dW then restructure", steps=10, prune_frac=0.10),
        Workload("stack16384x4_zipf_s99_bf16", ((16384, 16384),) * 4, 0.01, (1, 4), 0.02, "bf16", "zipf", 6,
                 "fwd of four layers, GELU between, one graph per token", gelu=True),
        # the pages' single-layer comparisons at 90% sparsity (training step and inference) on the
        # 4096-square shape
        Workload("linear4096_b16_s90", ((4096, 4096),), 0.10, (16,), 0.02, "f32", "uniform", 7, "fwd+dX+dW"),
    )
}


def nnz_for(out: int, in_: int, density: float) -> int:
    return int(round(density * out * in_))


def streams(seed: int, n: int = 8):
    """Independent numpy generators spawned from one master seed."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to the nearest bf16, ties to even; returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((b >> 16) & 1)
    return ((b + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniform_positions(out: int, in_: int, nnz: int, rng) -> tuple[np.ndarray, np.ndarray]:
    """nnz distinct flat positions, uniform without replacement, in random order."""
    flat = rng.choice(out * in_, size=nnz, replace=False, shuffle=True)
    return (flat // in_).astype(np.int32), (flat % in_).astype(np.int32)


def zipf_row_counts(out: int, in_: int, nnz: int, s: float, rng) -> np.ndarray:
    """Per-row nnz with a capped power law over rows.

    Row ranks are a seeded random permutation.  The row of rank q (1-based)
    gets min(in, floor(c * q^-s)) entries, with c the largest value (found by
    bisection) for which the total does not exceed nnz; the shortfall then
    goes one by one to the highest-ranked rows that are not yet full.
    """
    ranks = np.arange(1, out + 1, dtype=np.float64)
    w = ranks ** (-s)

    def total(c):
        return int(np.minimum(in_, np.floor(c * w)).sum())

    lo, hi = 0.0, float(in_) * out
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if total(mid) <= nnz:
            lo = mid
        else:
            hi = mid
    counts_by_rank = np.minimum(in_, np.floor(lo * w)).astype(np.int64)
    short = nnz - int(counts_by_rank.sum())
    q = 0
    while short > 0:
        if counts_by_rank[q] < in_:
            counts_by_rank[q] += 1
            short -= 1
        q = (q + 1) % out
    perm = rng.permutation(out)          # perm[q] = row that has rank q+1
    counts = np.empty(out, np.int64)
    counts[perm] = counts_by_rank
    return counts, lo


def zipf_positions(out: int, in_: int, nnz: int, s: float, rng):
    counts, _ = zipf_row_counts(out, in_, nnz, s, rng)
    rows = np.repeat(np.arange(out, dtype=np.int32), counts)
    cols = np.empty(nnz, np.int32)
    pos = 0
    for r in range(out):
        n = int(counts[r])
        if n:
            cols[pos:pos + n] = rng.choice(in_, size=n, replace=False)
            pos += n
    order = rng.permutation(nnz)
    return rows[order], cols[order]


def make_weights(out: int, in_: int, density: float, w_std, dtype: str, structure: str, rng_pos, rng_val,
                 zipf_s: float = 1.1) -> CooWeights:
    nnz = nnz_for(out, in_, density)
    if structure == "uniform":
        rows, cols = uniform_positions(out, in_, nnz, rng_pos)
    elif structure == "zipf":
        rows, cols = zipf_positions(out, in_, nnz, zipf_s, rng_pos)
    else:
        raise ValueError(structure)
    std = 1.0 / math.sqrt(nnz / out) if w_std == "inv_sqrt_row" else float(w_std)
    v = (rng_val.standard_normal(nnz) * std).astype(np.float32)
    vals = f32_to_bf16_bits(v) if dtype == "bf16" else v
    return CooWeights(out, in_, rows, cols, vals, dtype)


def dense(shape, dtype: str, rng, std: float = 1.0) -> np.ndarray:
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def build(name: str):
    """All arrays of one workload: layers, and per batch size the X and dY draws."""
    w = WORKLOADS[name]
    rs = streams(w.seed, 4 + 4 * len(w.layers))
    layers = []
    for li, (out, in_) in enumerate(w.layers):
        layers.append(make_weights(out, in_, w.density, w.w_std, w.dtype, w.structure, rs[4 * li],
                                   rs[4 * li + 1], w.zipf_s))
    acts = {}
    for B in w.batches:
        first_in = w.layers[0][1]
        last_out = w.layers[-1][0]
        acts[B] = dict(X=dense((B, first_in), w.dtype, rs[2]), dY=dense((B, last_out), w.dtype, rs[3]))
    return w, layers, acts


def random_layer(out: int, in_: int, nnz: int, seed: int, dtype: str = "f32", integer: bool = False,
                 std: float = 1.0) -> CooWeights:
    """Small seeded layer for tests; integer=True draws values in {-3..3}."""
    r_pos, r_val = streams(seed, 2)
    rows, cols = uniform_positions(out, in_, nnz, r_pos)
    if integer:
        v = r_val.integers(-3, 4, size=nnz).astype(np.float32)
    else:
        v = (r_val.standard_normal(nnz) * std).astype(np.float32)
    vals = f32_to_bf16_bits(v) if dtype == "bf16" else v
    return CooWeights(out, in_, rows, cols, vals, dtype)


def random_dense(shape, seed: int, dtype: str = "f32", integer: bool = False) -> np.ndarray:
    rng = streams(seed, 1)[0]
    if integer:
        x = rng.integers(-4, 5, size=shape).astype(np.float32)
    else:
        x = rng.standard_normal(shape).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x
