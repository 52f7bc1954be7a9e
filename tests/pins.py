"""Pins for the CPU oracle: checks against what mathematics and libraries fix.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with an independent fact: a dense matmul, exact integer
arithmetic, the adjoint identity, finite differences, brute-force sorting,
numpy's own Philox generator, torch's bf16 conversion, scipy's erf.  None of
them re-types the oracle's loops.  The same battery runs against planted
mutants of the oracle, each of which must fail at least one pin.
"""
from __future__ import annotations

import numpy as np

from coo_spmm_fwd_amd import workloads as W


# ---------------------------------------------------------------- helpers
def densify(out, in_, rows, cols, vals):
    Wd = np.zeros((out, in_), np.float64)
    Wd[rows, cols] = vals.astype(np.float64) if vals.dtype != np.uint16 else W.bf16_bits_to_f32(vals)
    return Wd


def f64(a):
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _layer(out, in_, nnz, seed, integer=False, dtype="f32"):
    return W.random_layer(out, in_, nnz, seed, dtype=dtype, integer=integer)


def _close(a, b, S, rel):
    err = np.abs(a - b)
    bound = rel * np.maximum(S, 1e-300)
    assert np.all((err <= bound) | (err == 0)), f"max err/S {np.max(err / np.maximum(S, 1e-300)):.3e}"


# ---------------------------------------------------------------- products
def pin_dense_tiny(orc):
    """Densified W and numpy matmul agree with the oracle on tiny shapes and several sparsities."""
    for (out, in_, B), frac, seed in [((5, 7, 3), 0.0, 1), ((5, 7, 3), 0.3, 2), ((5, 7, 3), 1.0, 3),
                                       ((1, 9, 1), 0.5, 4), ((8, 1, 2), 0.5, 5), ((6, 6, 4), 0.2, 6),
                                       ((13, 11, 5), 0.15, 7)]:
        nnz = int(round(frac * out * in_))
        L = _layer(out, in_, nnz, seed)
        X = W.random_dense((B, in_), seed + 100)
        dY = W.random_dense((B, out), seed + 200)
        Wd = densify(out, in_, L.rows, L.cols, L.vals)
        Y, S = orc.spmm_fwd(out, in_, L.rows, L.cols, L.vals, X)
        _close(Y, f64(X) @ Wd.T, S, 1e-13)
        dX, S2 = orc.spmm_bwd_input(out, in_, L.rows, L.cols, L.vals, dY)
        _close(dX, f64(dY) @ Wd, S2, 1e-13)
        dW, S3 = orc.spmm_bwd_values(out, in_, L.rows, L.cols, dY, X)
        G = f64(dY).T @ f64(X)
        _close(dW, G[L.rows, L.cols], S3, 1e-13)
        # magnitude sums are sums of |terms|: compare with |W| and |X| products
        _close(S, np.abs(f64(X)) @ np.abs(Wd).T, S, 1e-13)


def pin_integer_exact(orc):
    """Integer-valued inputs: every partial sum is an exact small integer, so results are bit-exact."""
    out, in_, B = 37, 29, 6
    L = _layer(out, in_, 300, 11, integer=True)
    X = W.random_dense((B, in_), 12, integer=True)
    dY = W.random_dense((B, out), 13, integer=True)
    Wd = densify(out, in_, L.rows, L.cols, L.vals)
    Y, _ = orc.spmm_fwd(out, in_, L.rows, L.cols, L.vals, X)
    assert np.array_equal(Y, f64(X) @ Wd.T)
    dX, _ = orc.spmm_bwd_input(out, in_, L.rows, L.cols, L.vals, dY)
    assert np.array_equal(dX, f64(dY) @ Wd)
    dW, _ = orc.spmm_bwd_values(out, in_, L.rows, L.cols, dY, X)
    assert np.array_equal(dW, (f64(dY).T @ f64(X))[L.rows, L.cols])


def pin_zero_sparsity(orc):
    """At 0% sparsity the layer is a dense layer: bit-identical to a naive fp64 loop in the same order."""
    out, in_, B = 6, 5, 3
    rows = np.repeat(np.arange(out), in_).astype(np.int32)
    cols = np.tile(np.arange(in_), out).astype(np.int32)
    vals = W.random_dense((out * in_,), 21)
    X = W.random_dense((B, in_), 22)
    Y, _ = orc.spmm_fwd(out, in_, rows, cols, vals, X)
    ref = np.zeros((B, out))
    for b in range(B):
        for r in range(out):
            acc = 0.0
            for c in range(in_):
                acc += float(vals[r * in_ + c]) * float(X[b, c])
            ref[b, r] = acc
    assert np.array_equal(Y, ref)
    np.testing.assert_allclose(Y, f64(X) @ f64(vals).reshape(out, in_).T, rtol=1e-13, atol=1e-14)


def pin_adjoint(orc):
    """<dY, X W^T> = <dY W, X> = <dW, v> for random fp32 data (fp64 rounding only)."""
    out, in_, B = 300, 200, 5
    L = _layer(out, in_, 6000, 31)
    X = W.random_dense((B, in_), 32)
    dY = W.random_dense((B, out), 33)
    Y, _ = orc.spmm_fwd(out, in_, L.rows, L.cols, L.vals, X)
    dX, _ = orc.spmm_bwd_input(out, in_, L.rows, L.cols, L.vals, dY)
    dW, _ = orc.spmm_bwd_values(out, in_, L.rows, L.cols, dY, X)
    a = float(np.sum(f64(dY) * Y))
    b = float(np.sum(dX * f64(X)))
    c = float(np.dot(dW, f64(L.vals)))
    scale = float(np.sum(np.abs(f64(dY)) @ np.abs(densify(out, in_, L.rows, L.cols, L.vals)) * np.abs(f64(X))))
    assert abs(a - b) <= 1e-12 * scale and abs(a - c) <= 1e-12 * scale, (a, b, c)


def pin_finite_differences(orc):
    """L(v) = <dY, fwd(X; v)> is linear in v and X, so central differences equal dW and dX up to rounding."""
    out, in_, B = 9, 8, 4
    rng = np.random.default_rng(41)
    L = _layer(out, in_, 30, 41)
    # values on a 2^-10 grid so that v +- h is exact in fp32
    L.vals = (np.round(rng.standard_normal(L.nnz) * 1024) / 1024).astype(np.float32)
    X = (np.round(rng.standard_normal((B, in_)) * 1024) / 1024).astype(np.float32)
    dY = W.random_dense((B, out), 42)
    h = np.float32(2.0 ** -4)

    def loss(vals, Xa):
        Y, _ = orc.spmm_fwd(out, in_, L.rows, L.cols, vals, Xa)
        return float(np.sum(f64(dY) * Y))

    dW, _ = orc.spmm_bwd_values(out, in_, L.rows, L.cols, dY, X)
    for k in range(L.nnz):
        vp = L.vals.copy(); vp[k] += h
        vm = L.vals.copy(); vm[k] -= h
        fd = (loss(vp, X) - loss(vm, X)) / (2 * float(h))
        assert abs(fd - dW[k]) <= 1e-12 * (1 + abs(dW[k])), (k, fd, dW[k])
    dX, _ = orc.spmm_bwd_input(out, in_, L.rows, L.cols, L.vals, dY)
    for b in range(B):
        for c in range(in_):
            xp = X.copy(); xp[b, c] += h
            xm = X.copy(); xm[b, c] -= h
            fd = (loss(L.vals, xp) - loss(L.vals, xm)) / (2 * float(h))
            assert abs(fd - dX[b, c]) <= 1e-12 * (1 + abs(dX[b, c])), (b, c, fd, dX[b, c])


def pin_special_cases(orc):
    """Permutation W, single nnz, empty layer, one full row, B = 1."""
    rng = np.random.default_rng(51)
    n, B = 17, 3
    perm = rng.permutation(n)
    rows = np.arange(n, dtype=np.int32)
    cols = perm.astype(np.int32)
    ones = np.ones(n, np.float32)
    X = W.random_dense((B, n), 52)
    Y, _ = orc.spmm_fwd(n, n, rows, cols, ones, X)
    assert np.array_equal(Y, f64(X)[:, perm])            # Y[:, r] = X[:, perm[r]]
    dX, _ = orc.spmm_bwd_input(n, n, rows, cols, ones, X)
    inv = np.argsort(perm)
    assert np.array_equal(dX, f64(X)[:, inv])
    # single nnz
    Y, _ = orc.spmm_fwd(4, 6, np.array([2], np.int32), np.array([5], np.int32), np.array([1.5], np.float32),
                        np.arange(12, dtype=np.float32).reshape(2, 6))
    exp = np.zeros((2, 4)); exp[0, 2] = 1.5 * 5; exp[1, 2] = 1.5 * 11
    assert np.array_equal(Y, exp)
    # empty layer
    e = np.zeros(0, np.int32)
    Y, S = orc.spmm_fwd(3, 4, e, e, np.zeros(0, np.float32), np.ones((2, 4), np.float32))
    assert np.array_equal(Y, np.zeros((2, 3))) and np.array_equal(S, np.zeros((2, 3)))
    dW, _ = orc.spmm_bwd_values(3, 4, e, e, np.ones((2, 3), np.float32), np.ones((2, 4), np.float32))
    assert dW.shape == (0,)
    # one full row, B = 1: the row's output is a dot product
    in_ = 40
    rows = np.full(in_, 3, np.int32)
    cols = rng.permutation(in_).astype(np.int32)
    vals = W.random_dense((in_,), 53)
    x = W.random_dense((1, in_), 54)
    Y, _ = orc.spmm_fwd(5, in_, rows, cols, vals, x)
    Wd = densify(5, in_, rows, cols, vals)
    assert np.all(Y[0, [0, 1, 2, 4]] == 0)
    assert abs(Y[0, 3] - float(np.dot(Wd[3], f64(x)[0]))) <= 1e-13 * float(np.sum(np.abs(Wd[3] * f64(x)[0])))


def pin_bf16(orc):
    """bf16 words decode like torch's bfloat16 -> float32 conversion; bf16 products follow."""
    import torch
    x = np.random.default_rng(61).standard_normal(1000).astype(np.float32)
    bits = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(W.bf16_bits_to_f32(bits), ref)    # generator rounding is torch's RNE
    dec = orc.decode(bits[:200])
    assert np.array_equal(dec, ref[:200].astype(np.float64))
    out, in_, B = 11, 13, 2
    L = _layer(out, in_, 40, 62, dtype="bf16")
    Xb = W.random_dense((B, in_), 63, dtype="bf16")
    Y, S = orc.spmm_fwd(out, in_, L.rows, L.cols, L.vals, Xb)
    _close(Y, f64(Xb) @ densify(out, in_, L.rows, L.cols, L.vals).T, S, 1e-13)


# ---------------------------------------------------------------- canonical order
def pin_canonicalize(orc):
    """Canonical arrays equal a brute-force Python sort; invariants hold; errors are reported."""
    out, in_ = 9, 12
    L = _layer(out, in_, 50, 71)
    res = orc.canonicalize(out, in_, L.rows, L.cols, L.vals)
    assert res["status"] == 0
    trip = sorted(zip(L.rows.tolist(), L.cols.tolist(), range(L.nnz)))
    assert res["rows"].tolist() == [t[0] for t in trip]
    assert res["cols"].tolist() == [t[1] for t in trip]
    assert res["src"].tolist() == [t[2] for t in trip]
    assert np.array_equal(res["vals"].view(np.uint32), L.vals[res["src"]].view(np.uint32))
    counts = np.bincount(L.rows, minlength=out)
    assert res["row_ptr"].tolist() == [0] + np.cumsum(counts).tolist()
    tr = sorted(range(L.nnz), key=lambda k: (trip[k][1], trip[k][0]))
    assert res["perm_c"].tolist() == tr
    assert res["rows_by_col"].tolist() == [trip[k][0] for k in tr]
    ccounts = np.bincount(L.cols, minlength=in_)
    assert res["col_ptr"].tolist() == [0] + np.cumsum(ccounts).tolist()
    again = orc.canonicalize(out, in_, res["rows"], res["cols"], res["vals"])
    assert again["src"].tolist() == list(range(L.nnz))
    bad = orc.canonicalize(out, in_, np.array([0, 9], np.int32), np.array([0, 0], np.int32),
                           np.zeros(2, np.float32))
    assert bad["status"] == -2
    bad = orc.canonicalize(out, in_, np.array([0, 1], np.int32), np.array([0, -1], np.int32),
                           np.zeros(2, np.float32))
    assert bad["status"] == -2
    dup = orc.canonicalize(out, in_, np.array([3, 1, 3], np.int32), np.array([4, 0, 4], np.int32),
                           np.zeros(3, np.float32))
    assert dup["status"] == -3


# ---------------------------------------------------------------- random stream
def numpy_philox_block(seed: int, step: int, block: int):
    """Block (block, step, 0, 0) under key (seed, 0), taken from numpy's own Philox4x64-10.

    numpy increments its 256-bit counter before each block, so it is started
    one below the wanted counter."""
    import numpy.random as npr
    ctr = (block | (step << 64)) - 1
    ctr %= 1 << 256
    words = [(ctr >> (64 * i)) & ((1 << 64) - 1) for i in range(4)]
    bg = npr.Philox(key=np.array([seed, 0], np.uint64), counter=np.array(words, np.uint64))
    return [int(v) for v in bg.random_raw(4)]


def pin_philox(orc):
    """The oracle's Philox4x64-10 equals numpy.random.Philox block for block."""
    for seed, step, block in [(0, 0, 0), (5, 0, 0), (5, 3, 0), (5, 3, 7), (2**64 - 1, 9, 123456),
                              (123456789, 2**40 + 3, 2**33 + 5), (1, 1, 1)]:
        got = orc.philox4x64_10([block, step, 0, 0], [seed, 0]).tolist()
        assert got == numpy_philox_block(seed, step, block), (seed, step, block)
    for i in range(12):
        assert orc.regrow_draw(7, 2, i) == numpy_philox_block(7, 2, i // 4)[i % 4]


def pin_position_map(orc):
    """floor(u * n / 2^64) in exact integer arithmetic; end points and monotonicity."""
    rng = np.random.default_rng(81)
    for n_out, n_in in [(1, 1), (3, 5), (4096, 4096), (16384, 16384), (8192, 8192), (65535, 65537)]:
        n = n_out * n_in
        us = [0, 1, 2**63, 2**64 - 1] + [int(x) for x in rng.integers(0, 2**63, 20, dtype=np.int64)]
        for u in us:
            p = orc.regrow_position(u, n_out, n_in)
            assert p == (u * n) >> 64 and 0 <= p < n
        assert orc.regrow_position(2**64 - 1, n_out, n_in) == n - 1


# ---------------------------------------------------------------- restructure
def brute_restructure(out, in_, rows_c, cols_c, vals_c, n_prune, seed, step, regrow_value):
    """Set-based re-implementation of the restructure reading, fed by numpy's Philox."""
    mag = vals_c.view(np.uint32) & 0x7FFFFFFF
    order = sorted(range(len(rows_c)), key=lambda k: (int(mag[k]), k))
    pruned = set(order[:n_prune])
    kept = [(int(rows_c[k]), int(cols_c[k]), float(vals_c[k])) for k in range(len(rows_c)) if k not in pruned]
    occ = {r * in_ + c for r, c, _ in kept}
    new, i, block_cache = [], 0, {}
    while len(new) < n_prune:
        blk = i // 4
        if blk not in block_cache:
            block_cache = {blk: numpy_philox_block(seed, step, blk)}
        p = (block_cache[blk][i % 4] * (out * in_)) >> 64
        i += 1
        if p in occ:
            continue
        occ.add(p)
        new.append((p // in_, p % in_, regrow_value))
    allt = sorted(kept + new)
    return (np.array([t[0] for t in allt], np.int32), np.array([t[1] for t in allt], np.int32),
            np.array([t[2] for t in allt], np.float32), i)


def pin_restructure(orc):
    """Restructure equals the set-based brute force and keeps every invariant."""
    cases = [(6, 7, 12, 3, 1, 0), (6, 7, 12, 0, 1, 1), (6, 7, 42, 5, 2, 3), (6, 7, 40, 40, 3, 4),
             (20, 30, 200, 20, 5, 9), (1, 50, 10, 4, 6, 2), (50, 1, 10, 4, 7, 2)]
    for out, in_, nnz, n_prune, seed, step in cases:
        L = _layer(out, in_, nnz, 90 + seed)
        # plant ties: some equal magnitudes and a signed zero pair
        v = L.vals.copy()
        if nnz >= 6:
            v[1] = -v[0]
            v[2] = 0.0
            v[3] = -0.0
        c = orc.canonicalize(out, in_, L.rows, L.cols, v)
        r2, c2, v2, draws = orc.restructure(out, in_, c["rows"], c["cols"], c["vals"], n_prune, seed, step, 0.25)
        br, bc, bv, bdraws = brute_restructure(out, in_, c["rows"], c["cols"], c["vals"], n_prune, seed, step, 0.25)
        assert np.array_equal(r2, br) and np.array_equal(c2, bc), (out, in_, nnz, n_prune)
        assert np.array_equal(v2.view(np.uint32), bv.view(np.uint32))
        assert draws == bdraws
        # invariants
        keys = r2.astype(np.int64) * in_ + c2
        assert len(keys) == nnz and np.all(np.diff(keys) > 0)
        mag = c["vals"].view(np.uint32) & 0x7FFFFFFF
        old = dict(zip((c["rows"].astype(np.int64) * in_ + c["cols"]).tolist(), c["vals"].view(np.uint32).tolist()))
        new = dict(zip(keys.tolist(), v2.view(np.uint32).tolist()))
        kept = [k for k in old if k in new and new[k] == old[k]]
        assert len(kept) >= nnz - n_prune
        if 0 < n_prune < nnz:
            order = sorted(range(nnz), key=lambda k: (int(mag[k]), k))
            assert int(mag[order[n_prune - 1]]) <= int(mag[order[n_prune]])
    # determinism and dependence on seed / step
    L = _layer(30, 30, 200, 99)
    c = orc.canonicalize(30, 30, L.rows, L.cols, L.vals)
    a = orc.restructure(30, 30, c["rows"], c["cols"], c["vals"], 20, 1, 1)
    b = orc.restructure(30, 30, c["rows"], c["cols"], c["vals"], 20, 1, 1)
    d = orc.restructure(30, 30, c["rows"], c["cols"], c["vals"], 20, 1, 2)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3]))
    assert not np.array_equal(a[1], d[1])


# ------------------------------------------------ gradient-informed regrow
def brute_restructure_grad(out, in_, rows_c, cols_c, vals_c, n_prune, dY, X, regrow_value):
    """Set-based reading of the gradient-informed restructure with exact integer scores:
    the same prune, then the empty positions ranked by |(dY^T X)[r, c]| (computed exactly in
    int64, so no summation order matters), ties to the smaller position."""
    mag = vals_c.view(np.uint32) & 0x7FFFFFFF
    order = sorted(range(len(rows_c)), key=lambda k: (int(mag[k]), k))
    pruned = set(order[:n_prune])
    kept = [(int(rows_c[k]), int(cols_c[k]), float(vals_c[k])) for k in range(len(rows_c)) if k not in pruned]
    occ = {r * in_ + c for r, c, _ in kept}
    G = np.abs(dY.astype(np.int64).T @ X.astype(np.int64))  # [out, in], exact
    empty = [p for p in range(out * in_) if p not in occ]
    empty.sort(key=lambda p: (-int(G[p // in_, p % in_]), p))
    new = [(p // in_, p % in_, regrow_value) for p in empty[:n_prune]]
    allt = sorted(kept + new)
    return (np.array([t[0] for t in allt], np.int32), np.array([t[1] for t in allt], np.int32),
            np.array([t[2] for t in allt], np.float32))


def pin_restructure_grad(orc):
    """Gradient-informed regrow: equals the exact brute force on integer-valued operands (every score
    exact, many ties), and on random operands the regrown positions outscore every position left empty."""
    rng = np.random.default_rng(17)
    for out, in_, nnz, n_prune, B in [(7, 9, 25, 6, 4), (12, 5, 30, 12, 3), (1, 40, 12, 5, 2), (30, 1, 12, 5, 6)]:
        L = _layer(out, in_, nnz, 70 + out)
        c = orc.canonicalize(out, in_, L.rows, L.cols, L.vals)
        dY = rng.integers(-2, 3, size=(B, out)).astype(np.float32)
        X = rng.integers(-2, 3, size=(B, in_)).astype(np.float32)
        r2, c2, v2 = orc.restructure_grad(out, in_, c["rows"], c["cols"], c["vals"], n_prune, dY, X, -0.5)
        br, bc, bv = brute_restructure_grad(out, in_, c["rows"], c["cols"], c["vals"], n_prune, dY, X, -0.5)
        assert np.array_equal(r2, br) and np.array_equal(c2, bc), (out, in_, nnz, n_prune)
        assert np.array_equal(v2.view(np.uint32), bv.view(np.uint32))
    # random operands: ranking invariant against numpy's fp64 scores (within fp32 rounding)
    out, in_, nnz, n_prune, B = 40, 50, 400, 60, 8
    L = _layer(out, in_, nnz, 5)
    c = orc.canonicalize(out, in_, L.rows, L.cols, L.vals)
    dY = rng.standard_normal((B, out)).astype(np.float32)
    X = rng.standard_normal((B, in_)).astype(np.float32)
    r2, c2, v2 = orc.restructure_grad(out, in_, c["rows"], c["cols"], c["vals"], n_prune, dY, X, 0.0)
    keys = r2.astype(np.int64) * in_ + c2
    assert len(keys) == nnz and np.all(np.diff(keys) > 0)
    mag = c["vals"].view(np.uint32) & 0x7FFFFFFF
    order = sorted(range(nnz), key=lambda k: (int(mag[k]), k))
    kept = {int(c["rows"][k]) * in_ + int(c["cols"][k]) for k in order[n_prune:]}
    new = [int(k) for k in keys if int(k) not in kept]
    assert len(new) == n_prune
    G = np.abs(dY.astype(np.float64).T @ X.astype(np.float64))
    S = np.abs(dY.astype(np.float64)).T @ np.abs(X.astype(np.float64))
    left = [p for p in range(out * in_) if p not in kept and p not in set(new)]
    lo = min(G[p // in_, p % in_] + 1e-6 * S[p // in_, p % in_] for p in new)
    hi = max(G[p // in_, p % in_] - 1e-6 * S[p // in_, p % in_] for p in left)
    assert lo >= hi


# ---------------------------------------------------------------- GELU
def pin_gelu(orc):
    from scipy.special import erf
    x = np.linspace(-8, 8, 2001)
    ref = 0.5 * x * (1 + erf(x / np.sqrt(2)))
    np.testing.assert_allclose(orc.gelu(x), ref, rtol=1e-14, atol=1e-15)
    h = 1e-5
    fd = (0.5 * (x + h) * (1 + erf((x + h) / np.sqrt(2))) - 0.5 * (x - h) * (1 + erf((x - h) / np.sqrt(2)))) / (2 * h)
    np.testing.assert_allclose(orc.gelu_grad(x), fd, rtol=1e-8, atol=1e-9)


ALL_PINS = [pin_dense_tiny, pin_integer_exact, pin_zero_sparsity, pin_adjoint, pin_finite_differences,
            pin_special_cases, pin_bf16, pin_canonicalize, pin_philox, pin_position_map, pin_restructure,
            pin_restructure_grad, pin_gelu]
