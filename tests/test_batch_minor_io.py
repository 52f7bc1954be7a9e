"""Batch-minor operands passed between calls: spmm_batch_minor, spmm_fwd_bm, spmm_bwd_bm.

A batch-minor copy of A [B, n] is T [n, ld] with T[c, b] = A[b, c] for b < B and zero pad slots
(ld = the power of two >= B).  spmm_batch_minor must write exactly that; spmm_fwd_bm / spmm_bwd_bm must
give bitwise the outputs of spmm_fwd_act / spmm_bwd_act (or the plain calls) whether or not the caller
hands them the copies of their operands, and their output copies must be the copies of their outputs.
Every path that stores an output is covered: task kernels with split rows and columns (power-law layer:
grouped splits at B <= 8 and the split fixup above), the LDS-table path (small operand tables), the
packed path (B <= 4), the LDS tiles (an 8192-square fp32 layer at B = 48), and a bf16 layer; B = 20
and 3 leave pad slots.  The operand copies feed the products' own gathers, so equality also checks
that a caller's copy is read exactly as the call's own would be.
"""
import numpy as np
import pytest
import torch

from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import bits, dev, host

pytestmark = pytest.mark.gpu


def layout(A, ld):
    """Reference batch-minor copy of a host array A [B, n]."""
    B, n = A.shape
    T = np.zeros((n, ld), dtype=A.dtype)
    T[:, :B] = A.T
    return T


def zipf_layer(out, in_, nnz, seed, dtype="f32"):
    r_pos, r_val = W.streams(seed, 2)
    rows, cols = W.zipf_positions(out, in_, nnz, 1.1, r_pos)
    v = r_val.standard_normal(nnz).astype(np.float32)
    return W.CooWeights(out, in_, rows, cols, W.f32_to_bf16_bits(v) if dtype == "bf16" else v, dtype)


CASES = {
    # name: (layer factory, batches)
    "power-law splits": (lambda: zipf_layer(3000, 4000, 400000, 5), (3, 8, 20, 32)),
    "lds tables": (lambda: W.random_layer(300, 260, 9000, seed=6), (3, 20, 64)),
    "uniform": (lambda: W.random_layer(3072, 768, 235930, seed=7), (32,)),
    "bf16": (lambda: zipf_layer(2000, 2500, 150000, 8, "bf16"), (4, 20)),
    "tiles": (lambda: W.random_layer(8192, 8192, 3355443, seed=9), (48,)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_bm_calls_match_plain_calls(case):
    make, batches = CASES[case]
    L = make()
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        td = torch.bfloat16 if L.dtype == "bf16" else torch.float32
        cast = (lambda a: dev(a).to(td)) if L.dtype == "bf16" else dev
        for B in batches:
            ld = csp.batch_minor_ld(B)
            X = cast(W.random_dense((B, L.in_), 10 + B))
            dY = cast(W.random_dense((B, L.out), 11 + B))
            Hin = cast(W.random_dense((B, L.in_), 12 + B))
            bias = cast(W.random_dense((L.out,), 13))
            tag = f"{case} B={B}"
            # the copy itself
            XT = csp.spmm_batch_minor(X)
            dYT = csp.spmm_batch_minor(dY)
            assert np.array_equal(host(XT).view(np.uint8), layout(host(X), ld).view(np.uint8)), f"{tag}: X copy"
            # forward: plain and with bias + GELU + pre-activation
            Y0 = csp.spmm_fwd(h, X)
            H0 = torch.empty_like(Y0)
            A0 = csp.spmm_fwd_act(h, X, bias=bias, act="gelu", H=H0)
            for xt in (None, XT):
                YT = torch.zeros((L.out, ld), dtype=td, device="cuda")
                Y = csp.spmm_fwd_bm(h, X, XT=xt, YT=YT)
                assert np.array_equal(host(Y).view(np.uint8), host(Y0).view(np.uint8)), f"{tag}: plain forward"
                assert np.array_equal(host(YT).view(np.uint8), layout(host(Y0), ld).view(np.uint8)), f"{tag}: Y copy"
                H = torch.empty_like(Y0)
                AT = torch.zeros((L.out, ld), dtype=td, device="cuda")
                A = csp.spmm_fwd_bm(h, X, XT=xt, bias=bias, act="gelu", H=H, YT=AT)
                assert np.array_equal(host(A).view(np.uint8), host(A0).view(np.uint8)), f"{tag}: GELU forward"
                assert np.array_equal(host(H).view(np.uint8), host(H0).view(np.uint8)), f"{tag}: pre-activation"
                assert np.array_equal(host(AT).view(np.uint8), layout(host(A0), ld).view(np.uint8)), f"{tag}: A copy"
            # backward: plain and through GELU'
            dX0, dW0 = csp.spmm_bwd(h, dY, X)
            dXa0, dWa0 = csp.spmm_bwd_act(h, dY, X, Hin, act="gelu")
            for dyt, xt in ((None, None), (dYT, None), (None, XT), (dYT, XT)):
                dXT = torch.zeros((L.in_, ld), dtype=td, device="cuda")
                dX, dW = csp.spmm_bwd_bm(h, dY, X, dYT=dyt, XT=xt, dXT=dXT)
                assert np.array_equal(host(dX).view(np.uint8), host(dX0).view(np.uint8)), f"{tag}: dX"
                assert np.array_equal(bits(host(dW)), bits(host(dW0))), f"{tag}: dW"
                assert np.array_equal(host(dXT).view(np.uint8), layout(host(dX0), ld).view(np.uint8)), f"{tag}: dX copy"
                dX, dW = csp.spmm_bwd_bm(h, dY, X, dYT=dyt, XT=xt, H_in=Hin, act="gelu")
                assert np.array_equal(host(dX).view(np.uint8), host(dXa0).view(np.uint8)), f"{tag}: dX * GELU'"
                assert np.array_equal(bits(host(dW)), bits(host(dWa0))), f"{tag}: dW (act)"
    finally:
        csp.sparse_layer_destroy(h)


def test_mlp_chain_with_copies_matches_plain_chain():
    """The two-layer step of the sparse MLP written with the copies handed along (X's copy made once,
    A's copy from the first forward, dH's copy from the second layer's backward) against the same step
    with plain calls: every output bitwise equal."""
    L1 = W.random_layer(3072, 768, 235930, seed=21)
    L2 = W.random_layer(768, 3072, 235930, seed=22)
    h1 = csp.sparse_layer_create(L1.out, L1.in_, dev(L1.rows), dev(L1.cols), dev(L1.vals))
    h2 = csp.sparse_layer_create(L2.out, L2.in_, dev(L2.rows), dev(L2.cols), dev(L2.vals))
    try:
        B = 32
        X = dev(W.random_dense((B, 768), 23))
        dY = dev(W.random_dense((B, 768), 24))
        # plain
        H0 = torch.empty((B, 3072), device="cuda")
        A0 = csp.spmm_fwd_act(h1, X, act="gelu", H=H0)
        Y0 = csp.spmm_fwd(h2, A0)
        dH0, dW20 = csp.spmm_bwd_act(h2, dY, A0, H0, act="gelu")
        dX0, dW10 = csp.spmm_bwd(h1, dH0, X)
        # with copies
        XT = csp.spmm_batch_minor(X)
        H = torch.empty_like(H0)
        AT = torch.zeros((3072, 32), device="cuda")
        A = csp.spmm_fwd_bm(h1, X, XT=XT, act="gelu", H=H, YT=AT)
        Y = csp.spmm_fwd_bm(h2, A, XT=AT)
        dHT = torch.zeros((3072, 32), device="cuda")
        dH, dW2 = csp.spmm_bwd_bm(h2, dY, A, XT=AT, H_in=H, act="gelu", dXT=dHT)
        dX, dW1 = csp.spmm_bwd_bm(h1, dH, X, dYT=dHT, XT=XT)
        for name, a, b in (("A", A, A0), ("Y", Y, Y0), ("dH", dH, dH0), ("dW2", dW2, dW20), ("dX", dX, dX0),
                           ("dW1", dW1, dW10)):
            assert torch.equal(a, b), name
    finally:
        csp.sparse_layer_destroy(h1)
        csp.sparse_layer_destroy(h2)


def test_bm_refusals():
    L = W.random_layer(300, 260, 9000, seed=31)
    h = csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals))
    try:
        for B in (1, 65):
            X = dev(W.random_dense((B, L.in_), 32))
            with pytest.raises(csp.CspError, match="2 <= B"):
                csp.spmm_fwd_bm(h, X)
            with pytest.raises(csp.CspError, match="2 <= B"):
                csp.spmm_bwd_bm(h, dev(W.random_dense((B, L.out), 33)), X)
            with pytest.raises(csp.CspError):
                csp.spmm_batch_minor(X)
    finally:
        csp.sparse_layer_destroy(h)
