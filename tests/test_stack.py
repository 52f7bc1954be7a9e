"""Multi-layer single-stream inference: four 16384 x 16384 bf16 layers at 99% (Zipf rows), GELU
between them fused into each producing layer's forward epilogue (spmm_fwd_act), one token batch
per HIP-graph replay -- the chain the inference bench times.  Each layer's output is compared with
the oracle on the GPU's own input to that layer (GELU through the oracle's fp64 erf; a per-layer
error never compounds into a failure), and every graph replay must equal the eager chain bit for
bit.  Tolerance of a fused bf16 GELU output: 1.2e-2 * S (derivation in tests/test_epilogue.py)."""
import numpy as np
import pytest
import torch

import oracle
from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import BF16_REL, assert_within, dev, host

pytestmark = pytest.mark.gpu
ACT_REL_BF16 = 1.2e-2


@pytest.mark.parametrize("B", [1, 4])
def test_stack_graph_matches_oracle_per_layer(B):
    orc = oracle.default()
    w, layers, acts = W.build("stack16384x4_zipf_s99_bf16")
    hs = [csp.sparse_layer_create(L.out, L.in_, dev(L.rows), dev(L.cols), dev(L.vals)) for L in layers]
    try:
        X = dev(acts[B]["X"])
        outs = [torch.empty((B, L.out), dtype=torch.bfloat16, device="cuda") for L in layers]
        ins = [X] + outs[:-1]

        def chain():
            for li, h in enumerate(hs):
                last = li + 1 == len(hs)
                csp.spmm_fwd_act(h, ins[li], act="none" if last else "gelu", Y=outs[li])

        chain()
        torch.cuda.synchronize()
        eager = [host(o.clone()) for o in outs]
        # per layer: the fused output against the oracle on the GPU's own input to that layer
        for li, L in enumerate(layers):
            ref, S = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, host(ins[li]))
            if li + 1 < len(layers):
                assert_within(eager[li], orc.gelu(ref), S, ACT_REL_BF16, f"stack layer {li + 1} GELU B={B}")
            else:
                assert_within(eager[li], ref, S, BF16_REL, f"stack layer {li + 1} B={B}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            chain()
        for rep in range(3):
            for o in outs:
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for li, o in enumerate(outs):
                assert np.array_equal(host(o), eager[li]), (rep, li)
        del g
    finally:
        torch.cuda.synchronize()
        for h in hs:
            csp.sparse_layer_destroy(h)
