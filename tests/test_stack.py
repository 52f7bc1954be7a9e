"""Multi-layer single-stream inference: four 16384 x 16384 bf16 layers at 99% (Zipf rows), GELU
between them, one token batch per HIP-graph replay.  Each layer's output is compared with the
oracle on the GPU's own input to that layer (a per-layer error never compounds into a failure),
and every graph replay must equal the eager chain bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from coo_spmm_fwd_amd import binding as csp
from coo_spmm_fwd_amd import workloads as W
from tests.gpu_util import BF16_REL, assert_within, dev, host

pytestmark = pytest.mark.gpu


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
                csp.spmm_fwd(h, ins[li], outs[li])
                if li + 1 < len(hs):
                    outs[li].copy_(torch.nn.functional.gelu(outs[li]))

        chain()
        torch.cuda.synchronize()
        eager = [host(o.clone()) for o in outs]
        # per layer: the pre-activation output against the oracle on the GPU's own input
        for li, (h, L) in enumerate(zip(hs, layers)):
            Y = host(csp.spmm_fwd(h, ins[li]))
            ref, S = orc.spmm_fwd(L.out, L.in_, L.rows, L.cols, L.vals, host(ins[li]))
            assert_within(Y, ref, S, BF16_REL, f"stack layer {li + 1} B={B}")
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
