"""SparseLinear: a torch module over one truly sparse COO layer.

"Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks on GPU"
(Abstract): the layer stores only its non-zero connections, trains them with
gradients computed in the sparse paradigm, and is restructured during dynamic
sparse training.  This module is the torch-facing side of that: forward calls
spmm_fwd, its autograd backward calls spmm_bwd (input gradient and the
gradient of the stored values), and restructure() calls restructure.

The module's parameter `values` is a zero-copy view of the layer's own value
buffer (canonical (row, col) order), so an optimizer updates the layer in
place; the next forward refreshes the layer's column-ordered copy when the
parameter's version counter shows a write.  A restructure may move the
buffer: the parameter is re-pointed at the new one, and any optimizer state
indexed by entry is the caller's to reset (the entries changed).

Argument marshalling only: every step runs in the HIP library.
"""
from __future__ import annotations

import torch

from . import binding as csp


class _SparseLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, X, values, module):  # values: the parameter, for autograd bookkeeping only
        ctx.module = module
        ctx.save_for_backward(X)
        return csp.spmm_fwd(module.handle, X)

    @staticmethod
    def backward(ctx, dY):
        (X,) = ctx.saved_tensors
        m = ctx.module
        need_x, need_v = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        dY = dY.contiguous()
        if need_x and need_v:
            dX, dW = csp.spmm_bwd(m.handle, dY, X)
        elif need_x:
            dX, dW = csp.spmm_bwd_input(m.handle, dY), None
        elif need_v:
            dX, dW = None, csp.spmm_bwd_values(m.handle, dY, X)
        else:
            dX = dW = None
        return dX, dW, None


class SparseLinear(torch.nn.Module):
    """Y[B, out] = X[B, in] @ W^T with W stored as COO triples (no dense weight, no mask).

    rows, cols: int32 device tensors of the stored positions (any order, no
    duplicates); vals: float32 or bfloat16 device tensor of their values.  No
    bias (a dense add outside the layer).  On a bf16 layer the input gradient
    flows through autograd but the values take no gradient (the library's
    value gradient is fp32: call spmm_bwd_values for it).
    """

    def __init__(self, rows, cols, vals, out_features: int, in_features: int):
        super().__init__()
        self.out_features, self.in_features = int(out_features), int(in_features)
        # the owner destroys the layer once neither the module nor any view of its values is left
        self._owner = csp.LayerOwner(csp.sparse_layer_create(self.out_features, self.in_features, rows, cols, vals))
        self.values = torch.nn.Parameter(csp.sparse_layer_values_tensor(self.handle, self._owner),
                                         requires_grad=vals.dtype == torch.float32)
        self._seen_version = self.values._version

    @property
    def handle(self) -> int:
        return self._owner.handle

    @property
    def nnz(self) -> int:
        return csp.sparse_layer_nnz(self.handle)

    def _sync_values(self):
        """Refresh the layer's column-ordered copy after in-place writes to `values`."""
        if self.values._version != self._seen_version:
            csp.sparse_layer_set_values(self.handle, None)
            self._seen_version = self.values._version

    def forward(self, X):
        if X.dim() != 2 or X.shape[1] != self.in_features:
            raise ValueError(f"X must be [B, {self.in_features}], got {tuple(X.shape)}")
        self._sync_values()
        return _SparseLinearFn.apply(X.contiguous(), self.values, self)

    @torch.no_grad()
    def restructure(self, n_prune: int, seed: int, step: int, regrow_value: float = 0.0):
        """One prune-and-regrow step (the n_prune smallest |v| go, as many empty positions are drawn)."""
        self._sync_values()
        csp.restructure(self.handle, int(n_prune), int(seed), int(step), float(regrow_value))
        self.values.data = csp.sparse_layer_values_tensor(self.handle, self._owner)
        self._seen_version = self.values._version

    @torch.no_grad()
    def restructure_by_gradient(self, n_prune: int, dY, X, regrow_value: float = 0.0):
        """Prune the n_prune smallest |v|; regrow the empty positions where |dY^T X| is largest."""
        self._sync_values()
        csp.restructure_grad(self.handle, int(n_prune), dY.contiguous(), X.contiguous(), float(regrow_value))
        self.values.data = csp.sparse_layer_values_tensor(self.handle, self._owner)
        self._seen_version = self.values._version

    def coo(self):
        """(rows, cols, values) in canonical (row, col) order, as new device tensors."""
        self._sync_values()
        return csp.sparse_layer_export(self.handle)

    def to_dense(self):
        """Dense [out, in] copy of W (for checks on small layers)."""
        r, c, v = self.coo()
        W = torch.zeros(self.out_features, self.in_features, dtype=v.dtype, device=v.device)
        W[r.long(), c.long()] = v
        return W

    def extra_repr(self) -> str:
        return f"in_features={self.in_features}, out_features={self.out_features}, nnz={self.nnz}"
