"""ctypes binding of libcoospmm.so -- same names as the C ABI in include/coospmm.h.

Argument marshalling only: every step runs in the HIP library.  Tensors are
torch tensors on the GPU (torch provides device memory and streams); pointers
and the current HIP stream are passed straight through.  When the library is
missing the calls raise; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcoospmm.so")

CSP_F32, CSP_BF16 = 0, 1
STATUS = {0: "CSP_OK", -1: "CSP_ERR_INVALID_ARG", -2: "CSP_ERR_INDEX_RANGE", -3: "CSP_ERR_DUPLICATE",
          -4: "CSP_ERR_NO_MEMORY", -5: "CSP_ERR_HIP", -6: "CSP_ERR_DTYPE"}
CSP_ACT_NONE, CSP_ACT_GELU = 0, 1
EXPORTED = ["sparse_layer_create", "sparse_layer_destroy", "spmm_fwd", "spmm_fwd_static", "spmm_bwd_input", "spmm_bwd_values", "spmm_bwd",
            "spmm_fwd_act", "spmm_bwd_input_act", "spmm_bwd_act", "restructure_grad",
            "restructure", "sparse_layer_nnz", "sparse_layer_shape", "sparse_layer_export",
            "sparse_layer_export_index", "sparse_layer_values", "sparse_layer_set_values", "sparse_layer_time_next",
            "sparse_layer_last_error", "restructure_async", "sparse_layer_sync", "spmm_batch_minor", "spmm_fwd_bm",
            "spmm_bwd_bm"]


class CspError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"coospmm HIP library not found at {path}; build it with "
                           "`python -m coo_spmm_fwd_amd.build` (there is no CPU fallback)")
    L = ctypes.CDLL(path)
    L.sparse_layer_create.restype = c_int
    L.sparse_layer_create.argtypes = [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                      POINTER(c_void_p)]
    L.sparse_layer_destroy.restype = None
    L.sparse_layer_destroy.argtypes = [c_void_p]
    L.spmm_fwd.restype = c_int
    L.spmm_fwd.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_void_p]
    L.spmm_fwd_static.restype = c_int
    L.spmm_fwd_static.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_void_p]
    L.spmm_bwd_input.restype = c_int
    L.spmm_bwd_input.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_void_p]
    L.spmm_bwd_values.restype = c_int
    L.spmm_bwd_values.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p]
    L.spmm_bwd.restype = c_int
    L.spmm_bwd.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p]
    L.spmm_fwd_act.restype = c_int
    L.spmm_fwd_act.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_void_p, c_void_p]
    L.spmm_bwd_input_act.restype = c_int
    L.spmm_bwd_input_act.argtypes = [c_void_p, c_void_p, c_int64, c_int, c_void_p, c_void_p, c_void_p]
    L.spmm_bwd_act.restype = c_int
    L.spmm_bwd_act.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_int, c_void_p, c_void_p, c_void_p, c_void_p]
    L.restructure.restype = c_int
    L.restructure.argtypes = [c_void_p, c_int64, c_uint64, c_uint64, c_float, c_void_p]
    L.spmm_batch_minor.restype = c_int
    L.spmm_batch_minor.argtypes = [c_void_p, c_int64, c_int64, c_int32, c_void_p, c_void_p]
    L.spmm_fwd_bm.restype = c_int
    L.spmm_fwd_bm.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_int, c_void_p, c_void_p, c_void_p,
                              c_void_p]
    L.spmm_bwd_bm.restype = c_int
    L.spmm_bwd_bm.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p]
    L.restructure_async.restype = c_int
    L.restructure_async.argtypes = [c_void_p, c_int64, c_uint64, c_void_p, c_float, c_void_p]
    L.sparse_layer_sync.restype = c_int
    L.sparse_layer_sync.argtypes = [c_void_p, c_void_p]
    L.restructure_grad.restype = c_int
    L.restructure_grad.argtypes = [c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_float, c_void_p]
    L.sparse_layer_nnz.restype = c_int64
    L.sparse_layer_nnz.argtypes = [c_void_p]
    L.sparse_layer_shape.restype = c_int
    L.sparse_layer_shape.argtypes = [c_void_p, POINTER(c_int64), POINTER(c_int64), POINTER(c_int32)]
    L.sparse_layer_export.restype = c_int
    L.sparse_layer_export.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    L.sparse_layer_export_index.restype = c_int
    L.sparse_layer_export_index.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    L.sparse_layer_values.restype = c_void_p
    L.sparse_layer_values.argtypes = [c_void_p]
    L.sparse_layer_set_values.restype = c_int
    L.sparse_layer_set_values.argtypes = [c_void_p, c_void_p, c_void_p]
    L.sparse_layer_time_next.restype = c_int
    L.sparse_layer_time_next.argtypes = [c_void_p, c_void_p, c_void_p]
    L.sparse_layer_last_error.restype = c_char_p
    L.sparse_layer_last_error.argtypes = []
    _lib = L
    return L


def sparse_layer_last_error() -> str:
    return load().sparse_layer_last_error().decode()


def _check(st: int):
    if st != 0:
        raise CspError(st, sparse_layer_last_error())


# ------------------------------------------------------------ marshalling
def _torch():
    import torch
    return torch


def _stream(stream):
    if stream is None:
        return c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return c_void_p(stream)
    return c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return CSP_F32
    if t.dtype == torch.bfloat16:
        return CSP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return c_void_p(t.data_ptr())


def _torch_dtype(code: int):
    torch = _torch()
    return torch.bfloat16 if code == CSP_BF16 else torch.float32


# ------------------------------------------------------------ the C ABI
def sparse_layer_create(out_features: int, in_features: int, rows, cols, vals, stream=None) -> int:
    """Build a layer from device int32 rows/cols and fp32/bf16 values; returns the handle (int)."""
    L = load()
    torch = _torch()
    nnz = int(rows.numel())
    dt = _dtype_code(vals)
    rp = _dev(rows, "rows", torch.int32, (nnz,))
    cp = _dev(cols, "cols", torch.int32, (nnz,))
    vp = _dev(vals, "vals", None, (nnz,))
    h = c_void_p()
    _check(L.sparse_layer_create(out_features, in_features, nnz, rp, cp, vp, dt, _stream(stream), ctypes.byref(h)))
    return h.value


def sparse_layer_destroy(layer: int):
    load().sparse_layer_destroy(c_void_p(layer))


def sparse_layer_nnz(layer: int) -> int:
    return int(load().sparse_layer_nnz(c_void_p(layer)))


def sparse_layer_shape(layer: int):
    o, i, d = c_int64(), c_int64(), c_int32()
    _check(load().sparse_layer_shape(c_void_p(layer), ctypes.byref(o), ctypes.byref(i), ctypes.byref(d)))
    return o.value, i.value, d.value


def spmm_fwd(layer: int, X, Y=None, stream=None):
    """Y[B, out] = X[B, in] W^T."""
    out, in_, dt = sparse_layer_shape(layer)
    B = int(X.shape[0])
    xp = _dev(X, "X", _torch_dtype(dt), (B, in_))
    if Y is None:
        Y = _torch().empty((B, out), dtype=X.dtype, device=X.device)
    yp = _dev(Y, "Y", _torch_dtype(dt), (B, out))
    _check(load().spmm_fwd(c_void_p(layer), xp, B, yp, _stream(stream)))
    return Y


def spmm_fwd_static(layer: int, X, Y=None, stream=None):
    """Y[B, out] = X[B, in] W^T with the call's workspace in the library's static per-GPU array
    (no allocation by the library; calls overlapping on one GPU race)."""
    out, in_, dt = sparse_layer_shape(layer)
    B = int(X.shape[0])
    xp = _dev(X, "X", _torch_dtype(dt), (B, in_))
    if Y is None:
        Y = _torch().empty((B, out), dtype=X.dtype, device=X.device)
    yp = _dev(Y, "Y", _torch_dtype(dt), (B, out))
    _check(load().spmm_fwd_static(c_void_p(layer), xp, B, yp, _stream(stream)))
    return Y


def spmm_bwd_input(layer: int, dY, dX=None, stream=None):
    """dX[B, in] = dY[B, out] W."""
    out, in_, dt = sparse_layer_shape(layer)
    B = int(dY.shape[0])
    gp = _dev(dY, "dY", _torch_dtype(dt), (B, out))
    if dX is None:
        dX = _torch().empty((B, in_), dtype=dY.dtype, device=dY.device)
    xp = _dev(dX, "dX", _torch_dtype(dt), (B, in_))
    _check(load().spmm_bwd_input(c_void_p(layer), gp, B, xp, _stream(stream)))
    return dX


def spmm_bwd_values(layer: int, dY, X, dW=None, stream=None):
    """dW[k] = sum_b dY[b, row_k] X[b, col_k], canonical order, fp32."""
    out, in_, dt = sparse_layer_shape(layer)
    nnz = sparse_layer_nnz(layer)
    B = int(X.shape[0])
    gp = _dev(dY, "dY", _torch_dtype(dt), (B, out))
    xp = _dev(X, "X", _torch_dtype(dt), (B, in_))
    if dW is None:
        dW = _torch().empty((nnz,), dtype=_torch().float32, device=X.device)
    wp = _dev(dW, "dW", _torch().float32, (nnz,))
    _check(load().spmm_bwd_values(c_void_p(layer), gp, xp, B, wp, _stream(stream)))
    return dW


def spmm_bwd(layer: int, dY, X, dX=None, dW=None, stream=None):
    """Both gradients in one pass: dX = dY W and dW[k] = sum_b dY[b, row_k] X[b, col_k]."""
    out, in_, dt = sparse_layer_shape(layer)
    nnz = sparse_layer_nnz(layer)
    B = int(X.shape[0])
    gp = _dev(dY, "dY", _torch_dtype(dt), (B, out))
    xp = _dev(X, "X", _torch_dtype(dt), (B, in_))
    if dX is None:
        dX = _torch().empty((B, in_), dtype=X.dtype, device=X.device)
    if dW is None:
        dW = _torch().empty((nnz,), dtype=_torch().float32, device=X.device)
    dxp = _dev(dX, "dX", _torch_dtype(dt), (B, in_))
    wp = _dev(dW, "dW", _torch().float32, (nnz,))
    _check(load().spmm_bwd(c_void_p(layer), gp, xp, B, dxp, wp, _stream(stream)))
    return dX, dW


def _act_code(act) -> int:
    codes = {None: CSP_ACT_NONE, "none": CSP_ACT_NONE, "gelu": CSP_ACT_GELU, CSP_ACT_NONE: CSP_ACT_NONE,
             CSP_ACT_GELU: CSP_ACT_GELU}
    if act not in codes:
        raise ValueError(f"unknown activation {act!r}")
    return codes[act]


def spmm_fwd_act(layer: int, X, bias=None, act="gelu", Y=None, H=None, stream=None):
    """Y = act(X W^T + bias); H (optional output) receives the pre-activation X W^T + bias."""
    out, in_, dt = sparse_layer_shape(layer)
    B = int(X.shape[0])
    td = _torch_dtype(dt)
    xp = _dev(X, "X", td, (B, in_))
    bp = None if bias is None else _dev(bias, "bias", td, (out,))
    if Y is None:
        Y = _torch().empty((B, out), dtype=X.dtype, device=X.device)
    yp = _dev(Y, "Y", td, (B, out))
    hp = None if H is None else _dev(H, "H", td, (B, out))
    _check(load().spmm_fwd_act(c_void_p(layer), xp, B, bp, _act_code(act), yp, hp, _stream(stream)))
    return Y


def spmm_bwd_input_act(layer: int, dY, H_in, act="gelu", dX=None, stream=None):
    """dX = (dY W) * act'(H_in): the input gradient through the activation that produced the layer's input."""
    out, in_, dt = sparse_layer_shape(layer)
    B = int(dY.shape[0])
    td = _torch_dtype(dt)
    gp = _dev(dY, "dY", td, (B, out))
    hp = None if H_in is None else _dev(H_in, "H_in", td, (B, in_))
    if dX is None:
        dX = _torch().empty((B, in_), dtype=dY.dtype, device=dY.device)
    xp = _dev(dX, "dX", td, (B, in_))
    _check(load().spmm_bwd_input_act(c_void_p(layer), gp, B, _act_code(act), hp, xp, _stream(stream)))
    return dX


def spmm_bwd_act(layer: int, dY, X, H_in, act="gelu", dX=None, dW=None, stream=None):
    """spmm_bwd with dX = (dY W) * act'(H_in); dW as in spmm_bwd_values."""
    out, in_, dt = sparse_layer_shape(layer)
    nnz = sparse_layer_nnz(layer)
    B = int(X.shape[0])
    td = _torch_dtype(dt)
    gp = _dev(dY, "dY", td, (B, out))
    xp = _dev(X, "X", td, (B, in_))
    hp = None if H_in is None else _dev(H_in, "H_in", td, (B, in_))
    if dX is None:
        dX = _torch().empty((B, in_), dtype=X.dtype, device=X.device)
    if dW is None:
        dW = _torch().empty((nnz,), dtype=_torch().float32, device=X.device)
    dxp = _dev(dX, "dX", td, (B, in_))
    wp = _dev(dW, "dW", _torch().float32, (nnz,))
    _check(load().spmm_bwd_act(c_void_p(layer), gp, xp, B, _act_code(act), hp, dxp, wp, _stream(stream)))
    return dX, dW


def batch_minor_ld(B: int) -> int:
    """Row length of a batch-minor copy at batch B (the power of two >= B)."""
    ld = 1
    while ld < B:
        ld *= 2
    return ld


def spmm_batch_minor(src, dst=None, stream=None):
    """dst[c, b] = src[b, c] for b < B, zero pad slots up to batch_minor_ld(B); src [B, n], 2 <= B <= 64."""
    torch = _torch()
    B, n = int(src.shape[0]), int(src.shape[1])
    ld = batch_minor_ld(B)
    sp = _dev(src, "src", None, (B, n))
    if dst is None:
        dst = torch.empty((n, ld), dtype=src.dtype, device=src.device)
    dp = _dev(dst, "dst", src.dtype, (n, ld))
    _check(load().spmm_batch_minor(sp, n, B, _dtype_code(src), dp, _stream(stream)))
    return dst


def spmm_fwd_bm(layer: int, X, XT=None, bias=None, act="none", Y=None, H=None, YT=None, stream=None):
    """spmm_fwd_act with X's batch-minor copy XT (optional input) and Y's copy YT (optional output,
    [out, ld], pad slots kept zero by the caller).  2 <= B <= 64."""
    out, in_, dt = sparse_layer_shape(layer)
    B = int(X.shape[0])
    ld = batch_minor_ld(B)
    td = _torch_dtype(dt)
    xp = _dev(X, "X", td, (B, in_))
    xtp = None if XT is None else _dev(XT, "XT", td, (in_, ld))
    bp = None if bias is None else _dev(bias, "bias", td, (out,))
    if Y is None:
        Y = _torch().empty((B, out), dtype=X.dtype, device=X.device)
    yp = _dev(Y, "Y", td, (B, out))
    hp = None if H is None else _dev(H, "H", td, (B, out))
    ytp = None if YT is None else _dev(YT, "YT", td, (out, ld))
    _check(load().spmm_fwd_bm(c_void_p(layer), xp, xtp, B, bp, _act_code(act), yp, hp, ytp, _stream(stream)))
    return Y


def spmm_bwd_bm(layer: int, dY, X, dYT=None, XT=None, H_in=None, act="none", dX=None, dXT=None, dW=None,
                stream=None):
    """spmm_bwd_act with the batch-minor copies dYT and XT (optional inputs) and dX's copy dXT
    (optional output, [in, ld]).  2 <= B <= 64."""
    torch = _torch()
    out, in_, dt = sparse_layer_shape(layer)
    nnz = sparse_layer_nnz(layer)
    B = int(X.shape[0])
    ld = batch_minor_ld(B)
    td = _torch_dtype(dt)
    gp = _dev(dY, "dY", td, (B, out))
    xp = _dev(X, "X", td, (B, in_))
    gtp = None if dYT is None else _dev(dYT, "dYT", td, (out, ld))
    xtp = None if XT is None else _dev(XT, "XT", td, (in_, ld))
    hp = None if H_in is None else _dev(H_in, "H_in", td, (B, in_))
    if dX is None:
        dX = torch.empty((B, in_), dtype=X.dtype, device=X.device)
    if dW is None:
        dW = torch.empty((nnz,), dtype=torch.float32, device=X.device)
    dxp = _dev(dX, "dX", td, (B, in_))
    dxtp = None if dXT is None else _dev(dXT, "dXT", td, (in_, ld))
    wp = _dev(dW, "dW", torch.float32, (nnz,))
    _check(load().spmm_bwd_bm(c_void_p(layer), gp, gtp, xp, xtp, B, _act_code(act), hp, dxp, dxtp, wp,
                              _stream(stream)))
    return dX, dW


def restructure(layer: int, n_prune: int, seed: int, step: int, regrow_value: float = 0.0, stream=None):
    """Prune n_prune smallest-|v| entries and regrow as many at empty positions (synchronizes)."""
    _check(load().restructure(c_void_p(layer), int(n_prune), int(seed) & (2**64 - 1), int(step) & (2**64 - 1),
                              float(regrow_value), _stream(stream)))


def restructure_async(layer: int, n_prune: int, seed: int, step_dev, regrow_value: float = 0.0, stream=None):
    """restructure with the step read from (and advanced in) step_dev, a one-element int64 GPU
    tensor; no host synchronization (capturable).  See the C header for what stays pending."""
    torch = _torch()
    sp = _dev(step_dev, "step_dev", torch.int64, (1,))
    _check(load().restructure_async(c_void_p(layer), int(n_prune), int(seed) & (2**64 - 1), sp,
                                    float(regrow_value), _stream(stream)))


def sparse_layer_sync(layer: int, stream=None):
    """Finish the bookkeeping of earlier restructure_async calls: build the task lists they left
    pending, then read back their counts and the short-regrow flag (synchronizes)."""
    _check(load().sparse_layer_sync(c_void_p(layer), _stream(stream)))


def restructure_grad(layer: int, n_prune: int, dY, X, regrow_value: float = 0.0, stream=None):
    """Prune n_prune smallest-|v| entries and regrow as many at the empty positions with the largest
    |(dY^T X)[r, c]| (fp32 multiply-add chain in batch order; synchronizes)."""
    out, in_, dt = sparse_layer_shape(layer)
    B = int(X.shape[0])
    td = _torch_dtype(dt)
    gp = _dev(dY, "dY", td, (B, out))
    xp = _dev(X, "X", td, (B, in_))
    _check(load().restructure_grad(c_void_p(layer), int(n_prune), gp, xp, B, float(regrow_value), _stream(stream)))


def sparse_layer_export(layer: int, stream=None):
    """Canonical (rows, cols, vals) as new device tensors."""
    torch = _torch()
    out, in_, dt = sparse_layer_shape(layer)
    nnz = sparse_layer_nnz(layer)
    dev = torch.device("cuda", torch.cuda.current_device())
    rows = torch.empty(nnz, dtype=torch.int32, device=dev)
    cols = torch.empty(nnz, dtype=torch.int32, device=dev)
    vals = torch.empty(nnz, dtype=_torch_dtype(dt), device=dev)
    _check(load().sparse_layer_export(c_void_p(layer), c_void_p(rows.data_ptr()), c_void_p(cols.data_ptr()),
                                      c_void_p(vals.data_ptr()), _stream(stream)))
    return rows, cols, vals


def sparse_layer_export_index(layer: int, stream=None):
    """(row_ptr, perm_c, rows_by_col, col_ptr) as new device tensors."""
    torch = _torch()
    out, in_, _ = sparse_layer_shape(layer)
    nnz = sparse_layer_nnz(layer)
    dev = torch.device("cuda", torch.cuda.current_device())
    row_ptr = torch.empty(out + 1, dtype=torch.int32, device=dev)
    perm_c = torch.empty(nnz, dtype=torch.int32, device=dev)
    rows_by_col = torch.empty(nnz, dtype=torch.int32, device=dev)
    col_ptr = torch.empty(in_ + 1, dtype=torch.int32, device=dev)
    _check(load().sparse_layer_export_index(c_void_p(layer), c_void_p(row_ptr.data_ptr()),
                                            c_void_p(perm_c.data_ptr()), c_void_p(rows_by_col.data_ptr()),
                                            c_void_p(col_ptr.data_ptr()), _stream(stream)))
    return row_ptr, perm_c, rows_by_col, col_ptr


def sparse_layer_values(layer: int) -> int:
    """Device address of the canonical values (for in-place optimizer updates)."""
    return int(load().sparse_layer_values(c_void_p(layer)) or 0)


def sparse_layer_set_values(layer: int, vals, stream=None):
    """Overwrite the canonical values with the device tensor vals[nnz] (layer dtype) and refresh
    the column-ordered copy; vals=None only refreshes the copy after in-place updates."""
    _, _, dt = sparse_layer_shape(layer)
    nnz = sparse_layer_nnz(layer)
    vp = None if vals is None else _dev(vals, "vals", _torch_dtype(dt), (nnz,))
    _check(load().sparse_layer_set_values(c_void_p(layer), vp, _stream(stream)))


class LayerOwner:
    """Owns a layer handle and destroys it when the last reference goes away.  Zero-copy views of
    the layer's device arrays hold a reference to it, so the layer outlives every view (an optimizer
    may keep a parameter after its module is gone)."""

    def __init__(self, handle: int, destroy=None):
        self.handle = handle
        self._destroy = destroy if destroy is not None else sparse_layer_destroy

    def __del__(self):
        h, self.handle = self.handle, None
        if h:
            self._destroy(h)


class _DeviceArray:
    """Minimal __cuda_array_interface__ holder for a library-owned device array; `owner` (a
    LayerOwner, or None) is kept alive as long as this object, and torch keeps this object alive as
    long as a tensor made from it."""

    def __init__(self, ptr: int, n: int, typestr: str, owner=None):
        self.owner = owner
        self.__cuda_array_interface__ = {"shape": (n,), "typestr": typestr, "data": (ptr, False),
                                         "strides": None, "version": 2}


def sparse_layer_values_tensor(layer: int, owner=None):
    """Zero-copy torch view of the layer's canonical values, valid until the next
    restructure (which may move them).  With `owner` (the layer's LayerOwner) the
    view keeps the layer alive; without it the caller must keep the layer until the
    view is gone.  After writing into it, call sparse_layer_set_values(layer, None)."""
    torch = _torch()
    _, _, dt = sparse_layer_shape(layer)
    nnz = sparse_layer_nnz(layer)
    ptr = sparse_layer_values(layer)
    if nnz == 0:
        return torch.empty(0, dtype=_torch_dtype(dt), device="cuda")
    t = torch.as_tensor(_DeviceArray(ptr, nnz, "<u2" if dt == CSP_BF16 else "<f4", owner), device="cuda")
    return t.view(torch.bfloat16) if dt == CSP_BF16 else t


def sparse_layer_time_next(layer: int, ev_before, ev_after):
    """Bracket the main kernel of the next product call with two torch.cuda.Event objects."""
    _check(load().sparse_layer_time_next(c_void_p(layer), c_void_p(ev_before.cuda_event),
                                         c_void_p(ev_after.cuda_event)))
