"""CPU oracle for the truly sparse COO layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``coo_spmm_fwd_amd``) never
imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C loops, fp64 accumulation), built
with the host ``gcc`` into ``liboracle.so``; this module is argument marshalling
over ctypes.  Method source: "Beyond Masked Sparsity: SNACK Enables Truly Sparse
Neural Networks on GPU" (arXiv:2610.04093), Abstract.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from ctypes import POINTER, c_double, c_int, c_int64, c_uint32, c_uint64, c_void_p

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
F32, BF16 = 0, 1
OK, ERR_ARG, ERR_RANGE, ERR_DUP, ERR_NOMEM = 0, -1, -2, -3, -4


def lib_path(mutant: int = 0) -> str:
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(HERE, name)


def build(mutant: int = 0, out_dir: str | None = None) -> str:
    """Compile oracle.c with gcc (no fast-math: IEEE fp64 throughout)."""
    path = lib_path(mutant) if out_dir is None else os.path.join(out_dir, os.path.basename(lib_path(mutant)))
    tmp = path + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           f"-DORACLE_MUTANT={int(mutant)}", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, path)
    return path


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(c_void_p)


class Oracle:
    """ctypes view of one build of oracle.c (the default or a planted mutant)."""

    def __init__(self, path: str | None = None, mutant: int = 0):
        if path is None:
            path = lib_path(mutant)
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
                build(mutant)
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.oracle_canonicalize.restype = c_int
        L.oracle_canonicalize.argtypes = [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_int,
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p]
        for name in ("oracle_spmm_fwd", "oracle_spmm_bwd_input"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int64,
                          c_void_p, c_void_p]
        L.oracle_spmm_bwd_values.restype = None
        L.oracle_spmm_bwd_values.argtypes = [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_int, c_void_p,
                                             c_void_p, c_int64, c_void_p, c_void_p]
        L.oracle_philox4x64_10.restype = None
        L.oracle_philox4x64_10.argtypes = [c_void_p, c_void_p, c_void_p]
        L.oracle_regrow_draw.restype = c_uint64
        L.oracle_regrow_draw.argtypes = [c_uint64, c_uint64, c_uint64]
        L.oracle_regrow_position.restype = c_int64
        L.oracle_regrow_position.argtypes = [c_uint64, c_int64, c_int64]
        L.oracle_restructure.restype = c_int
        L.oracle_restructure.argtypes = [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_int,
                                         c_int64, c_uint64, c_uint64, c_uint32, c_void_p, c_void_p, c_void_p,
                                         c_void_p]
        L.oracle_gelu.restype = None
        L.oracle_restructure_grad.restype = c_int
        L.oracle_restructure_grad.argtypes = [c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_int,
                                              c_int64, c_void_p, c_void_p, c_int64, c_uint32, c_void_p, c_void_p,
                                              c_void_p]
        L.oracle_gelu.argtypes = [c_int64, c_void_p, c_void_p]
        L.oracle_gelu_grad.restype = None
        L.oracle_gelu_grad.argtypes = [c_int64, c_void_p, c_void_p]
        L.oracle_decode.restype = c_double
        L.oracle_decode.argtypes = [c_void_p, c_int, c_int64]
        L.oracle_mutant_id.restype = c_int
        self.mutant = L.oracle_mutant_id()

    # -- helpers -----------------------------------------------------
    @staticmethod
    def _words(vals: np.ndarray):
        """Raw value words and dtype code: float32 -> fp32, uint16 -> bf16 bit patterns."""
        if vals.dtype == np.float32:
            return np.ascontiguousarray(vals), F32
        if vals.dtype == np.uint16:
            return np.ascontiguousarray(vals), BF16
        raise TypeError(f"oracle values must be float32 or uint16 (bf16 bits), got {vals.dtype}")

    @staticmethod
    def _i32(a):
        return np.ascontiguousarray(a, dtype=np.int32)

    # -- canonical order ---------------------------------------------
    def canonicalize(self, out: int, in_: int, rows, cols, vals):
        rows, cols = self._i32(rows), self._i32(cols)
        vals, dt = self._words(vals)
        nnz = rows.shape[0]
        res = dict(
            src=np.empty(nnz, np.int64), rows=np.empty(nnz, np.int32), cols=np.empty(nnz, np.int32),
            vals=np.empty(nnz, vals.dtype), row_ptr=np.empty(out + 1, np.int32),
            perm_c=np.empty(nnz, np.int32), rows_by_col=np.empty(nnz, np.int32),
            col_ptr=np.empty(in_ + 1, np.int32))
        st = self.lib.oracle_canonicalize(out, in_, nnz, _ptr(rows), _ptr(cols), _ptr(vals), dt,
                                          _ptr(res["src"]), _ptr(res["rows"]), _ptr(res["cols"]),
                                          _ptr(res["vals"]), _ptr(res["row_ptr"]), _ptr(res["perm_c"]),
                                          _ptr(res["rows_by_col"]), _ptr(res["col_ptr"]))
        res["status"] = st
        return res

    # -- products (any triple order; outputs fp64 plus magnitude sums) --
    def spmm_fwd(self, out, in_, rows, cols, vals, X):
        rows, cols = self._i32(rows), self._i32(cols)
        vals, dt = self._words(vals)
        X, dtx = self._words(X)
        assert dtx == dt, "X and W must share the layer dtype"
        B = X.shape[0]
        assert X.shape == (B, in_)
        Y = np.empty((B, out), np.float64)
        S = np.empty((B, out), np.float64)
        self.lib.oracle_spmm_fwd(out, in_, rows.shape[0], _ptr(rows), _ptr(cols), _ptr(vals), dt, _ptr(X), B,
                                 _ptr(Y), _ptr(S))
        return Y, S

    def spmm_bwd_input(self, out, in_, rows, cols, vals, dY):
        rows, cols = self._i32(rows), self._i32(cols)
        vals, dt = self._words(vals)
        dY, dty = self._words(dY)
        assert dty == dt
        B = dY.shape[0]
        assert dY.shape == (B, out)
        dX = np.empty((B, in_), np.float64)
        S = np.empty((B, in_), np.float64)
        self.lib.oracle_spmm_bwd_input(out, in_, rows.shape[0], _ptr(rows), _ptr(cols), _ptr(vals), dt, _ptr(dY),
                                       B, _ptr(dX), _ptr(S))
        return dX, S

    def spmm_bwd_values(self, out, in_, rows, cols, dY, X):
        rows, cols = self._i32(rows), self._i32(cols)
        dY, dt = self._words(dY)
        X, dtx = self._words(X)
        assert dt == dtx
        B = X.shape[0]
        assert X.shape == (B, in_) and dY.shape == (B, out)
        nnz = rows.shape[0]
        dW = np.empty(nnz, np.float64)
        S = np.empty(nnz, np.float64)
        self.lib.oracle_spmm_bwd_values(out, in_, nnz, _ptr(rows), _ptr(cols), dt, _ptr(dY), _ptr(X), B,
                                        _ptr(dW), _ptr(S))
        return dW, S

    # -- random stream and restructure ---------------------------------
    def philox4x64_10(self, ctr, key):
        c = np.ascontiguousarray(ctr, dtype=np.uint64)
        k = np.ascontiguousarray(key, dtype=np.uint64)
        o = np.empty(4, np.uint64)
        self.lib.oracle_philox4x64_10(_ptr(c), _ptr(k), _ptr(o))
        return o

    def regrow_draw(self, seed: int, step: int, i: int) -> int:
        return int(self.lib.oracle_regrow_draw(seed, step, i))

    def regrow_position(self, u: int, out: int, in_: int) -> int:
        return int(self.lib.oracle_regrow_position(u, out, in_))

    def restructure(self, out, in_, rows_c, cols_c, vals_c, n_prune, seed, step, regrow_value=0.0):
        rows_c, cols_c = self._i32(rows_c), self._i32(cols_c)
        vals_c, dt = self._words(vals_c)
        nnz = rows_c.shape[0]
        if dt == F32:
            bits = int(np.array([regrow_value], np.float32).view(np.uint32)[0])
        else:
            bits = int(np.asarray(regrow_value, dtype=np.uint16))  # caller passes bf16 bits
        r = np.empty(nnz, np.int32)
        c = np.empty(nnz, np.int32)
        v = np.empty(nnz, vals_c.dtype)
        draws = np.zeros(1, np.int64)
        st = self.lib.oracle_restructure(out, in_, nnz, _ptr(rows_c), _ptr(cols_c), _ptr(vals_c), dt, n_prune,
                                         seed, step, bits, _ptr(r), _ptr(c), _ptr(v), _ptr(draws))
        if st != OK:
            raise ValueError(f"oracle_restructure failed with status {st}")
        return r, c, v, int(draws[0])

    def restructure_grad(self, out, in_, rows_c, cols_c, vals_c, n_prune, dY, X, regrow_value=0.0):
        """Prune as restructure; regrow the n_prune empty positions with the largest |(dY^T X)[r, c]|
        (fp32 fused-multiply-add chain in batch order; ties to the smaller position)."""
        rows_c, cols_c = self._i32(rows_c), self._i32(cols_c)
        vals_c, dt = self._words(vals_c)
        dY, dty = self._words(dY)
        X, dtx = self._words(X)
        assert dt == dty == dtx
        B = X.shape[0]
        assert X.shape == (B, in_) and dY.shape == (B, out)
        nnz = rows_c.shape[0]
        if dt == F32:
            bits = int(np.array([regrow_value], np.float32).view(np.uint32)[0])
        else:
            bits = int(np.asarray(regrow_value, dtype=np.uint16))  # caller passes bf16 bits
        r = np.empty(nnz, np.int32)
        c = np.empty(nnz, np.int32)
        v = np.empty(nnz, vals_c.dtype)
        st = self.lib.oracle_restructure_grad(out, in_, nnz, _ptr(rows_c), _ptr(cols_c), _ptr(vals_c), dt, n_prune,
                                              _ptr(dY), _ptr(X), B, bits, _ptr(r), _ptr(c), _ptr(v))
        if st != OK:
            raise ValueError(f"oracle_restructure_grad failed with status {st}")
        return r, c, v

    # -- GELU -----------------------------------------------------------
    def gelu(self, x):
        x = np.ascontiguousarray(x, dtype=np.float64)
        y = np.empty_like(x)
        self.lib.oracle_gelu(x.size, _ptr(x), _ptr(y))
        return y

    def gelu_grad(self, x):
        x = np.ascontiguousarray(x, dtype=np.float64)
        g = np.empty_like(x)
        self.lib.oracle_gelu_grad(x.size, _ptr(x), _ptr(g))
        return g

    def decode(self, words):
        w, dt = self._words(np.ascontiguousarray(words).ravel())
        return np.array([self.lib.oracle_decode(_ptr(w), dt, i) for i in range(w.size)], np.float64)


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
