"""All-core fp32 CPU baseline (``parallel.c``) -- BENCHMARK INFRASTRUCTURE ONLY.

Only ``bench.py``'s ``cpu_baseline`` leg and its CPU test load this module.  It
is not the oracle: ``oracle.c`` (fp64, one core) is what parity is checked
against.  This is the same three loops with fp32 accumulation, parallel over
rows (forward, value gradient) and over columns of the transposed view (input
gradient) with OpenMP on every host core, reading batch-minor copies of the
dense operands that each call makes first; timed as a reported baseline.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from ctypes import c_int, c_int64, c_void_p

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "parallel.c")
LIB = os.path.join(HERE, "libparallel.so")


def build() -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run(["gcc", "-O3", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


def _p(a):
    """Data pointer of a numpy array; the caller keeps the array referenced while C uses it."""
    return c_void_p(a.ctypes.data)


class Parallel:
    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        L.par_threads.restype = c_int
        L.par_spmm_fwd.argtypes = [c_int64] * 3 + [c_void_p] * 7
        L.par_spmm_bwd_input.argtypes = [c_int64] * 3 + [c_void_p] * 8
        L.par_spmm_bwd_values.argtypes = [c_int64] * 3 + [c_void_p] * 7
        for f in (L.par_spmm_fwd, L.par_spmm_bwd_input, L.par_spmm_bwd_values):
            f.restype = None
        self.lib = L
        self.threads = int(L.par_threads())

    def _acc(self, B):
        return np.empty(self.threads * B, np.float32)

    def spmm_fwd(self, canon, out, in_, X):
        B = X.shape[0]
        X = np.ascontiguousarray(X, np.float32)
        Y = np.empty((B, out), np.float32)
        acc = self._acc(B)
        xt = np.empty(in_ * B, np.float32)
        self.lib.par_spmm_fwd(out, in_, B, _p(canon["row_ptr"]), _p(canon["cols"]), _p(canon["vals"]), _p(X),
                              _p(Y), _p(acc), _p(xt))
        return Y

    def spmm_bwd_input(self, canon, out, in_, dY):
        B = dY.shape[0]
        dY = np.ascontiguousarray(dY, np.float32)
        dX = np.empty((B, in_), np.float32)
        acc = self._acc(B)
        gt = np.empty(out * B, np.float32)
        self.lib.par_spmm_bwd_input(out, in_, B, _p(canon["col_ptr"]), _p(canon["perm_c"]), _p(canon["rows_by_col"]),
                                    _p(canon["vals"]), _p(dY), _p(dX), _p(acc), _p(gt))
        return dX

    def spmm_bwd_values(self, canon, out, in_, dY, X):
        B = X.shape[0]
        X = np.ascontiguousarray(X, np.float32)
        dY = np.ascontiguousarray(dY, np.float32)
        dW = np.empty(canon["cols"].shape[0], np.float32)
        gt = np.empty(out * B, np.float32)
        xt = np.empty(in_ * B, np.float32)
        self.lib.par_spmm_bwd_values(out, in_, B, _p(canon["row_ptr"]), _p(canon["cols"]), _p(dY), _p(X), _p(dW),
                                     _p(gt), _p(xt))
        return dW
