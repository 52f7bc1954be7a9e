"""The C ABI library loads, exports every declared symbol, and rejects bad arguments on the host.

No GPU is needed: every call below returns before the library touches the HIP runtime.
"""
import ctypes
import os
import re
from ctypes import POINTER, c_int64, c_void_p

import pytest

from coo_spmm_fwd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coospmm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["sparse_layer_create", "spmm_fwd", "spmm_bwd_input", "spmm_bwd_values", "restructure"]:
        assert n in names
    assert set(names) == set(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_create_rejects_bad_arguments_on_host(lib):
    h = c_void_p(123)
    st = lib.sparse_layer_create(0, 4, 0, None, None, None, 0, None, ctypes.byref(h))
    assert st == -1 and h.value is None
    assert "shape" in binding.sparse_layer_last_error()
    assert lib.sparse_layer_create(4, 4, 17, None, None, None, 0, None, ctypes.byref(h)) == -1   # nnz > out*in
    assert lib.sparse_layer_create(4, 4, -1, None, None, None, 0, None, ctypes.byref(h)) == -1
    assert lib.sparse_layer_create(4, 4, 3, None, None, None, 0, None, ctypes.byref(h)) == -1    # NULL arrays
    assert lib.sparse_layer_create(4, 4, 0, None, None, None, 7, None, ctypes.byref(h)) == -6    # dtype
    assert lib.sparse_layer_create(4, 4, 0, None, None, None, 0, None, None) == -1               # out_layer
    assert lib.sparse_layer_create(2**31, 4, 0, None, None, None, 0, None, ctypes.byref(h)) == -1


def test_calls_reject_null_layer(lib):
    assert lib.spmm_fwd(None, c_void_p(16), 4, c_void_p(16), None) == -1
    assert lib.spmm_bwd_input(None, c_void_p(16), 4, c_void_p(16), None) == -1
    assert lib.spmm_bwd_values(None, c_void_p(16), c_void_p(16), 4, c_void_p(16), None) == -1
    assert lib.spmm_fwd_act(None, c_void_p(16), 4, None, 1, c_void_p(16), None, None) == -1
    assert lib.spmm_bwd_input_act(None, c_void_p(16), 4, 1, c_void_p(16), c_void_p(16), None) == -1
    assert lib.spmm_bwd_act(None, c_void_p(16), c_void_p(16), 4, 1, c_void_p(16), c_void_p(16), c_void_p(16),
                            None) == -1
    assert lib.restructure_grad(None, 1, c_void_p(16), c_void_p(16), 4, ctypes.c_float(0.0), None) == -1
    assert lib.restructure(None, 0, 1, 1, 0.0, None) == -1
    assert lib.sparse_layer_nnz(None) == -1
    assert lib.sparse_layer_values(None) is None
    assert lib.sparse_layer_export(None, None, None, None, None) == -1
    lib.sparse_layer_destroy(None)
