"""bench.py's contract pieces that run without a GPU: the byte models behind
`value` and `roofline.achieved`, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("nnz,out,in_,B,fwd,dx,dw", [
    # stored entries, shape and batch of the 1024-square B=8 and 4096-square B=16 layers; bytes written
    # out from the models (fwd: 8 B per entry + row offsets + X and Y once; dX: 12 B per entry + column
    # offsets + dY and dX once; dW: 8 B per entry + row offsets + X and dY once)
    (104858, 1024, 1024, 8, 104858 * 8 + 4 * 1025 + 4 * 8 * 2048, 104858 * 12 + 4 * 1025 + 4 * 8 * 2048,
     104858 * 8 + 4 * 1025 + 4 * 8 * 2048),
    (838861, 4096, 4096, 16, 7_251_564, 10_607_008, 7_251_564),
])
def test_byte_models(nnz, out, in_, B, fwd, dx, dw):
    assert bench.bytes_fwd(nnz, out, in_, B) == fwd
    assert bench.bytes_dx(nnz, out, in_, B) == dx
    assert bench.bytes_dw(nnz, out, in_, B) == dw


def test_fused_gradient_bytes():
    """One launch for both gradients: 16 B per entry (row index and column-ordered value for dX,
    column index read and dW written for dW), both offset arrays, X and dY read once, dX written once."""
    nnz, out, in_, B = 838861, 4096, 4096, 16
    assert bench.bytes_gradients(nnz, out, in_, B) == 14_240_984


def test_bf16_forward_bytes():
    """bf16 values and activations with int32 column indices: 6 B per entry."""
    nnz, out, in_ = 2684355, 16384, 16384
    assert bench.bytes_fwd(nnz, out, in_, 1, sv=2, sx=2) == 16_237_206


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
