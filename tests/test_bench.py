"""bench.py's contract pieces that run without a GPU: the byte models behind
`value` and `roofline.achieved`, the cold replica cycle, and the refusal of more
than one GPU."""
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


def test_mirror_and_restructure_bytes():
    """The input gradient over the column-ordered value copy moves 8 B per entry (row index and copied
    value); restructure 36 B per entry; the products step of the 8192-square B=64 layer adds up the
    three per-op models."""
    nnz, out, in_, B = 3355443, 8192, 8192, 64
    assert bench.bytes_dx_mirror(nnz, out, in_, B) == nnz * 8 + 4 * 8193 + 4 * 64 * 16384
    assert bench.bytes_restructure(nnz) == 120_795_948

    class L:
        pass
    lay = L()
    lay.nnz, lay.out, lay.in_, lay.dtype = nnz, out, in_, "f32"
    assert bench.step_bytes("dst", [lay], B) == (bench.bytes_fwd(nnz, out, in_, B) + bench.bytes_dx_mirror(nnz, out, in_, B)
                                                 + bench.bytes_dw(nnz, out, in_, B))
    assert bench.step_bytes("inference", [lay], B) == bench.bytes_fwd(nnz, out, in_, B)


def test_cold_cycle_reuse_distance():
    """Every step, whatever the warm-up and step counts, reuses its replica R - 1 steps later, and R
    is chosen so that R - 1 replicas exceed twice the last-level cache."""
    for touched in (10 << 20, 94 << 20, 300 << 20):
        R = bench.replicas_for(touched, warm=False)
        assert (R - 1) * touched >= 2 * bench.MALL_BYTES
        cyc = bench.Cycle(R)
        last = {}
        for g in range(5 * R + 3):
            r = cyc.next()
            if r in last:
                assert g - last[r] == R
            last[r] = g
    assert bench.replicas_for(94 << 20, warm=True) == 1
