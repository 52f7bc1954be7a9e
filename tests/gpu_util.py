"""Helpers shared by the GPU tests: device transfer and the comparison rules.

Comparison rules (applied to every output element):
  fp32 ops   |gpu - ref| <= 1e-5 * S, with ref and S = sum |terms| from the fp64 oracle;
  bf16 ops   |gpu - ref| <= 1e-2 * S;
  integers, indices and moved values: bit-exact.
A row or column with no terms has S = 0, so it must be exactly 0.
"""
from __future__ import annotations

import numpy as np
import torch

from coo_spmm_fwd_amd import workloads as W

FP32_REL = 1e-5
BF16_REL = 1e-2


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:   # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def assert_within(gpu: np.ndarray, ref: np.ndarray, S: np.ndarray, rel: float, what: str = ""):
    g = as_f64(gpu)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bad = err > rel * S
    if np.any(bad):
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(S, 1e-300), 0)), g.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside {rel:g}*S; worst at {idx}: "
                             f"gpu={g[idx]!r} ref={ref[idx]!r} S={S[idx]!r}")


def err_ratio(gpu, ref, S) -> float:
    g = as_f64(gpu)
    m = S > 0
    return float(np.max(np.abs(g - ref)[m] / S[m])) if np.any(m) else 0.0


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype in (np.uint16,) else a.view(np.uint32)
