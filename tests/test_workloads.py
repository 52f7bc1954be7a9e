"""Synthetic input generators: exact nnz, no duplicates, the capped-Zipf statistics, determinism."""
import numpy as np
import pytest

from coo_spmm_fwd_amd import workloads as W


@pytest.mark.parametrize("out,in_,density,expect", [
    (1024, 1024, 0.10, 104858), (4096, 4096, 0.05, 838861), (3072, 768, 0.10, 235930),
    (768, 3072, 0.10, 235930), (16384, 16384, 0.01, 2684355), (8192, 8192, 0.05, 3355443)])
def test_nnz_rule(out, in_, density, expect):
    assert W.nnz_for(out, in_, density) == expect


def test_uniform_positions_distinct_and_in_range():
    rng = W.streams(2, 1)[0]
    r, c = W.uniform_positions(4096, 4096, 838861, rng)
    assert r.dtype == np.int32 and c.dtype == np.int32
    assert r.min() >= 0 and r.max() < 4096 and c.min() >= 0 and c.max() < 4096
    flat = r.astype(np.int64) * 4096 + c
    assert np.unique(flat).size == 838861
    assert not np.all(np.diff(flat) > 0)          # random order: the builder must sort


def test_zipf_statistics():
    """Capped power law over 16384 rows at 1% density (s = 1.1)."""
    counts, c = W.zipf_row_counts(16384, 16384, 2684355, 1.1, W.streams(4, 1)[0])
    assert counts.sum() == 2684355
    assert abs(c - 664004) < 1.0
    assert int((counts == 16384).sum()) == 28
    assert float(np.median(counts)) == 32.0
    assert int(counts.min()) == 15
    top = np.sort(counts)[::-1][:164].sum() / counts.sum()
    assert 0.45 < top < 0.46


def test_zipf_positions_distinct():
    r, c = W.zipf_positions(512, 512, 20000, 1.1, W.streams(9, 1)[0])
    flat = r.astype(np.int64) * 512 + c
    assert np.unique(flat).size == 20000


def test_build_is_deterministic():
    w1, l1, a1 = W.build("linear1024_b8_s90")
    w2, l2, a2 = W.build("linear1024_b8_s90")
    assert np.array_equal(l1[0].rows, l2[0].rows) and np.array_equal(l1[0].vals, l2[0].vals)
    assert np.array_equal(a1[8]["X"], a2[8]["X"])
    assert l1[0].nnz == 104858 and a1[8]["X"].shape == (8, 1024) and a1[8]["dY"].shape == (8, 1024)
    std = float(np.std(l1[0].vals))
    assert abs(std - 1 / np.sqrt(102.4)) < 0.002


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 0.0, -0.0], np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2**-6 and back[3] == -2.5
    assert bits[5] == 0x8000
