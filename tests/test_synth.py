"""The seeded input generator: deterministic, the stated distributions, exact outlier counts."""
import numpy as np
import pytest
from scipy import stats

import synth


def test_deterministic_and_seed_dependent():
    a = synth.normal_f64(5, 100000, sigma=0.02)
    b = synth.normal_f64(5, 100000, sigma=0.02)
    c = synth.normal_f64(6, 100000, sigma=0.02)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # counter-based: a window equals the same slice of a longer draw
    w = synth.normal_f64(5, 1000, sigma=0.02, start=5000)
    assert np.array_equal(w, a[5000:6000])


def test_normal_distribution():
    x = synth.normal_f64(11, 1 << 20)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    assert stats.kstest(x, "norm").pvalue > 1e-3


def test_laplace_distribution():
    x = synth.laplace_f64(12, 1 << 20, 0.015)
    assert stats.kstest(x, "laplace", args=(0, 0.015)).pvalue > 1e-3


def test_outliers_exact_count_distinct_signed():
    W = synth.weight_normal(256, 512, 0.02, seed=3, outlier_frac=0.001, outlier_k=10.0)
    cnt = synth.outlier_count(W.size, 0.001)
    assert cnt == 131
    pos, sign = synth.outlier_positions(3, W.size, cnt)
    assert np.unique(pos).size == cnt and pos.min() >= 0 and pos.max() < W.size
    vals = W.reshape(-1)[pos]
    assert (np.abs(vals.astype(np.float64)) == np.float64(np.float16(0.2))).all()
    assert (np.sign(vals) == sign).all()
    assert 30 < (sign > 0).sum() < 100


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_workload_table(name):
    spec = synth.WORKLOADS[name]
    for t in spec["tensors"]:
        assert t.rows > 0 and t.cols > 0
        for q in spec["quant"]:
            assert (t.cols if q.axis == 1 else t.rows) % q.group_size == 0


def test_small_workload_values():
    W = synth.WORKLOADS["single_1024"]["tensors"][0].make()
    assert W.dtype == np.float16 and W.shape == (1024, 1024)
    assert synth.outlier_count(W.size, 0.001) == 1049
    assert (np.abs(W.astype(np.float64)) >= 0.1999).sum() >= 1049
    core = W.astype(np.float64)[np.abs(W.astype(np.float64)) < 0.15]
    assert abs(core.std() - 0.02) < 5e-4
