"""The seeded generators draw what their recipes say (CPU only)."""
import numpy as np

import workloads


def test_tiny_is_reproducible_and_in_range():
    a = workloads.TINY.generate()
    b = workloads.TINY.generate()
    assert a.shape == (4, 64, 8) and a.dtype == np.uint8 and np.array_equal(a, b)


def test_nvfp4_outliers_avoid_window_and_non_finite_bytes():
    x = workloads.nvfp4_stack(8, 200, 64, seed=5, exc_rate=0.2)
    rng = np.random.default_rng(5)
    base = rng.integers(0x28, 0x48, (8, 200), endpoint=True, dtype=np.uint8)
    d = x.astype(int) - base[:, :, None]
    out = (d < 0) | (d > 15)
    assert abs(out.mean() - 0.2) < 0.01
    assert not np.any(x == 0x7F) and not np.any(x == 0xFF)


def test_hot_rows_hold_outliers_only():
    x = workloads.nvfp4_stack(4, 500, 50, seed=2, exc_rate=0.10, hot_row_frac=0.01)
    rng = np.random.default_rng(2)
    base = rng.integers(0x28, 0x48, (4, 500), endpoint=True, dtype=np.uint8)
    d = x.astype(int) - base[:, :, None]
    out = ((d < 0) | (d > 15)).reshape(-1, 50)
    assert (out.all(axis=1)).sum() >= 20  # the 20 hot rows
    assert abs(out.mean() - 0.10) < 0.01


def test_mxfp4_values():
    x = workloads.mxfp4_stack(4, 100, 160, seed=4, exc_rate=0.15)
    assert x.min() >= 100 and x.max() <= 140


def test_routing_counts():
    es = workloads.routing(512, 8, 64, seed=3)
    assert es.dtype == np.int32 and es.shape == (513,) and es[0] == 0
    cnt = np.diff(es)
    assert (cnt > 0).sum() == 8 and cnt.max() <= 64 and cnt.min() >= 0
