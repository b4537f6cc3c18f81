"""The comparison rules of the GPU parity tests, checked on the CPU: a single
wrong row fails even when the block norm passes, and the float32 per-row
scale (row_magnitude) is never below the row's own norm and still fails a
row whose error exceeds its rounding bound."""
import numpy as np
import pytest

from helpers import Y_TOL, check_y, oracle_rows, row_magnitude
from activation_sparse_feed_amd import workloads as wl


def _ref(T=40, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, 24))


def test_exact_output_passes():
    y = _ref()
    e = check_y("f32", y.copy(), y, np.zeros(len(y), dtype=bool))
    assert e["all"] == 0.0 and e["max_row"] == 0.0


def test_one_wrong_row_fails_though_the_block_passes():
    y = _ref(T=400)
    bad = y.copy()
    bad[7] *= 1.0 + 3 * Y_TOL["bf16"]  # one row 3x over the tolerance
    from helpers import rel_fro
    assert rel_fro(bad, y) <= Y_TOL["bf16"]  # the block norm alone would pass
    with pytest.raises(AssertionError, match="rows over"):
        check_y("bf16", bad, y, np.zeros(len(y), dtype=bool))


def test_zero_rows_must_be_exact():
    y = _ref()
    y[3] = 0.0
    bad = y.copy()
    bad[3, 0] = 1e-30
    with pytest.raises(AssertionError, match="should be 0"):
        check_y("f32", bad, y, np.zeros(len(y), dtype=bool))


def test_magnitude_scale_bounds_the_row_norm():
    inp = wl.generate_custom(T=64, d_model=96, d_ff=256, dtype="f32", beta=1.5, seed_base=3)
    rows = np.arange(64)
    m = row_magnitude(inp, rows)
    y = oracle_rows(inp, rows, 128, 128, dense=False)["y"]
    assert np.all(m >= np.linalg.norm(y, axis=1) * (1 - 1e-12))


def test_magnitude_scale_still_fails_a_wrong_row():
    y = _ref(T=40000)  # enough rows that the block norms pass
    mag = 50.0 * np.linalg.norm(y, axis=1)  # rows whose terms cancel 50-fold
    ok = y.copy()
    ok[5] += 20 * Y_TOL["f32"] * y[5]  # 20x tol relative, 0.4x tol against the scale
    check_y("f32", ok, y, np.zeros(len(y), dtype=bool), mag)
    bad = y.copy()
    bad[5] += 100 * Y_TOL["f32"] * y[5]  # 2x tol against the scale
    with pytest.raises(AssertionError, match="rows over"):
        check_y("f32", bad, y, np.zeros(len(y), dtype=bool), mag)
