"""Shared helpers of the GPU parity tests: device upload of seeded inputs,
oracle evaluation on a row subset, and the comparison rules."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from activation_sparse_feed_amd import workloads as wl

# Relative Frobenius tolerance on y: float32 workloads and bf16 storage with
# float32 accumulation.
Y_TOL = {"f32": 1e-5, "bf16": 5e-3}
# Relative tolerance of a stored TwELL value against the exact h (the value is
# the float32 accumulation rounded to the storage type).
VAL_RHO = {"f32": 2.0 ** -20, "bf16": 2.0 ** -8}


def to_device(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def device_inputs(inp: wl.Inputs) -> dict:
    dt = inp.workload.dtype
    return {"x": to_device(inp.x, dt), "wg_t": to_device(inp.wg_t, dt),
            "wu_t": to_device(inp.wu_t, dt), "wd": to_device(inp.wd, dt),
            "b_g": torch.from_numpy(inp.b_g).cuda()}


def to_f64(t: torch.Tensor) -> np.ndarray:
    with np.errstate(invalid="ignore"):  # unwritten TwELL padding may hold any bits
        return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_rows(inp: wl.Inputs, rows, tile: int, cap: int) -> dict:
    """Oracle forward of a subset of rows (rows are independent)."""
    x = inp.rows_f64("x", rows)
    wg, wu, wd = inp.as_f64("wg_t"), inp.as_f64("wu_t"), inp.as_f64("wd")
    out = oracle.sparse_forward(x, wg, inp.b_g, wu, wd, tile, cap)
    out["y_dense"] = oracle.ffn_dense(x, wg, inp.b_g, wu, wd)
    out["xnorm"] = np.linalg.norm(x, axis=1)
    out["wnorm"] = np.linalg.norm(wg, axis=1)
    return out


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b)) / nb


def check_twell(dt: str, count, idx, val, ref: dict, cap: int) -> None:
    """count and live idx bit-exact; live val within the storage rounding.
    Arguments are host arrays of the compared rows."""
    c = np.asarray(count).astype(np.int64)
    assert np.array_equal(c, ref["count"]), f"count mismatch at {np.argwhere(c != ref['count'])[:8]}"
    if cap == 0:
        return
    i = np.asarray(idx).astype(np.int64)
    v = np.asarray(val, dtype=np.float64)
    live = np.arange(cap)[None, None, :] < np.minimum(ref["count"], cap)[:, :, None]
    assert np.array_equal(np.where(live, i, -1), np.where(live, ref["idx"], -1)), "idx mismatch"
    h = ref["val"]
    rr, kk, ss = np.nonzero(live)
    jj = ref["idx"][rr, kk, ss]
    slack = 2.0 ** -18 * ref["xnorm"][rr] * ref["wnorm"][jj]
    err = np.abs(v[rr, kk, ss] - h[rr, kk, ss])
    bad = err > VAL_RHO[dt] * np.abs(h[rr, kk, ss]) + slack
    assert not bad.any(), f"{bad.sum()} TwELL values off, worst {err.max()}"


def check_y(dt: str, y: np.ndarray, y_ref: np.ndarray, routed_mask: np.ndarray) -> dict:
    tol = Y_TOL[dt]
    out = {"all": rel_fro(y, y_ref)}
    assert out["all"] <= tol, out
    if routed_mask.any():
        out["routed"] = rel_fro(y[routed_mask], y_ref[routed_mask])
        assert out["routed"] <= tol, out
    if (~routed_mask).any():
        out["not_routed"] = rel_fro(y[~routed_mask], y_ref[~routed_mask])
        assert out["not_routed"] <= tol, out
    return out


def sample_rows(T: int, n: int, must=(), seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = rng.choice(T, size=min(n, T), replace=False)
    return np.unique(np.concatenate([pick, np.asarray(must, dtype=np.int64),
                                     [0, T - 1]])).astype(np.int64)


def beta_density(beta: float) -> float:
    return 0.5 * math.erfc(beta / math.sqrt(2.0))
