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


def oracle_rows(inp: wl.Inputs, rows, tile: int, cap: int, dense: bool = True) -> dict:
    """Oracle forward of a subset of rows (rows are independent).  With
    dense=False the oracle's dense FFN (y_dense) is not computed."""
    x = inp.rows_f64("x", rows)
    wg, wu, wd = inp.as_f64("wg_t"), inp.as_f64("wu_t"), inp.as_f64("wd")
    out = oracle.sparse_forward(x, wg, inp.b_g, wu, wd, tile, cap)
    if dense:
        out["y_dense"] = oracle.ffn_dense(x, wg, inp.b_g, wu, wd)
    out["xnorm"] = np.linalg.norm(x, axis=1)
    out["wnorm"] = np.linalg.norm(wg, axis=1)
    return out


def oracle_twell_all_rows(inp: wl.Inputs, tile: int, cap: int, chunk: int = 1024) -> dict:
    """The oracle's gate and TwELL pack over every row, in row chunks (rows are
    independent), without the up and down projections: count, idx, val and the
    routed rows, for all-row comparisons at full size."""
    T = inp.workload.T
    wg = inp.as_f64("wg_t")
    counts, idxs, vals = [], [], []
    for r0 in range(0, T, chunk):
        rows = np.arange(r0, min(T, r0 + chunk))
        z = oracle.gate_preact(inp.rows_f64("x", rows), wg, inp.b_g)
        c, i, v = oracle.twell_pack(z, tile, cap)
        counts.append(c)
        idxs.append(i)
        vals.append(v)
    count = np.concatenate(counts)
    return {"count": count, "idx": np.concatenate(idxs), "val": np.concatenate(vals),
            "routed": oracle.route(count, cap),
            "xnorm": np.linalg.norm(inp.as_f64("x"), axis=1),
            "wnorm": np.linalg.norm(wg, axis=1)}


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


def row_rel_err(y: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Relative Euclidean error of every row; rows whose exact output is zero
    get their absolute error (they must come out exactly zero)."""
    num = np.linalg.norm(y - y_ref, axis=1)
    den = np.linalg.norm(y_ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def row_magnitude(inp: wl.Inputs, rows) -> np.ndarray:
    """Per row, the norm of the forward computed on absolute values,
    || sum_j |g_tj| (sum_k |x_tk| |wu_jk|) |wd_j| ||: the scale that bounds a
    row's floating-point error (each dot product's rounding error is at most
    a small multiple of the unit roundoff times the sum of the absolute values
    of its terms), and never below ||y_t||."""
    x = inp.rows_f64("x", rows)
    g = oracle.relu(oracle.gate_preact(x, inp.as_f64("wg_t"), inp.b_g))
    ua = np.abs(x) @ np.abs(inp.as_f64("wu_t")).T
    return np.linalg.norm((g * ua) @ np.abs(inp.as_f64("wd")), axis=1)


def check_y(dt: str, y: np.ndarray, y_ref: np.ndarray, routed_mask: np.ndarray,
            mag: np.ndarray | None = None) -> dict:
    """y against the oracle: the relative Frobenius error over all compared
    rows, separately over routed and non-routed rows, AND on every single row
    (so that a few wrong rows cannot hide in a block norm); rows whose exact
    output is zero must be exactly zero.  With mag (row_magnitude, float32
    workloads), a row's error is taken relative to max(||y_t||, mag_t), so that
    a row whose few terms cancel is held to its rounding bound instead of to
    the relative error of a small result.  Returns the errors, including the
    largest per-row one."""
    tol = Y_TOL[dt]
    out = {"all": rel_fro(y, y_ref)}
    assert out["all"] <= tol, out
    if routed_mask.any():
        out["routed"] = rel_fro(y[routed_mask], y_ref[routed_mask])
        assert out["routed"] <= tol, out
    if (~routed_mask).any():
        out["not_routed"] = rel_fro(y[~routed_mask], y_ref[~routed_mask])
        assert out["not_routed"] <= tol, out
    rows = row_rel_err(y, y_ref)
    if mag is not None:
        den = np.linalg.norm(y_ref, axis=1)
        rows = np.where(den > 0, rows * den / np.maximum(den, mag), rows)
    out["max_row"] = float(rows.max()) if len(rows) else 0.0
    out["worst_row"] = int(rows.argmax()) if len(rows) else -1
    zero = np.linalg.norm(y_ref, axis=1) == 0
    assert not np.any(rows[zero] != 0.0), f"rows {np.nonzero(zero & (rows != 0))[0][:8]} should be 0"
    bad = np.nonzero(rows > tol)[0]
    assert len(bad) == 0, f"{len(bad)} rows over {tol}: {bad[:8]} (max {out['max_row']:.3e})"
    return out


def sample_rows(T: int, n: int, must=(), seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = rng.choice(T, size=min(n, T), replace=False)
    return np.unique(np.concatenate([pick, np.asarray(must, dtype=np.int64),
                                     [0, T - 1]])).astype(np.int64)


def beta_density(beta: float) -> float:
    return 0.5 * math.erfc(beta / math.sqrt(2.0))
