"""GPU parity of the separate-conversion baseline: gate_preact (the gate GEMM
storing the float32 pre-activation), twell_from_preact and ell_from_preact
(standalone conversions of it), against the oracle and against twell_pack.

  * z within the guard band of the float32 accumulation around the exact value;
  * TwELL from z: counts and live indices bit-exact against the oracle, and
    bit-identical to twell_pack's output (values included) where both use the
    same accumulation (more than 64 tokens);
  * row-wise ELLPACK: counts and live indices bit-exact against the oracle's
    ell_pack, values within the bf16 rounding; the row count equals the sum of
    the row's TwELL tile counts (checked on every row at full size).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from activation_sparse_feed_amd import workloads as wl
from helpers import check_twell, device_inputs, oracle_rows, sample_rows, to_f64

pytestmark = pytest.mark.gpu


def _sffn():
    from activation_sparse_feed_amd import sffn
    return sffn


def run_convert(inp: wl.Inputs, cap: int, widths):
    sffn = _sffn()
    w = inp.workload
    d = device_inputs(inp)
    s = sffn.make_shape(w.T, w.d_model, w.d_ff, cap, sffn.SFFN_BF16)
    z = torch.empty((w.T, w.d_ff), dtype=torch.float32, device="cuda")
    sffn.gate_preact(s, d["x"], d["wg_t"], d["b_g"], z)
    ws = sffn.alloc_workspace(s, sffn.WS_CONVERT)
    tw = sffn.alloc_twell(s)
    sffn.twell_from_preact(s, z, d["x"], d["wg_t"], d["b_g"], *tw, ws)
    fused = sffn.alloc_twell(s)
    sffn.twell_pack(s, d["x"], d["wg_t"], d["b_g"], *fused, sffn.alloc_workspace(s, sffn.WS_PACK))
    ell = {}
    for W in widths:
        if W == "max":
            W = int(tw[0].to(torch.int32).sum(1).max().item())
        e = sffn.alloc_ell(s, W)
        sffn.ell_from_preact(s, W, z, d["x"], d["wg_t"], d["b_g"], *e, ws)
        ell[W] = e
    torch.cuda.synchronize()
    return z, tw, fused, ell


def guard_band(K: int, xnorm, wnorm, b):
    """The accumulation-error bound the activity decision relies on (16x16x32
    MFMA chain: K/32 roundings plus the bias add, with a factor 4 margin)."""
    return 2.0 ** -22 * (K // 32 + 2) * np.outer(xnorm, wnorm) + 2.0 ** -22 * np.abs(b)[None, :]


def check_ell(count, idx, val, z_ref, width: int, xnorm, wnorm) -> None:
    c_ref, i_ref, v_ref = oracle.ell_pack(z_ref, width)
    c = np.asarray(count).astype(np.int64)
    assert np.array_equal(c, c_ref), f"ELL count mismatch at {np.argwhere(c != c_ref)[:8]}"
    if width == 0:
        return
    live = np.arange(width)[None, :] < np.minimum(c_ref, width)[:, None]
    i = np.asarray(idx).astype(np.int64)
    assert np.array_equal(np.where(live, i, -1), np.where(live, i_ref, -1)), "ELL idx mismatch"
    rr, ss = np.nonzero(live)
    jj = i_ref[rr, ss]
    err = np.abs(np.asarray(val, np.float64)[rr, ss] - v_ref[rr, ss])
    bad = err > 2.0 ** -8 * np.abs(v_ref[rr, ss]) + 2.0 ** -18 * xnorm[rr] * wnorm[jj]
    assert not bad.any(), f"{bad.sum()} ELL values off"


def check_all(inp: wl.Inputs, cap: int, rows, z, tw, fused, ell):
    w = inp.workload
    ref = oracle_rows(inp, rows, w.tile, cap)
    # z within the guard band around the exact pre-activation
    zg = z.cpu().numpy().astype(np.float64)[rows]
    band = guard_band(w.d_model, ref["xnorm"], ref["wnorm"], inp.b_g.astype(np.float64))
    assert np.all(np.abs(zg - ref["z"]) <= band), "z outside the guard band"
    c, i = tw[0].cpu().numpy(), tw[1].cpu().numpy()
    check_twell("bf16", c[rows], i[rows], to_f64(tw[2])[rows], ref, cap)
    # the converter and the fused epilogue agree on every row
    fc, fi = fused[0].cpu().numpy(), fused[1].cpu().numpy()
    assert np.array_equal(c, fc)
    live = np.arange(max(cap, 1))[None, None, :] < np.minimum(c, cap)[:, :, None]
    assert np.array_equal(np.where(live, i, -1), np.where(live, fi, -1))
    if w.T > 128 and cap > 0:  # the few-token gate (split-K) sums in another order
        v16 = tw[2].view(torch.int16).cpu().numpy()
        f16 = fused[2].view(torch.int16).cpu().numpy()
        assert np.array_equal(np.where(live, v16, 0), np.where(live, f16, 0))
    for W, (ec, ei, ev) in ell.items():
        ecn = ec.cpu().numpy().astype(np.int64)
        assert np.array_equal(ecn, c.astype(np.int64).sum(1)), "ELL count != sum of tile counts"
        check_ell(ecn[rows], ei.cpu().numpy()[rows], to_f64(ev)[rows], ref["z"], W,
                  ref["xnorm"], ref["wnorm"])


@pytest.mark.parametrize("T,d_model,d_ff,beta,cap", [
    (300, 512, 1024, 1.9, 4),    # ragged row block, overflowing tiles
    (33, 256, 128, 1.0, 2),      # one column tile, few tokens (different fused summation)
    (1, 288, 384, 1.5, 3),       # a single token
    (257, 256, 512, 2.3, 0),     # capacity 0: counts only
])
def test_convert_all_rows(T, d_model, d_ff, beta, cap):
    inp = wl.generate_custom(T=T, d_model=d_model, d_ff=d_ff, dtype="bf16", beta=beta,
                             seed_base=21 + T, cap=cap)
    z, tw, fused, ell = run_convert(inp, cap, [0, 3, "max"])
    check_all(inp, cap, np.arange(T), z, tw, fused, ell)


def test_convert_prefill_full_size_sampled():
    w = wl.WORKLOADS["prefill_1pct"]
    inp = wl.generate(w)
    z, tw, fused, ell = run_convert(inp, w.cap, [16, "max"])
    rows = sample_rows(w.T, 96, seed=3)
    check_all(inp, w.cap, rows, z, tw, fused, ell)


def test_convert_decode_all_rows():
    w = wl.WORKLOADS["decode_1pct"]
    inp = wl.generate(w)
    z, tw, fused, ell = run_convert(inp, w.cap, ["max"])
    check_all(inp, w.cap, np.arange(w.T), z, tw, fused, ell)


def test_preact_rejects_float32():
    sffn = _sffn()
    s = sffn.make_shape(64, 256, 512, 8, sffn.SFFN_F32)
    x = torch.zeros((64, 256), device="cuda")
    z = torch.empty((64, 512), device="cuda")
    with pytest.raises(sffn.SffnError):
        sffn.gate_preact(s, x, torch.zeros((512, 256), device="cuda"), None, z)
