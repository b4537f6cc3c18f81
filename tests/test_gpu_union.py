"""GPU parity of sparse_ffn_fwd_union, the fused up(.)gate->down kernel that
stages each token block's column union in LDS (the pages' fused-kernel
organisation, pwwt.cn article, section 02), on the TwELL that twell_pack
writes: y of every non-routed row against the CPU oracle (relative Frobenius
error and per-row error within 5e-3, bf16 with float32 accumulation) and
against the row walk of sparse_ffn_fwd on every row; routed rows are left
untouched.  (The refusal of unsupported shapes is a host check, tested on the
CPU in test_abi.py.)
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from activation_sparse_feed_amd import workloads as wl
from helpers import check_y, device_inputs, oracle_rows, rel_fro, row_rel_err, sample_rows, to_f64

pytestmark = pytest.mark.gpu

SENTINEL = 12288.0  # 1.5 * 2^13: exact in bf16, never an FFN output of these workloads


def _sffn():
    from activation_sparse_feed_amd import sffn
    return sffn


def run_union(inp: wl.Inputs, cap: int, rows=None):
    sffn = _sffn()
    w = inp.workload
    d = device_inputs(inp)
    ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, cap, torch.bfloat16)
    y_walk = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"]).clone()
    y_u = torch.full((w.T, w.d_model), SENTINEL, dtype=torch.bfloat16, device="cuda")
    print(f"union {w.name}: T={w.T} d_model={w.d_model} d_ff={w.d_ff} cap={cap}", flush=True)
    sffn.sparse_ffn_fwd_union(ffn.shape, d["x"], d["wu_t"], d["wd"], ffn.count, ffn.idx,
                              ffn.val, y_u)
    torch.cuda.synchronize()
    n_r = int(ffn.n_routed.item())
    routed = ffn.routed[:n_r].cpu().numpy().astype(np.int64)
    yu = to_f64(y_u)
    yw = to_f64(y_walk)
    # routed rows are not written
    assert np.all(yu[routed] == SENTINEL)
    keep = np.ones(w.T, dtype=bool)
    keep[routed] = False
    # against the row walk on every non-routed row (same sum, other rounding order)
    assert np.all(np.isfinite(yu[keep]))
    per_row = row_rel_err(yu[keep], yw[keep])
    assert rel_fro(yu[keep], yw[keep]) <= 2e-3 and per_row.max(initial=0.0) <= 5e-3, per_row.max()
    # against the oracle on the compared rows (all rows, or a sample)
    if rows is None:
        rows = np.arange(w.T)
    rows = rows[keep[rows]]
    ref = oracle_rows(inp, rows, w.tile, cap, dense=False)
    assert len(ref["routed"]) == 0
    errs = check_y("bf16", yu[rows], ref["y"], np.zeros(len(rows), dtype=bool))
    print(f"  routed {n_r}, oracle rows {len(rows)}: rel_err {errs['all']:.3e} "
          f"max_row {errs['max_row']:.3e}; vs row walk max_row {per_row.max(initial=0.0):.3e}")
    return n_r


def test_union_prefill_full_size():
    inp = wl.generate(wl.WORKLOADS["prefill_1pct"])
    run_union(inp, 8, sample_rows(4096, 600, seed=5))


def test_union_hybrid_routed_rows_untouched():
    w = wl.WORKLOADS["hybrid_mix"]
    inp = wl.generate(w)
    n_r = run_union(inp, w.cap, sample_rows(w.T, 400, seed=6))
    assert n_r > 0


def test_union_decode_d4096():
    inp = wl.generate(wl.WORKLOADS["decode_1pct"])
    run_union(inp, 8)


@pytest.mark.parametrize("T,d_model,d_ff,beta,cap", [
    (1, 512, 1024, 1.2, 32),     # one token, one partly filled block
    (37, 1024, 2048, 1.6, 16),   # ragged last block, unions larger than one staged chunk
    (300, 512, 1152, 2.0, 4),    # routed rows, ragged tail, 9 tiles
    (64, 512, 1024, 3.0, 0),     # capacity 0: every row with an active entry routed, the rest 0
    (520, 4096, 2048, 2.3, 8),   # d_model 4096 (8 tokens per workgroup, 8 staged columns), 65 blocks
])
def test_union_small_shapes(T, d_model, d_ff, beta, cap):
    inp = wl.generate_custom(T, d_model, d_ff, "bf16", beta, seed_base=70 + T, cap=cap)
    run_union(inp, cap)
