"""GPU parity of the sparse backward (sparse_ffn_bwd) against the oracle.

The forward runs first (twell_pack, sparse_ffn_fwd, hybrid_route) and its
TwELL arrays and routed rows feed the backward, as in training.  Each gradient
is compared with the oracle's sparse backward on the same TwELL values and with
its dense backward (exact h), by relative Frobenius error within the bf16
tolerance 5e-3 (float32 shapes: 1e-5); gx separately over routed and
non-routed rows.  The weight gradients are float32 sums in a fixed order: two
calls give the same bits.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from activation_sparse_feed_amd import workloads as wl
from helpers import device_inputs, rel_fro, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

TOL = 5e-3
TOL_F32 = 1e-5


def _sffn():
    from activation_sparse_feed_amd import sffn
    return sffn


def run_backward(inp: wl.Inputs, cap: int, gy_np: np.ndarray, repeat: int = 1, lam: float = 0.0,
                 exact_ws: bool = False):
    """exact_ws: size the routed part of the workspace for the forward's own
    routed count (max_routed = n_routed) instead of for every token."""
    sffn = _sffn()
    w = inp.workload
    d = device_inputs(inp)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, cap, dt)
    ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    s = ffn.shape
    gy = to_device(gy_np, w.dtype)
    mr = int(ffn.n_routed.item()) if exact_ws else None
    if exact_ws:
        ws = torch.empty(max(sffn.backward_workspace_bytes(s, mr), 16), dtype=torch.uint8,
                         device="cuda")
    else:
        ws = sffn.alloc_workspace(s, sffn.WS_BACKWARD)
    outs = []
    for _ in range(repeat):
        gx = torch.empty((w.T, w.d_model), dtype=dt, device="cuda")
        g = [torch.full((w.d_ff, w.d_model), float("nan"), device="cuda") for _ in range(3)]
        gb = torch.full((w.d_ff,), float("nan"), device="cuda")
        sffn.sparse_ffn_bwd(s, d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"], ffn.count, ffn.idx,
                            ffn.val, ffn.routed, ffn.n_routed, gy, gx, *g, gb, ws, l1_lambda=lam,
                            max_routed=mr)
        outs.append({"gx": gx, "gwg_t": g[0], "gwu_t": g[1], "gwd": g[2], "gb": gb})
    torch.cuda.synchronize()
    return ffn, outs


def check(inp: wl.Inputs, cap: int, dense: bool, rows=None, lam: float = 0.0,
          exact_ws: bool = False):
    w = inp.workload
    gy_np = wl.upstream_grad(w)
    ffn, outs = run_backward(inp, cap, gy_np, repeat=2, lam=lam, exact_ws=exact_ws)
    o = outs[0]
    for k in o:  # deterministic
        assert torch.equal(o[k].view(torch.int16) if o[k].dtype == torch.bfloat16 else o[k],
                           outs[1][k].view(torch.int16) if o[k].dtype == torch.bfloat16 else outs[1][k]), k
    x, wg, wu, wd = inp.as_f64("x"), inp.as_f64("wg_t"), inp.as_f64("wu_t"), inp.as_f64("wd")
    gy = (wl.bf16_bits_to_f32(gy_np) if w.dtype == "bf16" else gy_np).astype(np.float64)
    tol = TOL if w.dtype == "bf16" else TOL_F32
    n_r = int(ffn.n_routed.item())
    routed = ffn.routed[:n_r].cpu().numpy().astype(np.int64)
    ref = oracle.ffn_sparse_backward(x, wg, inp.b_g, wu, wd, gy, ffn.count.cpu().numpy(),
                                     ffn.idx.cpu().numpy().astype(np.int64), to_f64(ffn.val), cap,
                                     lam)
    refs = [ref]
    if dense:
        refs.append(oracle.ffn_dense_backward(x, wg, inp.b_g, wu, wd, gy, lam))
    got = {k: to_f64(v) for k, v in o.items()}
    mask = np.zeros(w.T, dtype=bool)
    mask[routed] = True
    errs = {}
    for r in refs:
        for k in ("gwg_t", "gwu_t", "gwd", "gb"):
            errs[k] = rel_fro(got[k], r[k])
            assert errs[k] <= tol, (k, errs[k])
        sel = np.arange(w.T) if rows is None else rows
        errs["gx"] = rel_fro(got["gx"][sel], r["gx"][sel])
        assert errs["gx"] <= tol, errs
        for name, m in (("routed", mask[sel]), ("not_routed", ~mask[sel])):
            if m.any():
                errs["gx_" + name] = rel_fro(got["gx"][sel][m], r["gx"][sel][m])
                assert errs["gx_" + name] <= tol, errs
    errs["n_routed"] = n_r
    return errs


@pytest.mark.parametrize("T,d_model,d_ff,beta,cap", [
    (300, 512, 1024, 1.9, 4),     # ragged rows, routed rows (complete lists)
    (64, 1024, 512, 1.2, 8),      # two 512-wide chunks, many routed rows
    (33, 512, 256, 2.0, 8),       # few tokens (the forward's split-K gate)
    (130, 1536, 384, 1.5, 0),     # capacity 0: every active row routed
    (40, 4096, 640, 2.0, 4),      # the widest model dimension (eight 512-wide chunks)
    (97, 2560, 256, 1.7, 2),      # five chunks, odd d-chunk count for the weight gradients
    # more than 256 tokens, d_model <= 2048: per-entry gradients in the column pass
    (400, 1024, 512, 1.2, 8),     # two chunks
    (280, 1536, 384, 1.5, 0),     # three chunks, capacity 0: empty column lists
    (270, 2048, 384, 2.0, 3),     # four chunks, ragged rows
    (300, 2560, 256, 1.7, 2),     # wider than 2048: row pass and column pass
])
def test_backward_small(T, d_model, d_ff, beta, cap):
    inp = wl.generate_custom(T=T, d_model=d_model, d_ff=d_ff, dtype="bf16", beta=beta,
                             seed_base=60 + T, cap=cap)
    e = check(inp, cap, dense=True)
    if cap == 0:
        assert e["n_routed"] > 0


def test_backward_decode_full_size():
    w = wl.WORKLOADS["decode_1pct"]
    check(wl.generate(w), w.cap, dense=True)


def test_backward_prefill_full_size():
    # 4096 tokens, 2048 -> 5632, no routed rows: the fused column order at full size;
    # the weight gradients and gb over every column, gx on 256 rows
    w = wl.WORKLOADS["prefill_1pct"]
    e = check(wl.generate(w), w.cap, dense=False, rows=sample_rows(w.T, 256, seed=5))
    assert e["n_routed"] == 0


def test_backward_hybrid_mix_full_size():
    w = wl.WORKLOADS["hybrid_mix"]
    inp = wl.generate(w)
    e = check(inp, w.cap, dense=False, rows=sample_rows(w.T, 256, seed=4))
    assert e["n_routed"] > 60


@pytest.mark.parametrize("T,d_model,d_ff,beta,cap,lam,exact_ws", [
    (8200, 1024, 1024, 1.0, 2, 0.0, False),  # fused column order, ragged row tiles
    (8192, 2560, 512, 1.0, 2, 0.5, False),   # row and column walk order, the L1 term
    (8200, 1024, 1024, 1.0, 2, 0.0, True),   # workspace sized for the routed count only
    (8192, 1536, 640, 1.0, 2, 0.25, False),  # d_ff not a multiple of 256: half-empty wide tiles
])
def test_backward_routed_rows_on_tiles(T, d_model, d_ff, beta, cap, lam, exact_ws):
    """More than 1024 routed rows with at least 8192 tokens: the routed rows'
    products run on MFMA tiles (per-entry gradients rounded to bf16 before the
    weight-gradient and gx products) and are added to the other rows' sums.
    The tile grid is sized for the workspace's row bound and numbered by the
    actual count, so both sizings are checked."""
    inp = wl.generate_custom(T=T, d_model=d_model, d_ff=d_ff, dtype="bf16", beta=beta,
                             seed_base=110 + d_model, cap=cap)
    e = check(inp, cap, dense=False, rows=sample_rows(T, 300, must=np.arange(T - 9, T), seed=8),
              lam=lam, exact_ws=exact_ws)
    assert e["n_routed"] > 1024


def test_backward_few_routed_rows_with_tile_kernels_launched():
    # at least 8192 tokens but few routed rows: the per-entry kernels take them
    # (the MFMA kernels are launched and return at once)
    inp = wl.generate_custom(T=8192, d_model=512, d_ff=512, dtype="bf16", beta=2.3,
                             seed_base=120, cap=4)
    e = check(inp, 4, dense=False, rows=sample_rows(8192, 300, seed=9))
    assert 0 < e["n_routed"] < 1024


@pytest.mark.parametrize("case", ["tiny_f32", "ragged_routed", "wide_masked"])
def test_backward_float32(case):
    """Float32 shapes: the backward from complete activity lists of every row
    (twell_pack's own kernels at the full capacity), against the oracle's
    sparse and dense backward within 1e-5."""
    if case == "tiny_f32":
        inp = wl.generate(wl.WORKLOADS["tiny_f32"])
        cap, lam = inp.workload.cap, 0.0
    elif case == "ragged_routed":   # many routed rows, d_model not a multiple of 256, L1 term
        inp = wl.generate_custom(T=130, d_model=200, d_ff=384, dtype="f32", beta=1.2,
                                 seed_base=140, cap=2)
        cap, lam = 2, 0.3
    else:                           # chunks of 4 floats per lane up to 8, the last one masked
        inp = wl.generate_custom(T=300, d_model=1544, d_ff=256, dtype="f32", beta=1.7,
                                 seed_base=150, cap=4)
        cap, lam = 4, 0.0
    e = check(inp, cap, dense=True, lam=lam)
    if case == "ragged_routed":
        assert e["n_routed"] > 10


@pytest.mark.parametrize("T,d_model,d_ff,beta,cap,lam", [
    (300, 264, 384, 1.5, 4, 0.0),    # one masked chunk per lane row, routed rows
    (64, 768, 512, 1.2, 8, 0.2),     # a common width, many routed rows, the L1 term
    (257, 1288, 256, 1.9, 2, 0.0),   # three chunks, the last one partly masked
    (100, 2304, 256, 1.7, 2, 0.0),   # wider than 2048: five chunks per lane
])
def test_backward_bf16_general_width(T, d_model, d_ff, beta, cap, lam):
    """bf16 widths that are not a multiple of 512 take the general path
    (complete lists of every row, as for float32) within the bf16 tolerance."""
    inp = wl.generate_custom(T=T, d_model=d_model, d_ff=d_ff, dtype="bf16", beta=beta,
                             seed_base=160 + d_model, cap=cap)
    e = check(inp, cap, dense=True, lam=lam)
    assert e["n_routed"] > 0


@pytest.mark.parametrize("T,d_model,d_ff,dtype,beta,cap", [
    (8200, 1024, 1024, "bf16", 1.0, 2),   # routed rows on MFMA tiles (recomputed gate)
    (300, 512, 1024, "bf16", 1.9, 4),     # per-entry routed rows
    (130, 200, 384, "f32", 1.2, 2),       # the general path (complete lists of every row)
])
def test_backward_precomputed_weight_norms(T, d_model, d_ff, dtype, beta, cap):
    """The gate-weight row norms only set the guard band of the recomputed
    activity decisions, which are exact: passing twell_weight_norms' result
    gives the same gradients, bit for bit, as letting the call compute them."""
    sffn = _sffn()
    inp = wl.generate_custom(T=T, d_model=d_model, d_ff=d_ff, dtype=dtype, beta=beta,
                             seed_base=170 + d_model, cap=cap)
    w = inp.workload
    d = device_inputs(inp)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ffn = sffn.SparseFFN(T, d_model, d_ff, cap, dt)
    wn = ffn.weight_norms(d["wg_t"])
    ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"], wn)
    s = ffn.shape
    gy = to_device(wl.upstream_grad(w), dtype)
    ws = sffn.alloc_workspace(s, sffn.WS_BACKWARD)
    outs = []
    for norms in (None, wn):
        gx = torch.empty((T, d_model), dtype=dt, device="cuda")
        g = [torch.empty((d_ff, d_model), device="cuda") for _ in range(3)]
        gb = torch.empty(d_ff, device="cuda")
        sffn.sparse_ffn_bwd(s, d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"], ffn.count,
                            ffn.idx, ffn.val, ffn.routed, ffn.n_routed, gy, gx, *g, gb, ws, norms)
        torch.cuda.synchronize()
        outs.append([gx.view(torch.int16) if dt == torch.bfloat16 else gx] + g + [gb])
    for a_, b_ in zip(*outs):
        assert torch.equal(a_, b_)
    assert int(ffn.n_routed.item()) > 0


def test_backward_rejects_unsupported_width():
    sffn = _sffn()
    s = sffn.make_shape(64, 4104, 256, 8, sffn.SFFN_BF16)  # wider than 4096
    ws = torch.empty(max(sffn.workspace_bytes(s, sffn.WS_BACKWARD), 16), dtype=torch.uint8,
                     device="cuda")
    b = torch.zeros((64, 4104), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((256, 4104), dtype=torch.bfloat16, device="cuda")
    g = [torch.zeros((256, 4104), device="cuda") for _ in range(3)]
    c = torch.zeros((64, 2), dtype=torch.uint16, device="cuda")
    i = torch.zeros((64, 2, 8), dtype=torch.uint16, device="cuda")
    v = torch.zeros((64, 2, 8), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(sffn.SffnError) as ei:
        sffn.sparse_ffn_bwd(s, b, w, None, w, w, c, i, v, r, r[:1], b, b, *g, None, ws)
    assert ei.value.status == sffn.SFFN_ERR_UNSUPPORTED


@pytest.mark.parametrize("T,d_model,d_ff,beta,cap", [
    (300, 512, 1024, 1.9, 4),     # row pass, routed rows (complete lists)
    (33, 512, 256, 2.0, 8),       # few tokens
    (400, 1024, 512, 1.2, 8),     # fused column order (per-entry gradients in the column pass)
    (130, 1536, 384, 1.5, 0),     # capacity 0: every active entry in a routed row
])
def test_backward_l1_regulariser(T, d_model, d_ff, beta, cap):
    """The L1 activation regulariser's gradient (lam / T on every active entry,
    routed rows' entries past the capacity included) through gz into gb,
    gwg_t and gx, against the oracle with the same lam; the lam-free
    gradients (gwu_t, gwd) are unchanged bit for bit."""
    inp = wl.generate_custom(T=T, d_model=d_model, d_ff=d_ff, dtype="bf16", beta=beta,
                             seed_base=71, cap=cap)
    lam = 0.5
    e = check(inp, cap, dense=True, lam=lam)
    gy_np = wl.upstream_grad(inp.workload)
    _, (with_l1,) = run_backward(inp, cap, gy_np, lam=lam)
    _, (without,) = run_backward(inp, cap, gy_np, lam=0.0)
    for k in ("gwu_t", "gwd"):
        assert torch.equal(with_l1[k], without[k]), k
    # gb moves by lam / T times the number of active rows of each column
    x, wg = inp.as_f64("x"), inp.as_f64("wg_t")
    act = (oracle.gate_preact(x, wg, inp.b_g) > 0).sum(0)
    dgb = to_f64(with_l1["gb"]) - to_f64(without["gb"])
    assert np.allclose(dgb, lam / T * act, rtol=1e-4, atol=1e-4 * (1 + np.abs(to_f64(without["gb"])).max()))
    print(f"l1 backward T={T} d={d_model}: {e}")


@pytest.mark.parametrize("case", ["ragged", "hybrid_mix"])
def test_backward_from_saved_state_alone(case):
    """The backward needs nothing of the forward but its TwELL arrays and the
    routed list: the forward's buffers and workspaces are freed first, and the
    backward workspace holds exactly the routed rows the forward produced
    (max_routed = n_routed, read after the forward)."""
    sffn = _sffn()
    if case == "ragged":
        inp = wl.generate_custom(T=300, d_model=512, d_ff=1024, dtype="bf16", beta=1.9,
                                 seed_base=73, cap=4)
    else:
        inp = wl.generate(wl.WORKLOADS["hybrid_mix"])
    w = inp.workload
    d = device_inputs(inp)
    ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, w.cap, torch.bfloat16)
    ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    saved = {k: getattr(ffn, k).clone() for k in ("count", "idx", "val", "routed", "n_routed")}
    s = ffn.shape
    del ffn
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    n_r = int(saved["n_routed"].item())
    assert n_r > 0
    ws = torch.empty(sffn.backward_workspace_bytes(s, n_r), dtype=torch.uint8, device="cuda")
    assert ws.numel() < sffn.workspace_bytes(s, sffn.WS_BACKWARD)
    gy_np = wl.upstream_grad(w)
    gy = to_device(gy_np, "bf16")
    gx = torch.empty((w.T, w.d_model), dtype=torch.bfloat16, device="cuda")
    g = [torch.empty((w.d_ff, w.d_model), device="cuda") for _ in range(3)]
    gb = torch.empty(w.d_ff, device="cuda")
    sffn.sparse_ffn_bwd(s, d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"], saved["count"],
                        saved["idx"], saved["val"], saved["routed"], saved["n_routed"], gy, gx, *g,
                        gb, ws, max_routed=n_r)
    torch.cuda.synchronize()
    x, wg, wu, wd = inp.as_f64("x"), inp.as_f64("wg_t"), inp.as_f64("wu_t"), inp.as_f64("wd")
    gyf = wl.bf16_bits_to_f32(gy_np).astype(np.float64)
    ref = oracle.ffn_dense_backward(x, wg, inp.b_g, wu, wd, gyf)
    got = {"gx": gx, "gwg_t": g[0], "gwu_t": g[1], "gwd": g[2], "gb": gb}
    for k, v in got.items():
        e = rel_fro(to_f64(v), ref[k])
        assert e <= TOL, (k, e)
    print(f"backward from saved state ({case}): {n_r} routed rows, workspace "
          f"{ws.numel() / 1e6:.1f} MB of {sffn.workspace_bytes(s, sffn.WS_BACKWARD) / 1e6:.1f} MB")


def test_backward_routed_overflow_is_flagged():
    """A routed-row bound below what the forward routed leaves those rows out;
    the call then sets gb and the first row of gx to NaN (forced from the host:
    the bound is one row short)."""
    sffn = _sffn()
    inp = wl.generate_custom(T=300, d_model=512, d_ff=1024, dtype="bf16", beta=1.9, seed_base=73,
                             cap=4)
    w = inp.workload
    d = device_inputs(inp)
    ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, w.cap, torch.bfloat16)
    ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    n_r = int(ffn.n_routed.item())
    assert n_r > 1
    s = ffn.shape
    ws = torch.empty(sffn.backward_workspace_bytes(s, n_r - 1), dtype=torch.uint8, device="cuda")
    gy = to_device(wl.upstream_grad(w), "bf16")
    gx = torch.zeros((w.T, w.d_model), dtype=torch.bfloat16, device="cuda")
    g = [torch.zeros((w.d_ff, w.d_model), device="cuda") for _ in range(3)]
    gb = torch.zeros(w.d_ff, device="cuda")
    sffn.sparse_ffn_bwd(s, d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"], ffn.count, ffn.idx,
                        ffn.val, ffn.routed, ffn.n_routed, gy, gx, *g, gb, ws, max_routed=n_r - 1)
    torch.cuda.synchronize()
    assert torch.isnan(gb).all()
    assert torch.isnan(gx[0].float()).all()
