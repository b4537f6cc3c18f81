"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

TwELL counts, live indices, the routed-row set and n_routed are compared bit
for bit; TwELL values within the storage rounding; y by relative Frobenius
error (1e-5 float32, 5e-3 bf16 with float32 accumulation), over all compared
rows, separately over routed and non-routed rows, and on every compared row
by itself.  The prefill and hybrid workloads are compared on all 4096 rows;
the large workload's counts, live indices and routed set on all 16384 rows,
its y on a sample of rows that includes routed ones.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from activation_sparse_feed_amd import workloads as wl
from helpers import (check_twell, check_y, device_inputs, oracle_rows, oracle_twell_all_rows,
                     row_magnitude, sample_rows, to_f64)

pytestmark = pytest.mark.gpu


def _sffn():
    from activation_sparse_feed_amd import sffn
    return sffn


def run_sparse(inp: wl.Inputs, cap: int):
    sffn = _sffn()
    w = inp.workload
    d = device_inputs(inp)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, cap, dt)
    y = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    torch.cuda.synchronize()
    return ffn, y, d


def compare(inp: wl.Inputs, cap: int, rows=None, ffn=None, y=None) -> dict:
    w = inp.workload
    if ffn is None:
        ffn, y, _ = run_sparse(inp, cap)
    T = w.T
    n_r = int(ffn.n_routed.item())
    routed_gpu = ffn.routed[:n_r].cpu().numpy().astype(np.int64)
    count_all = ffn.count.cpu().numpy().astype(np.int64)
    # the routed list is the ascending set of rows with a tile over capacity
    # in the GPU's own counts (full-size consistency) ...
    assert np.array_equal(routed_gpu, np.nonzero(count_all.max(1) > cap)[0])
    if rows is None:
        rows = np.arange(T)
    ref = oracle_rows(inp, rows, w.tile, cap, dense=False)
    # ... and those counts match the oracle bit for bit on the compared rows
    check_twell(w.dtype, count_all[rows], ffn.idx.cpu().numpy()[rows],
                to_f64(ffn.val)[rows], ref, cap)
    routed_ref = rows[ref["routed"]]
    assert np.array_equal(np.intersect1d(routed_gpu, rows), routed_ref)
    if len(rows) == T:
        assert n_r == len(ref["routed"])
    mask = np.zeros(len(rows), dtype=bool)
    mask[ref["routed"]] = True
    mag = row_magnitude(inp, rows) if w.dtype == "f32" else None
    errs = check_y(w.dtype, to_f64(y[rows]), ref["y"], mask, mag)
    errs["n_routed"] = n_r
    print(f"{w.name}: rows {len(rows)}/{T} routed {n_r} rel_err {errs['all']:.3e} "
          f"max_row {errs['max_row']:.3e}")
    return errs


# ------------------------------------------------------------------ workloads
def test_tiny_f32_all_rows():
    inp = wl.generate(wl.WORKLOADS["tiny_f32"])
    e = compare(inp, 8)
    assert e["n_routed"] == 0


@pytest.mark.parametrize("beta", [1.9, 2.3])  # most rows routed; about one in eight
def test_bf16_ragged_tail_with_routing(beta):
    # 300 tokens: the routed-row mask with a ragged last word (300 = 18 x 16 + 12),
    # compacted inside the fallback's gate+up kernel
    inp = wl.generate_custom(T=300, d_model=512, d_ff=1024, dtype="bf16", beta=beta,
                             seed_base=11, cap=4)
    e = compare(inp, 4)
    assert 0 < e["n_routed"] < 300


def test_f32_ragged_tail_with_routing():
    inp = wl.generate_custom(T=200, d_model=264, d_ff=384, dtype="f32", beta=1.7,
                             seed_base=12, cap=3)
    e = compare(inp, 3)
    assert e["n_routed"] > 0


def test_f32_many_tokens_with_routing():
    # more than 256 tokens in float32: the routed-row mask, then the separate
    # compaction kernel (the float32 fallback has no fused scan); a ragged last
    # mask word (600 = 37 x 16 + 8)
    inp = wl.generate_custom(T=600, d_model=264, d_ff=384, dtype="f32", beta=2.3,
                             seed_base=13, cap=3)
    e = compare(inp, 3)
    assert 0 < e["n_routed"] < 600


def test_prefill_full_size_all_rows():
    w = wl.WORKLOADS["prefill_1pct"]
    inp = wl.generate(w)
    ffn, y, _ = run_sparse(inp, w.cap)
    compare(inp, w.cap, None, ffn, y)


def test_hybrid_mix_full_size_all_rows():
    w = wl.WORKLOADS["hybrid_mix"]
    inp = wl.generate(w)
    ffn, y, _ = run_sparse(inp, w.cap)
    n_r = int(ffn.n_routed.item())
    heavy = np.nonzero(inp.scales > 1)[0]
    routed = ffn.routed[:n_r].cpu().numpy()
    assert set(heavy.tolist()) <= set(routed.tolist())
    assert 60 <= n_r <= 260
    e = compare(inp, w.cap, None, ffn, y)
    assert "routed" in e and "not_routed" in e


def test_decode_all_rows():
    inp = wl.generate(wl.WORKLOADS["decode_1pct"])
    compare(inp, 8)


def test_large_lognormal_full_size():
    """Counts, live indices, values and the routed set on all 16384 rows
    (the oracle's gate in row chunks); y on 320 rows, 64 of them routed."""
    w = wl.WORKLOADS["large_lognormal"]
    inp = wl.generate(w)
    ffn, y, _ = run_sparse(inp, w.cap)
    n_r = int(ffn.n_routed.item())
    assert 0.08 * w.T < n_r < 0.3 * w.T
    routed = ffn.routed[:n_r].cpu().numpy().astype(np.int64)
    ref = oracle_twell_all_rows(inp, w.tile, w.cap)
    check_twell(w.dtype, ffn.count.cpu().numpy(), ffn.idx.cpu().numpy(), to_f64(ffn.val), ref,
                w.cap)
    assert np.array_equal(routed, ref["routed"])
    rows = sample_rows(w.T, 256, must=routed[::max(1, n_r // 64)], seed=3)
    compare(inp, w.cap, rows, ffn, y)


def test_gate_tile_mix_with_odd_tile_count():
    # 129 row tiles (the last ragged) x 3 TwELL tiles: the 256-row gate kernel
    # runs one column of 256-wide tiles and one column of 128-wide tiles
    inp = wl.generate_custom(T=33000, d_model=256, d_ff=384, dtype="bf16", beta=1.5,
                             seed_base=70, cap=8)
    ffn, y, _ = run_sparse(inp, 8)
    compare(inp, 8, None, ffn, y)


# ------------------------------------------------------------- dense reference
@pytest.mark.parametrize("name,T", [("tiny_f32", None), ("prefill_1pct", 512),
                                    ("decode_1pct", None)])
def test_dense_reference(name, T):
    sffn = _sffn()
    w = wl.WORKLOADS[name]
    if T is not None:
        w = w.replace(T=T)
    inp = wl.generate(w)
    d = device_inputs(inp)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dense = sffn.DenseFFN(w.T, w.d_model, w.d_ff, dt)
    y = to_f64(dense.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"]))
    rows = np.arange(w.T)
    ref = oracle_rows(inp, rows, w.tile, w.cap)
    check_y(w.dtype, y, ref["y_dense"], np.zeros(w.T, dtype=bool))


def test_dense_reference_prefill_full_size_sampled():
    # 4096 tokens: the dense gate+up runs its 256 x 128 (eight-wave) tiles
    sffn = _sffn()
    w = wl.WORKLOADS["prefill_1pct"]
    inp = wl.generate(w)
    d = device_inputs(inp)
    dense = sffn.DenseFFN(w.T, w.d_model, w.d_ff, torch.bfloat16)
    y = to_f64(dense.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"]))
    rows = sample_rows(w.T, 64, seed=6)
    ref = oracle_rows(inp, rows, w.tile, w.cap)
    check_y(w.dtype, y[rows], ref["y_dense"], np.zeros(len(rows), dtype=bool))


def test_dense_reference_large_full_size_sampled():
    # 16384 tokens, 4096 -> 14336: the dense down runs its 256 x 256 (eight-wave)
    # tiles with the K-major weight staged in 512-byte rows
    sffn = _sffn()
    w = wl.WORKLOADS["large_lognormal"]
    inp = wl.generate(w)
    d = device_inputs(inp)
    dense = sffn.DenseFFN(w.T, w.d_model, w.d_ff, torch.bfloat16)
    y = to_f64(dense.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"]))
    rows = sample_rows(w.T, 96, seed=8)
    ref = oracle_rows(inp, rows, w.tile, w.cap)
    check_y(w.dtype, y[rows], ref["y_dense"], np.zeros(len(rows), dtype=bool))


def test_dense_reference_wide_down_ragged():
    # 256 x 256 down tiles over ragged rows (16000 = 62.5 tiles) and a ragged
    # last column tile (2184 = 8 x 256 + 136, a partial 16-column fragment)
    sffn = _sffn()
    inp = wl.generate_custom(T=16000, d_model=2184, d_ff=1024, dtype="bf16", beta=1.0,
                             seed_base=80)
    w = inp.workload
    d = device_inputs(inp)
    dense = sffn.DenseFFN(w.T, w.d_model, w.d_ff, torch.bfloat16)
    y = to_f64(dense.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"]))
    rows = sample_rows(w.T, 64, must=np.arange(w.T - 130, w.T, 7), seed=9)
    ref = oracle_rows(inp, rows, w.tile, w.cap, dense=True)
    check_y(w.dtype, y[rows], ref["y_dense"], np.zeros(len(rows), dtype=bool))


@pytest.mark.parametrize("T,K,N", [(1, 256, 512), (7, 384, 1280), (32, 1024, 4096)])
def test_dense_reference_few_tokens(T, K, N):
    """Split-K dense kernels (few tokens), ragged row fragments included."""
    sffn = _sffn()
    inp = wl.generate_custom(T=T, d_model=K, d_ff=N, dtype="bf16", beta=1.0, seed_base=51)
    d = device_inputs(inp)
    dense = sffn.DenseFFN(T, K, N, torch.bfloat16)
    y1 = dense.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"]).clone()
    y2 = dense.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ref = oracle_rows(inp, np.arange(T), 128, 8)
    check_y("bf16", to_f64(y1), ref["y_dense"], np.zeros(T, dtype=bool))


# ------------------------------------------------------- few-token kernels
@pytest.mark.parametrize("T,K,N,beta,cap", [
    (48, 1056, 1024, 1.6, 8),   # split-K gate with 4 row fragments, K tail in a 512-column chunk
    (64, 2048, 2048, 2.0, 8),   # split-K gate, several splits per tile
    (17, 4096, 1408, 2.3, 8),   # ragged row fragment, long K
    (5, 2048, 8192, 2.0, 8),    # one workgroup per column tile, ragged rows
    (65, 512, 1024, 1.5, 8),    # streaming gate with 8 row fragments, one valid row in the last
    (96, 1088, 2048, 1.8, 8),   # 8 row fragments, K not a multiple of 128
    (128, 2048, 5632, 2.3, 8),  # most tokens of the streaming gate
    (100, 264, 640, 1.5, 4),    # two-pass sparse kernels with K % 32 != 0, routing
    (256, 512, 1024, 1.9, 8),   # largest token count of the two-pass kernels
    (256, 512, 1024, 1.2, 8),   # many routed rows, route scan inside the routed gate+up kernel
    (257, 512, 1024, 1.2, 8),   # one row more: separate route kernels
])
def test_few_token_paths(T, K, N, beta, cap):
    inp = wl.generate_custom(T=T, d_model=K, d_ff=N, dtype="bf16", beta=beta, seed_base=41)
    e = compare(inp, cap)
    if beta < 1.5:
        assert e["n_routed"] > 10


@pytest.mark.parametrize("T,K,N,beta,cap", [
    (300, 1024, 1024, 0.8, 32),  # windowed kernel at its largest capacity: up to 128 listed entries per window
    (300, 1024, 1024, 0.8, 40),  # capacity above 32: the per-token kernel instead of the windowed one
])
def test_many_token_capacity_bounds(T, K, N, beta, cap):
    inp = wl.generate_custom(T=T, d_model=K, d_ff=N, dtype="bf16", beta=beta, seed_base=43)
    e = compare(inp, cap)
    assert 0 < e["n_routed"] < T


# ---------------------------------------------------------------- edge cases
def _small(beta, dtype="bf16", T=64, seed=21):
    return wl.generate_custom(T=T, d_model=256, d_ff=512, dtype=dtype, beta=beta, seed_base=seed)


def test_single_token():
    compare(_small(1.5, T=1), 8)


def test_capacity_zero_routes_every_active_row():
    e = compare(_small(2.0), 0)
    assert e["n_routed"] > 0


def test_capacity_full_tile_routes_nothing():
    e = compare(_small(0.0), 128)
    assert e["n_routed"] == 0


def test_huge_bias_gives_exact_zeros():
    inp = _small(1e4)
    ffn, y, _ = run_sparse(inp, 8)
    assert int(ffn.count.to(torch.int32).sum().item()) == 0
    assert int(ffn.n_routed.item()) == 0
    assert torch.count_nonzero(y).item() == 0


def test_positive_bias_routes_every_row():
    inp = _small(-50.0, T=40)
    e = compare(inp, 8)
    assert e["n_routed"] == 40


def test_many_routed_rows_use_the_large_tile_fallback():
    inp = _small(-50.0, T=1200)
    e = compare(inp, 8)
    assert e["n_routed"] == 1200


def test_many_routed_rows_wide_tiles_ragged():
    # 8200 tokens (the eight-wave fallback kernels are launched from 8192 on)
    # and nearly every row routed: 256-row tiles with a ragged last row tile
    # (8200 = 32 x 256 + 8), a ragged last column tile of the down GEMM
    # (2080 = 8 x 256 + 32) and K splits of the down GEMM; y on 300 rows
    inp = wl.generate_custom(T=8200, d_model=2080, d_ff=1024, dtype="bf16", beta=1.0,
                             seed_base=90, cap=2)
    rows = sample_rows(8200, 300, must=np.arange(8190, 8200), seed=4)
    e = compare(inp, 2, rows)
    assert e["n_routed"] > 1024


def test_zero_tokens_is_a_noop():
    sffn = _sffn()
    s = sffn.make_shape(0, 256, 512, 8, sffn.SFFN_BF16)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((512, 256), dtype=torch.bfloat16, device="cuda")
    c, i, v = sffn.alloc_twell(sffn.make_shape(1, 256, 512, 8, sffn.SFFN_BF16))
    ws = sffn.alloc_workspace(sffn.make_shape(1, 256, 512, 8, sffn.SFFN_BF16), sffn.WS_PACK)
    sffn.twell_pack(s, x, w, None, c, i, v, ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["prefill_1pct", "tiny_f32"])
def test_precomputed_weight_norms_give_identical_twell(name):
    w = wl.WORKLOADS[name]
    if w.T > 512:
        w = w.replace(T=512)
    inp = wl.generate(w)
    ffn, y1, d = run_sparse(inp, w.cap)
    c1, i1 = ffn.count.clone(), ffn.idx.clone()
    y1 = y1.clone()
    norms = ffn.weight_norms(d["wg_t"])
    y2 = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"], norms)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), ffn.count.view(torch.int16))
    assert torch.equal(y1, y2)
    ref = np.linalg.norm(inp.as_f64("wg_t"), axis=1)
    assert np.allclose(norms.cpu().numpy(), ref, rtol=1e-4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_sign_near_zero(dtype):
    """Entries whose float32 sum is 0 or of the wrong sign are decided on the
    exact value (both the float64 stage and the exact fixed-point stage)."""
    T, K, N = 5, 64, 256
    inp = wl.generate_custom(T=T, d_model=K, d_ff=N, dtype=dtype, beta=2.0, seed_base=31)
    x = inp.as_f64("x")
    wg = inp.as_f64("wg_t")
    b = inp.b_g.copy()
    # row 0: z = 2^-59 (needs the exact stage), 2^-59 negative, exact zero,
    # 2^-40 (decided by the float64 stage)
    x[0, :] = 0.0
    x[0, :3] = [1.0, 2.0 ** -30, 2.0 ** -30]
    wg[:4, :] = 0.0
    wg[0, :3] = [1.0, 2.0 ** -30, 2.0 ** -30]
    wg[1, :3] = [1.0, -2.0 ** -30, -2.0 ** -30]
    wg[2, 0] = 1.0
    wg[3, :2] = [1.0, 2.0 ** -10]
    b[:4] = -1.0
    # row 1: same cancellations with a large lane spread
    x[1, :] = 0.0
    x[1, 0], x[1, 40] = 1.0, 2.0 ** -30
    wg[4, :] = 0.0
    wg[4, 0], wg[4, 40] = 1.0, 2.0 ** -31
    b[4] = -1.0
    store = (lambda a: wl.f32_to_bf16_bits(a.astype(np.float32))) if dtype == "bf16" \
        else (lambda a: a.astype(np.float32))
    inp.x, inp.wg_t, inp.b_g = store(x), store(wg), b.astype(np.float32)
    assert np.array_equal(inp.as_f64("x"), x) and np.array_equal(inp.as_f64("wg_t"), wg)
    ffn, y, _ = run_sparse(inp, 8)
    ref = oracle_rows(inp, np.arange(T), 128, 8)
    assert ref["z"][0, 0] == 2.0 ** -59 and ref["z"][0, 2] == 0.0 and ref["z"][1, 4] > 0
    assert ref["z"][0, 3] > 0
    compare(inp, 8, None, ffn, y)


def test_repeat_runs_are_bitwise_identical():
    w = wl.WORKLOADS["prefill_1pct"].replace(T=1024)
    inp = wl.generate(w)
    ffn, y1, d = run_sparse(inp, w.cap)
    c1, i1, v1 = ffn.count.clone(), ffn.idx.clone(), ffn.val.clone()
    y1 = y1.clone()
    y2 = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), ffn.count.view(torch.int16))
    live = torch.arange(w.cap, device="cuda")[None, None, :] < torch.clamp(
        c1.to(torch.int32), max=w.cap)[:, :, None]
    assert torch.equal(torch.where(live, i1.to(torch.int32), -1),
                       torch.where(live, ffn.idx.to(torch.int32), -1))
    assert torch.equal(torch.where(live, v1.float(), 0.0), torch.where(live, ffn.val.float(), 0.0))
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("name", ["hybrid_mix", "decode_1pct"])
def test_forward_graph_replay(name):
    """The three calls of a forward launch kernels only (no allocation, copy,
    memset or synchronisation), so a caller can capture them in a HIP graph:
    each replay, with eager forwards and synchronisations between replays,
    gives the eager result bit for bit (TwELL arrays, routed set, y)."""
    inp = wl.generate(wl.WORKLOADS[name])
    cap = inp.workload.cap
    ffn, y0, d = run_sparse(inp, cap)
    ref = {"y": y0.clone(), "count": ffn.count.clone(), "idx": ffn.idx.clone(),
           "val": ffn.val.clone(), "n": int(ffn.n_routed.item()), "routed": ffn.routed.clone()}
    live = torch.arange(cap, device="cuda")[None, None, :] < torch.clamp(
        ref["count"].to(torch.int32), max=cap)[:, :, None]
    args = (d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            ffn.forward(*args, stream=side)
    torch.cuda.synchronize()
    for _ in range(3):
        ffn.y.zero_()
        ffn.count.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ffn.y.view(torch.int16), ref["y"].view(torch.int16))
        assert torch.equal(ffn.count.view(torch.int16), ref["count"].view(torch.int16))
        assert torch.equal(torch.where(live, ffn.idx.to(torch.int32), -1),
                           torch.where(live, ref["idx"].to(torch.int32), -1))
        assert torch.equal(torch.where(live, ffn.val.float(), 0.0),
                           torch.where(live, ref["val"].float(), 0.0))
        n = int(ffn.n_routed.item())
        assert n == ref["n"]
        assert torch.equal(ffn.routed[:n], ref["routed"][:n])
        ffn.forward(*args)  # eager work between the replays
        torch.cuda.synchronize()


def test_decode_two_pass_repeats():
    """The few-token bf16 kernels (two passes through the workspace) give
    bitwise identical results on repeated calls."""
    inp = wl.generate(wl.WORKLOADS["decode_1pct"])
    ffn, y1, d = run_sparse(inp, 8)
    y1 = y1.clone()
    for _ in range(3):
        y2 = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_f32_split_tickets_repeat():
    """The float32 few-token path splits each row's tiles and reduces the
    partials through per-row tickets: repeated calls on one workspace give
    bitwise identical results that match the oracle."""
    sffn = _sffn()
    w = wl.WORKLOADS["tiny_f32"]
    assert sffn.workspace_bytes(sffn.make_shape(w.T, w.d_model, w.d_ff, w.cap, sffn.SFFN_F32),
                                sffn.WS_SPARSE) > 0  # the ticket path
    inp = wl.generate(w)
    ffn, y1, d = run_sparse(inp, w.cap)
    y1 = y1.clone()
    for _ in range(3):
        y2 = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
    compare(inp, w.cap, None, ffn, y2)


def test_shared_sparse_workspace_across_shapes():
    """One sparse_ffn_fwd workspace, filled with garbage first, serves calls of
    different shapes and kernel paths in turn (bf16 two-pass with 32 tokens,
    bf16 split tickets with 512, float32 tickets with 64, twice each): every
    call matches a call on a fresh workspace bit for bit and the oracle."""
    sffn = _sffn()
    cases = [wl.WORKLOADS["decode_1pct"].replace(d_ff=2048),
             wl.WORKLOADS["decode_1pct"].replace(T=512, d_ff=2048),
             wl.WORKLOADS["tiny_f32"]]
    shapes = [sffn.make_shape(w.T, w.d_model, w.d_ff, w.cap,
                              sffn.SFFN_BF16 if w.dtype == "bf16" else sffn.SFFN_F32)
              for w in cases]
    n = max(sffn.workspace_bytes(s, sffn.WS_SPARSE) for s in shapes)
    shared = torch.randint(0, 256, (max(n, 16),), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for w, s in zip(cases, shapes):
            inp = wl.generate(w)
            d = device_inputs(inp)
            dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
            ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, w.cap, dt)
            ref_y = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"]).clone()
            y = torch.empty_like(ref_y)
            sffn.sparse_ffn_fwd(s, d["x"], d["wu_t"], d["wd"], ffn.count, ffn.idx, ffn.val, y,
                                shared)
            sffn.hybrid_route(s, d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"], ffn.count,
                              ffn.routed, ffn.n_routed, ffn.ws_hybrid, y)
            torch.cuda.synchronize()
            assert torch.equal(y, ref_y), (rep, w.name, w.T)
            if rep == 0:
                compare(inp, w.cap, None, ffn, y)
