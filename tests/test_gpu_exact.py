"""GPU results that must be exact, and the error model of the exact-sign
guard band.

* Integer fixture: x and the weights in {-1, 0, 1}, gate bias -(m + 1/2).
  Every pre-activation is a half-integer and every product and partial sum of
  the forward is a small dyadic rational that float32 (and, for the one-hot
  variant, bfloat16) holds exactly, whatever the summation order.  So the HIP
  path must reproduce the oracle's y BIT FOR BIT, together with the TwELL
  arrays (values included) and the routed set, on every kernel path the token
  count selects (few-token split-K gate, two-pass sparse kernels, split
  tickets, windowed kernel, dense fallback).  Each case first checks on the
  oracle's values that its premise holds (every intermediate representable).

* MFMA rounding: twell_pack decides activity on the exact sign of z.  Entries
  whose float32 accumulation lies within a guard band
  |z32| <= c_xw ||x_t|| ||w_j|| + c_b |b_j| are re-evaluated exactly, with
  c_xw = 2^-22 (K/32 + 2) for bf16 (K/32 chained 16x16x32 MFMAs) and
  2^-22 (K + 2) for float32 (one FMA per k), c_b = 2^-22.  The bf16 band
  rests on an error model of one v_mfma_f32_16x16x32_bf16 on this hardware,
  measured here with sffn_probe_mfma_step on adversarial operands (wide
  exponent ranges, cancellation, many tiny products beside a large one,
  products just below the truncation step, a large accumulator) against
  exact rational arithmetic:
      |D - (C + sum_k a_k b_k)| <= u (8 max_k |a_k b_k| + 2 |C + sum_k a_k b_k|)
  with u = 2^-24: the 32 products are aligned to the largest one and
  truncated a little below float32 precision (the measured loss of 31 tiny
  products beside a product of 1 is 6.5 u, so the instruction does NOT round
  only once), then added to the accumulator with one rounding.  Over a chain
  of K/32 instructions the truncation terms add up to at most
  8 u sum_k |x_k w_k| <= 8 u ||x|| ||w|| (each product belongs to one step)
  and the roundings to (K/32) 2 u ||x|| ||w||; with the bias add this stays
  below the band for every K >= 32.

* The band at full size: gate_preact stores the same float32 accumulation as
  twell_pack (more than 64 tokens); max |z32 - z| / band over every entry of
  the prefill and large workloads is printed and must be below 1.  A
  cancellation fixture (x = [v, v], half of the gate columns [a, -a] with one
  coordinate nudged by one bf16 step, so the large partial sums cancel exactly
  and every z of those columns is tiny) drives thousands of entries into the
  band: TwELL must still match the oracle bit for bit.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from activation_sparse_feed_amd import workloads as wl
from helpers import check_twell, device_inputs, oracle_rows, to_f64

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _sffn():
    from activation_sparse_feed_amd import sffn
    return sffn


def _bf16_exact(a: np.ndarray) -> bool:
    a32 = a.astype(np.float32)
    return bool(np.all(a32.astype(np.float64) == a)) and \
        bool(np.all(wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(a32)) == a32))


# ------------------------------------------------------------ integer fixture
INTEGER_CASES = [
    # dtype, T, variant, density, m, cap: kernel paths the token count selects
    ("f32", 64, "dense", 2 / 3, 15, 16),     # float32 gate, split tickets
    ("f32", 300, "dense", 2 / 3, 15, 16),    # float32, more rows than one split pass
    ("bf16", 48, "one_hot", 0.25, 7, 8),     # split-K gate (<= 64 tokens), two-pass sparse
    ("bf16", 200, "one_hot", 0.25, 7, 8),    # 256-row gate, two-pass sparse
    ("bf16", 600, "one_hot", 0.25, 7, 8),    # bf16 split tickets
    ("bf16", 2100, "one_hot", 0.25, 6, 12),  # windowed sparse kernel, routed fallback
]


@pytest.mark.parametrize("dt,T,variant,density,m,cap", INTEGER_CASES)
def test_integer_fixture_bitwise(dt, T, variant, density, m, cap):
    sffn = _sffn()
    K, N = 256, 1024
    inp = wl.generate_integer(T, K, N, dt, seed=17 + T, m=m, variant=variant, density=density)
    x, wg, wu, wd = (inp.as_f64(n) for n in ("x", "wg_t", "wu_t", "wd"))
    ref = oracle.sparse_forward(x, wg, inp.b_g, wu, wd, 128, cap)
    z, y_ref = ref["z"], ref["y"]
    act = z > 0
    u = oracle.up_proj(x, wu)
    h_dense = np.where(act, z, 0.0) * u
    # premise: every intermediate exact in the arithmetic under test
    assert np.all(np.abs(2 * z) % 2 == 1), "pre-activations are half-integers"
    assert 0 < len(ref["routed"]) < T, "the fixture exercises both paths"
    assert np.array_equal(oracle.ffn_dense(x, wg, inp.b_g, wu, wd), y_ref)
    if dt == "bf16":
        for name, a in (("z", z[act]), ("u", u), ("h", h_dense), ("y", y_ref)):
            assert _bf16_exact(a), f"{name} not exact in bf16"
    else:
        # every partial sum of the down projection (any order) below 2^22
        assert (np.abs(h_dense) @ np.abs(wd)).max() < 2 ** 22
        assert np.abs(x).sum(1).max() * 1.0 < 2 ** 22 and np.abs(h_dense).max() < 2 ** 22

    d = device_inputs(inp)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    ffn = sffn.SparseFFN(T, K, N, cap, dtype)
    y = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    dense = sffn.DenseFFN(T, K, N, dtype)
    yd = dense.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    torch.cuda.synchronize()

    count = ffn.count.cpu().numpy().astype(np.int64)
    assert np.array_equal(count, ref["count"])
    n_r = int(ffn.n_routed.item())
    assert np.array_equal(ffn.routed[:n_r].cpu().numpy(), ref["routed"])
    live = np.arange(cap)[None, None, :] < np.minimum(ref["count"], cap)[:, :, None]
    idx = ffn.idx.cpu().numpy().astype(np.int64)
    val = to_f64(ffn.val)
    assert np.array_equal(np.where(live, idx, -1), np.where(live, ref["idx"], -1))
    assert np.array_equal(np.where(live, val, 0.0), np.where(live, ref["val"], 0.0)), "values"
    yg = to_f64(y)
    bad = np.argwhere(yg != y_ref)
    assert len(bad) == 0, f"{len(bad)} y entries differ, first {bad[:4]}"
    assert np.array_equal(to_f64(yd), y_ref), "dense reference"
    print(f"integer {dt} T={T}: routed {n_r}, nnz {int(act.sum())}, bitwise equal")


# --------------------------------------------------------- MFMA rounding model
def _bf16_values(rng, shape, emin, emax):
    """Random bf16 values: 8-bit significands, exponents in [emin, emax],
    random signs (exact float32)."""
    mant = rng.integers(128, 256, size=shape).astype(np.float64) / 128.0
    e = rng.integers(emin, emax + 1, size=shape)
    s = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    return (s * mant * np.exp2(e)).astype(np.float32)


def _case(rng, kind):
    """A: [16, 32], B: [32, 16] (bf16 values as float32), C: [16, 16] float32."""
    if kind == "layout":
        A = rng.integers(-8, 9, size=(16, 32)).astype(np.float32)
        B = rng.integers(-8, 9, size=(32, 16)).astype(np.float32)
        C = rng.integers(-100, 101, size=(16, 16)).astype(np.float32)
    elif kind == "wide":
        A = _bf16_values(rng, (16, 32), -20, 20)
        B = _bf16_values(rng, (32, 16), -20, 20)
        C = (_bf16_values(rng, (16, 16), -20, 20) * np.float32(1 + 2 ** -20)).astype(np.float32)
    elif kind == "cancel":
        # products in +/- pairs of equal size plus one small term: large
        # partial sums, small exact result
        A = _bf16_values(rng, (16, 32), -4, 4)
        B = _bf16_values(rng, (32, 16), -4, 4)
        A[:, 16:] = A[:, :16]
        B[16:, :] = -B[:16, :]
        B[31, :] = _bf16_values(rng, (16,), -30, -20)
        C = np.zeros((16, 16), dtype=np.float32)
    elif kind == "tiny_beside_large":
        # one product of 1, 31 products just below half an ulp of it
        A = np.zeros((16, 32), dtype=np.float32)
        B = np.zeros((32, 16), dtype=np.float32)
        A[:, 0] = 1.0
        B[0, :] = 1.0
        A[:, 1:] = np.float32(2.0 ** -13) * rng.choice([1.0, 1.5, 1.75], size=(16, 31)).astype(np.float32)
        B[1:, :] = np.float32(2.0 ** -12)
        C = np.zeros((16, 16), dtype=np.float32)
    elif kind == "below_step":
        # a product of 1 and 31 products just below 2^-25 (largest bf16
        # significand): lost entirely if truncated at 2^-25 below the leader
        A = np.zeros((16, 32), dtype=np.float32)
        B = np.zeros((32, 16), dtype=np.float32)
        A[:, 31] = 1.0
        B[31, :] = 1.0
        A[:, :31] = np.float32(255.0 / 128.0 * 2.0 ** -13)
        B[:31, :] = np.float32(2.0 ** -13) * rng.choice([1.0, 0.5, 0.25], size=(31, 16)).astype(np.float32)
        C = np.zeros((16, 16), dtype=np.float32)
    elif kind == "large_acc":
        # accumulator 2^24 and products of 0.75: each alone is below half an
        # ulp of the accumulator, their sum is not
        A = np.full((16, 32), 0.75, dtype=np.float32)
        B = np.ones((32, 16), dtype=np.float32)
        C = np.full((16, 16), 2.0 ** 24, dtype=np.float32) * rng.choice([1.0, -1.0], size=(16, 16)).astype(np.float32)
    else:
        raise ValueError(kind)
    return A, B, C


def _to_lanes(A, B, C):
    """The instruction's lane layout: lane l holds A[l % 16, 8 (l // 16) + e],
    B[8 (l // 16) + e, l % 16] (e < 8) and accumulator rows 4 (l // 16) + i of
    column l % 16 (i < 4)."""
    lanes = np.arange(64)
    r, g = lanes % 16, lanes // 16
    e = np.arange(8)
    a = A[r[:, None], 8 * g[:, None] + e[None, :]]
    b = B[8 * g[:, None] + e[None, :], r[:, None]]
    i = np.arange(4)
    c = C[4 * g[:, None] + i[None, :], r[:, None]]
    return a, b, c


def _from_lanes(d):
    D = np.zeros((16, 16), dtype=np.float64)
    lanes = np.arange(64)
    r, g = lanes % 16, lanes // 16
    for i in range(4):
        D[4 * g + i, r] = d[:, i]
    return D


def test_mfma_step_error_model():
    sffn = _sffn()
    rng = np.random.default_rng(123)
    kinds = ["layout"] * 2 + ["wide"] * 6 + ["cancel"] * 4 + ["tiny_beside_large"] * 2 + \
        ["below_step"] * 2 + ["large_acc"] * 2
    cases = [_case(rng, k) for k in kinds]
    W = len(cases)
    a = np.zeros((W, 64, 8), dtype=np.uint16)
    b = np.zeros((W, 64, 8), dtype=np.uint16)
    c = np.zeros((W, 64, 4), dtype=np.float32)
    for w, (A, B, C) in enumerate(cases):
        la, lb, lc = _to_lanes(A, B, C)
        a[w], b[w], c[w] = wl.f32_to_bf16_bits(la), wl.f32_to_bf16_bits(lb), lc
        assert np.array_equal(wl.bf16_bits_to_f32(a[w]), la) and \
            np.array_equal(wl.bf16_bits_to_f32(b[w]), lb), "operands are bf16 values"
    dev = lambda t: torch.from_numpy(t).cuda()  # noqa: E731
    d = torch.zeros((W, 64, 4), dtype=torch.float32, device="cuda")
    sffn.probe_mfma_step(dev(a.view(np.int16)), dev(b.view(np.int16)), dev(c), d)
    torch.cuda.synchronize()
    d = d.cpu().numpy()
    worst, worst_mag = {}, {}
    for w, ((A, B, C), kind) in enumerate(zip(cases, kinds)):
        D = _from_lanes(d[w])
        for i in range(16):
            for j in range(16):
                terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(32)]
                exact = Fraction(float(C[i, j])) + sum(terms)
                mag = abs(Fraction(float(C[i, j]))) + sum(abs(t) for t in terms)
                err = abs(Fraction(float(D[i, j])) - exact)
                if kind == "layout":
                    assert err == 0, f"layout case: D[{i},{j}] = {D[i, j]}, exact {float(exact)}"
                    continue
                model = Fraction(U) * (8 * max(abs(t) for t in terms) + 2 * abs(exact))
                ratio = float(err / model) if model else float(err > 0)
                worst[kind] = max(worst.get(kind, 0.0), ratio)
                r2 = float(err / (Fraction(U) * mag)) if mag else float(err > 0)
                worst_mag[kind] = max(worst_mag.get(kind, 0.0), r2)
    print("MFMA error / (u (8 max|a b| + 2 |exact|)), worst per case kind:",
          {k: round(v, 3) for k, v in worst.items()})
    print("MFMA error / (u (|C| + sum |a b|)), worst per case kind:",
          {k: round(v, 3) for k, v in worst_mag.items()})
    assert max(worst.values()) <= 1.0, worst
    # the truncation is real: a single rounding would leave at most u |exact|
    assert worst_mag["tiny_beside_large"] > 1.0


# ------------------------------------------------------ the band at full size
def guard_band(dt: str, K: int, xnorm, wnorm, b):
    c_xw = 2.0 ** -22 * (K / 32 + 2) if dt == "bf16" else 2.0 ** -22 * (K + 2)
    return c_xw * np.outer(xnorm, wnorm) + 2.0 ** -22 * np.abs(b)[None, :]


@pytest.mark.parametrize("name", ["prefill_1pct", "large_lognormal"])
def test_guard_band_margin_full_size(name):
    """max |z32 - z| / band over every entry, z32 being twell_pack's own
    float32 accumulation (gate_preact, same kernel main loop)."""
    sffn = _sffn()
    w = wl.WORKLOADS[name]
    inp = wl.generate(w)
    d = device_inputs(inp)
    shape = sffn.make_shape(w.T, w.d_model, w.d_ff, w.cap, sffn.SFFN_BF16)
    z32 = torch.empty((w.T, w.d_ff), dtype=torch.float32, device="cuda")
    sffn.gate_preact(shape, d["x"], d["wg_t"], d["b_g"], z32)
    torch.cuda.synchronize()
    wg = inp.as_f64("wg_t")
    wnorm = np.linalg.norm(wg, axis=1)
    worst, inside = 0.0, 0
    chunk = 1024
    for r0 in range(0, w.T, chunk):
        rows = np.arange(r0, min(w.T, r0 + chunk))
        x = inp.rows_f64("x", rows)
        z = oracle.gate_preact(x, wg, inp.b_g)
        band = guard_band("bf16", w.d_model, np.linalg.norm(x, axis=1), wnorm, inp.b_g)
        zg = z32[r0:r0 + len(rows)].cpu().numpy().astype(np.float64)
        worst = max(worst, float((np.abs(zg - z) / band).max()))
        inside += int((np.abs(zg) <= band).sum())
    print(f"{name}: max |z32 - z| / band = {worst:.4f}; entries re-evaluated exactly: {inside}")
    assert worst < 1.0


def cancellation_fixture(T=256, K=2048, N=1024, seed=5):
    """x_t = [v_t, v_t]; gate column j even: [a_j, -a_j] with one coordinate of
    the first half moved by one bf16 step, bias -1.645 times that step (about
    5% active), so every z of the column is tiny while its partial sums reach
    ||x|| ||w|| / 2; odd columns ordinary N(0, 1/K) with bias -2.326."""
    rng = np.random.default_rng(seed)
    half = K // 2
    v = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(rng.standard_normal((T, half)).astype(np.float32)))
    x = np.concatenate([v, v], axis=1)
    wg = np.zeros((N, K), dtype=np.float32)
    b = np.full(N, -2.326, dtype=np.float32)
    for j in range(N):
        if j % 2:
            wg[j] = rng.standard_normal(K).astype(np.float32) / np.sqrt(K)
            continue
        a = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(
            (rng.standard_normal(half) / 32.0).astype(np.float32)))
        row = np.concatenate([a, -a])
        k0 = int(rng.integers(0, half))
        bits = wl.f32_to_bf16_bits(row[k0:k0 + 1].astype(np.float32))
        nudged = wl.bf16_bits_to_f32(bits + np.uint16(1))[0]  # next bf16 away from zero
        step = float(nudged) - float(row[k0])
        row[k0] = nudged
        wg[j] = row
        b[j] = np.float32(-1.645 * abs(step))
    wu = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    wd = (rng.standard_normal((N, K)) / np.sqrt(N)).astype(np.float32)
    st = wl.f32_to_bf16_bits
    w = wl.Workload("cancellation", T=T, d_model=K, d_ff=N, dtype="bf16", beta=2.326, cap=8)
    return wl.Inputs(w, st(x), st(wg), st(wu), st(wd), b, np.ones(T, dtype=np.float32))


def test_cancellation_fixture_exact_twell():
    sffn = _sffn()
    inp = cancellation_fixture()
    w = inp.workload
    d = device_inputs(inp)
    ffn = sffn.SparseFFN(w.T, w.d_model, w.d_ff, w.cap, torch.bfloat16)
    y = ffn.forward(d["x"], d["wg_t"], d["b_g"], d["wu_t"], d["wd"])
    z32 = torch.empty((w.T, w.d_ff), dtype=torch.float32, device="cuda")
    sffn.gate_preact(ffn.shape, d["x"], d["wg_t"], d["b_g"], z32)
    torch.cuda.synchronize()
    rows = np.arange(w.T)
    ref = oracle_rows(inp, rows, w.tile, w.cap, dense=False)
    band = guard_band("bf16", w.d_model, ref["xnorm"], ref["wnorm"], inp.b_g)
    zg = z32.cpu().numpy().astype(np.float64)
    inside = np.abs(zg) <= band
    ratio = float((np.abs(zg - ref["z"]) / band).max())
    even = np.zeros(w.d_ff, dtype=bool)
    even[::2] = True
    print(f"cancellation: entries in the band {int(inside.sum())} "
          f"(of {int(inside[:, even].size)} in cancelling columns), "
          f"max |z32 - z| / band = {ratio:.4f}, "
          f"active {int((ref['z'] > 0).sum())}, routed {len(ref['routed'])}")
    assert inside[:, even].mean() > 0.95, "the cancelling columns sit inside the band"
    assert ratio < 1.0
    check_twell("bf16", ffn.count.cpu().numpy(), ffn.idx.cpu().numpy(), to_f64(ffn.val), ref,
                w.cap)
    n_r = int(ffn.n_routed.item())
    assert np.array_equal(ffn.routed[:n_r].cpu().numpy(), ref["routed"])
    # rows within capacity: y from the exactly decided TwELL entries
    keep = np.ones(w.T, dtype=bool)
    keep[ref["routed"]] = False
    from helpers import check_y
    check_y("bf16", to_f64(y)[keep], ref["y"][keep], np.zeros(int(keep.sum()), dtype=bool))
