"""Pins of the CPU oracle against facts that do not come from the oracle itself.

  * exact rational brute force (pure-Python loops over Fractions) on tiny
    shapes, including partial tiles, overflow, routing and exact zeros;
  * an integer fixture at moderate size whose exact answer comes from integer
    matrix products;
  * the closed-form activation density given the row and weight norms;
  * symmetry (x and -x with zero bias) and the special cases of the capacity
    rule;
  * planted mistakes in the oracle that these pins must catch.
"""
from __future__ import annotations

import math
from fractions import Fraction as Fr

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import ffn as offn
from activation_sparse_feed_amd import workloads as wl


# ---------------------------------------------------------------- brute force
def brute_force(x, wg, b, wu, wd, tile, cap):
    """Exact rational evaluation with nested loops (no numpy arithmetic)."""
    T, K = len(x), len(x[0])
    d_ff, dm = len(wg), len(wd[0])
    X = [[Fr(float(v)) for v in row] for row in x]
    G = [[Fr(float(v)) for v in row] for row in wg]
    U_ = [[Fr(float(v)) for v in row] for row in wu]
    D = [[Fr(float(v)) for v in row] for row in wd]
    B = [Fr(float(v)) for v in b]
    z = [[B[j] + sum(X[t][k] * G[j][k] for k in range(K)) for j in range(d_ff)]
         for t in range(T)]
    nt = -(-d_ff // tile)
    count = [[0] * nt for _ in range(T)]
    lists = [[[] for _ in range(nt)] for _ in range(T)]
    for t in range(T):
        for kt in range(nt):
            for j in range(kt * tile, min((kt + 1) * tile, d_ff)):
                if z[t][j] > 0:
                    count[t][kt] += 1
                    lists[t][kt].append(j)
    row_lists = [[j for j in range(d_ff) if z[t][j] > 0] for t in range(T)]
    routed = [t for t in range(T) if any(c > cap for c in count[t])]
    u = [[sum(X[t][k] * U_[j][k] for k in range(K)) for j in range(d_ff)] for t in range(T)]
    y = [[sum((z[t][j] if z[t][j] > 0 else 0) * u[t][j] * D[j][c] for j in range(d_ff))
          for c in range(dm)] for t in range(T)]
    return {"z": z, "count": count, "lists": lists, "row_lists": row_lists, "routed": routed,
            "y": y}


def _bf16(a):
    return wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


def tiny_cases():
    """Tiny inputs: random bf16-valued data plus crafted exact-zero and
    cancellation entries."""
    cases = []
    rng = np.random.default_rng(12345)
    shapes = [(3, 6, 8, 4, 2), (2, 5, 10, 4, 1), (4, 4, 12, 4, 3), (3, 6, 8, 4, 0),
              (1, 3, 9, 4, 4), (4, 6, 8, 8, 2)]
    for (T, K, d_ff, tile, cap) in shapes:
        x = _bf16(rng.standard_normal((T, K)))
        wg = _bf16(rng.standard_normal((d_ff, K)) / math.sqrt(K))
        wu = _bf16(rng.standard_normal((d_ff, K)) / math.sqrt(K))
        wd = _bf16(rng.standard_normal((d_ff, 5)) / math.sqrt(d_ff))
        b = _bf16(rng.standard_normal(d_ff) * 0.5)
        # crafted entries in row 0: an exact zero and two cancellations that
        # float64 sums in natural order get wrong
        x[0, :3] = [1.0, 2.0 ** -30, 2.0 ** -30]
        wg[0, :3] = [1.0, 2.0 ** -30, 2.0 ** -30]
        wg[0, 3:] = 0.0
        b[0] = -1.0            # z[0,0] = 2^-59 > 0 exactly; naive float64 gives 0
        wg[1, :3] = [1.0, -2.0 ** -30, -2.0 ** -30]
        wg[1, 3:] = 0.0
        b[1] = -1.0            # z[0,1] = -2^-59 - (x terms) ... negative
        wg[2, :] = 0.0
        wg[2, 0] = 1.0
        b[2] = -1.0            # z[0,2] = 0 exactly: inactive
        cases.append((x, wg, b, wu, wd, tile, cap))
    return cases


def check_against_brute(x, wg, b, wu, wd, tile, cap):
    ref = brute_force(x, wg, b, wu, wd, tile, cap)
    out = oracle.sparse_forward(x, wg, b, wu, wd, tile, cap)
    T, d_ff = len(x), len(wg)
    # gate sign exact; value within a few float64 ulps of the exact value
    for t in range(T):
        for j in range(d_ff):
            ze = ref["z"][t][j]
            assert (out["z"][t, j] > 0) == (ze > 0), (t, j)
            assert abs(Fr(float(out["z"][t, j])) - ze) <= Fr(2.0 ** -50) * (abs(ze) + 1)
    # TwELL: counts exact, live slots exact and ascending, values equal h
    cnt = out["count"]
    assert cnt.shape == (T, -(-d_ff // tile))
    for t in range(T):
        for kt in range(cnt.shape[1]):
            assert cnt[t, kt] == ref["count"][t][kt]
            live = ref["lists"][t][kt][:cap]
            assert list(out["idx"][t, kt, :len(live)]) == live
            for s, j in enumerate(live):
                assert out["val"][t, kt, s] == out["z"][t, j]
    assert list(out["routed"]) == ref["routed"]
    # unpack reproduces ReLU(z) on every row that is not routed
    H = oracle.twell_unpack(out["count"], out["idx"], out["val"], d_ff)
    Hr = oracle.relu(out["z"])
    keep = np.setdiff1d(np.arange(T), out["routed"])
    assert np.array_equal(H[keep], Hr[keep])
    # row-wise ELLPACK: row counts, ascending live columns, values equal h;
    # the widest row fixes the classic width, which makes it lossless
    longest = max(len(r) for r in ref["row_lists"])
    for width in sorted({0, 1, 3, longest, longest + 2}):
        ec, ei, ev = oracle.ell_pack(out["z"], width)
        assert ei.shape == (T, width)
        for t in range(T):
            assert ec[t] == len(ref["row_lists"][t])
            live = ref["row_lists"][t][:width]
            assert list(ei[t, :len(live)]) == live
            assert all(v == -1 for v in ei[t, len(live):])
            for s, j in enumerate(live):
                assert ev[t, s] == out["z"][t, j]
        if width >= longest:
            assert np.array_equal(oracle.ell_unpack(ec, ei, ev, d_ff), oracle.relu(out["z"]))
    # L1 regulariser: lam / T times the exact sum of the positive z
    for lam in (1.0, 0.25):
        exact = Fr(lam) * sum((v for row in ref["z"] for v in row if v > 0), Fr(0)) / T
        got = oracle.l1_term(out["z"], lam)
        assert abs(Fr(got) - exact) <= Fr(2.0 ** -50) * (abs(exact) + 1)
    # dense and sparse y against the exact result
    yex = np.array([[float(v) for v in row] for row in ref["y"]])
    scale = max(1e-300, float(np.abs(yex).max()))
    yd = oracle.ffn_dense(x, wg, b, wu, wd)
    assert np.abs(yd - yex).max() <= 1e-12 * scale
    assert np.abs(out["y"] - yex).max() <= 1e-12 * scale


@pytest.mark.parametrize("case", range(len(tiny_cases())))
def test_brute_force_tiny(case):
    check_against_brute(*tiny_cases()[case])


def test_crafted_signs():
    x, wg, b, wu, wd, tile, cap = tiny_cases()[0]
    z = oracle.gate_preact(x, wg, b)
    assert z[0, 0] == 2.0 ** -59      # exact, although 1 + 2^-60 rounds to 1
    assert z[0, 1] < 0
    assert z[0, 2] == 0.0 and oracle.relu(z)[0, 2] == 0.0


# -------------------------------------------------------- integer fixture
def test_integer_fixture_exact():
    """x, W in {-1, 0, 1} and a half-integer bias: every quantity is a small
    dyadic rational, so the oracle must agree exactly with integer products."""
    rng = np.random.default_rng(7)
    T, K, d_ff, dm, tile = 24, 64, 256, 48, 128
    X = rng.integers(-1, 2, size=(T, K))
    Wg = rng.integers(-1, 2, size=(d_ff, K))
    Wu = rng.integers(-1, 2, size=(d_ff, K))
    Wd = rng.integers(-1, 2, size=(d_ff, dm))
    m = 7
    b = np.full(d_ff, -(m + 0.5))
    z2 = 2 * (X @ Wg.T) - (2 * m + 1)           # 2 z, integer, odd
    act = z2 > 0
    Uint = X @ Wu.T
    y2 = (np.where(act, z2, 0) * Uint) @ Wd      # 2 y, integer
    for cap in (0, 4, 8, 128):
        out = oracle.sparse_forward(X.astype(float), Wg.astype(float), b,
                                    Wu.astype(float), Wd.astype(float), tile, cap)
        assert np.array_equal(out["z"] * 2, z2)
        cnt = np.stack([act[:, k * tile:(k + 1) * tile].sum(1) for k in range(2)], 1)
        assert np.array_equal(out["count"], cnt)
        assert np.array_equal(out["routed"], np.nonzero(cnt.max(1) > cap)[0])
        assert np.array_equal(out["y"] * 2, y2)
        assert np.array_equal(oracle.ffn_dense(X, Wg, b, Wu, Wd) * 2, y2)
    assert 0 < len(oracle.route(out["count"], 8)) < T   # the fixture does exercise routing


# ---------------------------------------------------------- density closed form
def _p_active(xn, wn, beta, d):
    """P(x.w > beta) for fixed norms and independent uniform directions:
    cos^2 of the angle is Beta(1/2, (d-1)/2)."""
    a = beta / np.outer(xn, wn)
    a = np.clip(a, 0.0, None)
    inside = a < 1.0
    p = np.zeros_like(a)
    p[inside] = 0.5 * (1.0 - scipy.special.betainc(0.5, (d - 1) / 2.0, a[inside] ** 2))
    return p


@pytest.mark.parametrize("name,rows", [("tiny_f32", None), ("prefill_1pct", 96),
                                       ("hybrid_mix", 128)])
def test_density_closed_form(name, rows):
    w = wl.WORKLOADS[name]
    inp = wl.generate(w)
    sel = np.arange(w.T) if rows is None else np.linspace(0, w.T - 1, rows).astype(int)
    if name == "hybrid_mix":   # make sure the heavy rows are in the sample
        sel = np.union1d(sel, np.nonzero(inp.scales > 1)[0])
    x = inp.rows_f64("x", sel)
    wg = inp.as_f64("wg_t")
    z = oracle.gate_preact(x, wg, inp.b_g)
    count, _, _ = oracle.twell_pack(z, w.tile, w.cap)
    p = _p_active(np.linalg.norm(x, axis=1), np.linalg.norm(wg, axis=1), w.beta, w.d_model)
    mean, sd = p.sum(), math.sqrt((p * (1 - p)).sum())
    obs = count.sum()
    assert abs(obs - mean) <= 5 * sd + 0.005 * mean, (obs, mean, sd)
    # per-row counts follow the per-row expectation (heavy rows included)
    per_row = p.sum(1)
    assert np.corrcoef(count.sum(1), per_row)[0, 1] > (0.95 if name == "hybrid_mix" else 0.3)


def test_unit_rows_density_matches_gaussian_tail():
    """With unit row scale, the mean density is close to 1 - Phi(beta)."""
    w = wl.WORKLOADS["prefill_1pct"]
    inp = wl.generate(w)
    sel = np.arange(0, w.T, 32)
    z = oracle.gate_preact(inp.rows_f64("x", sel), inp.as_f64("wg_t"), inp.b_g)
    dens = (z > 0).mean()
    q = 0.5 * math.erfc(w.beta / math.sqrt(2))
    assert abs(dens / q - 1) < 0.05, (dens, q)


# --------------------------------------------------------- symmetry, special cases
def test_symmetry_zero_bias():
    """With b = 0, z(-x) = -z(x): across a row pair every column is active in
    exactly one of the two rows unless z is exactly zero."""
    inp = wl.generate_custom(T=16, d_model=128, d_ff=512, dtype="bf16", beta=0.0, seed_base=77)
    x = inp.as_f64("x")
    x2 = np.concatenate([x, -x])
    z = oracle.gate_preact(x2, inp.as_f64("wg_t"), np.zeros(512, np.float32))
    count, _, _ = oracle.twell_pack(z, 128, 128)
    zeros = (z[:16] == 0).sum(1)
    assert np.array_equal(count[:16].sum(1) + count[16:].sum(1), 512 - zeros)


def _small_inputs(beta, dtype="bf16", seed=5):
    return wl.generate_custom(T=12, d_model=64, d_ff=384, dtype=dtype, beta=beta, seed_base=seed)


def test_capacity_full_tile_routes_nothing():
    inp = _small_inputs(0.0)
    out = oracle.sparse_forward(inp.as_f64("x"), inp.as_f64("wg_t"), inp.b_g,
                                inp.as_f64("wu_t"), inp.as_f64("wd"), 128, 128)
    assert len(out["routed"]) == 0
    yd = oracle.ffn_dense(inp.as_f64("x"), inp.as_f64("wg_t"), inp.b_g,
                          inp.as_f64("wu_t"), inp.as_f64("wd"))
    assert np.allclose(out["y"], yd, rtol=1e-12, atol=1e-12 * np.abs(yd).max())


def test_capacity_zero_routes_every_active_row():
    inp = _small_inputs(2.0)
    x, wg, wu, wd = (inp.as_f64(n) for n in ("x", "wg_t", "wu_t", "wd"))
    out = oracle.sparse_forward(x, wg, inp.b_g, wu, wd, 128, 0)
    z = oracle.gate_preact(x, wg, inp.b_g)
    assert np.array_equal(out["routed"], np.nonzero((z > 0).any(1))[0])
    assert np.array_equal(out["y"][out["routed"]],
                          oracle.ffn_dense(x[out["routed"]], wg, inp.b_g, wu, wd))


def test_huge_bias_gives_zero_output():
    inp = _small_inputs(1e6)
    out = oracle.sparse_forward(inp.as_f64("x"), inp.as_f64("wg_t"), inp.b_g,
                                inp.as_f64("wu_t"), inp.as_f64("wd"), 128, 8)
    assert out["count"].sum() == 0 and len(out["routed"]) == 0
    assert np.array_equal(out["y"], np.zeros_like(out["y"]))


def test_large_positive_bias_routes_every_row():
    inp = _small_inputs(-1e3)
    out = oracle.sparse_forward(inp.as_f64("x"), inp.as_f64("wg_t"), inp.b_g,
                                inp.as_f64("wu_t"), inp.as_f64("wd"), 128, 8)
    assert np.array_equal(out["routed"], np.arange(12))
    assert np.all(out["count"] == 128)


def test_empty_token_batch():
    inp = _small_inputs(2.0)
    x = inp.as_f64("x")[:0]
    out = oracle.sparse_forward(x, inp.as_f64("wg_t"), inp.b_g, inp.as_f64("wu_t"),
                                inp.as_f64("wd"), 128, 8)
    assert out["count"].shape == (0, 3) and out["y"].shape == (0, 64)


# ------------------------------------------------------------ planted mistakes
def _mut_pack_zero_active(orig):
    return lambda z, tile, cap: orig(np.where(np.asarray(z) == 0, 1e-300, z), tile, cap)


def _mut_pack_local_index(orig):
    def f(z, tile, cap):
        c, i, v = orig(z, tile, cap)
        i = i.copy()
        for k in range(i.shape[1]):
            i[:, k][i[:, k] >= 0] -= k * tile
        return c, i, v
    return f


def _mut_pack_descending(orig):
    def f(z, tile, cap):
        c, i, v = orig(np.asarray(z, float)[:, ::-1], tile, cap)
        d_ff = np.asarray(z).shape[1]
        i = np.where(i >= 0, d_ff - 1 - i, i)
        return c[:, ::-1], i[:, ::-1], v[:, ::-1]
    return f


def _mut_ell_count_capped(orig):
    def f(z, width):
        c, i, v = orig(z, width)
        return np.minimum(c, width), i, v
    return f


def _mut_ell_zero_active(orig):
    return lambda z, width: orig(np.where(np.asarray(z) == 0, 1e-300, z), width)


def _mut_ell_no_running_slot(orig):
    # every 4-column tile writes its list from slot 0 (a converter that forgets
    # the running count across tiles): later tiles overwrite earlier ones
    def f(z, width):
        z = np.asarray(z, float)
        c, i, v = orig(z, width)
        i, v = np.full_like(i, -1), np.zeros_like(v)
        for t in range(z.shape[0]):
            for lo in range(0, z.shape[1], 4):
                cols = [lo + j for j in np.nonzero(z[t, lo:lo + 4] > 0)[0]][:width]
                i[t, :len(cols)] = cols
                v[t, :len(cols)] = z[t, cols]
        return c, i, v
    return f


def _mut_l1_abs(orig):
    return lambda z, lam: float(lam) * float(np.abs(np.asarray(z, float)).sum()) / max(1, len(z))


def _mut_l1_no_mean(orig):
    return lambda z, lam: orig(z, lam) * max(1, len(z))


def _mut_route_ge(orig):
    return lambda count, cap: np.nonzero(np.asarray(count).max(1) >= cap)[0]


def _mut_gate_naive(orig):
    return lambda x, w, b=None: np.asarray(x, float) @ np.asarray(w, float).T + np.asarray(b, float)


def _mut_gate_bias_sign(orig):
    return lambda x, w, b=None: orig(x, w, -np.asarray(b, float))


def _mut_up_from_gate(orig):
    def f(x, wg, b, wu, wd, count, idx, val, cap):
        return orig(x, wg, b, wg, wd, count, idx, val, cap)
    return f


def _mut_drop_val(orig):
    def f(x, wg, b, wu, wd, count, idx, val, cap):
        return orig(x, wg, b, wu, wd, count, idx, np.ones_like(val), cap)
    return f


def _mut_skip_last_slot(orig):
    def f(x, wg, b, wu, wd, count, idx, val, cap):
        return orig(x, wg, b, wu, wd, np.maximum(np.asarray(count) - 1, 0), idx, val, cap)
    return f


MUTATIONS = {
    "pack_zero_active": ("twell_pack", _mut_pack_zero_active),
    "pack_local_index": ("twell_pack", _mut_pack_local_index),
    "pack_descending": ("twell_pack", _mut_pack_descending),
    "route_ge": ("route", _mut_route_ge),
    "l1_sums_abs": ("l1_term", _mut_l1_abs),
    "l1_no_token_mean": ("l1_term", _mut_l1_no_mean),
    "ell_count_capped": ("ell_pack", _mut_ell_count_capped),
    "ell_zero_active": ("ell_pack", _mut_ell_zero_active),
    "ell_no_running_slot": ("ell_pack", _mut_ell_no_running_slot),
    "gate_naive_sum": ("gate_preact", _mut_gate_naive),
    "gate_bias_sign": ("gate_preact", _mut_gate_bias_sign),
    "up_from_gate": ("ffn_sparse", _mut_up_from_gate),
    "drop_val": ("ffn_sparse", _mut_drop_val),
    "skip_last_slot": ("ffn_sparse", _mut_skip_last_slot),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, make = MUTATIONS[name]
    orig = getattr(offn, attr)
    monkeypatch.setattr(offn, attr, make(orig))
    monkeypatch.setattr(oracle, attr, getattr(offn, attr), raising=False)
    caught = False
    for case in tiny_cases():
        try:
            check_against_brute(*case)
        except (AssertionError, ValueError, IndexError):
            caught = True
            break
    assert caught, f"planted mistake {name} was not detected"


# ------------------------------------------------------------ L1 regulariser
def test_l1_closed_form_when_every_entry_is_active():
    """With a bias large enough that every z > 0, sum_tj z = sum_t x_t . (sum_j w_j)
    + T sum_j b_j: an independent closed form of the L1 sum."""
    rng = np.random.default_rng(7)
    T, K, d_ff = 5, 16, 12
    x = _bf16(rng.standard_normal((T, K)))
    w = _bf16(rng.standard_normal((d_ff, K)) / 4)
    b = np.full(d_ff, 64.0)
    z = oracle.gate_preact(x, w, b)
    assert (z > 0).all()
    closed = (sum((Fr(float(x[t, k])) * sum(Fr(float(w[j, k])) for j in range(d_ff))
                   for t in range(T) for k in range(K)), Fr(0)) + T * Fr(float(b.sum())))
    got = oracle.l1_term(z, 0.5)
    assert abs(Fr(got) - Fr(1, 2) * closed / T) <= Fr(2.0 ** -48) * abs(closed)


def test_l1_special_cases():
    z = np.array([[-1.0, 0.0, -3.0], [0.0, -0.5, -2.0]])
    assert oracle.l1_term(z, 3.0) == 0.0          # nothing active (z = 0 is inactive)
    assert oracle.l1_term(np.zeros((0, 4)), 1.0) == 0.0
    assert oracle.l1_term(np.array([[2.0, -1.0], [1.0, 4.0]]), 1.0) == 3.5

