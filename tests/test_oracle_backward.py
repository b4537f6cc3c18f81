"""Pins of the oracle's backward (ffn_dense_backward, ffn_sparse_backward)
against facts that do not come from the oracle itself:

  * exact rational brute force of the chain rule (pure-Python loops over
    Fractions) on the tiny cases of the forward pins, exact zeros included;
  * torch.autograd in float64 on the CPU (an independent implementation of the
    derivative) at a moderate size;
  * central finite differences of L = sum(y * gy) along random directions,
    on inputs whose pre-activations stay clear of the ReLU kink;
  * the sparse form against the dense one, and planted mistakes that the pins
    must catch;
  * all of the above also with the L1 activation regulariser lam / T *
    sum ReLU(z) added to the loss (its gradient lam / T on the active
    entries).
"""
from __future__ import annotations

from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

import oracle
from oracle import ffn as offn
from test_oracle_pins import _bf16, tiny_cases


def brute_backward(x, wg, b, wu, wd, gy, lam=0.0):
    """Exact chain rule with nested loops (no numpy arithmetic); lam weights
    the L1 term lam / T * sum ReLU(z) added to the loss."""
    F = lambda m: [[Fr(float(v)) for v in row] for row in m]
    X, G, U_, D, GY = F(x), F(wg), F(wu), F(wd), F(gy)
    B = [Fr(float(v)) for v in b]
    T, K, d_ff, dm = len(X), len(X[0]), len(G), len(D[0])
    l1 = Fr(float(lam)) / T if T else Fr(0)
    z = [[B[j] + sum(X[t][k] * G[j][k] for k in range(K)) for j in range(d_ff)] for t in range(T)]
    u = [[sum(X[t][k] * U_[j][k] for k in range(K)) for j in range(d_ff)] for t in range(T)]
    h = [[z[t][j] if z[t][j] > 0 else Fr(0) for j in range(d_ff)] for t in range(T)]
    ga = [[sum(GY[t][c] * D[j][c] for c in range(dm)) for j in range(d_ff)] for t in range(T)]
    gz = [[ga[t][j] * u[t][j] + l1 if z[t][j] > 0 else Fr(0) for j in range(d_ff)]
          for t in range(T)]
    gu = [[ga[t][j] * h[t][j] for j in range(d_ff)] for t in range(T)]
    gx = [[sum(gz[t][j] * G[j][k] + gu[t][j] * U_[j][k] for j in range(d_ff)) for k in range(K)]
          for t in range(T)]
    gwg = [[sum(gz[t][j] * X[t][k] for t in range(T)) for k in range(K)] for j in range(d_ff)]
    gwu = [[sum(gu[t][j] * X[t][k] for t in range(T)) for k in range(K)] for j in range(d_ff)]
    gwd = [[sum(h[t][j] * u[t][j] * GY[t][c] for t in range(T)) for c in range(dm)]
           for j in range(d_ff)]
    gb = [sum(gz[t][j] for t in range(T)) for j in range(d_ff)]
    return {"gx": gx, "gwg_t": gwg, "gwu_t": gwu, "gwd": gwd, "gb": gb}


def _close(got, exact, tol=2.0 ** -40) -> None:
    ex = np.array(exact, dtype=object)
    flat = [Fr(v) for v in np.asarray(ex).ravel()] if ex.size else []
    scale = max([abs(v) for v in flat] + [Fr(1, 10 ** 30)])
    g = np.asarray(got, dtype=np.float64).ravel()
    assert g.size == len(flat)
    for a, e in zip(g.tolist(), flat):
        assert abs(Fr(a) - e) <= Fr(tol) * scale, (a, float(e))


def _gy(case, seed=3):
    x, wg, b, wu, wd, tile, cap = case
    return _bf16(np.random.default_rng(seed).standard_normal((x.shape[0], wd.shape[1])))


def check_backward_against_brute(case, lam=0.0):
    x, wg, b, wu, wd, tile, cap = case
    gy = _gy(case)
    ref = brute_backward(x, wg, b, wu, wd, gy, lam)
    dense = oracle.ffn_dense_backward(x, wg, b, wu, wd, gy, lam)
    z = oracle.gate_preact(x, wg, b)
    count, idx, val = oracle.twell_pack(z, tile, cap)
    sparse = oracle.ffn_sparse_backward(x, wg, b, wu, wd, gy, count, idx, val, cap, lam)
    for out in (dense, sparse):
        for k in ("gx", "gwg_t", "gwu_t", "gwd", "gb"):
            _close(out[k], ref[k])


@pytest.mark.parametrize("lam", [0.0, 0.75])
@pytest.mark.parametrize("case", range(len(tiny_cases())))
def test_backward_brute_force_tiny(case, lam):
    check_backward_against_brute(tiny_cases()[case], lam)


def _moderate(seed=11, T=20, K=32, d_ff=48, dm=None, margin=None):
    rng = np.random.default_rng(seed)
    dm = dm or K
    x = _bf16(rng.standard_normal((T, K)))
    wg = _bf16(rng.standard_normal((d_ff, K)) / np.sqrt(K))
    wu = _bf16(rng.standard_normal((d_ff, K)) / np.sqrt(K))
    wd = _bf16(rng.standard_normal((d_ff, dm)) / np.sqrt(d_ff))
    b = _bf16(rng.standard_normal(d_ff) * 0.3)
    gy = _bf16(rng.standard_normal((T, dm)))
    if margin is not None:  # move b so that every |z| >= margin
        z = x @ wg.T + b
        near = np.abs(z) < margin
        while near.any():
            b = b + np.where(near.any(0), 0.125, 0.0)  # exact in float32
            z = x @ wg.T + b
            near = np.abs(z) < margin
    return x, wg, b, wu, wd, gy


@pytest.mark.parametrize("lam", [0.0, 0.3])
def test_backward_matches_torch_autograd_float64(lam):
    x, wg, b, wu, wd, gy = _moderate()
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in dict(x=x, wg=wg, b=b, wu=wu, wd=wd).items()}
    h = torch.relu(t["x"] @ t["wg"].T + t["b"])
    y = (h * (t["x"] @ t["wu"].T)) @ t["wd"]
    loss = (y * torch.tensor(gy, dtype=torch.float64)).sum() + lam / x.shape[0] * h.sum()
    loss.backward()
    got = oracle.ffn_dense_backward(x, wg, b, wu, wd, gy, lam)
    pairs = {"gx": "x", "gwg_t": "wg", "gwu_t": "wu", "gwd": "wd", "gb": "b"}
    for k, tk in pairs.items():
        ref = t[tk].grad.numpy()
        assert np.abs(got[k] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), k


@pytest.mark.parametrize("lam", [0.0, 1.5])
def test_backward_finite_differences(lam):
    x, wg, b, wu, wd, gy = _moderate(seed=12, T=6, K=8, d_ff=12, dm=5, margin=0.0625)

    def loss(x_, wg_, b_, wu_, wd_):
        z = x_ @ wg_.T + b_
        h = np.maximum(z, 0.0)
        return float(((h * (x_ @ wu_.T)) @ wd_ * gy).sum()) + lam / x_.shape[0] * float(h.sum())

    g = oracle.ffn_dense_backward(x, wg, b, wu, wd, gy, lam)
    rng = np.random.default_rng(5)
    args = [x, wg, b, wu, wd]
    names = ["gx", "gwg_t", "gb", "gwu_t", "gwd"]
    order = ["x", "wg", "b", "wu", "wd"]
    for i, name in enumerate(order):
        v = rng.standard_normal(args[i].shape)
        eps = 1e-6
        plus = list(args); plus[i] = args[i] + eps * v
        minus = list(args); minus[i] = args[i] - eps * v
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = float((g[{"x": "gx", "wg": "gwg_t", "b": "gb", "wu": "gwu_t", "wd": "gwd"}[name]] * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    assert set(names) == set(g)


@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_sparse_backward_equals_dense_with_routing(lam):
    x, wg, b, wu, wd, gy = _moderate(seed=13, T=24, K=32, d_ff=64)
    z = oracle.gate_preact(x, wg, b)
    for cap in (0, 2, 4, 64):
        count, idx, val = oracle.twell_pack(z, 16, cap)
        sp = oracle.ffn_sparse_backward(x, wg, b, wu, wd, gy, count, idx, val, cap, lam)
        de = oracle.ffn_dense_backward(x, wg, b, wu, wd, gy, lam)
        for k in de:
            assert np.abs(sp[k] - de[k]).max() <= 1e-12 * max(1.0, np.abs(de[k]).max()), (cap, k)


# ------------------------------------------------------------ planted mistakes
def _mut_no_relu_mask(orig):
    def f(x, wg_t, b_g, wu_t, wd, gy, lam=0.0):
        out = orig(x, wg_t, b_g, wu_t, wd, gy, lam)
        z = offn.gate_preact(x, wg_t, b_g)
        u = np.asarray(x, float) @ np.asarray(wu_t, float).T
        ga = np.asarray(gy, float) @ np.asarray(wd, float).T
        out["gb"] = (ga * u).sum(0)  # ReLU' dropped
        return out
    return f


def _mut_gu_from_u(orig):
    def f(x, wg_t, b_g, wu_t, wd, gy, lam=0.0):
        out = orig(x, wg_t, b_g, wu_t, wd, gy, lam)
        x64 = np.asarray(x, float)
        u = x64 @ np.asarray(wu_t, float).T
        ga = np.asarray(gy, float) @ np.asarray(wd, float).T
        out["gwu_t"] = (ga * u).T @ x64  # gu = ga * u instead of ga * h
        return out
    return f


def _mut_gwd_from_h(orig):
    def f(x, wg_t, b_g, wu_t, wd, gy, lam=0.0):
        out = orig(x, wg_t, b_g, wu_t, wd, gy, lam)
        h = offn.relu(offn.gate_preact(x, wg_t, b_g))
        out["gwd"] = h.T @ np.asarray(gy, float)  # a = h * u lost
        return out
    return f


def _mut_gx_gate_only(orig):
    def f(x, wg_t, b_g, wu_t, wd, gy, lam=0.0):
        out = orig(x, wg_t, b_g, wu_t, wd, gy, lam)
        z = offn.gate_preact(x, wg_t, b_g)
        x64 = np.asarray(x, float)
        u = x64 @ np.asarray(wu_t, float).T
        ga = np.asarray(gy, float) @ np.asarray(wd, float).T
        out["gx"] = np.where(z > 0, ga * u, 0.0) @ np.asarray(wg_t, float)  # up path dropped
        return out
    return f


def _mut_l1_everywhere(orig):
    def f(x, wg_t, b_g, wu_t, wd, gy, lam=0.0):
        out = orig(x, wg_t, b_g, wu_t, wd, gy, lam)
        z = offn.gate_preact(x, wg_t, b_g)
        T = np.asarray(x).shape[0]
        out["gb"] = out["gb"] + lam / T * (z <= 0).sum(0)  # regulariser on inactive entries too
        return out
    return f


def _mut_l1_no_mean(orig):
    def f(x, wg_t, b_g, wu_t, wd, gy, lam=0.0):
        return orig(x, wg_t, b_g, wu_t, wd, gy, lam * np.asarray(x).shape[0])  # lam, not lam / T
    return f


BWD_MUTATIONS = {"no_relu_mask": _mut_no_relu_mask, "gu_from_u": _mut_gu_from_u,
                 "gwd_from_h": _mut_gwd_from_h, "gx_gate_only": _mut_gx_gate_only,
                 "l1_everywhere": _mut_l1_everywhere, "l1_no_mean": _mut_l1_no_mean}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_backward_planted_mistake_is_caught(name, monkeypatch):
    orig = offn.ffn_dense_backward
    monkeypatch.setattr(offn, "ffn_dense_backward", BWD_MUTATIONS[name](orig))
    monkeypatch.setattr(oracle, "ffn_dense_backward", offn.ffn_dense_backward)
    lam = 0.75 if name.startswith("l1_") else 0.0
    caught = False
    for case in tiny_cases():
        try:
            check_backward_against_brute(case, lam)
        except AssertionError:
            caught = True
            break
    assert caught, name
