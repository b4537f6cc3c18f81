"""CPU oracle of the activation-sparse gated FFN forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

Plain numpy float64, written from the pages' description of the method
("Sparser, Faster, Lighter Transformer Language Models"; pwwt.cn article
sections 01-03, kongchang.com article "TwELL" and "custom CUDA kernels"
sections, neo-ai.one article on TwELL and the Hybrid format):

  gate   z = x . W_g + b_g                       (gated FFN, pwwt.cn section 01)
  ReLU   h = z where z > 0, else 0               (ReLU gate gives unstructured
                                                  sparsity, pwwt.cn section 01)
  TwELL  per row and per 1D column tile, an ELLPACK list of the active columns
         and their values                        (pwwt.cn section 02; the ELLPACK
                                                  value + column-index arrays,
                                                  kongchang.com "TwELL" section)
  hybrid rows whose tile lists overflow the capacity go to a dense path
                                                 (pwwt.cn section 03)
  fused  y_t = sum over packed (j, h_tj) of h_tj * (x_t . W_u[:, j]) * W_d[j, :]
         (up projection only on the packed nonzeros, scaled by the gate value,
         accumulated into the down projection; pwwt.cn section 02)

The pages lose every formula in extraction; the readings taken here (gated FFN
y = (ReLU(x W_g + b_g) * x W_u) W_d, strict z > 0, ascending slot order, global
column indices, true per-tile counts) are the plainest ones the prose supports.

Inputs must be finite and exactly representable in float32 (float32 or
bfloat16 data widened to float64).  Then every product x_k * w_k is exact in
float64, which ``gate_preact`` uses to make the sign of z exact.

Parity pins: every function here is pinned in tests/test_oracle_pins.py
(exact rational brute force on tiny shapes, an integer fixture at moderate size,
closed-form density, symmetry and special cases).
"""
from __future__ import annotations

import math

import numpy as np
import scipy.sparse

_U64 = 2.0 ** -53  # unit roundoff of float64


def _f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return a


def _check_f32_representable(name: str, a: np.ndarray) -> None:
    if not np.all(np.isfinite(a)):
        raise ValueError(f"{name} holds non-finite values")
    if not np.array_equal(a.astype(np.float32).astype(np.float64), a):
        raise ValueError(f"{name} is not exactly representable in float32")


def gate_preact(x, wg_t, b_g=None) -> np.ndarray:
    """Gate pre-activation z[t, j] = sum_k x[t, k] * wg_t[j, k] + b_g[j].

    (Gate projection of the gated FFN, pwwt.cn article section 01.)

    The bulk is a float64 matrix product.  Its error is at most
    (K + 1) * u * (sum_k |x_tk w_jk| + |b_j|) for any summation order, so every
    entry whose magnitude is within twice that bound is recomputed with
    ``math.fsum`` over the exact float64 products and the bias, which returns
    the correctly rounded sum.  The sign of every returned entry is therefore
    the sign of the exact value, and near-zero entries are correctly rounded.
    """
    x = _f64(x)
    w = _f64(wg_t)
    T, K = x.shape
    d_ff = w.shape[0]
    b = np.zeros(d_ff) if b_g is None else _f64(b_g)
    _check_f32_representable("x", x)
    _check_f32_representable("wg_t", w)
    _check_f32_representable("b_g", b)
    z = x @ w.T + b
    a = np.abs(x) @ np.abs(w).T + np.abs(b)
    bound = 2.0 * (K + 2) * _U64 * a * (1.0 + 1e-6)
    ts, js = np.nonzero(np.abs(z) <= bound)
    for t, j in zip(ts.tolist(), js.tolist()):
        prods = (x[t] * w[j]).tolist()  # exact: float32 x float32 fits float64
        prods.append(float(b[j]))
        z[t, j] = math.fsum(prods)
    return z


def relu(z) -> np.ndarray:
    """h = z where z > 0 (strictly), else 0 (pwwt.cn article section 01)."""
    z = _f64(z)
    return np.where(z > 0.0, z, 0.0)


def n_tiles(d_ff: int, tile: int) -> int:
    return -(-d_ff // tile)


def twell_pack(z, tile: int, cap: int):
    """Tile-wise ELLPACK of the ReLU output (pwwt.cn article section 02).

    The columns are cut into 1D tiles of ``tile`` consecutive columns (the last
    tile may be narrower).  For each row t and tile k:
      count[t, k]   number of active columns (z > 0) in the tile, uncapped;
      idx[t, k, s]  for s < min(count, cap): the s-th active column, ascending,
                    as a global column index; -1 in unused slots;
      val[t, k, s]  h at that column; 0 in unused slots.
    """
    z = _f64(z)
    T, d_ff = z.shape
    nt = n_tiles(d_ff, tile)
    count = np.zeros((T, nt), dtype=np.int64)
    idx = np.full((T, nt, cap), -1, dtype=np.int64)
    val = np.zeros((T, nt, cap), dtype=np.float64)
    for k in range(nt):
        lo, hi = k * tile, min((k + 1) * tile, d_ff)
        act = z[:, lo:hi] > 0.0
        count[:, k] = act.sum(axis=1)
        slot = np.cumsum(act, axis=1) - 1
        keep = act & (slot < cap)
        rr, cc = np.nonzero(keep)
        ss = slot[rr, cc]
        idx[rr, k, ss] = lo + cc
        val[rr, k, ss] = z[rr, lo + cc]
    return count, idx, val


def twell_unpack(count, idx, val, d_ff: int) -> np.ndarray:
    """Dense [T, d_ff] matrix holding the live TwELL entries, zeros elsewhere."""
    count = np.asarray(count)
    idx = np.asarray(idx)
    val = _f64(val)
    T, nt, cap = idx.shape
    h = np.zeros((T, d_ff), dtype=np.float64)
    live = np.arange(cap)[None, None, :] < np.minimum(count, cap)[:, :, None]
    rr, kk, ss = np.nonzero(live)
    h[rr, idx[rr, kk, ss]] = val[rr, kk, ss]
    return h


def ell_pack(z, width: int):
    """Classic row-wise ELLPACK of the ReLU output: one list per row over all
    columns, padded to a common width (the "traditional ELLPACK" that the
    pwwt.cn article, section 01, contrasts with TwELL; value and column-index
    arrays of the kongchang.com article's ELLPACK passage).

      count[t]     number of active columns (z > 0) in row t, uncapped;
      idx[t, s]    for s < min(count, width): the s-th active column,
                   ascending; -1 in unused slots;
      val[t, s]    h at that column; 0 in unused slots.
    The classic format sets width to the longest row, max_t count[t].
    """
    z = _f64(z)
    T, d_ff = z.shape
    count = np.zeros(T, dtype=np.int64)
    idx = np.full((T, width), -1, dtype=np.int64)
    val = np.zeros((T, width), dtype=np.float64)
    for t in range(T):
        cols = np.nonzero(z[t] > 0.0)[0]
        count[t] = len(cols)
        keep = cols[:width]
        idx[t, :len(keep)] = keep
        val[t, :len(keep)] = z[t, keep]
    return count, idx, val


def ell_unpack(count, idx, val, d_ff: int) -> np.ndarray:
    """Dense [T, d_ff] matrix holding the live row-ELLPACK entries."""
    count = np.asarray(count)
    idx = np.asarray(idx)
    val = _f64(val)
    T, width = idx.shape
    h = np.zeros((T, d_ff), dtype=np.float64)
    live = np.arange(width)[None, :] < np.minimum(count, width)[:, None]
    rr, ss = np.nonzero(live)
    h[rr, idx[rr, ss]] = val[rr, ss]
    return h


def l1_term(z, lam: float) -> float:
    """L1 activation regulariser of the sparse training recipe (pwwt.cn article,
    section 04; besthub.dev page): lam times the mean over tokens of the summed
    ReLU activations, lam / T * sum_t sum_j h[t, j].  The formula itself was lost
    from the pages; this is the plainest reading of an L1 penalty on the FFN
    activations averaged over tokens.  Its gradient with respect to z is lam / T
    wherever z > 0.  No tokens: 0."""
    z = _f64(z)
    T = z.shape[0]
    if T == 0:
        return 0.0
    return float(lam) * math.fsum(z[z > 0.0].tolist()) / T


def route(count, cap: int) -> np.ndarray:
    """Rows sent to the dense path: any tile with more active columns than the
    capacity (hybrid routing, pwwt.cn article section 03).  Ascending."""
    count = np.asarray(count)
    if count.shape[1] == 0:
        return np.zeros(0, dtype=np.int64)
    return np.nonzero(count.max(axis=1) > cap)[0].astype(np.int64)


def up_proj(x, wu_t) -> np.ndarray:
    """u[t, j] = x_t . wu_t[j] (up projection, pwwt.cn article section 01)."""
    return _f64(x) @ _f64(wu_t).T


def ffn_dense(x, wg_t, b_g, wu_t, wd) -> np.ndarray:
    """Dense gated FFN y = (ReLU(x W_g + b_g) * x W_u) W_d."""
    h = relu(gate_preact(x, wg_t, b_g))
    return (h * up_proj(x, wu_t)) @ _f64(wd)


def ffn_sparse(x, wg_t, b_g, wu_t, wd, count, idx, val, cap: int) -> np.ndarray:
    """Hybrid sparse forward from a TwELL encoding.

    Rows within capacity: y_t = sum over live (k, s) of
    val * (x_t . wu_t[idx]) * wd[idx]  (pwwt.cn article section 02: the up
    projection is computed only for the packed nonzeros, scaled by the gate
    value and accumulated into the down projection; h is never formed).
    Routed rows: the dense gated FFN, gate recomputed from x (section 03).
    """
    x = _f64(x)
    wu = _f64(wu_t)
    wdd = _f64(wd)
    count = np.asarray(count)
    idx = np.asarray(idx)
    val = _f64(val)
    T, nt, cap_ = idx.shape
    d_ff = wu.shape[0]
    R = route(count, cap)
    routed = np.zeros(T, dtype=bool)
    routed[R] = True
    live = np.arange(cap_)[None, None, :] < np.minimum(count, cap_)[:, :, None]
    live &= ~routed[:, None, None]
    rr, kk, ss = np.nonzero(live)
    jj = idx[rr, kk, ss]
    vv = val[rr, kk, ss]
    # up projection on the packed nonzeros only, in bounded chunks
    u = np.empty(len(rr), dtype=np.float64)
    step = max(1, (1 << 22) // max(1, x.shape[1]))
    for a in range(0, len(rr), step):
        u[a:a + step] = np.einsum("ek,ek->e", x[rr[a:a + step]], wu[jj[a:a + step]])
    g = vv * u
    G = scipy.sparse.csr_matrix((g, (rr, jj)), shape=(T, d_ff))
    y = np.asarray(G @ wdd)
    if len(R):
        y[R] = ffn_dense(x[R], wg_t, b_g, wu_t, wd)
    return y


def sparse_forward(x, wg_t, b_g, wu_t, wd, tile: int, cap: int) -> dict:
    """Gate -> ReLU -> TwELL pack -> route -> fused sparse forward."""
    z = gate_preact(x, wg_t, b_g)
    count, idx, val = twell_pack(z, tile, cap)
    R = route(count, cap)
    y = ffn_sparse(x, wg_t, b_g, wu_t, wd, count, idx, val, cap)
    return {"z": z, "count": count, "idx": idx, "val": val, "routed": R, "y": y}


def ffn_dense_backward(x, wg_t, b_g, wu_t, wd, gy, lam: float = 0.0) -> dict:
    """Gradients of the gated FFN y = (ReLU(x W_g + b_g) * x W_u) W_d for an
    upstream gradient gy = dL/dy, by the chain rule on the plain definition
    (the pages give the forward only; training through the format is their
    pwwt.cn section 03-04 result), with the L1 activation regulariser
    lam / T * sum_t sum_j ReLU(z) of the training recipe (section 04; see
    l1_term) added to the loss:

      a  = h * u,  h = ReLU(z),  u = x wu_t^T       (forward)
      ga = gy wd^T                                   dL/da
      gz = (ga * u + lam / T) * [z > 0]   (ReLU' = 1 strictly above 0, 0 at and below)
      gu = ga * h
      gx = gz wg_t + gu wu_t
      g_wg_t = gz^T x,  g_wu_t = gu^T x,  g_wd = a^T gy,  g_b = sum_t gz
    """
    x = _f64(x)
    T = x.shape[0]
    return _dense_backward(x, wg_t, b_g, wu_t, wd, gy, float(lam) / T if T else 0.0)


def _dense_backward(x, wg_t, b_g, wu_t, wd, gy, l1g: float) -> dict:
    """ffn_dense_backward with the regulariser's per-entry gradient l1g given
    (lam / T of the whole batch, also when x holds only some of its rows)."""
    x = _f64(x)
    z = gate_preact(x, wg_t, b_g)
    act = z > 0.0
    h = np.where(act, z, 0.0)
    wg, wu, wdd, gy = _f64(wg_t), _f64(wu_t), _f64(wd), _f64(gy)
    u = x @ wu.T
    a = h * u
    ga = gy @ wdd.T
    gz = np.where(act, ga * u + l1g, 0.0)
    gu = ga * h
    return {"gx": gz @ wg + gu @ wu, "gwg_t": gz.T @ x, "gwu_t": gu.T @ x,
            "gwd": a.T @ gy, "gb": gz.sum(axis=0)}


def ffn_sparse_backward(x, wg_t, b_g, wu_t, wd, gy, count, idx, val, cap: int,
                        lam: float = 0.0) -> dict:
    """The same gradients from the forward's TwELL encoding: for rows within
    capacity only the packed entries (j, h) exist, so the up projection, the
    down-projection gradient and every product are taken per entry
    (u_e = x_t . wu_t[j], ga_e = gy_t . wd[j], gz_e = ga_e u_e, gu_e = ga_e h_e,
    a_e = h_e u_e), and the weight gradients are sums over the entries of each
    column; routed rows go through the dense formulas (hybrid routing, pwwt.cn
    article section 03).  Uses val as h, as the sparse kernels do.  The L1
    regulariser adds lam / T (T: all rows) to gz of every active entry: the
    packed ones and, for routed rows, all of theirs."""
    x = _f64(x)
    wg, wu, wdd, gy = _f64(wg_t), _f64(wu_t), _f64(wd), _f64(gy)
    count = np.asarray(count)
    idx = np.asarray(idx)
    val = _f64(val)
    T, nt, cap_ = idx.shape
    d_ff = wg.shape[0]
    R = route(count, cap)
    routed = np.zeros(T, dtype=bool)
    routed[R] = True
    live = np.arange(cap_)[None, None, :] < np.minimum(count, cap_)[:, :, None]
    live &= ~routed[:, None, None]
    rr, kk, ss = np.nonzero(live)
    jj = idx[rr, kk, ss]
    hh = val[rr, kk, ss]
    l1g = float(lam) / T if T else 0.0
    u = np.einsum("ek,ek->e", x[rr], wu[jj]) if len(rr) else np.zeros(0)
    ga = np.einsum("ek,ek->e", gy[rr], wdd[jj]) if len(rr) else np.zeros(0)
    gz, gu, a = ga * u + l1g, ga * hh, hh * u
    GZ = scipy.sparse.csr_matrix((gz, (rr, jj)), shape=(T, d_ff))
    GU = scipy.sparse.csr_matrix((gu, (rr, jj)), shape=(T, d_ff))
    A = scipy.sparse.csr_matrix((a, (rr, jj)), shape=(T, d_ff))
    out = {"gx": np.asarray(GZ @ wg + GU @ wu),
           "gwg_t": np.asarray(GZ.T @ x), "gwu_t": np.asarray(GU.T @ x),
           "gwd": np.asarray(A.T @ gy), "gb": np.asarray(GZ.sum(axis=0)).ravel()}
    if len(R):
        d = _dense_backward(x[R], wg_t, b_g, wu_t, wd, gy[R], l1g)
        out["gx"][R] = d["gx"]
        for k in ("gwg_t", "gwu_t", "gwd", "gb"):
            out[k] = out[k] + d[k]
    return out

