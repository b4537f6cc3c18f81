"""Seeded synthetic inputs for the activation-sparse gated FFN.

This module only draws numbers: the token activations x, the three weight
matrices and the gate bias, rounded to the storage dtype.  It holds none of the
method's arithmetic (no projection, no ReLU, no packing), so both the HIP path
and the CPU oracle can take their inputs from it without sharing any step of
the computation.

Workloads follow the synthetic data recipe of the pages' setting: a ReLU-gated
FFN whose gate pre-activation is shifted by a bias -beta so that a fixed
fraction of the gate outputs survive (the pages describe ReLU gating producing
unstructured activation sparsity, "Sparser, Faster, Lighter Transformer
Language Models" (pwwt.cn article), section 01), and per-token row scales that
model the strongly varying number of active neurons per token (same article,
sections 03 and 05).

Drawing rule (fixed so that any run can regenerate the same arrays):
  * one numpy ``Generator(PCG64(seed))`` per tensor, with
    ``seed = seed_base + {x: 1, wg: 2, wu: 3, wd: 4, rows: 5}``;
  * samples are drawn as float32 standard normals and scaled by the standard
    deviation in float32 (variances are the ``N(0, v)`` second argument);
  * for bf16 workloads the float32 samples are rounded to bfloat16 with
    round-to-nearest-even; those rounded values are what every consumer uses;
  * the gate bias is ``-beta`` in float32.

Layouts: ``x [T, d_model]``; ``wg_t, wu_t, wd`` all ``[d_ff, d_model]``
row-major, i.e. row ``j`` holds the d_model weights attached to FFN neuron j
(for the gate and up projections, the column of W_g / W_u; for the down
projection, the row of W_d).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_OFFSETS = {"x": 1, "wg": 2, "wu": 3, "wd": 4, "rows": 5, "gy": 6}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, dtype and data recipe of one synthetic FFN workload."""

    name: str
    T: int
    d_model: int
    d_ff: int
    dtype: str  # "f32" or "bf16": storage and arithmetic type of x, weights, val, y
    beta: float
    cap: int = 8
    tile: int = 128
    seed_base: int = 0
    rows: str = "unit"  # "unit" | "mixture" | "lognormal"
    heavy_frac: float = 0.0  # mixture: fraction of rows with the large scale
    heavy_scale: float = 1.0  # mixture: scale of those rows
    log_sigma: float = 0.0  # lognormal: sigma of log(row scale)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def n_tiles(self) -> int:
        return -(-self.d_ff // self.tile)


# Seed base of the tiny float32 workload: the first base in the sequence
# 0, 100, 200, ... whose gate activations overflow no TwELL tile at capacity 8.
# Chosen by tests/golden/choose_tiny_seed.py (which calls only the oracle) and
# recorded in tests/golden/tiny_f32_seed.json.
TINY_F32_SEED_BASE = 100

WORKLOADS = {
    # 64 tokens, 256 -> 1024, float32 end to end, ~2% density, no overflow.
    "tiny_f32": Workload("tiny_f32", T=64, d_model=256, d_ff=1024, dtype="f32",
                         beta=2.054, cap=8, seed_base=TINY_F32_SEED_BASE),
    # Prefill: 4096 tokens, 2048 -> 5632, bf16, ~1% density (~56 nnz/row).
    "prefill_1pct": Workload("prefill_1pct", T=4096, d_model=2048, d_ff=5632,
                             dtype="bf16", beta=2.326, cap=8, seed_base=1000),
    # Same shapes; 99% light rows (~0.5%) and 1% heavy rows (scale 3.8, ~25%),
    # capacity 4: the heavy rows and a few light ones overflow and go dense.
    "hybrid_mix": Workload("hybrid_mix", T=4096, d_model=2048, d_ff=5632,
                           dtype="bf16", beta=2.576, cap=4, seed_base=2000,
                           rows="mixture", heavy_frac=0.01, heavy_scale=3.8),
    # Decode: 32 tokens, 4096 -> 11008, bf16, ~1% density.
    "decode_1pct": Workload("decode_1pct", T=32, d_model=4096, d_ff=11008,
                            dtype="bf16", beta=2.326, cap=8, seed_base=3000),
    # Large: 16384 tokens, 4096 -> 14336, bf16, lognormal row scales.
    "large_lognormal": Workload("large_lognormal", T=16384, d_model=4096,
                                d_ff=14336, dtype="bf16", beta=2.75, cap=8,
                                seed_base=4000, rows="lognormal",
                                log_sigma=0.35),
}

# Gate-bias sweep of the large workload (density ~50%, 10%, 1%, 0.3%).
LARGE_BETA_SWEEP = (0.0, 1.28, 2.33, 2.75)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Only finite inputs are supported (the generator draws finite normals).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return z


def row_scales(w: Workload) -> np.ndarray:
    """Per-token scale s_t (float32) of the workload's row recipe."""
    seed = w.seed_base + SEED_OFFSETS["rows"]
    if w.rows == "unit":
        return np.ones(w.T, dtype=np.float32)
    if w.rows == "mixture":
        rng = np.random.Generator(np.random.PCG64(seed))
        n_heavy = int(round(w.heavy_frac * w.T))
        s = np.ones(w.T, dtype=np.float32)
        if n_heavy > 0:
            pos = rng.choice(w.T, size=n_heavy, replace=False)
            s[pos] = np.float32(w.heavy_scale)
        return s
    if w.rows == "lognormal":
        rng = np.random.Generator(np.random.PCG64(seed))
        return np.exp(np.float32(w.log_sigma)
                      * rng.standard_normal(size=w.T, dtype=np.float32)).astype(np.float32)
    raise ValueError(f"unknown row recipe {w.rows!r}")


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs.

    ``x, wg_t, wu_t, wd`` hold the storage encoding: float32 arrays for
    ``dtype == "f32"``, uint16 bfloat16 bit patterns for ``"bf16"``.
    ``b_g`` is always float32.  ``as_f64`` widens a storage array exactly.
    """

    workload: Workload
    x: np.ndarray
    wg_t: np.ndarray
    wu_t: np.ndarray
    wd: np.ndarray
    b_g: np.ndarray
    scales: np.ndarray

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def rows_f64(self, name: str, rows) -> np.ndarray:
        a = getattr(self, name)[rows]
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def generate(w: Workload, beta: float | None = None) -> Inputs:
    """Draw the workload's inputs (see the module docstring for the rule)."""
    beta = w.beta if beta is None else beta
    sb = w.seed_base
    s = row_scales(w)
    x = _normal(sb + SEED_OFFSETS["x"], (w.T, w.d_model), 1.0)
    x *= s[:, None]
    wg = _normal(sb + SEED_OFFSETS["wg"], (w.d_ff, w.d_model), math.sqrt(1.0 / w.d_model))
    wu = _normal(sb + SEED_OFFSETS["wu"], (w.d_ff, w.d_model), math.sqrt(1.0 / w.d_model))
    wd = _normal(sb + SEED_OFFSETS["wd"], (w.d_ff, w.d_model), math.sqrt(1.0 / w.d_ff))
    b = np.full(w.d_ff, -beta, dtype=np.float32)
    return Inputs(w, _store(x, w.dtype), _store(wg, w.dtype), _store(wu, w.dtype),
                  _store(wd, w.dtype), b, s)


def generate_custom(T: int, d_model: int, d_ff: int, dtype: str, beta: float,
                    seed_base: int, cap: int = 8, rows: str = "unit", **kw) -> Inputs:
    """Inputs for an ad-hoc shape with the same drawing rule."""
    w = Workload("custom", T=T, d_model=d_model, d_ff=d_ff, dtype=dtype,
                 beta=beta, cap=cap, seed_base=seed_base, rows=rows, **kw)
    return generate(w)


def upstream_grad(w: Workload) -> np.ndarray:
    """A seeded upstream gradient dL/dy for the backward, [T, d_model]: unit
    normals in the workload's storage format (bf16 bit patterns or float32)."""
    return _store(_normal(w.seed_base + SEED_OFFSETS["gy"], (w.T, w.d_model), 1.0), w.dtype)



def generate_integer(T: int, d_model: int, d_ff: int, dtype: str, seed: int, m: int,
                     variant: str = "dense", density: float = 2.0 / 3.0) -> Inputs:
    """An exact-arithmetic fixture: x, wg_t, wu_t, wd hold only -1, 0 and 1
    and the gate bias is -(m + 1/2), so every pre-activation is a half-integer
    (never zero) and every product and sum of the forward is a small dyadic
    rational.  Draws only; the caller checks that its sizes keep every
    intermediate exactly representable in the arithmetic under test.

    variant "dense": every entry of x and the three weights is nonzero with
    probability ``density``, sign uniform.
    variant "one_hot": x and wg_t as above; each row of wu_t and of wd has a
    single +1 or -1 at a uniform position, so x_t . wu_t[j] is -1, 0 or 1 and
    each output column sums few terms (exact in bfloat16 at moderate sizes).
    """
    rng = np.random.Generator(np.random.PCG64(seed))

    def tern(shape):
        nz = rng.random(shape) < density
        sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        return np.where(nz, sign, 0.0).astype(np.float32)

    def one_hot(rows, cols):
        a = np.zeros((rows, cols), dtype=np.float32)
        pos = rng.integers(0, cols, size=rows)
        a[np.arange(rows), pos] = np.where(rng.random(rows) < 0.5, -1.0, 1.0)
        return a

    x = tern((T, d_model))
    wg = tern((d_ff, d_model))
    if variant == "dense":
        wu, wd = tern((d_ff, d_model)), tern((d_ff, d_model))
    elif variant == "one_hot":
        wu, wd = one_hot(d_ff, d_model), one_hot(d_ff, d_model)
    else:
        raise ValueError(f"unknown variant {variant!r}")
    b = np.full(d_ff, -(m + 0.5), dtype=np.float32)
    w = Workload("integer", T=T, d_model=d_model, d_ff=d_ff, dtype=dtype, beta=m + 0.5,
                 seed_base=seed)
    return Inputs(w, _store(x, dtype), _store(wg, dtype), _store(wu, dtype), _store(wd, dtype), b,
                  np.ones(T, dtype=np.float32))
