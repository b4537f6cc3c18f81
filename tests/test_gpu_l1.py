"""GPU parity of the L1 activation regulariser fused into the gate epilogue
(twell_pack_l1) against the oracle's l1_term, on every gate kernel: the
256-row bf16 GEMM, the few-token split-K kernels, the 128-row bf16 kernel
(d_model not a multiple of 32) and the float32 kernel.

The bound is rigorous: each active z carries at most the accumulation error
of its guard band (taken here with the float32 coefficient 2^-22 (K + 2),
which covers every kernel's summation order), the float32 partial sums of
positive terms (at most about 30 additions deep, under 2^-19 relative) are
taken with 2^-17, and the result is rounded to float32 once; the 128-row bf16 kernel sums z rounded to bf16 (2^-8 relative).
Activity is exact on both sides, so inactive entries add nothing to either.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from activation_sparse_feed_amd import workloads as wl
from helpers import device_inputs

pytestmark = pytest.mark.gpu


def _sffn():
    from activation_sparse_feed_amd import sffn
    return sffn


def run_l1(inp: wl.Inputs, cap: int, lam: float):
    sffn = _sffn()
    w = inp.workload
    d = device_inputs(inp)
    dt = sffn.SFFN_BF16 if w.dtype == "bf16" else sffn.SFFN_F32
    s = sffn.make_shape(w.T, w.d_model, w.d_ff, cap, dt)
    out = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    tw = sffn.alloc_twell(s)
    sffn.twell_pack_l1(s, d["x"], d["wg_t"], d["b_g"], *tw, lam, out,
                       sffn.alloc_workspace(s, sffn.WS_PACK_L1))
    ref_tw = sffn.alloc_twell(s)
    sffn.twell_pack(s, d["x"], d["wg_t"], d["b_g"], *ref_tw, sffn.alloc_workspace(s, sffn.WS_PACK))
    torch.cuda.synchronize()
    return float(out.item()), tw, ref_tw


def l1_bound(inp: wl.Inputs, z: np.ndarray, lam: float, value: float) -> float:
    w = inp.workload
    x, wg = inp.as_f64("x"), inp.as_f64("wg_t")
    act = z > 0
    band = (2.0 ** -22 * (w.d_model + 2) * np.outer(np.linalg.norm(x, axis=1), np.linalg.norm(wg, axis=1))
            + 2.0 ** -22 * np.abs(inp.b_g.astype(np.float64))[None, :])
    hsum = float(z[act].sum())
    rel = 2.0 ** -17 + (2.0 ** -8 if (w.dtype == "bf16" and w.d_model % 32) else 0.0)
    return lam / w.T * (float(band[act].sum()) + rel * hsum) + 2.0 ** -23 * abs(value)


@pytest.mark.parametrize("T,d_model,d_ff,dtype,beta,cap", [
    (300, 512, 1024, "bf16", 1.9, 4),    # 256-row GEMM, ragged rows, overflowing tiles
    (48, 512, 768, "bf16", 1.5, 8),      # few tokens: split-K stream + epilogue
    (130, 264, 384, "bf16", 1.2, 8),     # d_model % 32 != 0: 128-row bf16 kernel
    (70, 264, 384, "f32", 1.7, 3),       # float32 kernel
])
def test_l1_value(T, d_model, d_ff, dtype, beta, cap):
    inp = wl.generate_custom(T=T, d_model=d_model, d_ff=d_ff, dtype=dtype, beta=beta,
                             seed_base=40 + T, cap=cap)
    lam = 0.03
    got, tw, ref_tw = run_l1(inp, cap, lam)
    z = oracle.gate_preact(inp.as_f64("x"), inp.as_f64("wg_t"), inp.b_g)
    want = oracle.l1_term(z, lam)
    assert want > 0
    assert abs(got - want) <= l1_bound(inp, z, lam, want), (got, want)
    # the TwELL outputs are twell_pack's
    assert torch.equal(tw[0], ref_tw[0])


def test_l1_decode_and_prefill_full_size():
    for name in ("decode_1pct", "prefill_1pct"):
        w = wl.WORKLOADS[name]
        inp = wl.generate(w)
        got, _, _ = run_l1(inp, w.cap, 1.0)
        z = oracle.gate_preact(inp.as_f64("x"), inp.as_f64("wg_t"), inp.b_g)
        want = oracle.l1_term(z, 1.0)
        assert abs(got - want) <= l1_bound(inp, z, 1.0, want), (name, got, want)


def test_l1_no_tokens_writes_zero():
    sffn = _sffn()
    s = sffn.make_shape(0, 256, 512, 8, sffn.SFFN_BF16)
    out = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    sffn.twell_pack_l1(s, e, e, None, e, e, e, 1.0, out, torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert out.item() == 0.0
