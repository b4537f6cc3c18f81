"""twell_pack_noalloc against twell_pack: the allocation-free entry point
(static device scratch instead of a workspace) must give the same TwELL
arrays bit for bit, and the oracle's counts and live indices, on two calls in
a row whose second input is smaller (the scratch keeps the first call's
contents), for the 256-row gate and for the few-token split-K gate whose
partial tiles live in the scratch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from activation_sparse_feed_amd import workloads as wl
from helpers import check_twell, device_inputs, oracle_rows, sample_rows, to_f64

pytestmark = pytest.mark.gpu


def _pack_both(inp, cap, norms):
    from activation_sparse_feed_amd import sffn
    w = inp.workload
    code = sffn.SFFN_BF16 if w.dtype == "bf16" else sffn.SFFN_F32
    shape = sffn.make_shape(w.T, w.d_model, w.d_ff, cap, code)
    d = device_inputs(inp)
    wn = None
    if norms:
        wn = torch.empty(w.d_ff, dtype=torch.float32, device="cuda")
        sffn.twell_weight_norms(shape, d["wg_t"], wn)
    ws = sffn.alloc_workspace(shape, sffn.WS_PACK)
    ref = sffn.alloc_twell(shape)
    sffn.twell_pack(shape, d["x"], d["wg_t"], d["b_g"], *ref, ws, wn)
    out = sffn.alloc_twell(shape)
    sffn.twell_pack_noalloc(shape, d["x"], d["wg_t"], d["b_g"], *out, wn)
    torch.cuda.synchronize()
    return ref, out


def _same(ref, out, cap):
    c1, i1, v1 = ref
    c2, i2, v2 = out
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    live = torch.arange(cap, device="cuda")[None, None, :] < torch.clamp(
        c1.to(torch.int32), max=cap)[:, :, None]
    assert torch.equal(torch.where(live, i1.to(torch.int32), -1),
                       torch.where(live, i2.to(torch.int32), -1))
    assert torch.equal(torch.where(live, v1.float(), 0.0), torch.where(live, v2.float(), 0.0))


@pytest.mark.parametrize("first,second", [
    # 256-row gate: prefill shape, then a smaller ragged one
    (dict(T=4096, d_model=2048, d_ff=5632, beta=2.326, cap=8, norms=False),
     dict(T=300, d_model=512, d_ff=1024, beta=1.9, cap=4, norms=True)),
    # few-token split-K gate (partial tiles in the scratch): decode, then fewer
    (dict(T=48, d_model=4096, d_ff=11008, beta=2.326, cap=8, norms=True),
     dict(T=7, d_model=1024, d_ff=2048, beta=1.5, cap=8, norms=False)),
])
def test_noalloc_matches_twell_pack(first, second):
    for n, spec in enumerate((first, second)):
        spec = dict(spec)
        norms, cap = spec.pop("norms"), spec["cap"]
        inp = wl.generate_custom(dtype="bf16", seed_base=90 + n, **spec)
        ref, out = _pack_both(inp, cap, norms)
        _same(ref, out, cap)
        rows = sample_rows(spec["T"], 64, seed=n)
        o = oracle_rows(inp, rows, 128, cap, dense=False)
        c, i, v = out
        check_twell("bf16", c.cpu().numpy()[rows], i.cpu().numpy()[rows], to_f64(v)[rows], o, cap)
        print(f"noalloc T={spec['T']} K={spec['d_model']} N={spec['d_ff']}: identical to twell_pack")
