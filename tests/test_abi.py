"""The C ABI on the host: every symbol the header declares is exported, and
argument errors are reported before anything is launched (no GPU needed)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
HEADER = os.path.join(ROOT, "include", "sffn.h")


@pytest.fixture(scope="module")
def sffn():
    from activation_sparse_feed_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from activation_sparse_feed_amd import sffn as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("twell_pack", "sparse_ffn_fwd", "hybrid_route", "dense_ffn_ref",
              "sffn_workspace_bytes", "sffn_strerror"):
        assert n in names


def test_every_declared_symbol_is_exported(sffn):
    lib = ctypes.CDLL(sffn.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(sffn.EXPORTED)


def _shape(sffn, **kw):
    base = dict(T=64, d_model=256, d_ff=512, cap=8, dtype=sffn.SFFN_BF16)
    base.update(kw)
    s = sffn.make_shape(base["T"], base["d_model"], base["d_ff"], base["cap"], base["dtype"])
    for k in ("tile",):
        if k in kw:
            setattr(s, k, kw[k])
    return s


P = ctypes.c_void_p(0x10000)        # aligned fake device pointer: never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)


WS = ctypes.c_void_p(0x20000)


def _pack(sffn, s, x=P, w=P, b=None, c=P, i=P, v=P, n=None, ws=WS, ws_n=1 << 30):
    return sffn._lib.twell_pack(ctypes.byref(s) if s is not None else None, x, w, b, n, c, i, v,
                                ws, ws_n, None)


@pytest.mark.parametrize("kw,status", [
    (dict(tile=64), -2), (dict(d_ff=100), -2), (dict(d_ff=65536 + 128), -2),
    (dict(cap=129), -2), (dict(cap=-1), -1), (dict(T=-1), -1), (dict(d_model=12), -2),
    (dict(d_model=8200), -2), (dict(dtype=7), -1), (dict(d_model=0), -1),
])
def test_shape_errors(sffn, kw, status):
    assert _pack(sffn, _shape(sffn, **kw)) == status


def test_null_and_misaligned_pointers(sffn):
    s = _shape(sffn)
    assert _pack(sffn, None) == sffn.SFFN_ERR_ARG
    assert _pack(sffn, s, x=None) == sffn.SFFN_ERR_ARG
    assert _pack(sffn, s, w=MISALIGNED) == sffn.SFFN_ERR_ARG
    assert _pack(sffn, s, b=MISALIGNED) == sffn.SFFN_ERR_ARG
    assert _pack(sffn, s, c=None) == sffn.SFFN_ERR_ARG
    assert _pack(sffn, s, n=MISALIGNED) == sffn.SFFN_ERR_ARG
    assert sffn._lib.twell_weight_norms(ctypes.byref(s), P, None, None) == sffn.SFFN_ERR_ARG


def test_zero_tokens_is_ok_without_buffers(sffn):
    s = _shape(sffn, T=0)
    assert _pack(sffn, s, x=None, w=None, c=None, i=None, v=None, ws=None, ws_n=0) == sffn.SFFN_OK
    lib = sffn._lib
    assert lib.dense_ffn_ref(ctypes.byref(s), None, None, None, None, None, None, 0, None, None) == 0


def test_workspace_errors(sffn):
    s = _shape(sffn)
    lib = sffn._lib
    need_p = sffn.workspace_bytes(s, sffn.WS_PACK)
    assert need_p >= (64 + 512) * 4
    assert _pack(sffn, s, ws_n=need_p - 1) == -3
    assert _pack(sffn, s, ws=None) == -3
    # activations too large for 32-bit buffer offsets
    big = _shape(sffn, T=1 << 17, d_model=8192)
    assert _pack(sffn, big) == -2
    need = sffn.workspace_bytes(s, sffn.WS_DENSE)
    assert need >= 64 * 512 * 2
    assert lib.dense_ffn_ref(ctypes.byref(s), P, P, None, P, P, P, need - 1, P, None) == -3
    assert lib.dense_ffn_ref(ctypes.byref(s), P, P, None, P, P, None, need, P, None) == -3
    need_h = sffn.workspace_bytes(s, sffn.WS_HYBRID)
    assert need_h > 64 * 512 * 2
    assert lib.hybrid_route(ctypes.byref(s), P, P, None, P, P, P, P, P, P, need_h - 1, P, None) == -3
    # few tokens: the fused kernel splits columns and needs a partial buffer
    sd = _shape(sffn, T=4)
    need_s = sffn.workspace_bytes(sd, sffn.WS_SPARSE)
    assert need_s > 0
    assert lib.sparse_ffn_fwd(ctypes.byref(sd), P, P, P, P, P, P, P, None, 0, None) == -3
    assert sffn.workspace_bytes(_shape(sffn, T=4096), sffn.WS_SPARSE) == 0


def test_union_variant_refuses_unsupported_shapes(sffn):
    # checked on the host before any launch: d_model outside {512, ..., 4096},
    # cap above 32, float32
    lib = sffn._lib
    for d_model, cap, dt in ((768, 8, sffn.SFFN_BF16), (512, 33, sffn.SFFN_BF16),
                             (512, 8, sffn.SFFN_F32), (8192, 8, sffn.SFFN_BF16)):
        s = sffn.make_shape(16, d_model, 1024, cap, dt)
        assert lib.sparse_ffn_fwd_union(ctypes.byref(s), P, P, P, P, P, P, P, None) == -2
    s = sffn.make_shape(16, 512, 1000, 8, sffn.SFFN_BF16)  # d_ff not a multiple of 128
    assert lib.sparse_ffn_fwd_union(ctypes.byref(s), P, P, P, P, P, P, P, None) == -2
    s = sffn.make_shape(16, 512, 1024, 8, sffn.SFFN_BF16)
    assert lib.sparse_ffn_fwd_union(ctypes.byref(s), P, None, P, P, P, P, P, None) == -1


def test_workspace_query_of_invalid_shape_is_zero(sffn):
    assert sffn.workspace_bytes(_shape(sffn, tile=32), sffn.WS_DENSE) == 0
    assert sffn.workspace_bytes(_shape(sffn), 9) == 0


def test_strerror(sffn):
    for code in (0, -1, -2, -3, -4, 5):
        assert isinstance(sffn.strerror(code), str) and sffn.strerror(code)
    assert sffn.strerror(-3) != sffn.strerror(-1)


def test_conversion_baseline_errors(sffn):
    lib = sffn._lib
    s = _shape(sffn)
    ws_n = sffn.workspace_bytes(s, sffn.WS_CONVERT)
    assert ws_n >= (64 + 512) * 4
    sf = _shape(sffn, dtype=sffn.SFFN_F32)
    assert lib.gate_preact(ctypes.byref(sf), P, P, None, P, None) == -2
    assert lib.gate_preact(ctypes.byref(_shape(sffn, d_model=264)), P, P, None, P, None) == -2
    assert lib.gate_preact(ctypes.byref(s), P, P, None, None, None) == -1
    assert lib.twell_from_preact(ctypes.byref(s), P, P, P, None, None, P, P, P, WS, ws_n - 1,
                                 None) == -3
    assert lib.twell_from_preact(ctypes.byref(s), None, P, P, None, None, P, P, P, WS, ws_n,
                                 None) == -1
    assert lib.ell_from_preact(ctypes.byref(s), -1, P, P, P, None, None, P, P, P, WS, ws_n,
                               None) == -1
    assert lib.ell_from_preact(ctypes.byref(s), 513, P, P, P, None, None, P, P, P, WS, ws_n,
                               None) == -1
    assert lib.ell_from_preact(ctypes.byref(s), 4, P, P, P, None, None, P, None, P, WS, ws_n,
                               None) == -1
    assert lib.ell_from_preact(ctypes.byref(sf), 4, P, P, P, None, None, P, P, P, WS, ws_n,
                               None) == -2
    s0 = _shape(sffn, T=0)
    assert lib.ell_from_preact(ctypes.byref(s0), 0, None, None, None, None, None, None, None,
                               None, None, 0, None) == 0


def test_pack_l1_errors(sffn):
    lib = sffn._lib
    s = _shape(sffn)
    need = sffn.workspace_bytes(s, sffn.WS_PACK_L1)
    assert need > sffn.workspace_bytes(s, sffn.WS_PACK) + 64 * 4 * 4
    nan = float("nan")
    assert lib.twell_pack_l1(ctypes.byref(s), P, P, None, None, P, P, P, 1.0, P, WS, need - 1,
                             None) == -3
    assert lib.twell_pack_l1(ctypes.byref(s), P, P, None, None, P, P, P, 1.0, None, WS, need,
                             None) == -1
    assert lib.twell_pack_l1(ctypes.byref(s), P, P, None, None, P, P, P, nan, P, WS, need,
                             None) == -1
    assert lib.twell_pack_l1(ctypes.byref(_shape(sffn, tile=64)), P, P, None, None, P, P, P, 1.0,
                             P, WS, need, None) == -2


def test_backward_errors(sffn):
    lib = sffn._lib
    s = _shape(sffn, d_model=512)
    need = sffn.workspace_bytes(s, sffn.WS_BACKWARD)
    assert need >= 20 * 64 * 512
    # ..., routed, n_routed, max_routed, gy, l1_lambda, gx, gwg_t, gwu_t, gwd, gb
    args = [P] * 11 + [64, P, 0.25] + [P] * 5
    args[2] = None   # b_g
    args[5] = None   # wg_norms
    args[18] = None  # gb
    assert lib.sparse_ffn_bwd(ctypes.byref(s), *args, WS, need - 1, None) == -3
    bad = list(args)
    bad[14] = None   # gx
    assert lib.sparse_ffn_bwd(ctypes.byref(s), *bad, WS, need, None) == -1
    bad = list(args)
    bad[13] = float("nan")  # l1_lambda
    assert lib.sparse_ffn_bwd(ctypes.byref(s), *bad, WS, need, None) == -1
    for mr in (-1, 65):   # max_routed outside 0..T
        bad = list(args)
        bad[11] = mr
        assert lib.sparse_ffn_bwd(ctypes.byref(s), *bad, WS, need, None) == -1
    # a smaller routed-row bound needs a smaller workspace, and that one is enough
    small = sffn.backward_workspace_bytes(s, 4)
    assert 0 < small < need and sffn.backward_workspace_bytes(s, 64) == need
    assert sffn.backward_workspace_bytes(s, 65) == 0
    bad = list(args)
    bad[11] = 4
    assert lib.sparse_ffn_bwd(ctypes.byref(s), *bad, WS, small - 1, None) == -3
    bad = list(args)
    bad[9] = MISALIGNED  # routed
    assert lib.sparse_ffn_bwd(ctypes.byref(s), *bad, WS, need, None) == -1
    # bf16 is taken up to d_model 4096
    s264 = _shape(sffn, d_model=4104)
    n264 = sffn.workspace_bytes(s264, sffn.WS_BACKWARD)
    assert lib.sparse_ffn_bwd(ctypes.byref(s264), *args, WS, n264, None) == -2
    # float32 is taken up to d_model 2048
    sf = _shape(sffn, d_model=2056, dtype=sffn.SFFN_F32)
    assert lib.sparse_ffn_bwd(ctypes.byref(sf), *args, WS, sffn.workspace_bytes(sf, 6), None) == -2
    sf512 = _shape(sffn, d_model=512, dtype=sffn.SFFN_F32)
    assert sffn.workspace_bytes(sf512, 6) >= 40 * 64 * 512  # complete lists and their gradients
    s0 = _shape(sffn, T=0)
    assert lib.sparse_ffn_bwd(ctypes.byref(s0), *([None] * 11), 0, None, 0.0, *([None] * 5), None,
                              0, None) == 0



def test_probe_errors(sffn):
    lib = sffn._lib
    ARG = sffn.SFFN_ERR_ARG
    assert lib.sffn_probe_hbm(None, None, 1024, 64, None) == ARG
    assert lib.sffn_probe_hbm(MISALIGNED, None, 1024, 64, None) == ARG
    assert lib.sffn_probe_hbm(P, MISALIGNED, 1024, 64, None) == ARG
    assert lib.sffn_probe_hbm(P, None, 1000, 64, None) == ARG      # not a multiple of 16
    assert lib.sffn_probe_hbm(P, None, 1024, 0, None) == ARG
    assert lib.sffn_probe_hbm(P, None, 0, 64, None) == sffn.SFFN_OK  # nothing to do
    assert lib.sffn_probe_mfma(None, 4, 16, None) == ARG
    assert lib.sffn_probe_mfma(P, 0, 16, None) == ARG
    assert lib.sffn_probe_mfma(P, 4, 0, None) == ARG
    assert lib.sffn_probe_mfma(P, 4, 8192, None) == ARG
    assert lib.sffn_probe_mfma_step(None, P, P, P, 1, None) == ARG
    assert lib.sffn_probe_mfma_step(P, P, P, MISALIGNED, 1, None) == ARG
    assert lib.sffn_probe_mfma_step(P, P, P, P, 0, None) == ARG
    assert lib.sffn_probe_cached(None, 1024, 1, 1, None) == ARG
    assert lib.sffn_probe_cached(P, 1000, 1, 1, None) == ARG
    assert lib.sffn_probe_cached(P, 1024, 0, 1, None) == ARG
    assert lib.sffn_probe_cached(P, 1024, 1, 0, None) == ARG
    assert lib.sffn_probe_gather(P, P, P, -1, 8192, None) == ARG
    assert lib.sffn_probe_gather(P, P, P, 4, 3000, None) == ARG
    assert lib.sffn_probe_gather(P, P, P, 0, 8192, None) == sffn.SFFN_OK
    assert lib.sffn_probe_bf16_round(None, P, 4, None) == ARG
    assert lib.sffn_probe_bf16_round(P, None, 4, None) == ARG
    assert lib.sffn_probe_bf16_round(P, P, 0, None) == sffn.SFFN_OK


def test_noalloc_rejects_shapes_beyond_its_scratch(sffn):
    """twell_pack_noalloc checks the workspace its shape needs against its
    static scratch on the host, before any device call."""
    lib = sffn._lib
    cap_bytes = sffn.twell_pack_noalloc_max_bytes()
    assert cap_bytes == 32 << 20
    big = _shape(sffn, T=9_000_000, d_model=8, d_ff=512)   # row norms alone exceed 32 MiB
    assert sffn.workspace_bytes(big, sffn.WS_PACK) > cap_bytes
    assert lib.twell_pack_noalloc(ctypes.byref(big), P, P, None, None, P, P, P, None) == \
        sffn.SFFN_ERR_TOO_LARGE
    assert "scratch" in sffn.strerror(sffn.SFFN_ERR_TOO_LARGE)
    ok = _shape(sffn)
    assert lib.twell_pack_noalloc(ctypes.byref(ok), None, P, None, None, P, P, P, None) == \
        sffn.SFFN_ERR_ARG
    assert lib.twell_pack_noalloc(ctypes.byref(_shape(sffn, T=0)), None, None, None, None, None,
                                  None, None, None) == sffn.SFFN_OK
