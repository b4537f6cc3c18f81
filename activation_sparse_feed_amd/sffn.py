"""Python binding of libsffn.so: argument marshalling only.

Every function takes torch tensors that live on the GPU, checks their dtype,
shape and contiguity, and passes raw device pointers plus the current HIP
stream to the C entry point of the same name.  All arithmetic happens in the
library's kernels; there is no fallback: if the library is missing, importing
this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsffn.so")

SFFN_OK, SFFN_ERR_ARG, SFFN_ERR_UNSUPPORTED, SFFN_ERR_WORKSPACE, SFFN_ERR_HIP = 0, -1, -2, -3, -4
SFFN_ERR_TOO_LARGE = -5
SFFN_F32, SFFN_BF16 = 0, 1
WS_HYBRID, WS_DENSE, WS_SPARSE, WS_PACK, WS_CONVERT, WS_PACK_L1, WS_BACKWARD = 0, 1, 2, 3, 4, 5, 6
TILE = 128

EXPORTED = ("twell_weight_norms", "twell_pack", "twell_pack_noalloc",
            "twell_pack_noalloc_max_bytes", "twell_pack_l1", "sparse_ffn_fwd", "sparse_ffn_fwd_union",
            "hybrid_route",
            "dense_ffn_ref", "sparse_ffn_bwd", "gate_preact", "twell_from_preact",
            "ell_from_preact", "sffn_probe_hbm", "sffn_probe_mfma", "sffn_probe_mfma_step",
            "sffn_probe_cached", "sffn_probe_gather", "sffn_probe_bf16_round",
            "sffn_workspace_bytes", "sparse_ffn_bwd_workspace_bytes", "sffn_strerror")


class SffnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("cap", ctypes.c_int32), ("dtype", ctypes.c_int32)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m activation_sparse_feed_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    sp = ctypes.POINTER(Shape)
    lib.twell_weight_norms.argtypes = [sp, vp, vp, vp]
    lib.twell_pack.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.twell_pack_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.twell_pack_noalloc_max_bytes.argtypes = []
    lib.twell_pack_noalloc_max_bytes.restype = sz
    lib.twell_pack_l1.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, sz, vp]
    lib.sparse_ffn_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sparse_ffn_fwd_union.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hybrid_route.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.dense_ffn_ref.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.gate_preact.argtypes = [sp, vp, vp, vp, vp, vp]
    lib.sparse_ffn_bwd.argtypes = [sp] + [vp] * 11 + [i32, vp, ctypes.c_float] + [vp] * 5 + [vp, sz, vp]
    lib.sparse_ffn_bwd_workspace_bytes.argtypes = [sp, i32]
    lib.sparse_ffn_bwd_workspace_bytes.restype = sz
    lib.sffn_probe_hbm.argtypes = [vp, vp, sz, i32, vp]
    lib.sffn_probe_mfma.argtypes = [vp, i32, i32, vp]
    lib.sffn_probe_mfma_step.argtypes = [vp, vp, vp, vp, i32, vp]
    lib.sffn_probe_cached.argtypes = [vp, sz, i32, i32, vp]
    lib.sffn_probe_gather.argtypes = [vp, vp, vp, i32, i32, vp]
    lib.sffn_probe_bf16_round.argtypes = [vp, vp, sz, vp]
    lib.twell_from_preact.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ell_from_preact.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    for fn in ("twell_weight_norms", "twell_pack", "twell_pack_noalloc", "twell_pack_l1",
               "sparse_ffn_fwd", "sparse_ffn_fwd_union", "hybrid_route", "dense_ffn_ref", "sparse_ffn_bwd", "gate_preact", "twell_from_preact",
               "ell_from_preact", "sffn_probe_hbm", "sffn_probe_mfma", "sffn_probe_mfma_step",
               "sffn_probe_cached", "sffn_probe_gather", "sffn_probe_bf16_round"):
        getattr(lib, fn).restype = i32
    lib.sffn_workspace_bytes.argtypes = [sp, i32]
    lib.sffn_workspace_bytes.restype = sz
    lib.sffn_strerror.argtypes = [i32]
    lib.sffn_strerror.restype = ctypes.c_char_p
    return lib


_lib = load_library()


def strerror(status: int) -> str:
    return _lib.sffn_strerror(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != SFFN_OK:
        raise SffnError(fn, status, strerror(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SFFN_BF16
    if t.dtype == torch.float32:
        return SFFN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_shape(T: int, d_model: int, d_ff: int, cap: int, dtype: int, tile: int = TILE) -> Shape:
    return Shape(int(T), int(d_model), int(d_ff), int(tile), int(cap), int(dtype))


def shape_of(x: torch.Tensor, w: torch.Tensor, cap: int) -> Shape:
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [T, d_model] and weights [d_ff, d_model]")
    if x.dtype != w.dtype:
        raise TypeError("x and the weights must share a dtype")
    return make_shape(x.shape[0], x.shape[1], w.shape[0], cap, _dtype_code(x))


def workspace_bytes(shape: Shape, which: int) -> int:
    return int(_lib.sffn_workspace_bytes(ctypes.byref(shape), int(which)))


def alloc_workspace(shape: Shape, which: int, device=None) -> torch.Tensor:
    """Device workspace for one call kind (no call needs initial contents; it
    is zero-filled only so that its bytes are defined)."""
    n = workspace_bytes(shape, which)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device or "cuda")


def alloc_twell(shape: Shape, device=None):
    """count [T, n_tiles] u16, idx [T, n_tiles, cap] u16, val [T, n_tiles, cap] dtype."""
    nt = shape.d_ff // shape.tile
    dt = torch.bfloat16 if shape.dtype == SFFN_BF16 else torch.float32
    dev = device or "cuda"
    count = torch.empty((shape.T, nt), dtype=torch.uint16, device=dev)
    idx = torch.empty((shape.T, nt, max(shape.cap, 1)), dtype=torch.uint16, device=dev)
    val = torch.empty((shape.T, nt, max(shape.cap, 1)), dtype=dt, device=dev)
    return count, idx, val


def twell_weight_norms(shape: Shape, wg_t, wg_norms, stream=None) -> None:
    _check("twell_weight_norms", _lib.twell_weight_norms(ctypes.byref(shape), _ptr(wg_t),
                                                         _ptr(wg_norms), _stream(stream)))


def twell_pack(shape: Shape, x, wg_t, b_g, count, idx, val, workspace, wg_norms=None,
               stream=None) -> None:
    ws_n = workspace.numel() * workspace.element_size()
    _check("twell_pack", _lib.twell_pack(ctypes.byref(shape), _ptr(x), _ptr(wg_t), _ptr(b_g),
                                         _ptr(wg_norms), _ptr(count), _ptr(idx), _ptr(val),
                                         _ptr(workspace), ws_n, _stream(stream)))


def twell_pack_noalloc(shape: Shape, x, wg_t, b_g, count, idx, val, wg_norms=None,
                       stream=None) -> None:
    _check("twell_pack_noalloc", _lib.twell_pack_noalloc(
        ctypes.byref(shape), _ptr(x), _ptr(wg_t), _ptr(b_g), _ptr(wg_norms), _ptr(count),
        _ptr(idx), _ptr(val), _stream(stream)))


def twell_pack_noalloc_max_bytes() -> int:
    return int(_lib.twell_pack_noalloc_max_bytes())


def twell_pack_l1(shape: Shape, x, wg_t, b_g, count, idx, val, lam: float, l1_value, workspace,
                  wg_norms=None, stream=None) -> None:
    if l1_value.dtype != torch.float32 or l1_value.numel() < 1:
        raise ValueError("l1_value must be a float32 device tensor with one element")
    ws_n = workspace.numel() * workspace.element_size()
    _check("twell_pack_l1", _lib.twell_pack_l1(
        ctypes.byref(shape), _ptr(x), _ptr(wg_t), _ptr(b_g), _ptr(wg_norms), _ptr(count),
        _ptr(idx), _ptr(val), float(lam), _ptr(l1_value), _ptr(workspace), ws_n, _stream(stream)))


def sparse_ffn_fwd(shape: Shape, x, wu_t, wd, count, idx, val, y, workspace=None,
                   stream=None) -> None:
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("sparse_ffn_fwd", _lib.sparse_ffn_fwd(
        ctypes.byref(shape), _ptr(x), _ptr(wu_t), _ptr(wd), _ptr(count), _ptr(idx), _ptr(val),
        _ptr(y), _ptr(workspace), ws_n, _stream(stream)))


def sparse_ffn_fwd_union(shape: Shape, x, wu_t, wd, count, idx, val, y, stream=None) -> None:
    _check("sparse_ffn_fwd_union", _lib.sparse_ffn_fwd_union(
        ctypes.byref(shape), _ptr(x), _ptr(wu_t), _ptr(wd), _ptr(count), _ptr(idx), _ptr(val),
        _ptr(y), _stream(stream)))


def hybrid_route(shape: Shape, x, wg_t, b_g, wu_t, wd, count, routed, n_routed, workspace, y,
                 stream=None) -> None:
    ws_n = workspace.numel() * workspace.element_size()
    _check("hybrid_route", _lib.hybrid_route(
        ctypes.byref(shape), _ptr(x), _ptr(wg_t), _ptr(b_g), _ptr(wu_t), _ptr(wd), _ptr(count),
        _ptr(routed), _ptr(n_routed), _ptr(workspace), ws_n, _ptr(y), _stream(stream)))


def probe_hbm(src, dst=None, workgroups: int = 4096, stream=None) -> None:
    """One streaming pass over src (copied to dst, or only read when dst is None)."""
    n = src.numel() * src.element_size()
    _check("sffn_probe_hbm", _lib.sffn_probe_hbm(_ptr(src), _ptr(dst), n, int(workgroups),
                                                 _stream(stream)))


def probe_mfma(out, iters: int, stream=None) -> None:
    """out: float32 with a multiple of 256 elements (one workgroup per 256)."""
    wgs = out.numel() // 256
    _check("sffn_probe_mfma", _lib.sffn_probe_mfma(_ptr(out), int(wgs), int(iters),
                                                   _stream(stream)))


def probe_cached(src, window_bytes: int, reps: int, workgroups: int, stream=None) -> None:
    """Every workgroup reads src[0:window_bytes] reps times (cached-load rate)."""
    if window_bytes > src.numel() * src.element_size():
        raise ValueError("window larger than the buffer")
    _check("sffn_probe_cached", _lib.sffn_probe_cached(_ptr(src), int(window_bytes), int(reps),
                                                       int(workgroups), _stream(stream)))


def probe_bf16_round(x, out, stream=None) -> None:
    """out = the library's float32 -> bfloat16 rounding of x (uint16 bits)."""
    if x.dtype != torch.float32 or out.dtype not in (torch.int16, torch.uint16):
        raise TypeError("x must be float32 and out 16-bit integer")
    if out.numel() < x.numel():
        raise ValueError("out too small")
    _check("sffn_probe_bf16_round", _lib.sffn_probe_bf16_round(_ptr(x), _ptr(out), int(x.numel()),
                                                               _stream(stream)))


def probe_gather(a, b, rows, row_bytes: int, max_row=None, stream=None) -> None:
    """Read rows[i] of a and of b (row_bytes per row) for every listed row.
    max_row: the largest entry of rows when the caller knows it (then rows is
    not read back from the device here, e.g. inside a timed region)."""
    if rows.dtype != torch.int32:
        raise TypeError("rows must be int32")
    n_a = a.numel() * a.element_size() // row_bytes
    n_b = b.numel() * b.element_size() // row_bytes
    top = (int(rows.max().item()) if rows.numel() else -1) if max_row is None else int(max_row)
    if top >= min(n_a, n_b):
        raise ValueError("row index beyond the matrices")
    _check("sffn_probe_gather", _lib.sffn_probe_gather(_ptr(a), _ptr(b), _ptr(rows),
                                                       int(rows.numel()), int(row_bytes),
                                                       _stream(stream)))


def probe_mfma_step(a, b, c, d, stream=None) -> None:
    """a, b: uint16/int16 [waves, 64, 8] operand registers; c, d: float32
    [waves, 64, 4] accumulators in and out (one MFMA per wave)."""
    waves = d.numel() // 256
    if a.numel() != waves * 512 or b.numel() != waves * 512 or c.numel() != waves * 256 \
            or d.numel() != waves * 256 or waves <= 0:
        raise ValueError("a, b: [waves, 64, 8]; c, d: [waves, 64, 4]")
    if c.dtype != torch.float32 or d.dtype != torch.float32:
        raise TypeError("c and d must be float32")
    _check("sffn_probe_mfma_step", _lib.sffn_probe_mfma_step(_ptr(a), _ptr(b), _ptr(c), _ptr(d),
                                                             int(waves), _stream(stream)))


def dense_ffn_ref(shape: Shape, x, wg_t, b_g, wu_t, wd, workspace, y, stream=None) -> None:
    ws_n = workspace.numel() * workspace.element_size()
    _check("dense_ffn_ref", _lib.dense_ffn_ref(
        ctypes.byref(shape), _ptr(x), _ptr(wg_t), _ptr(b_g), _ptr(wu_t), _ptr(wd),
        _ptr(workspace), ws_n, _ptr(y), _stream(stream)))


def backward_workspace_bytes(shape: Shape, max_routed: int) -> int:
    return int(_lib.sparse_ffn_bwd_workspace_bytes(ctypes.byref(shape), int(max_routed)))


def sparse_ffn_bwd(shape: Shape, x, wg_t, b_g, wu_t, wd, count, idx, val, routed, n_routed, gy,
                   gx, gwg_t, gwu_t, gwd, gb, workspace, wg_norms=None, l1_lambda: float = 0.0,
                   max_routed=None, stream=None) -> None:
    """max_routed: routed rows the workspace holds (default T, the workspace of
    alloc_workspace(shape, WS_BACKWARD)); see backward_workspace_bytes."""
    mr = shape.T if max_routed is None else int(max_routed)
    for name, t in (("gwg_t", gwg_t), ("gwu_t", gwu_t), ("gwd", gwd)):
        if t.dtype != torch.float32 or tuple(t.shape) != (shape.d_ff, shape.d_model):
            raise ValueError(f"{name} must be float32 [d_ff, d_model]")
    if gb is not None and (gb.dtype != torch.float32 or gb.numel() != shape.d_ff):
        raise ValueError("gb must be float32 [d_ff]")
    ws_n = workspace.numel() * workspace.element_size()
    _check("sparse_ffn_bwd", _lib.sparse_ffn_bwd(
        ctypes.byref(shape), _ptr(x), _ptr(wg_t), _ptr(b_g), _ptr(wu_t), _ptr(wd), _ptr(wg_norms),
        _ptr(count), _ptr(idx), _ptr(val), _ptr(routed), _ptr(n_routed), mr, _ptr(gy),
        float(l1_lambda), _ptr(gx), _ptr(gwg_t), _ptr(gwu_t), _ptr(gwd), _ptr(gb), _ptr(workspace),
        ws_n, _stream(stream)))


def gate_preact(shape: Shape, x, wg_t, b_g, z, stream=None) -> None:
    if z.dtype != torch.float32 or tuple(z.shape) != (shape.T, shape.d_ff):
        raise ValueError("z must be float32 [T, d_ff]")
    _check("gate_preact", _lib.gate_preact(ctypes.byref(shape), _ptr(x), _ptr(wg_t), _ptr(b_g),
                                           _ptr(z), _stream(stream)))


def twell_from_preact(shape: Shape, z, x, wg_t, b_g, count, idx, val, workspace, wg_norms=None,
                      stream=None) -> None:
    ws_n = workspace.numel() * workspace.element_size()
    _check("twell_from_preact", _lib.twell_from_preact(
        ctypes.byref(shape), _ptr(z), _ptr(x), _ptr(wg_t), _ptr(b_g), _ptr(wg_norms), _ptr(count),
        _ptr(idx), _ptr(val), _ptr(workspace), ws_n, _stream(stream)))


def alloc_ell(shape: Shape, width: int, device=None):
    """Row-wise ELLPACK buffers: count [T] u16, idx [T, width] u16, val [T, width] bf16."""
    dev = device or "cuda"
    count = torch.empty(shape.T, dtype=torch.uint16, device=dev)
    idx = torch.empty((shape.T, max(width, 1)), dtype=torch.uint16, device=dev)
    val = torch.empty((shape.T, max(width, 1)), dtype=torch.bfloat16, device=dev)
    return count, idx, val


def ell_from_preact(shape: Shape, width: int, z, x, wg_t, b_g, count, idx, val, workspace,
                    wg_norms=None, stream=None) -> None:
    ws_n = workspace.numel() * workspace.element_size()
    _check("ell_from_preact", _lib.ell_from_preact(
        ctypes.byref(shape), int(width), _ptr(z), _ptr(x), _ptr(wg_t), _ptr(b_g), _ptr(wg_norms),
        _ptr(count), _ptr(idx), _ptr(val), _ptr(workspace), ws_n, _stream(stream)))


class SparseFFN:
    """Buffers for repeated sparse forwards of one shape: TwELL arrays, routed
    list, workspaces.  ``forward`` issues twell_pack, sparse_ffn_fwd and
    hybrid_route on one stream with no host synchronisation.  ``wg_norms``
    (from ``weight_norms``) may be passed to skip recomputing the gate-weight
    row norms on every call."""

    def __init__(self, T: int, d_model: int, d_ff: int, cap: int, dtype: torch.dtype,
                 device="cuda"):
        code = SFFN_BF16 if dtype == torch.bfloat16 else SFFN_F32
        self.shape = make_shape(T, d_model, d_ff, cap, code)
        self.dtype = dtype
        self.count, self.idx, self.val = alloc_twell(self.shape, device)
        self.routed = torch.empty(max(T, 1), dtype=torch.int32, device=device)
        self.n_routed = torch.zeros(1, dtype=torch.int32, device=device)
        self.ws_sparse = alloc_workspace(self.shape, WS_SPARSE, device)
        self.ws_pack = alloc_workspace(self.shape, WS_PACK, device)
        self.ws_hybrid = alloc_workspace(self.shape, WS_HYBRID, device)
        self.y = torch.empty((T, d_model), dtype=dtype, device=device)

    def weight_norms(self, wg_t, stream=None) -> torch.Tensor:
        n = torch.empty(self.shape.d_ff, dtype=torch.float32, device=wg_t.device)
        twell_weight_norms(self.shape, wg_t, n, stream)
        return n

    def forward(self, x, wg_t, b_g, wu_t, wd, wg_norms=None, stream=None) -> torch.Tensor:
        s = self.shape
        twell_pack(s, x, wg_t, b_g, self.count, self.idx, self.val, self.ws_pack, wg_norms, stream)
        sparse_ffn_fwd(s, x, wu_t, wd, self.count, self.idx, self.val, self.y, self.ws_sparse,
                       stream)
        hybrid_route(s, x, wg_t, b_g, wu_t, wd, self.count, self.routed, self.n_routed,
                     self.ws_hybrid, self.y, stream)
        return self.y


class DenseFFN:
    """Buffers for repeated dense reference forwards of one shape."""

    def __init__(self, T: int, d_model: int, d_ff: int, dtype: torch.dtype, device="cuda"):
        code = SFFN_BF16 if dtype == torch.bfloat16 else SFFN_F32
        self.shape = make_shape(T, d_model, d_ff, 0, code)
        self.ws = alloc_workspace(self.shape, WS_DENSE, device)
        self.y = torch.empty((T, d_model), dtype=dtype, device=device)

    def forward(self, x, wg_t, b_g, wu_t, wd, stream=None) -> torch.Tensor:
        dense_ffn_ref(self.shape, x, wg_t, b_g, wu_t, wd, self.ws, self.y, stream)
        return self.y
