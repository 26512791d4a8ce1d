"""qdec: weight-only quantized matmul for MI355X (gfx950), y = W_hat x.

A thin ctypes binding over the C ABI of ``libqdec.so`` (``include/qdec.h``).
The functions carry the C names (``qdec_gemv`` ...) and only marshal
arguments: every step of the computation runs in the library's HIP kernels.
PyTorch provides device memory and streams.  Importing this package fails
loudly when the library has not been built (``__graft_entry__.build()``);
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqdec.so")

QDEC_OK, QDEC_EINVAL, QDEC_EUNSUPPORTED, QDEC_EWORKSPACE, QDEC_EHIP, QDEC_ENODEV = 0, -1, -2, -3, -4, -5
QDEC_CODE_HYB, QDEC_CODE_1MAD, QDEC_CODE_3INST, QDEC_CODE_NUQ, QDEC_CODE_VQ, QDEC_CODE_LUT = 1, 2, 3, 4, 5, 6
QDEC_OP_GEMV, QDEC_OP_GEMM, QDEC_OP_ENCODE = 1, 2, 3
QDEC_ABI_VERSION = 2

# The exported symbols, as declared in include/qdec.h.
EXPORTS = ("qdec_abi_version", "qdec_status_string", "qdec_last_error", "qdec_workspace_bytes",
           "qdec_rht", "qdec_gemv", "qdec_gemm", "qdec_decode_tile", "qdec_encode",
           "qdec_gemv_group", "qdec_gemv_group_workspace_bytes", "qdec_gemv_noalloc",
           "qdec_noalloc_scratch_bytes", "qdec_debug_fail_launches")
GEMV_GROUP_MAX = 8


class QdecError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = ""
        if status == QDEC_EHIP:
            detail = ": " + _lib.qdec_last_error().decode()
        super().__init__("%s failed: %s (%d)%s" % (what, _status_string(status), status, detail))


class qdec_layer(ctypes.Structure):
    """Mirror of ``struct qdec_layer`` (include/qdec.h)."""
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("code", ctypes.c_int32),
        ("L", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32), ("Q", ctypes.c_int32),
        ("kv", ctypes.c_int32), ("kv_b", ctypes.c_int32), ("m_a", ctypes.c_int64),
        ("m", ctypes.c_int64), ("n", ctypes.c_int64),
        ("codes", ctypes.c_void_p), ("lut", ctypes.c_void_p), ("group_scale", ctypes.c_void_p),
        ("group", ctypes.c_int32), ("layer_scale", ctypes.c_float),
        ("sign_in", ctypes.c_void_p), ("sign_out", ctypes.c_void_p),
        ("had_in", ctypes.c_int32), ("had_out", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqdec.so is not built (%s); run __graft_entry__.build() -- "
                          "there is no fallback path" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.qdec_abi_version.restype = ctypes.c_uint32
    lib.qdec_abi_version.argtypes = []
    lib.qdec_debug_fail_launches.restype = ctypes.c_int
    lib.qdec_debug_fail_launches.argtypes = [ctypes.c_int32]
    lib.qdec_status_string.restype = ctypes.c_char_p
    lib.qdec_status_string.argtypes = [ctypes.c_int]
    lib.qdec_last_error.restype = ctypes.c_char_p
    lib.qdec_last_error.argtypes = []
    lib.qdec_workspace_bytes.restype = ctypes.c_size_t
    lib.qdec_workspace_bytes.argtypes = [P, i64, i32]
    lib.qdec_rht.restype = ctypes.c_int
    lib.qdec_rht.argtypes = [P, i32, P, i32, i64, i64, i32, P, i32, ctypes.c_float, P]
    for fn in (lib.qdec_gemv, lib.qdec_gemm):
        fn.restype = ctypes.c_int
        fn.argtypes = [P, P, P, i64, P, ctypes.c_size_t, P]
    lib.qdec_decode_tile.restype = ctypes.c_int
    lib.qdec_decode_tile.argtypes = [P, i64, i64, P, P]
    lib.qdec_encode.restype = ctypes.c_int
    lib.qdec_encode.argtypes = [P, P, P, P, ctypes.c_size_t, P]
    lib.qdec_gemv_group.restype = ctypes.c_int
    lib.qdec_gemv_group.argtypes = [P, i32, P, P, P, ctypes.c_size_t, P]
    lib.qdec_gemv_group_workspace_bytes.restype = ctypes.c_size_t
    lib.qdec_gemv_group_workspace_bytes.argtypes = [P, i32]
    lib.qdec_gemv_noalloc.restype = ctypes.c_int
    lib.qdec_gemv_noalloc.argtypes = [P, P, P, i64, P]
    lib.qdec_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.qdec_noalloc_scratch_bytes.argtypes = []
    if lib.qdec_abi_version() != QDEC_ABI_VERSION:
        raise ImportError("libqdec.so ABI version mismatch")
    return lib


_lib = _load()


def _status_string(status: int) -> str:
    return _lib.qdec_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != QDEC_OK:
        raise QdecError(status, what)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class Layer:
    """A quantized layer whose buffers live in device tensors.  Holds the
    tensors (so they outlive the descriptor) and the C descriptor."""
    code: int
    L: int
    k: int
    V: int
    Q: int
    m: int
    n: int
    codes: object
    lut: object = None
    group_scale: object = None
    group: int = 0
    layer_scale: float = 1.0
    sign_in: object = None
    sign_out: object = None
    had_in: int = 1
    had_out: int = 1
    kv: int = 0       # bits per trellis step of rows [0, m_a) (0: k * V)
    kv_b: int = 0     # half-TCQ: bits per step of rows [m_a, m)
    m_a: int = 0      # half-TCQ: rows of the first part (0: one part)
    _desc: qdec_layer = field(default=None, repr=False)

    def desc(self) -> qdec_layer:
        if self._desc is None:
            self._desc = qdec_layer(QDEC_ABI_VERSION, self.code, self.L, self.k, self.V, self.Q,
                                    self.kv, self.kv_b, self.m_a,
                                    self.m, self.n, _ptr(self.codes), _ptr(self.lut),
                                    _ptr(self.group_scale), self.group, self.layer_scale,
                                    _ptr(self.sign_in), _ptr(self.sign_out), self.had_in, self.had_out)
        return self._desc

    @property
    def n_tiles(self) -> int:
        return (self.m // 16) * (self.n // 16)

    @property
    def code_bytes(self) -> int:
        kva = self.kv if self.kv else self.k * self.V
        rows_a = self.m_a if self.m_a else self.m
        bits = rows_a * self.n * kva // self.V
        if self.m_a:
            bits += (self.m - self.m_a) * self.n * self.kv_b // self.V
        return bits // 8


def qdec_workspace_bytes(layer: Layer, batch: int, op: int) -> int:
    return int(_lib.qdec_workspace_bytes(ctypes.byref(layer.desc()), batch, op))


def qdec_rht(inp, in_dtype: int, out, out_dtype: int, rows: int, n: int, block: int,
             signs=None, mode: int = 0, scale: float = 1.0, stream=None) -> None:
    _check(_lib.qdec_rht(_ptr(inp), in_dtype, _ptr(out), out_dtype, rows, n, block, _ptr(signs),
                         mode, scale, _stream(stream)), "qdec_rht")


def qdec_gemv(layer: Layer, x, y, batch: int, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.qdec_gemv(ctypes.byref(layer.desc()), _ptr(x), _ptr(y), batch, _ptr(ws), ws_bytes,
                          _stream(stream)), "qdec_gemv")


def qdec_gemv_noalloc(layer: Layer, x, y, batch: int, stream=None) -> None:
    _check(_lib.qdec_gemv_noalloc(ctypes.byref(layer.desc()), _ptr(x), _ptr(y), batch, _stream(stream)),
           "qdec_gemv_noalloc")


def qdec_noalloc_scratch_bytes() -> int:
    return int(_lib.qdec_noalloc_scratch_bytes())


def qdec_gemm(layer: Layer, x, y, batch: int, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.qdec_gemm(ctypes.byref(layer.desc()), _ptr(x), _ptr(y), batch, _ptr(ws), ws_bytes,
                          _stream(stream)), "qdec_gemm")


def qdec_decode_tile(layer: Layer, first_tile: int, n_tiles: int, out, stream=None) -> None:
    _check(_lib.qdec_decode_tile(ctypes.byref(layer.desc()), first_tile, n_tiles, _ptr(out),
                                 _stream(stream)), "qdec_decode_tile")


def qdec_encode(layer: Layer, w, codes, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.qdec_encode(ctypes.byref(layer.desc()), _ptr(w), _ptr(codes), _ptr(ws), ws_bytes,
                            _stream(stream)), "qdec_encode")


class GroupCall:
    """The host-side pointer arrays of one qdec_gemv_group call (built once,
    so a call only passes them by reference)."""

    def __init__(self, layers, xs, ys):
        count = len(layers)
        self.count = count
        self.layers = list(layers)
        self.keep = (list(xs), list(ys))
        self._descs = [l.desc() for l in self.layers]
        self.lp = (ctypes.c_void_p * count)(*[ctypes.addressof(d) for d in self._descs])
        self.xp = (ctypes.c_void_p * count)(*[_ptr(x) for x in xs])
        self.yp = (ctypes.c_void_p * count)(*[_ptr(y) for y in ys])


def qdec_gemv_group_workspace_bytes(layers) -> int:
    descs = [l.desc() for l in layers]
    arr = (ctypes.c_void_p * len(descs))(*[ctypes.addressof(d) for d in descs])
    return int(_lib.qdec_gemv_group_workspace_bytes(arr, len(descs)))


def qdec_gemv_group(call: GroupCall, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.qdec_gemv_group(call.lp, call.count, call.xp, call.yp, _ptr(ws), ws_bytes,
                                _stream(stream)), "qdec_gemv_group")


def raw_status(fn_name: str, *args) -> int:
    """Call an entry point with raw ctypes arguments and return its status
    (for error-path tests)."""
    return int(getattr(_lib, fn_name)(*args))


# ---------------------------------------------------------------------------
# Convenience wrappers over torch tensors (allocation is torch's).

def upload_layer(host, device="cuda") -> Layer:
    """Copy a host layer (numpy arrays: codes, lut, gscale, sign_in, sign_out)
    to device tensors."""
    import numpy as np
    import torch

    def t(a, dtype):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).to(device)

    codes = t(host.codes, np.int32)
    return Layer(code=host.code, L=host.L, k=host.k, V=host.V, Q=host.Q, m=host.m, n=host.n,
                 codes=codes, lut=t(host.lut, np.int32), group_scale=t(host.gscale, np.int16),
                 group=host.group, layer_scale=host.scale, sign_in=t(host.sign_in, np.int32),
                 sign_out=t(host.sign_out, np.int32), had_in=host.had_in, had_out=host.had_out,
                 kv=getattr(host, "kv", 0), kv_b=getattr(host, "kv_b", 0), m_a=getattr(host, "m_a", 0))


def workspace(layer: Layer, batch: int, op: int, device="cuda"):
    """A workspace tensor for qdec_gemv / qdec_gemm (zero-filled, although
    no call depends on its contents)."""
    import torch
    nbytes = qdec_workspace_bytes(layer, batch, op)
    if nbytes == 0:
        raise QdecError(QDEC_EINVAL, "qdec_workspace_bytes")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def gemv(layer: Layer, x, ws=None, y=None):
    """y = layer(x) for x of shape [b, n] (fp16, b <= 8), one launch."""
    import torch
    b = x.shape[0]
    if ws is None:
        ws = workspace(layer, b, QDEC_OP_GEMV, x.device)
    if y is None:
        y = torch.empty((b, layer.m), dtype=torch.float16, device=x.device)
    qdec_gemv(layer, x, y, b, ws, ws.numel())
    return y


def gemv_group(layers, xs, ws=None, ys=None):
    """ys[l] = layers[l](xs[l]) for one-column inputs xs[l] of shape [n_l] or
    [1, n_l] (fp16), in one grouped call (two launches)."""
    import torch
    dev = xs[0].device
    if ys is None:
        ys = [torch.empty((1, l.m), dtype=torch.float16, device=dev) for l in layers]
    if ws is None:
        nbytes = qdec_gemv_group_workspace_bytes(layers)
        if nbytes == 0:
            raise QdecError(QDEC_EINVAL, "qdec_gemv_group_workspace_bytes")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    qdec_gemv_group(GroupCall(layers, xs, ys), ws, ws.numel())
    return ys


def gemm(layer: Layer, x, ws=None, y=None):
    """y = layer(x) for x of shape [b, n] (fp16, b <= 256), MFMA path."""
    import torch
    b = x.shape[0]
    if ws is None:
        ws = workspace(layer, b, QDEC_OP_GEMM, x.device)
    if y is None:
        y = torch.empty((b, layer.m), dtype=torch.float16, device=x.device)
    qdec_gemm(layer, x, y, b, ws, ws.numel())
    return y


def encode(layer: Layer, w, codes=None, ws=None):
    """Codes of the layer's format for the fp32 matrix w [m, n] (the
    tail-biting trellis encoder); returns the int32 tensor of code words."""
    import torch
    if codes is None:
        codes = torch.empty(layer.code_bytes // 4, dtype=torch.int32, device=w.device)
    if ws is None:
        ws = workspace(layer, 1, QDEC_OP_ENCODE, w.device)
    qdec_encode(layer, w, codes, ws, ws.numel())
    return codes
