"""CPU oracle for the quantized matmul -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper around ``qdec_oracle.c`` (plain C, fp64, bit-serial
trellis walk, Hadamard by its definition).  Only ``tests/``, the smoke check
and the bench's CPU-baseline leg may import this package; the HIP library never
does.  See ``qdec_oracle.c`` for the page sections each function follows and
for the readings taken where the pages are silent.

Parity status of each function (what pins it is in ``tests/test_oracle_pins.py``):
  walk_bits / window_state   pinned: worked example of the bitshift trellis,
                             brute-force bijection on tiny trellises,
                             L = kV reduces to a direct table lookup
  f16_from_double            pinned: numpy's IEEE binary16 conversion
  state_value (HYB)          pinned: every output is +/- a LUT pair (V = 2)
                             or value (V = 1); each of the 2^(Q+1) signed
                             entries is hit equally often; hand-computed
                             hashes of single states
  state_value (LUT)          pinned: with a codebook whose entry e is the fp16
                             pattern e, the decoded patterns are the states of
                             the worked example of the bitshift trellis
  state_value (1MAD/3INST)   pinned by statistics only (near-Gaussian moments,
                             uncorrelated trellis neighbours) and closed forms
                             of single states; the exact constants of the
                             original codes are not on the pages, so parity
                             with them is unpinned
  fractional kV, half-TCQ    pinned: bits per weight of the Q-Palette
                             examples (2.5; 2.5 and 3 giving 2.75); each
                             tile the cyclic walk of its 128 kV-bit stream
                             (numpy slicing); even kV equals the integer k;
                             a two-part layer decodes as two layers stacked
  viterbi / encode_stream    pinned: brute force over every bit string of
                             tiny trellises (free ends, constrained ends,
                             tail-biting with every wrap tried); L = kV is
                             the nearest codeword; the returned stream's
                             cyclic walk is the returned path
  encode_layer               pinned: MSE on N(0,1) between the rate-
                             distortion limit 2^(-2k) and the Lloyd-Max
                             scalar MSE (2 and 3 bits); the decoded layer's
                             error equals the reported cost
  rht                        pinned: H H^T = B I, Kronecker recursion,
                             Parseval, round trip, numpy's matrix product
  forward / forward_block    pinned: a small layer against an independent
                             numpy evaluation built from decode_tile and the
                             Kronecker-built Hadamard
  lloyd_max_gauss            pinned: the textbook 8-level Gaussian table
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qdec_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A sanitizer build of the same source (tests/test_sanitizers.py) is loaded
# in place of the plain one when this names it.
_SAN_LIB = os.environ.get("QDEC_ORACLE_SANITIZED_LIB")

HYB, MAD1, INST3, NUQ, VQ, LUT = 1, 2, 3, 4, 5, 6
CODE_NAMES = {HYB: "HYB", MAD1: "1MAD", INST3: "3INST", NUQ: "NUQ", VQ: "VQ", LUT: "LUT"}


def build(force: bool = True) -> str:
    """Compile qdec_oracle.c with gcc into liboracle.so (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _SAN_LIB:
            L = ctypes.CDLL(_SAN_LIB)
        else:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build(force=True)
            L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.orc_f16_from_double.restype = ctypes.c_uint16
        L.orc_f16_from_double.argtypes = [ctypes.c_double]
        L.orc_f16_from_float_array.restype = None
        L.orc_f16_from_float_array.argtypes = [P, i64, P]
        L.orc_f16_to_double.restype = ctypes.c_double
        L.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_walk_bits.argtypes = [P, i64, i32, i32, i64, i32, P]
        L.orc_window_state.restype = ctypes.c_uint32
        L.orc_window_state.argtypes = [P, i64, i32, i32, i64]
        L.orc_validate.argtypes = [P]
        L.orc_tile_index.restype = i64
        L.orc_tile_index.argtypes = [i64, i64, i64]
        L.orc_tile_coords.argtypes = [i64, i64, P, P]
        L.orc_decode_tile.argtypes = [P, i64, i64, P]
        L.orc_decode_dense.argtypes = [P, P]
        L.orc_decode_storage.argtypes = [P, i64, i64, P]
        L.orc_hadamard_entry.argtypes = [i64, i64]
        L.orc_rht.argtypes = [P, P, i64, i64, i64, P, i32, ctypes.c_double]
        L.orc_forward.argtypes = [P, P, i64, P, P]
        L.orc_forward_block.argtypes = [P, P, i64, P, i64, i64, P]
        L.orc_state_value.argtypes = [i32, i32, i32, P, ctypes.c_uint32, P]
        L.orc_lloyd_max_gauss.argtypes = [i32, i32, P, P]
        f32 = ctypes.c_float
        L.orc_viterbi.restype = f32
        L.orc_viterbi.argtypes = [i32, i32, i32, i32, P, P, f32, i32, i64, i64, P]
        L.orc_encode_stream.restype = f32
        L.orc_encode_stream.argtypes = [i32, i32, i32, i32, P, P, f32, i32, P, P]
        L.orc_encode_layer.argtypes = [P, P, P, i32, P]
        L.orc_omp_threads.restype = i32
        L.orc_set_threads.argtypes = [i32]
        L.orc_set_threads.restype = None
        _lib = L
    return _lib


class _OrcLayer(ctypes.Structure):
    _fields_ = [
        ("code", ctypes.c_int32), ("L", ctypes.c_int32), ("k", ctypes.c_int32),
        ("V", ctypes.c_int32), ("Q", ctypes.c_int32),
        ("kv", ctypes.c_int32), ("kv_b", ctypes.c_int32), ("m_a", ctypes.c_int64),
        ("m", ctypes.c_int64), ("n", ctypes.c_int64),
        ("codes", ctypes.c_void_p), ("lut", ctypes.c_void_p),
        ("gscale", ctypes.c_void_p), ("group", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("sign_in", ctypes.c_void_p), ("sign_out", ctypes.c_void_p),
        ("had_in", ctypes.c_int32), ("had_out", ctypes.c_int32),
    ]


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _struct(layer) -> tuple:
    """Build the oracle's own descriptor from a host layer object (any object
    with the attributes below, holding numpy arrays)."""
    keep = []

    def arr(a, dt):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dt)
        keep.append(a)
        return a

    codes = arr(layer.codes, np.uint32)
    lut = arr(layer.lut, np.uint32)
    gs = arr(layer.gscale, np.uint16)
    si = arr(layer.sign_in, np.uint32)
    so = arr(layer.sign_out, np.uint32)
    s = _OrcLayer(layer.code, layer.L, layer.k, layer.V, layer.Q,
                  getattr(layer, "kv", 0), getattr(layer, "kv_b", 0), getattr(layer, "m_a", 0),
                  layer.m, layer.n, _ptr(codes), _ptr(lut), _ptr(gs), layer.group,
                  layer.scale, _ptr(si), _ptr(so), layer.had_in, layer.had_out)
    return s, keep


def validate(layer) -> bool:
    s, keep = _struct(layer)
    return lib().orc_validate(ctypes.byref(s)) == 0


def f16_from_double(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    f = lib().orc_f16_from_double
    return np.array([f(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def f16_from_float32(v) -> np.ndarray:
    """fp16 bit patterns (round to nearest even) of an fp32 array, in one call."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.zeros(v.shape, dtype=np.uint16)
    lib().orc_f16_from_float_array(_ptr(v), v.size, _ptr(out))
    return out


def f16_to_double(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    f = lib().orc_f16_to_double
    return np.array([f(int(x)) for x in h.ravel()], dtype=np.float64).reshape(h.shape)


def walk_bits(bits, L: int, kV: int, nsteps: int, tailbiting: bool) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8))
    out = np.zeros(max(nsteps, 1), dtype=np.uint32)
    rc = lib().orc_walk_bits(_ptr(b), b.size, L, kV, nsteps, int(tailbiting), _ptr(out))
    if rc:
        raise ValueError("walk_bits: invalid arguments")
    return out[:nsteps]


def window_state(bits, L: int, kV: int, t: int) -> int:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8))
    return int(lib().orc_window_state(_ptr(b), b.size, L, kV, t))


def tile_index(n: int, R: int, C: int) -> int:
    return int(lib().orc_tile_index(n, R, C))


def tile_coords(n: int, index: int) -> tuple:
    R, C = ctypes.c_int64(), ctypes.c_int64()
    lib().orc_tile_coords(n, index, ctypes.byref(R), ctypes.byref(C))
    return R.value, C.value


def decode_tile(layer, R: int, C: int) -> np.ndarray:
    s, keep = _struct(layer)
    out = np.zeros(256, dtype=np.uint16)
    if lib().orc_decode_tile(ctypes.byref(s), R, C, _ptr(out)):
        raise ValueError("decode_tile: invalid layer or tile")
    return out


def decode_tiles_storage(layer, first: int, count: int) -> np.ndarray:
    """Decode tiles by storage index (the order they sit in memory)."""
    s, keep = _struct(layer)
    out = np.zeros((count, 256), dtype=np.uint16)
    if lib().orc_decode_storage(ctypes.byref(s), first, count, _ptr(out)):
        raise ValueError("decode_storage: invalid layer or range")
    return out


def decode_dense(layer) -> np.ndarray:
    s, keep = _struct(layer)
    W = np.zeros((layer.m, layer.n), dtype=np.float64)
    if lib().orc_decode_dense(ctypes.byref(s), _ptr(W)):
        raise ValueError("decode_dense: invalid layer")
    return W


def hadamard_entry(i: int, j: int) -> int:
    return int(lib().orc_hadamard_entry(i, j))


def rht(x, B: int, signs=None, mode: int = 0, scale: float = 1.0) -> np.ndarray:
    x = np.ascontiguousarray(np.atleast_2d(np.asarray(x, dtype=np.float64)))
    y = np.zeros_like(x)
    sg = None if signs is None else np.ascontiguousarray(signs, dtype=np.uint32)
    if lib().orc_rht(_ptr(x), _ptr(y), x.shape[0], x.shape[1], B, _ptr(sg), mode, scale):
        raise ValueError("rht: invalid arguments")
    return y


def forward(layer, x_f16: np.ndarray) -> np.ndarray:
    """y (b x m, fp64) for x given as fp16 bit patterns (b x n)."""
    x = np.ascontiguousarray(np.atleast_2d(x_f16), dtype=np.uint16)
    b = x.shape[0]
    s, keep = _struct(layer)
    W = np.zeros((layer.m, layer.n), dtype=np.float64)
    y = np.zeros((b, layer.m), dtype=np.float64)
    if lib().orc_forward(ctypes.byref(s), _ptr(x), b, _ptr(W), _ptr(y)):
        raise ValueError("forward: invalid layer")
    return y


def forward_block(layer, x_f16: np.ndarray, cols, block: int) -> np.ndarray:
    """Outputs of one output-Hadamard block (rows block*had_out ...) for the
    selected batch columns: len(cols) x had_out, fp64."""
    x = np.ascontiguousarray(np.atleast_2d(x_f16), dtype=np.uint16)
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    s, keep = _struct(layer)
    y = np.zeros((cols.size, layer.had_out), dtype=np.float64)
    if lib().orc_forward_block(ctypes.byref(s), _ptr(x), x.shape[0], _ptr(cols),
                               cols.size, block, _ptr(y)):
        raise ValueError("forward_block: invalid arguments")
    return y


def state_value(code: int, s: int, Q: int = 9, lut=None, V: int = 2) -> tuple:
    """fp16 bit patterns of the value(s) of state s (V matters for HYB only)."""
    lt = None if lut is None else np.ascontiguousarray(lut, dtype=np.uint32)
    out = np.zeros(2, dtype=np.uint16)
    nv = lib().orc_state_value(code, V, Q, _ptr(lt), s, _ptr(out))
    if nv < 0:
        raise ValueError("state_value: bad code")
    return tuple(int(v) for v in out[:nv])


def state_values_all(code: int, L: int = 16, Q: int = 9, lut=None, V: int = 2) -> np.ndarray:
    """Values of all 2^L states as fp16 bit patterns, shape (2^L, V)."""
    rows = [state_value(code, s, Q, lut, V) for s in range(1 << L)]
    return np.array(rows, dtype=np.uint16)


def viterbi(L: int, kV: int, V: int, vals, x, scale: float = 1.0, r: int = 0,
            start_P: int = -1, end_P: int = -1) -> tuple:
    """Best path of the bitshift trellis for the targets x (T x V): returns
    (fp32 cost, states).  vals: 2^L x V code values."""
    vals = np.ascontiguousarray(vals, dtype=np.float32).reshape(-1)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    T = x.size // V
    st = np.zeros(T, dtype=np.uint32)
    c = lib().orc_viterbi(L, kV, V, T, _ptr(vals), _ptr(x), scale, r, start_P, end_P, _ptr(st))
    return float(c), st


def encode_stream(L: int, kV: int, V: int, vals, x, scale: float = 1.0, exact: bool = False) -> tuple:
    """Tail-biting encode of the targets x (T x V) into T*kV stream bits:
    returns (fp32 cost, words, states)."""
    vals = np.ascontiguousarray(vals, dtype=np.float32).reshape(-1)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    T = x.size // V
    words = np.zeros((T * kV + 31) // 32, dtype=np.uint32)
    st = np.zeros(T, dtype=np.uint32)
    c = lib().orc_encode_stream(L, kV, V, T, _ptr(vals), _ptr(x), scale, int(exact), _ptr(words), _ptr(st))
    if np.isnan(c):
        raise ValueError("encode_stream: invalid arguments")
    return float(c), words, st


def encode_layer(layer, W, exact: bool = False) -> tuple:
    """Codes of the layer's format (its code, V, Q, lut, widths and scale)
    that minimise each tile's squared error against W (m x n): returns
    (codes, sum of the tiles' fp32 costs).  layer.codes only sizes the
    output."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    assert W.shape == (layer.m, layer.n)
    out = np.zeros_like(np.asarray(layer.codes, dtype=np.uint32))
    s, keep = _struct(layer)
    sse = ctypes.c_double()
    if lib().orc_encode_layer(ctypes.byref(s), _ptr(W), _ptr(out), int(exact), ctypes.byref(sse)):
        raise ValueError("encode_layer: invalid layer")
    return out, sse.value


def lloyd_max_gauss(nlev: int, iters: int = 2000) -> tuple:
    lv = np.zeros(nlev, dtype=np.float64)
    mse = ctypes.c_double()
    if lib().orc_lloyd_max_gauss(nlev, iters, _ptr(lv), ctypes.byref(mse)):
        raise ValueError("lloyd_max_gauss: bad arguments")
    return lv, mse.value


def omp_threads() -> int:
    return int(lib().orc_omp_threads())


def set_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops from now on."""
    lib().orc_set_threads(int(n))
