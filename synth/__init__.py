"""Seeded synthetic inputs for the quantized matmul.

Shared by the tests, the bench and the smoke check; imported by neither the
HIP library nor the oracle.  It holds none of the method's arithmetic: only
random code words (any bit string is a valid tail-biting trellis walk),
random sign bits, N(0,1) values rounded to fp16, the textbook Lloyd-Max
levels for N(0,1) (data, not computed here), random group scales, and the
layer shapes of the workloads.

Every array is a numpy array; fp16 values are carried as uint16 bit patterns.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

HYB, MAD1, INST3, NUQ, VQ, LUT = 1, 2, 3, 4, 5, 6
CODE_NAMES = {HYB: "HYB", MAD1: "1MAD", INST3: "3INST", NUQ: "NUQ", VQ: "VQ", LUT: "LUT"}

# Optimal 4-, 8- and 16-level quantizers for a unit Gaussian (J. Max,
# "Quantizing for minimum distortion", IRE Trans. IT-6, 1960, the Gaussian
# rows N = 4, 8, 16): the output levels, stored as data.
LLOYD_MAX_4 = (-1.510, -0.4528, 0.4528, 1.510)
LLOYD_MAX_8 = (-2.152, -1.344, -0.7560, -0.2451, 0.2451, 0.7560, 1.344, 2.152)
LLOYD_MAX_16 = (-2.733, -2.069, -1.618, -1.256, -0.9424, -0.6568, -0.3881, -0.1284,
                0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733)
LLOYD_MAX = {2: LLOYD_MAX_4, 3: LLOYD_MAX_8, 4: LLOYD_MAX_16}


def rng_for(*tags) -> np.random.Generator:
    """A numpy Generator seeded by a hash of the tags (stable across runs)."""
    h = hashlib.sha256("/".join(str(t) for t in tags).encode()).digest()
    return np.random.default_rng(int.from_bytes(h[:8], "little"))


def f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float16)).view(np.uint16)


def normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return f16_bits(rng.standard_normal(shape))


def random_words(rng: np.random.Generator, count: int) -> np.ndarray:
    return rng.integers(0, 1 << 32, size=count, dtype=np.uint64).astype(np.uint32)


def sign_words(rng: np.random.Generator, nbits: int) -> np.ndarray:
    return random_words(rng, (nbits + 31) // 32)


def largest_pow2_divisor(x: int) -> int:
    return x & -x


@dataclass
class HostLayer:
    """Host copy of one quantized linear layer (W_hat is m out x n in)."""
    code: int
    L: int
    k: int
    V: int
    Q: int
    m: int
    n: int
    codes: np.ndarray                   # uint32, m*n*k/32 words
    lut: Optional[np.ndarray] = None    # uint32 table
    gscale: Optional[np.ndarray] = None  # uint16 fp16 [m][n/group]
    group: int = 0
    scale: float = 1.0
    sign_in: Optional[np.ndarray] = None
    sign_out: Optional[np.ndarray] = None
    had_in: int = 1
    had_out: int = 1
    name: str = ""
    kv: int = 0       # bits per trellis step of rows [0, m_a) (0: k * V)
    kv_b: int = 0     # bits per step of rows [m_a, m) (half-TCQ), else 0
    m_a: int = 0      # rows of the first part (half-TCQ), else 0

    @property
    def bits_per_weight(self) -> float:
        return self.codes.size * 32 / (self.m * self.n)

    @property
    def n_tiles(self) -> int:
        return (self.m // 16) * (self.n // 16)

    @property
    def code_bytes(self) -> int:
        return self.codes.size * 4

    @property
    def side_bytes(self) -> int:
        b = 0
        for a in (self.lut, self.gscale, self.sign_in, self.sign_out):
            if a is not None:
                b += a.nbytes
        return b


def code_words(code: int, m: int, n: int, k: int, V: Optional[int] = None, kv: int = 0,
               kv_b: int = 0, m_a: int = 0) -> int:
    """uint32 words of packed codes: per 256-weight tile, 256/V steps of kV
    bits (kV = kv, or k * V), the rows split at m_a when kv_b is given."""
    if V is None:
        V = 2 if code in (HYB, VQ) else 1
    kva = kv if kv else k * V
    rows_a = m_a if m_a else m
    words = (rows_a // 16) * (n // 16) * (256 // V) * kva // 32
    if m_a:
        words += ((m - m_a) // 16) * (n // 16) * (256 // V) * kv_b // 32
    return words


def make_layer(code: int, m: int, n: int, k: int, *, tag: str, V: Optional[int] = None,
               Q: int = 9, scale: float = 0.02, signs: bool = True,
               had_in: Optional[int] = None, had_out: Optional[int] = None,
               group: int = 128, codes: Optional[np.ndarray] = None,
               kv: int = 0, kv_b: int = 0, m_a: int = 0) -> HostLayer:
    """A seeded random layer.  Trellis codes use L = 16; NUQ uses L = k, V = 1;
    VQ uses L = 2k, V = 2 (one index per weight pair).  Trellis codes may give
    the bits per step kv instead of k (pass k = 0; V = 2 and kv = 5 is 2.5
    bits per weight), and a second width kv_b for rows [m_a, m)."""
    if code == HYB:
        V = 2 if V is None else V
        L = 16
    elif code == LUT:
        V, L = 1, 16
    elif code in (MAD1, INST3):
        V = 1
        L = 16
    elif code == NUQ:
        V, L = 1, k
    elif code == VQ:
        V, L = 2, 2 * k
    else:
        raise ValueError("unknown code %r" % code)
    nwords = code_words(code, m, n, k, V, kv, kv_b, m_a)
    if codes is None:
        codes = random_words(rng_for(tag, "codes"), nwords)
    assert codes.size == nwords
    lut = gscale = None
    grp = 0
    if code == HYB and V == 2:
        lut = normal_f16(rng_for(tag, "lut"), (1 << Q) * 2).view(np.uint32).copy()
    elif code == HYB:        # V = 1: one fp16 value in the low half of each word
        lut = normal_f16(rng_for(tag, "lut"), 1 << Q).astype(np.uint32)
    elif code == LUT:        # 2^16 fp16 values, two per word
        lut = normal_f16(rng_for(tag, "lut"), 1 << 16).view(np.uint32).copy()
    elif code == NUQ:
        if k not in LLOYD_MAX:
            raise ValueError("the textbook tables here have 4, 8 and 16 levels (k = 2, 3, 4)")
        lv = f16_bits(np.array(LLOYD_MAX[k])).astype(np.uint32)
        lut = lv
        grp = group
        gscale = f16_bits(rng_for(tag, "gscale").uniform(0.01, 0.03, size=(m, n // group)))
        scale = 1.0
    elif code == VQ:
        lut = normal_f16(rng_for(tag, "lut"), (1 << L) * 2).view(np.uint32).copy()
    si = sign_words(rng_for(tag, "sign_in"), n) if signs else None
    so = sign_words(rng_for(tag, "sign_out"), m) if signs else None
    return HostLayer(code=code, L=L, k=k, V=V, Q=Q if code == HYB else 0, m=m, n=n,
                     codes=codes, lut=lut, gscale=gscale, group=grp, scale=float(scale),
                     sign_in=si, sign_out=so,
                     had_in=largest_pow2_divisor(n) if had_in is None else had_in,
                     had_out=largest_pow2_divisor(m) if had_out is None else had_out,
                     name=tag, kv=kv, kv_b=kv_b, m_a=m_a)


def activations(tag: str, b: int, n: int) -> np.ndarray:
    """x ~ N(0,1) rounded to fp16, b x n bit patterns."""
    return normal_f16(rng_for(tag, "x"), (b, n))


# ---------------------------------------------------------------------------
# Workloads: layer shapes and code settings of the five configurations.

@dataclass
class LayerSpec:
    name: str
    code: int
    m: int
    n: int
    k: int
    scale: float = 0.02
    had_in: Optional[int] = None
    had_out: Optional[int] = None

    def build(self, tag: str) -> HostLayer:
        return make_layer(self.code, self.m, self.n, self.k, tag=tag + "/" + self.name,
                          scale=self.scale, had_in=self.had_in, had_out=self.had_out)


@dataclass
class Workload:
    name: str
    layers: List[LayerSpec]
    batches: List[int]
    description: str = ""

    @property
    def code_bytes(self) -> int:
        return sum(s.m * s.n * s.k // 8 for s in self.layers)


WORKLOADS = {
    # 4096x4096, HYB k=2 V=2 Q=9, scale 0.02, RHT 4096 both sides, batch 1
    "hyb4096": Workload("hyb4096", [LayerSpec("w", HYB, 4096, 4096, 2)], [1],
                        "single 4096x4096 linear, 2-bit HYB trellis"),
    # 4096x4096 with computed codes, k in {2,3,4}, V = 1, batch 1
    "computed4096": Workload(
        "computed4096",
        [LayerSpec("%s_k%d" % (CODE_NAMES[c], k), c, 4096, 4096, k)
         for c in (MAD1, INST3) for k in (2, 3, 4)],
        [1], "4096x4096 with 1MAD and 3INST codes, k = 2, 3, 4"),
    # Llama-3-8B-shaped decoder layer, HYB k=2, batch 1 and 8
    "llama3_8b_layer": Workload(
        "llama3_8b_layer",
        [LayerSpec("q", HYB, 4096, 4096, 2), LayerSpec("k", HYB, 1024, 4096, 2),
         LayerSpec("v", HYB, 1024, 4096, 2), LayerSpec("o", HYB, 4096, 4096, 2),
         LayerSpec("gate", HYB, 14336, 4096, 2), LayerSpec("up", HYB, 14336, 4096, 2),
         LayerSpec("down", HYB, 4096, 14336, 2)],
        [1, 8], "Llama-3-8B-shaped decoder layer, 7 linears, HYB k=2"),
    # the same layer with the same-input projections fused: q, k, v as one
    # 6144-row layer and gate, up as one 28672-row layer (each quantized as one
    # matrix, so its output Hadamard block is the largest power of two
    # dividing the fused m: 2048 and 4096); 4 GEMVs per layer instead of 7
    "llama3_8b_layer_fused": Workload(
        "llama3_8b_layer_fused",
        [LayerSpec("qkv", HYB, 6144, 4096, 2), LayerSpec("o", HYB, 4096, 4096, 2),
         LayerSpec("gate_up", HYB, 28672, 4096, 2), LayerSpec("down", HYB, 4096, 14336, 2)],
        [1, 8], "Llama-3-8B-shaped layer with fused QKV and gate+up, HYB k=2"),
    # scalar / vector LUT variants on the down-projection shape, batch 1
    "down_nuq": Workload("down_nuq", [LayerSpec("down_nuq", NUQ, 4096, 14336, 3, scale=1.0)],
                         [1], "4096x14336 NUQ 3-bit, fp16 scale per 128 weights"),
    "down_vq": Workload("down_vq", [LayerSpec("down_vq", VQ, 4096, 14336, 4)],
                        [1], "4096x14336 2-D VQ, 8-bit index per weight pair"),
    # batched prefill on a 70B-class up-projection, HYB k=3, batch 64
    "up70b_prefill": Workload(
        "up70b_prefill", [LayerSpec("up", HYB, 28672, 8192, 3, had_in=8192, had_out=4096)],
        [64], "28672x8192 HYB k=3, X 64x8192"),
}


def with_codes(layer: HostLayer, codes: np.ndarray) -> HostLayer:
    return replace(layer, codes=codes)
