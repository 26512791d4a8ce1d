"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: the worked
example printed on the pages, brute force on tiny trellises, closed forms,
library routines (numpy's binary16 conversion, numpy matrix products,
np.kron), invariants (H H^T = B I, Parseval, exact LUT coverage) and
statistical properties the pages state for the computed codes.
"""
import dataclasses
import itertools
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals[k] = v
    return vals


def _bits(s):
    return np.array([int(c) for c in s], dtype=np.uint8)


# ---------------------------------------------------------------------------
# Bitshift trellis walk

def test_worked_example_linear():
    g = _read_golden("bitshift_trellis_example.txt")
    L, kV = int(g["L"]), int(g["kV"])
    want = [int(v) for v in g["states"].split(",")]
    got = oracle.walk_bits(_bits(g["bits"]), L, kV, len(want), tailbiting=False)
    assert list(got) == want


def test_worked_example_tailbiting():
    g = _read_golden("bitshift_trellis_example.txt")
    L, kV = int(g["L"]), int(g["kV"])
    want = [int(v) for v in g["tailbiting_states"].split(",")]
    got = oracle.walk_bits(_bits(g["tailbiting_bits"]), L, kV, len(want), tailbiting=True)
    assert list(got) == want


def test_short_linear_stream_rejected():
    with pytest.raises(ValueError):
        oracle.walk_bits(_bits("001011"), 2, 1, 6, tailbiting=False)


@pytest.mark.parametrize("L,kV,steps", [(4, 2, 4), (3, 1, 6), (4, 1, 8), (6, 3, 4)])
def test_bijection_onto_cyclic_walks(L, kV, steps):
    """Tail-biting: the map from the steps*kV-bit stream to state sequences
    is a bijection onto the cyclic walks of the bitshift trellis (every state
    shares its low L-kV bits with the high L-kV bits of the next, wrapping)."""
    nbits = steps * kV
    mask = (1 << (L - kV)) - 1
    seen = set()
    for v in range(1 << nbits):
        bits = [(v >> (nbits - 1 - i)) & 1 for i in range(nbits)]
        st = tuple(int(s) for s in oracle.walk_bits(np.array(bits, np.uint8), L, kV, steps, True))
        for t in range(steps):
            a, b = st[t], st[(t + 1) % steps]
            assert (a & mask) == (b >> kV), (bits, st)
        seen.add(st)
    assert len(seen) == 1 << nbits  # injective
    # brute force over all state sequences: the valid cyclic walks number
    # exactly 2^nbits when L <= nbits (each step adds kV free bits)
    if (1 << L) ** steps <= 1 << 20:
        valid = 0
        for st in itertools.product(range(1 << L), repeat=steps):
            if all((st[t] & mask) == (st[(t + 1) % steps] >> kV) for t in range(steps)):
                valid += 1
                assert st in seen
        assert valid == len(seen)


@pytest.mark.parametrize("L,kV", [(16, 2), (16, 3), (16, 4), (16, 6), (12, 5), (16, 1)])
def test_serial_walk_equals_random_access_window(L, kV):
    rng = np.random.default_rng(L * 100 + kV)
    steps = 64
    nbits = steps * kV
    bits = rng.integers(0, 2, size=nbits, dtype=np.uint8)
    serial = oracle.walk_bits(bits, L, kV, steps, True)
    for t in range(steps):
        assert serial[t] == oracle.window_state(bits, L, kV, t)
    # and a window by numpy's own bit handling: concatenate, slice, pack
    ext = np.concatenate([bits, bits])
    for t in range(0, steps, 7):
        w = ext[t * kV:t * kV + L]
        assert serial[t] == int("".join(str(int(b)) for b in w), 2)


@pytest.mark.parametrize("kV", [3, 8])
def test_L_equals_kV_is_plain_fields(kV):
    """L = kV: the trellis becomes plain kV-bit VQ (no overlap), so state t is
    field t of the stream ("Ablations and fast inference")."""
    rng = np.random.default_rng(kV)
    words = rng.integers(0, 1 << 32, size=24, dtype=np.uint64).astype(np.uint32)
    bits = np.unpackbits(words.astype(">u4").view(np.uint8))  # MSB-first per word
    steps = bits.size // kV
    st = oracle.walk_bits(bits, kV, kV, steps, True)
    fields = bits[:steps * kV].reshape(steps, kV)
    want = fields.dot(1 << np.arange(kV - 1, -1, -1))
    assert np.array_equal(st, want)


# ---------------------------------------------------------------------------
# fp16 rounding (own implementation) vs numpy's IEEE binary16 conversion

def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    vals = [0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 5.96e-8, 2.98e-8,
            2.9802322387695312e-08, 8.940696716308594e-08, 6.097555160522461e-05,
            6.103515625e-05, float("inf"), -float("inf")]
    # exact halfway points between neighbouring fp16 values, across binades
    h = np.arange(0, 0x7BFF, 37, dtype=np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).view(np.float16).astype(np.float64)
    mids = (a + b) / 2
    x = np.concatenate([np.array(vals), mids, -mids, rng.standard_normal(3000) * 10,
                        rng.standard_normal(2000) * 1e-5,
                        np.exp(rng.uniform(-20, 12, 2000))])
    got = oracle.f16_from_double(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    back = oracle.f16_to_double(np.arange(0, 0x7C00, 13, dtype=np.uint16))
    assert np.array_equal(back, np.arange(0, 0x7C00, 13, dtype=np.uint16).view(np.float16).astype(np.float64))


@pytest.mark.parametrize("e", [-26, -25, -15, -14, 0, 15])
def test_f16_rounding_exhaustive_binades(e):
    """Every fp32 value of the binade [2^e, 2^(e+1)), both signs, rounds to
    the fp16 that numpy's float32 -> float16 conversion gives: below half
    the smallest subnormal (to zero), around the smallest subnormal, the
    subnormal/normal boundary, the unit binade and the top binade (overflow
    to infinity from 65520 on)."""
    m = np.arange(1 << 23, dtype=np.uint32)
    for sign in (0, 1):
        bits = (np.uint32(sign) << np.uint32(31)) | (np.uint32(e + 127) << np.uint32(23)) | m
        v = bits.view(np.float32)
        with np.errstate(over="ignore"):
            want = v.astype(np.float16).view(np.uint16)
        assert np.array_equal(oracle.f16_from_float32(v), want), (e, sign)


# ---------------------------------------------------------------------------
# HYB code

def test_hyb_covers_signed_codebook_uniformly():
    """Over all 2^16 states the HYB decode yields only +/- LUT pairs, the sign
    flips both halves, and each of the 2^(Q+1) = 1024 signed entries appears
    exactly 64 times (the LUT of 512 words expands to 1024 entries at V = 2;
    untitled ALU-op comment and "Bit Accounting (Q2)")."""
    g = _read_golden("bit_accounting.txt")
    Q = int(g["hyb_Q"])
    lut = synth.normal_f16(synth.rng_for("pin", "hyb"), (1 << Q) * 2).view(np.uint32)
    assert lut.size == int(g["hyb_lut_words"])
    vals = oracle.state_values_all(oracle.HYB, 16, Q, lut)
    words = vals[:, 0].astype(np.uint32) | (vals[:, 1].astype(np.uint32) << 16)
    pos = {int(w): i for i, w in enumerate(lut)}
    neg = {int(w) ^ 0x80008000: i for i, w in enumerate(lut)}
    counts = {}
    for w in words:
        w = int(w)
        key = ("+", pos[w]) if w in pos else ("-", neg[w])
        counts[key] = counts.get(key, 0) + 1
    assert len(counts) == int(g["hyb_signed_entries"])
    assert set(counts.values()) == {64}
    # codebook size from the bit accounting: 2^Q x V x 16 bits
    assert (1 << Q) * int(g["hyb_V"]) * 16 // 8 == int(g["hyb_codebook_bytes"]) == lut.nbytes


@pytest.mark.parametrize("Q", [6, 9])
def test_hyb_v1_covers_signed_codebook_uniformly(Q):
    """HYB with a one-dimensional codebook ("Other hardware (W3)": Q = 6,
    V = 1): every value is +/- the fp16 in the low half of a LUT word, and each
    of the 2^(Q+1) signed entries is hit by exactly 2^16 / 2^(Q+1) states."""
    # distinct positive fp16 values, in a seeded random order
    lut = (synth.rng_for("pin", "hyb1_%d" % Q).permutation(1 << Q) + 0x2000).astype(np.uint32)
    vals = oracle.state_values_all(oracle.HYB, 16, Q, lut, V=1)
    assert vals.shape == (1 << 16, 1)
    pos = {int(w): i for i, w in enumerate(lut)}
    neg = {int(w) ^ 0x8000: i for i, w in enumerate(lut)}
    counts = {}
    for w in vals[:, 0]:
        w = int(w)
        key = ("+", pos[w]) if w in pos else ("-", neg[w])
        counts[key] = counts.get(key, 0) + 1
    assert len(counts) == 2 << Q
    assert set(counts.values()) == {(1 << 16) >> (Q + 1)}


# (state, Q, index, negative) worked out by hand from h = s*s + s mod 2^16,
# index = bits [15-Q, 15) of h, sign = bit 15 of h:
#   s = 0:      h = 0                                   -> index 0, +
#   s = 0xFFFF: h = 0xFFFF * 0x10000 = 0 mod 2^16        -> index 0, +
#   s = 0x00FF: h = 65025 + 255 = 65280 = 0xFF00         -> bit 15 set;
#               Q = 6: 0xFF00 >> 9 = 127, & 63 = 63;  Q = 9: 0xFF00 >> 6 = 1020, & 511 = 508
#   s = 0x0100: h = 65536 + 256 = 256 mod 2^16           -> Q = 6: 256 >> 9 = 0;  Q = 9: 256 >> 6 = 4
#   s = 181:    h = 32761 + 181 = 32942 = 0x80AE         -> bit 15 set;
#               Q = 6: 32942 >> 9 = 64, & 63 = 0;  Q = 9: 32942 >> 6 = 514, & 511 = 2
HYB_HAND = [(0, 6, 0, False), (0xFFFF, 6, 0, False), (0x00FF, 6, 63, True), (0x0100, 6, 0, False),
            (181, 6, 0, True), (0x00FF, 9, 508, True), (0x0100, 9, 4, False), (181, 9, 2, True)]


@pytest.mark.parametrize("s,Q,idx,negative", HYB_HAND)
def test_hyb_hash_of_single_states(s, Q, idx, negative):
    lut1 = (np.arange(1 << Q, dtype=np.uint32) + 0x3C00)                  # distinct positive fp16
    lut2 = lut1 | ((lut1 + 0x100) << 16)
    (v1,) = oracle.state_value(oracle.HYB, s, Q, lut1, V=1)
    assert v1 == (int(lut1[idx]) ^ (0x8000 if negative else 0))
    lo, hi = oracle.state_value(oracle.HYB, s, Q, lut2, V=2)
    flip = 0x8000 if negative else 0
    assert (lo, hi) == (int(lut2[idx] & 0xFFFF) ^ flip, int(lut2[idx] >> 16) ^ flip)


# Single states of the computed codes, worked by hand from the code rules
# (1MAD: one multiply-add of a 32-bit LCG, then the sum of the four bytes;
# 3INST: the LCG, a bit-field insert of the exponent pattern, one fp16 add;
# computed-codes reply and "LCG citation (O2)"; the constants are this
# library's own).  A wrong constant, byte, mask or insert order changes these
# values, while it could keep the statistical pins above.
#
# 1MAD, u = 0x00EA4F79 * s + 0xC2AA9973 (mod 2^32), C = fp32(1/sqrt(21845)):
#   s = 0:      u = 0xC2AA9973; bytes 0x73 0x99 0xAA 0xC2 = 115+153+170+194
#               = 632; 632 - 510 = 122; fp32(122 C) = 0.82543677; in [0.5, 1)
#               the fp16 step is 2^-11: 0.82543677 * 2048 = 1690.495, which
#               rounds down to 1690 (0.8251953) -- a near tie; bits 0x3800 |
#               (1690 - 1024) = 0x3A9A.
#   s = 1:      u = 0xC2AA9973 + 0x00EA4F79 = 0xC394E8EC (no carry out of the
#               low half: 0x9973 + 0x4F79 = 0xE8EC); bytes 0xEC 0xE8 0x94 0xC3
#               = 236+232+148+195 = 811; 811 - 510 = 301; fp32(301 C) =
#               2.0365283; in [2, 4) the step is 2^-9: 2.0365283 * 512 =
#               1042.70 -> 1043 (2.0371094); bits 0x4000 | (1043 - 1024) = 0x4013.
#   s = 0x1234: u = 0x6BD94007; bytes 0x07 0x40 0xD9 0x6B = 7+64+217+107 =
#               395; 395 - 510 = -115; fp32(-115 C) = -0.77807564;
#               0.77807564 * 2048 = 1593.50 -> 1593 (0.7778320, below the tie:
#               1593.4989); bits 0x8000 | 0x3800 | 569 = 0xBA39.
# 3INST, u = 0x00E77B2B * s + 0xEACB81D7, u' = (u & 0x8FFF8FFF) | 0x30003000,
# value = fp16(f16(low half of u') + f16(high half)):
#   s = 0:      u = 0xEACB81D7 -> & 0x8FFF8FFF = 0x8ACB81D7 -> | 0x30003000 =
#               0xBACBB1D7; low 0xB1D7 = -(1 + 471/1024) 2^-3 = -0.18249512,
#               high 0xBACB = -(1 + 715/1024) 2^-1 = -0.84912109; sum
#               -1.03161621; in [1, 2) the step is 2^-10: 1056.375 -> 1056
#               (1.03125); bits 0x8000 | 0x3C00 | 32 = 0xBC20.
#   s = 1:      u = 0xEACB81D7 + 0x00E77B2B = 0xEBB2FD02 -> u' = 0xBBB2BD02;
#               low 0xBD02 = -(1 + 258/1024) = -1.25195313, high 0xBBB2 =
#               -(1 + 946/1024) 2^-1 = -0.96191406; sum -2.21386719; in [2, 4)
#               the step is 2^-9: 1133.5 exactly, a tie, to even 1134
#               (2.21484375); bits 0x8000 | 0x4000 | 110 = 0xC06E.
#   s = 0xFFFF: u = 0x650F06AC -> u' = 0x350F36AC; low 0x36AC = (1 + 684/1024)
#               2^-2 = 0.41699219, high 0x350F = (1 + 271/1024) 2^-2 =
#               0.31616211; sum 0.73315430 = 1501.5 * 2^-11, a tie, to even
#               1502 (0.73339844); bits 0x3800 | (1502 - 1024) = 0x39DE.
COMPUTED_HAND = [
    (2, 0x0000, 0x3A9A), (2, 0x0001, 0x4013), (2, 0x1234, 0xBA39),
    (3, 0x0000, 0xBC20), (3, 0x0001, 0xC06E), (3, 0xFFFF, 0x39DE),
]


@pytest.mark.parametrize("code,s,bits", COMPUTED_HAND,
                         ids=["%s_%04x" % ("1MAD" if c == 2 else "3INST", s) for c, s, _ in COMPUTED_HAND])
def test_computed_code_single_states(code, s, bits):
    (v,) = oracle.state_value(code, s, V=1)
    assert v == bits, "state %#06x: oracle %#06x, worked by hand %#06x" % (s, v, bits)


@pytest.mark.parametrize("k", [2, 3])
def test_lut_code_decodes_the_states(k):
    """Pure-lookup code (L = 16, V = 1; "Ablations and fast inference",
    Table A): with a codebook whose entry e is the bit pattern e, a tile
    decodes to its own trellis states, which the bit-serial walk (pinned by
    the worked example) computes independently from the stream bits."""
    lay = synth.make_layer(synth.LUT, 128, 32, k, tag="lutpin%d" % k)
    ident = np.arange(1 << 16, dtype=np.uint32)
    lay = dataclasses.replace(lay, lut=(ident[0::2] | (ident[1::2] << 16)).astype(np.uint32))
    for R, C in [(0, 0), (3, 1), (7, 0)]:
        got = oracle.decode_tile(lay, R, C)
        i = oracle.tile_index(32, R, C)
        words = lay.codes[i * 8 * k:(i + 1) * 8 * k]
        bits = np.unpackbits(words.astype(">u4").view(np.uint8))
        want = oracle.walk_bits(bits, 16, k, 256, True)
        assert np.array_equal(got.astype(np.int64), want.astype(np.int64))


# ---------------------------------------------------------------------------
# Computed codes: statistics the pages state (approximately Gaussian for
# L >= 10, neighbouring trellis states not strongly correlated), and the
# FP8-cast negative control of the computed-codes reply.

def _neighbour_pairs(v, L, kV):
    s = np.arange(1 << L, dtype=np.int64)
    nxt = ((s[:, None] << kV) | np.arange(1 << kV)[None, :]) & ((1 << L) - 1)
    return np.repeat(v, 1 << kV), v[nxt.ravel()]


def _coverage(a, b, bins=12):
    qa = np.quantile(a, np.linspace(0, 1, bins + 1)[1:-1])
    qb = np.quantile(b, np.linspace(0, 1, bins + 1)[1:-1])
    ia, ib = np.searchsorted(qa, a), np.searchsorted(qb, b)
    occ = np.zeros((bins, bins), bool)
    occ[ia, ib] = True
    return occ.mean()


@pytest.fixture(scope="module")
def computed_values():
    out = {}
    for code in (oracle.MAD1, oracle.INST3):
        h = oracle.state_values_all(code, 16)[:, 0]
        out[code] = h.view(np.float16).astype(np.float64)
    return out


@pytest.mark.parametrize("code", [oracle.MAD1, oracle.INST3])
def test_computed_code_near_gaussian(code, computed_values):
    v = computed_values[code]
    assert np.all(np.isfinite(v))
    z = (v - v.mean()) / v.std()
    assert abs(v.mean()) < 0.02 * v.std()
    assert 2.5 < (z ** 4).mean() < 3.3        # kurtosis near 3
    assert abs((z ** 3).mean()) < 0.05         # symmetric
    assert len(np.unique(v)) > 200             # many distinct values


@pytest.mark.parametrize("code", [oracle.MAD1, oracle.INST3])
@pytest.mark.parametrize("kV", [1, 2, 3, 4])
def test_computed_code_neighbours_decorrelated(code, kV, computed_values):
    v = computed_values[code]
    a, b = _neighbour_pairs(v, 16, kV)
    rho = np.corrcoef(a, b)[0, 1]
    assert abs(rho) < 0.01
    assert _coverage(a, b) > 0.97


def _predictability(v, L, kV, classes=4):
    """Mean over states of the largest fraction of its 2^kV successors that
    fall in one value class (classes = quantiles of v).  Near the i.i.d.
    random-codebook value when the state does not predict its successor."""
    q = np.quantile(v, np.linspace(0, 1, classes + 1)[1:-1])
    cls = np.searchsorted(q, v, side="right")
    s = np.arange(1 << L, dtype=np.int64)
    nxt = ((s[:, None] << kV) | np.arange(1 << kV)[None, :]) & ((1 << L) - 1)
    c = cls[nxt]
    frac = np.stack([(c == i).mean(1) for i in range(classes)], 1)
    return frac.max(1).mean()


def _random_codebook_predictability(L, kV, seed=0):
    v = np.random.default_rng(seed).standard_normal(1 << L)
    return _predictability(v, L, kV)


@pytest.mark.parametrize("code", [oracle.MAD1, oracle.INST3])
@pytest.mark.parametrize("kV", [1, 2, 3, 4])
def test_computed_code_successors_unpredictable(code, kV, computed_values):
    """A one-multiply-add LCG code keeps a little of the shift structure of
    the bitshift trellis (the successor's LCG output is about 2^kV times the
    current one plus a d-dependent offset); an LCG with a full 32-bit
    multiplier shows an excess of about 0.04 on this statistic.  Require the
    excess over an i.i.d. Gaussian codebook to stay below 0.06."""
    got = _predictability(computed_values[code], 16, kV)
    ref = _random_codebook_predictability(16, kV)
    assert got - ref < 0.06, (got, ref)


def test_fp8_cast_negative_control():
    """The direct FP8 (e5m2) cast of the state, the counter-example in the
    computed-codes reply (L = 8, K = 4): the mantissa bits of a state become
    sign and exponent bits of the next, so the successor's value class is
    largely fixed by the state -- the same statistic must flag it."""
    L, K = 8, 4
    s = np.arange(1 << L)
    # e5m2 is the upper byte of a binary16 pattern; drop the inf/nan states
    v = (s.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    v = np.where(np.isfinite(v), v, 0.0)
    got = _predictability(v, L, K)
    ref = _random_codebook_predictability(L, K)
    assert got > ref + 0.25, (got, ref)


def test_1mad_values_are_scaled_integers(computed_values):
    """1MAD values are (integer in [-510, 510]) / sqrt(21845) up to fp16
    rounding: a sum of four bytes, centred."""
    v = computed_values[oracle.MAD1]
    scaled = v * np.sqrt(21845.0)
    assert np.all(np.abs(scaled) <= 510 * (1 + 2 ** -10))
    assert np.all(np.abs(scaled - np.round(scaled)) <= np.abs(scaled) * 2 ** -10 + 1e-9)
    assert abs(v.std() - 1.0) < 0.02           # unit variance by construction


# ---------------------------------------------------------------------------
# Hadamard

@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64])
def test_hadamard_orthogonal(B):
    H = np.array([[oracle.hadamard_entry(i, j) for j in range(B)] for i in range(B)])
    assert np.array_equal(H @ H.T, B * np.eye(B, dtype=np.int64))


def test_hadamard_kronecker():
    H = np.array([[1]])
    for _ in range(6):
        H = np.kron(np.array([[1, 1], [1, -1]]), H)
    B = H.shape[0]
    Ho = np.array([[oracle.hadamard_entry(i, j) for j in range(B)] for i in range(B)])
    assert np.array_equal(H, Ho)


def _kron_h(B):
    H = np.array([[1.0]])
    while H.shape[0] < B:
        H = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), H)
    return H


def _signs_pm(words, n):
    if words is None:
        return np.ones(n)
    bits = (words[np.arange(n) >> 5] >> (np.arange(n) & 31).astype(np.uint32)) & 1
    return np.where(bits == 1, -1.0, 1.0)


@pytest.mark.parametrize("B,n", [(16, 64), (64, 192), (256, 256)])
def test_rht_against_kron_matrix(B, n):
    rng = np.random.default_rng(B + n)
    x = rng.standard_normal((3, n))
    sw = synth.sign_words(rng, n)
    s = _signs_pm(sw, n)
    H = _kron_h(B) / np.sqrt(B)
    want0 = np.concatenate([(H @ (s[b:b + B, None] * x.T[b:b + B])) for b in range(0, n, B)]).T
    got0 = oracle.rht(x, B, sw, mode=0)
    assert np.allclose(got0, want0, atol=1e-12)
    want1 = np.concatenate([s[b:b + B, None] * (H @ x.T[b:b + B]) for b in range(0, n, B)]).T
    got1 = oracle.rht(x, B, sw, mode=1, scale=1.0)
    assert np.allclose(got1, want1, atol=1e-12)
    # Parseval and round trip (input transform undone by the output transform)
    assert np.allclose((got0 ** 2).sum(1), (x ** 2).sum(1))
    back = oracle.rht(got0, B, sw, mode=1)
    assert np.allclose(back, x, atol=1e-12)


# ---------------------------------------------------------------------------
# Layer geometry and sizes

def test_tile_index_panel_order():
    n = 16 * 5
    seen = set()
    for R in range(16):
        for C in range(5):
            i = oracle.tile_index(n, R, C)
            assert oracle.tile_coords(n, i) == (R, C)
            seen.add(i)
    assert seen == set(range(16 * 5))
    # the 8 tiles of one panel column sit next to each other
    assert [oracle.tile_index(n, r, 3) for r in range(8, 16)] == list(range(5 * 8 + 24, 5 * 8 + 32))


def test_bits_per_weight_and_side_info():
    g = _read_golden("bit_accounting.txt")
    for wl in synth.WORKLOADS.values():
        for spec in wl.layers:
            assert spec.m * spec.n * spec.k % 32 == 0
    lay = synth.make_layer(synth.HYB, 4096, 4096, 2, tag="acct")
    assert lay.code_bytes * 8 == 2 * 4096 * 4096           # exactly k bits per weight
    side_bits = (lay.lut.nbytes * 8) + (4096 + 4096)          # codebook + n+m sign bits
    assert side_bits / (4096 * 4096) < float(g["max_side_bits_per_weight"])


def test_validate_rejects_bad_layers():
    good = synth.make_layer(synth.HYB, 128, 64, 2, tag="val")
    assert oracle.validate(good)
    import dataclasses
    for bad in [dict(m=100), dict(n=40), dict(k=0), dict(Q=0), dict(V=3),
                dict(had_in=3), dict(had_out=256), dict(L=12)]:
        assert not oracle.validate(dataclasses.replace(good, **bad)), bad


# ---------------------------------------------------------------------------
# Lloyd-Max

def test_lloyd_max_textbook():
    lv, mse = oracle.lloyd_max_gauss(8, 3000)
    assert np.allclose(lv, synth.LLOYD_MAX_8, atol=6e-4)
    assert abs(mse - 0.03454) < 5e-5
    assert np.array_equal(synth.f16_bits(lv), synth.f16_bits(np.array(synth.LLOYD_MAX_8)))
    # the 4- and 16-level rows of the same table (MSE 0.1175 and 0.0095)
    lv4, mse4 = oracle.lloyd_max_gauss(4, 3000)
    assert np.allclose(lv4, synth.LLOYD_MAX_4, atol=6e-4) and abs(mse4 - 0.1175) < 1e-4
    lv16, mse16 = oracle.lloyd_max_gauss(16, 20000)
    assert np.allclose(lv16, synth.LLOYD_MAX_16, atol=6e-4) and abs(mse16 - 0.0095) < 1e-5
    lv2, mse2 = oracle.lloyd_max_gauss(2, 200)
    # two levels: +/- sqrt(2/pi), MSE 1 - 2/pi
    assert np.allclose(lv2, [-np.sqrt(2 / np.pi), np.sqrt(2 / np.pi)], atol=1e-12)
    assert abs(mse2 - (1 - 2 / np.pi)) < 1e-12


# ---------------------------------------------------------------------------
# The forward pass

def _numpy_forward(layer, x16):
    """Independent evaluation: dense W from tile decodes placed by hand,
    Kronecker-built Hadamards, numpy matrix products."""
    m, n = layer.m, layer.n
    W = np.zeros((m, n))
    for R in range(m // 16):
        for C in range(n // 16):
            t = oracle.decode_tile(layer, R, C).view(np.float16).astype(np.float64)
            W[R * 16:(R + 1) * 16, C * 16:(C + 1) * 16] = t.reshape(16, 16)
    W *= float(np.float32(layer.scale))   # the descriptor carries an fp32 scale
    x = np.atleast_2d(x16).view(np.float16).astype(np.float64)
    si, so = _signs_pm(layer.sign_in, n), _signs_pm(layer.sign_out, m)
    Hi = _kron_h(layer.had_in) / np.sqrt(layer.had_in)
    Ho = _kron_h(layer.had_out) / np.sqrt(layer.had_out)
    Hin = np.kron(np.eye(n // layer.had_in), Hi)
    Hout = np.kron(np.eye(m // layer.had_out), Ho)
    xr = (Hin @ (si[:, None] * x.T))
    z = W @ xr
    return (so[:, None] * (Hout @ z)).T


@pytest.mark.parametrize("code,k,V", [(synth.HYB, 2, 2), (synth.MAD1, 3, None), (synth.INST3, 2, None),
                                      (synth.VQ, 4, None), (synth.HYB, 3, 2), (synth.HYB, 2, 1),
                                      (synth.LUT, 3, None)])
def test_forward_matches_numpy(code, k, V):
    lay = synth.make_layer(code, 256, 96, k, tag="fwd%d%d" % (code, k), had_out=64, V=V,
                           Q=6 if V == 1 else 9)
    x = synth.activations("fwdx", 2, 96)
    got = oracle.forward(lay, x)
    want = _numpy_forward(lay, x)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    bi = lay.m // lay.had_out - 1
    blk = oracle.forward_block(lay, x, [1], bi)
    assert np.allclose(blk[0], want[1, bi * lay.had_out:(bi + 1) * lay.had_out],
                       rtol=1e-12, atol=1e-12)


def test_forward_nuq_matches_numpy_with_exact_products():
    lay = synth.make_layer(synth.NUQ, 128, 256, 3, tag="fwdnuq")
    x = synth.activations("fwdnuqx", 1, 256)
    got = oracle.forward(lay, x)
    # NUQ weights are level x group scale exactly; rebuild from the stream bits
    lvl = np.array(lay.lut, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    gs = lay.gscale.view(np.float16).astype(np.float64)
    W = np.zeros((128, 256))
    for R in range(8):
        for C in range(16):
            i = oracle.tile_index(256, R, C)
            words = lay.codes[i * 24:(i + 1) * 24]
            bits = np.unpackbits(words.astype(">u4").view(np.uint8))
            idx = bits.reshape(256, 3).dot([4, 2, 1])
            for j in range(256):
                r, c = R * 16 + j // 16, C * 16 + j % 16
                W[r, c] = lvl[idx[j]] * gs[r, c // 128]
    x64 = x.view(np.float16).astype(np.float64)
    si, so = _signs_pm(lay.sign_in, 256), _signs_pm(lay.sign_out, 128)
    xr = (_kron_h(256) / 16.0) @ (si * x64[0])
    want = so * ((_kron_h(128) / np.sqrt(128)) @ (W @ xr))
    assert np.allclose(got[0], want, rtol=1e-12, atol=1e-12)


def test_forward_closed_form_constant_rows():
    """A VQ layer whose codebook is (1, 0) everywhere has W[r][c] = scale for
    even c and 0 for odd c.  With x = e_j the input RHT gives the column j of
    H/sqrt(B) times s_in[j]; every row of z equals the sum of its even entries;
    the output RHT of a constant block is sqrt(B) times that value in the
    block's first row and 0 elsewhere, times the output signs."""
    m, n, k = 256, 64, 4
    lay = synth.make_layer(synth.VQ, m, n, k, tag="closed", scale=0.5)
    lay.lut[:] = np.uint32(0x3C00)              # (1.0, 0.0)
    j = 5
    x = np.zeros((1, n), dtype=np.float64)
    x[0, j] = 1.0
    x16 = synth.f16_bits(x)
    y = oracle.forward(lay, x16)[0]
    si, so = _signs_pm(lay.sign_in, n), _signs_pm(lay.sign_out, m)
    Bi, Bo = lay.had_in, lay.had_out
    col = np.array([(-1) ** bin(i & j).count("1") for i in range(Bi)]) / np.sqrt(Bi) * si[j]
    zval = 0.5 * col[0::2].sum()
    want = np.zeros(m)
    for b0 in range(0, m, Bo):
        want[b0] = np.sqrt(Bo) * zval * so[b0]
    assert np.allclose(y, want, atol=1e-12)


# ---------------------------------------------------------------------------
# Fractional bit widths and half-TCQ

def _frac_layer(kv, m=256, n=48, kv_b=0, m_a=0, tag="frac"):
    return synth.make_layer(synth.HYB, m, n, 0, tag=tag, kv=kv, kv_b=kv_b, m_a=m_a, had_out=64)


def test_fractional_bits_per_weight():
    """kV = 5 at V = 2 stores 2.5 bits per weight; two equal halves at 2.5
    and 3 bits store 2.75 on average (the Q-Palette half-TCQ example)."""
    g = _read_golden("bit_accounting.txt")
    lay = _frac_layer(5)
    assert lay.bits_per_weight == float(g["fractional_example_bits"])
    ka, kb = (float(v) for v in g["half_tcq_parts_bits"].split(","))
    half = _frac_layer(int(2 * ka), kv_b=int(2 * kb), m_a=128)
    assert half.bits_per_weight == float(g["half_tcq_average_bits"])
    assert oracle.validate(lay) and oracle.validate(half)


@pytest.mark.parametrize("kv", [5, 7])
def test_fractional_tile_is_cyclic_walk_of_its_stream(kv):
    """Each tile is a tail-biting stream of 128 kv bits (kv/2 bits per
    weight) in storage order: its states are the cyclic kv-bit-shift windows
    of that stream, taken here with numpy's own bit unpacking and slicing."""
    lay = _frac_layer(kv)
    tw = 128 * kv // 32
    n = lay.n
    for i in (0, 5, lay.n_tiles - 1):
        R, C = oracle.tile_coords(n, i)
        bits = np.unpackbits(lay.codes[i * tw:(i + 1) * tw].astype(">u4").view(np.uint8))
        assert bits.size == 128 * kv
        ext = np.concatenate([bits, bits[:16]])
        want = []
        for t in range(128):
            s = int(ext[t * kv:t * kv + 16].dot(1 << np.arange(15, -1, -1)))
            want.extend(oracle.state_value(synth.HYB, s, lay.Q, lay.lut, V=2))
        assert np.array_equal(oracle.decode_tile(lay, R, C), np.array(want, dtype=np.uint16))


def test_even_kv_equals_integer_k():
    """kv = 2k given as bits per step decodes exactly as the integer width k."""
    a = synth.make_layer(synth.HYB, 128, 64, 3, tag="evenkv")
    b = dataclasses.replace(a, k=0, kv=6)
    assert np.array_equal(oracle.decode_dense(a), oracle.decode_dense(b))


@pytest.mark.parametrize("kv,kv_b,m_a", [(5, 6, 128), (7, 4, 256), (4, 5, 128)])
def test_half_tcq_is_two_layers_stacked(kv, kv_b, m_a):
    """Rows [0, m_a) at kv and [m_a, m) at kv_b, stored one part after the
    other, decode as two separate layers (split at the part boundary of the
    code words) stacked row-wise; the storage order lists the first part's
    tiles, then the second's."""
    m, n = 384, 48
    lay = _frac_layer(kv, m=m, n=n, kv_b=kv_b, m_a=m_a, tag="half%d%d" % (kv, kv_b))
    wa = (m_a // 16) * (n // 16) * 128 * kv // 32
    assert lay.codes.size == wa + ((m - m_a) // 16) * (n // 16) * 128 * kv_b // 32
    top = dataclasses.replace(lay, m=m_a, kv=kv, kv_b=0, m_a=0, codes=lay.codes[:wa].copy())
    bot = dataclasses.replace(lay, m=m - m_a, kv=kv_b, kv_b=0, m_a=0, codes=lay.codes[wa:].copy())
    W = oracle.decode_dense(lay)
    assert np.array_equal(W[:m_a], oracle.decode_dense(top))
    assert np.array_equal(W[m_a:], oracle.decode_dense(bot))
    st = oracle.decode_tiles_storage(lay, 0, lay.n_tiles)
    ta = top.n_tiles
    assert np.array_equal(st[:ta], oracle.decode_tiles_storage(top, 0, ta))
    assert np.array_equal(st[ta:], oracle.decode_tiles_storage(bot, 0, bot.n_tiles))


def test_fractional_validate_rejects():
    good = _frac_layer(5, kv_b=6, m_a=128)
    assert oracle.validate(good)
    for bad in [dict(k=2), dict(m_a=100), dict(m_a=256), dict(kv_b=0), dict(kv=17),
                dict(m_a=0), dict(kv_b=20)]:
        assert not oracle.validate(dataclasses.replace(good, **bad)), bad
    nuq = synth.make_layer(synth.NUQ, 128, 128, 3, tag="valnuq")
    assert not oracle.validate(dataclasses.replace(nuq, kv=3, k=0))
    assert not oracle.validate(dataclasses.replace(nuq, kv_b=3, m_a=0))


@pytest.mark.parametrize("kv,kv_b,m_a", [(5, 0, 0), (7, 0, 0), (5, 6, 128)])
def test_forward_fractional_matches_numpy(kv, kv_b, m_a):
    lay = _frac_layer(kv, kv_b=kv_b, m_a=m_a, m=256, n=96, tag="fwdfrac%d%d" % (kv, kv_b))
    lay = dataclasses.replace(lay, had_out=256)      # the output RHT spans both parts
    x = synth.activations("fwdfracx", 2, 96)
    got = oracle.forward(lay, x)
    want = _numpy_forward(lay, x)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# The encoder (Viterbi on the bitshift trellis)

def _path_cost(vals, x, st, V, scale=1.0):
    """fp64 squared error of a state path (independent of the encoder)."""
    T = st.size
    return float(((x.reshape(T, V).astype(np.float64) -
                   scale * vals.reshape(-1, V)[st].astype(np.float64)) ** 2).sum())


def _all_streams(nbits):
    for v in range(1 << nbits):
        yield np.array([(v >> (nbits - 1 - i)) & 1 for i in range(nbits)], np.uint8)


TINY = [(4, 1, 1, 8), (6, 2, 1, 6), (6, 3, 2, 4), (5, 2, 2, 5)]


@pytest.mark.parametrize("L,kV,V,T", TINY)
def test_viterbi_linear_equals_brute_force(L, kV, V, T):
    """Free start and end: the Viterbi optimum is the minimum over every bit
    string of L + (T-1) kV bits, walked by the (pinned) shift register."""
    rng = np.random.default_rng(L * 1000 + kV * 10 + V)
    for trial in range(3):
        vals = rng.standard_normal((1 << L, V)).astype(np.float32)
        x = rng.standard_normal(T * V).astype(np.float32)
        best = min(_path_cost(vals, x, oracle.walk_bits(b, L, kV, T, False), V)
                   for b in _all_streams(L + (T - 1) * kV))
        c, st = oracle.viterbi(L, kV, V, vals, x)
        assert abs(c - best) <= 1e-5 * best
        assert abs(_path_cost(vals, x, st, V) - best) <= 1e-5 * best
        # consecutive states share L - kV bits
        G = 1 << (L - kV)
        assert all((st[t] & (G - 1)) == (st[t + 1] >> kV) for t in range(T - 1))


@pytest.mark.parametrize("L,kV,V,T", TINY)
def test_tailbiting_encoder_equals_brute_force(L, kV, V, T):
    """Trying every wrap P gives the minimum over all T*kV-bit tail-biting
    streams; the two-pass encoder returns a valid stream (so never below the
    minimum) whose cyclic walk is the path it reports."""
    rng = np.random.default_rng(L * 1000 + kV * 10 + V + 7)
    for trial in range(3):
        vals = rng.standard_normal((1 << L, V)).astype(np.float32)
        x = rng.standard_normal(T * V).astype(np.float32)
        costs = [_path_cost(vals, x, oracle.walk_bits(b, L, kV, T, True), V)
                 for b in _all_streams(T * kV)]
        best = min(costs)
        for exact in (True, False):
            c, words, st = oracle.encode_stream(L, kV, V, vals, x, exact=exact)
            bits = np.unpackbits(words.astype(">u4").view(np.uint8))[:T * kV]
            walk = oracle.walk_bits(bits, L, kV, T, True)
            assert np.array_equal(walk, st)
            assert abs(_path_cost(vals, x, walk, V) - c) <= 1e-5 * c
            if exact:
                assert abs(c - best) <= 1e-5 * best
            else:
                assert c >= best * (1 - 1e-6)


def test_viterbi_constraints_equal_brute_force():
    """start_P / end_P restrict the first state's high and the last state's
    low L - kV bits."""
    L, kV, V, T = 6, 2, 1, 5
    rng = np.random.default_rng(99)
    vals = rng.standard_normal((1 << L, V)).astype(np.float32)
    x = rng.standard_normal(T * V).astype(np.float32)
    G = 1 << (L - kV)
    for P0, P1 in [(3, 3), (0, 15), (9, -1), (-1, 5)]:
        best = None
        for b in _all_streams(L + (T - 1) * kV):
            st = oracle.walk_bits(b, L, kV, T, False)
            if P0 >= 0 and (st[0] >> kV) != P0:
                continue
            if P1 >= 0 and (st[-1] & (G - 1)) != P1:
                continue
            c = _path_cost(vals, x, st, V)
            best = c if best is None else min(best, c)
        c, st = oracle.viterbi(L, kV, V, vals, x, start_P=P0, end_P=P1)
        assert abs(c - best) <= 1e-5 * best, (P0, P1)


def test_encoder_L_equals_kV_is_nearest_neighbour():
    """L = kV: no overlap between steps, so each step takes its nearest
    codeword (plain kV-bit V-dim VQ, "Ablations and fast inference")."""
    rng = np.random.default_rng(3)
    for L, V in [(4, 1), (6, 2)]:
        T = 32
        vals = rng.standard_normal((1 << L, V)).astype(np.float32)
        x = rng.standard_normal(T * V).astype(np.float32)
        c, words, st = oracle.encode_stream(L, L, V, vals, x)
        d = ((x.reshape(T, 1, V).astype(np.float64) - vals[None].astype(np.float64)) ** 2).sum(2)
        assert np.array_equal(st, d.argmin(1))


@pytest.mark.parametrize("code,kV,V,lo,hi", [
    (synth.MAD1, 2, 1, "rd_limit_2bit", "lloyd_max_mse_2bit"),
    (synth.MAD1, 3, 1, "rd_limit_3bit", "lloyd_max_mse_3bit"),
    (synth.HYB, 4, 2, "rd_limit_2bit", "lloyd_max_mse_2bit")])
def test_encoder_mse_between_rate_distortion_and_lloyd_max(code, kV, V, lo, hi):
    """L = 16 trellis on i.i.d. N(0,1): the MSE per weight lies above the
    rate-distortion limit 2^(-2k) and well below the optimal scalar
    quantizer at the same rate; the tail-biting stream costs at most a few
    percent over the free-ended Viterbi optimum (a lower bound)."""
    g = _read_golden("bit_accounting.txt")
    k = kV / V
    lay = synth.make_layer(code, 128, 64, 0, kv=kV, V=V, tag="encmse%d%d" % (code, kV), scale=1.0)
    vals = oracle.state_values_all(code, 16, lay.Q, lay.lut, V).view(np.float16).astype(np.float32)
    rng = np.random.default_rng(kV)
    W = rng.standard_normal((lay.m, lay.n)).astype(np.float32)
    codes, sse = oracle.encode_layer(lay, W)
    mse = sse / W.size
    assert float(g[lo]) < mse < 0.7 * float(g[hi]), mse
    assert mse < float(g[lo]) * (1.25 if k == 2 else 1.3)
    # the reported cost is the error of the decoded layer
    What = oracle.decode_dense(dataclasses.replace(lay, codes=codes))
    assert abs(((W - What) ** 2).sum() - sse) <= 1e-4 * sse
    # a few tiles against the free-ended optimum
    for i in range(3):
        x = W[16 * i:16 * i + 16, :16].reshape(-1)
        c, _, _ = oracle.encode_stream(16, kV, V, vals, x)
        cl, _ = oracle.viterbi(16, kV, V, vals, x)
        assert cl <= c <= 1.12 * cl


def test_encode_layer_half_tcq_round_trip():
    """A half-TCQ layer encodes part by part at its own widths; decoding the
    codes gives back the reported error."""
    lay = synth.make_layer(synth.HYB, 256, 32, 0, kv=5, kv_b=6, m_a=128, tag="enchalf", scale=0.5)
    rng = np.random.default_rng(11)
    W = (0.5 * rng.standard_normal((256, 32))).astype(np.float32)
    codes, sse = oracle.encode_layer(lay, W)
    What = oracle.decode_dense(dataclasses.replace(lay, codes=codes))
    err = ((W - What) ** 2)
    assert abs(err.sum() - sse) <= 1e-4 * sse
    # more bits per weight, less error: the 3-bit half beats the 2.5-bit half
    assert err[128:].mean() < err[:128].mean()
