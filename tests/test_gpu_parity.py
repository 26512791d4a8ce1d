"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Bars: decoded weights bit-exact (qdec_decode_tile, every tile); outputs of
qdec_rht / qdec_gemv / qdec_gemm within ||y - y_ref|| / ||y_ref|| <= 2e-3 per
batch column (fp32 accumulation, fp16 in and out).  Every output is also held to an
element-wise bound (|y - y_ref| <= 2e-3 rms(y_ref) + 1 fp16 ulp).  Small
layers (several tiles, ragged chunking, odd shapes) and the full-size
workloads alike are checked whole: every tile of the decode, every output of
every batch column of the matmuls.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def q(dev):
    import dequant_matmul_packed_amd as q
    return q


def _f16_tensor(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


def _to_f64(t):
    import torch
    return t.cpu().view(torch.int16).numpy().view(np.float16).astype(np.float64)


def _rel(y, ref):
    y = np.atleast_2d(y)
    ref = np.atleast_2d(ref)
    errs = []
    for c in range(ref.shape[0]):
        d = np.linalg.norm(ref[c])
        errs.append(np.linalg.norm(y[c] - ref[c]) / (d if d > 0 else 1.0))
    return max(errs)


def _elementwise(y, ref, tol=REL_TOL):
    """Every output against the bound |y - y_ref| <= tol * rms(column of
    y_ref) + 1 fp16 ulp of y_ref (the last term is the output rounding), so a
    single wrong element cannot hide in a column norm.  Returns the largest
    ratio |y - y_ref| / bound (must be <= 1)."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    assert y.shape == ref.shape, (y.shape, ref.shape)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    bound = tol * rms + ulp
    return float(np.max(np.abs(y - ref) / bound))


def _check_output(y, ref, what=""):
    """Both bars: per-column relative L2 error and the element-wise bound."""
    rel = _rel(y, ref)
    ew = _elementwise(y, ref)
    assert rel < REL_TOL and ew <= 1.0, (what, rel, ew)
    return rel, ew


# ---------------------------------------------------------------------------
# decode: bit-exact

DECODE_CASES = [
    (synth.HYB, 2), (synth.HYB, 3), (synth.HYB, 4),
    (synth.MAD1, 2), (synth.MAD1, 3), (synth.MAD1, 4),
    (synth.INST3, 2), (synth.INST3, 3), (synth.INST3, 4),
    (synth.NUQ, 2), (synth.NUQ, 3), (synth.NUQ, 4), (synth.VQ, 2), (synth.VQ, 3), (synth.VQ, 4),
]


@pytest.mark.parametrize("code,k", DECODE_CASES)
def test_decode_tile_bit_exact_small(q, dev, code, k):
    import torch
    m, n = 384, 160 if code != synth.NUQ else 256
    _say("decode small", synth.CODE_NAMES[code], k, m, n)
    host = synth.make_layer(code, m, n, k, tag="dec%d_%d" % (code, k))
    lay = q.upload_layer(host, dev)
    want = oracle.decode_tiles_storage(host, 0, host.n_tiles)
    out = torch.zeros((host.n_tiles, 256), dtype=torch.int16, device=dev)
    q.qdec_decode_tile(lay, 0, host.n_tiles, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # a sub-range that is not a multiple of the 32 tiles of a workgroup
    first, cnt = 7, 45
    out2 = torch.zeros((cnt, 256), dtype=torch.int16, device=dev)
    q.qdec_decode_tile(lay, first, cnt, out2)
    torch.cuda.synchronize()
    assert np.array_equal(out2.cpu().numpy().view(np.uint16), want[first:first + cnt])


def _full_layers():
    out = []
    for wl in synth.WORKLOADS.values():
        for spec in wl.layers:
            out.append((wl.name, spec))
    return out


@pytest.mark.parametrize("wname,spec", _full_layers(), ids=[w + "/" + s.name for w, s in _full_layers()])
def test_decode_tile_bit_exact_full_size(q, dev, wname, spec):
    """Every tile of every layer of every workload."""
    import torch
    _say("decode full", wname, spec.name, spec.m, spec.n, spec.k)
    host = spec.build(wname)
    lay = q.upload_layer(host, dev)
    want = oracle.decode_tiles_storage(host, 0, host.n_tiles)
    out = torch.empty((host.n_tiles, 256), dtype=torch.int16, device=dev)
    q.qdec_decode_tile(lay, 0, host.n_tiles, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    bad = np.nonzero((got != want).any(1))[0]
    assert bad.size == 0, "first mismatching tiles %s" % bad[:8]


# ---------------------------------------------------------------------------
# RHT

@pytest.mark.parametrize("B,n,rows", [(1, 64, 3), (16, 592, 2), (256, 1024, 5), (4096, 4096, 2),
                                      (2048, 14336, 1), (8192, 8192, 2), (16384, 16384, 1),
                                      (8192, 8192, 64), (4096, 4096, 160)])
@pytest.mark.parametrize("mode", [0, 1])
def test_rht_matches_oracle(q, dev, B, n, rows, mode):
    import torch
    _say("rht", B, n, rows, mode)
    rng = synth.rng_for("rht", B, n, mode)
    x16 = synth.normal_f16(rng, (rows, n))
    sg = synth.sign_words(rng, n)
    xt = _f16_tensor(x16, dev)
    st = torch.from_numpy(sg.view(np.int32)).to(dev)
    ref = oracle.rht(x16.view(np.float16).astype(np.float64), B, sg, mode=mode, scale=0.5)
    out32 = torch.empty((rows, n), dtype=torch.float32, device=dev)
    q.qdec_rht(xt, 0, out32, 1, rows, n, B, st, mode, 0.5)
    out16 = torch.empty((rows, n), dtype=torch.int16, device=dev)
    q.qdec_rht(xt, 0, out16, 0, rows, n, B, st, mode, 0.5)
    # fp32 in place, back to the input
    inplace = out32.clone()
    q.qdec_rht(inplace, 1, inplace, 1, rows, n, B, st, 1 - mode, 2.0)
    # fp16 in place (where the out-of-place call cuts a block over several
    # workgroups, an in-place call must not)
    ip16 = xt.clone()
    q.qdec_rht(ip16, 0, ip16, 0, rows, n, B, st, mode, 0.5)
    torch.cuda.synchronize()
    assert _rel(out32.cpu().numpy().astype(np.float64), ref) < 1e-5
    _check_output(_to_f64(out16), ref, "fp16 out")
    _check_output(_to_f64(ip16), ref, "fp16 in place")
    back = inplace.cpu().numpy().astype(np.float64)
    assert _rel(back, x16.view(np.float16).astype(np.float64)) < 1e-5


# ---------------------------------------------------------------------------
# GEMV (fused, batch <= 8)

GEMV_SHAPES = [(256, 96), (384, 592), (1024, 1024), (128, 16), (640, 2048)]


@pytest.mark.parametrize("code,k", [(synth.HYB, 2), (synth.HYB, 3), (synth.MAD1, 2), (synth.MAD1, 4),
                                    (synth.INST3, 3), (synth.NUQ, 3), (synth.VQ, 4), (synth.HYB, 4),
                                    (synth.INST3, 2), (synth.MAD1, 3), (synth.NUQ, 2), (synth.NUQ, 4),
                                    (synth.VQ, 2), (synth.VQ, 3)])
@pytest.mark.parametrize("b", [1, 3, 8])
def test_gemv_small_matches_oracle(q, dev, code, k, b):
    import torch
    for (m, n) in GEMV_SHAPES:
        if code == synth.NUQ and n % 128:
            continue
        _say("gemv small", synth.CODE_NAMES[code], k, b, m, n)
        host = synth.make_layer(code, m, n, k, tag="gv%d_%d_%d_%d" % (code, k, m, n))
        x16 = synth.activations("gvx%d" % n, b, n)
        ref = oracle.forward(host, x16)
        lay = q.upload_layer(host, dev)
        y = q.gemv(lay, _f16_tensor(x16, dev))
        torch.cuda.synchronize()
        _check_output(_to_f64(y), ref, (m, n))


@pytest.mark.parametrize("Q", [6, 10, 11])
def test_hyb_table_sizes(q, dev, Q):
    """HYB with lookup tables of 2^Q pairs other than the default 512: the
    GEMV (one and three batch columns, fused and precomputed input RHT) and
    the GEMM against the oracle, and the decode bit-exact."""
    import torch
    m, n = 384, 1024
    host = synth.make_layer(synth.HYB, m, n, 2, Q=Q, tag="q%d" % Q)
    lay = q.upload_layer(host, dev)
    for b in (1, 3):
        _say("hyb Q", Q, "gemv b", b)
        x16 = synth.activations("qx%d" % b, b, n)
        y = q.gemv(lay, _f16_tensor(x16, dev))
        torch.cuda.synchronize()
        _check_output(_to_f64(y), oracle.forward(host, x16), b)
    _say("hyb Q", Q, "gemm")
    x16 = synth.activations("qx64", 64, n)
    y = q.gemm(lay, _f16_tensor(x16, dev))
    torch.cuda.synchronize()
    _check_output(_to_f64(y), oracle.forward(host, x16))
    out = torch.zeros((host.n_tiles, 256), dtype=torch.int16, device=dev)
    q.qdec_decode_tile(lay, 0, host.n_tiles, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), oracle.decode_tiles_storage(host, 0, host.n_tiles))


# HYB with a one-dimensional codebook (V = 1) and the pure-lookup code (a
# 128 KiB table of 2^16 fp16 values in LDS): decode, GEMV and GEMM.
NEW_CODES = [(synth.HYB, 1, 6, 2), (synth.HYB, 1, 6, 3), (synth.HYB, 1, 9, 4),
             (synth.LUT, None, 9, 2), (synth.LUT, None, 9, 3), (synth.LUT, None, 9, 4)]


@pytest.mark.parametrize("code,V,Q,k", NEW_CODES, ids=["%s_V%s_Q%d_k%d" % (synth.CODE_NAMES[c], v, qq, kk)
                                                      for c, v, qq, kk in NEW_CODES])
def test_hyb1_and_lut_codes(q, dev, code, V, Q, k):
    import torch
    for (m, n) in [(384, 160), (256, 592), (1024, 1024)]:
        host = synth.make_layer(code, m, n, k, V=V, Q=Q, tag="nc%d_%s_%d_%d_%d" % (code, V, Q, k, n))
        lay = q.upload_layer(host, dev)
        _say("new code decode", synth.CODE_NAMES[code], V, Q, k, m, n)
        out = torch.zeros((host.n_tiles, 256), dtype=torch.int16, device=dev)
        q.qdec_decode_tile(lay, 0, host.n_tiles, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), oracle.decode_tiles_storage(host, 0, host.n_tiles))
        for b in (1, 3, 8):
            _say("new code gemv", b)
            x16 = synth.activations("ncx%d_%d" % (b, n), b, n)
            y = q.gemv(lay, _f16_tensor(x16, dev))
            torch.cuda.synchronize()
            _check_output(_to_f64(y), oracle.forward(host, x16), (m, n, b))
        for b in (70, 9):    # 64- and 16-column batch tiles
            _say("new code gemm", b)
            x16 = synth.activations("ncx64_%d" % n, b, n)
            y = q.gemm(lay, _f16_tensor(x16, dev))
            torch.cuda.synchronize()
            _check_output(_to_f64(y), oracle.forward(host, x16), (m, n, b))


@pytest.mark.parametrize("code,V,Q", [(synth.HYB, 1, 6), (synth.LUT, None, 9)])
def test_hyb1_and_lut_full_size_whole(q, dev, code, V, Q):
    """4096 x 4096 at k = 2, b = 1 (the launch the bench would time)."""
    import torch
    host = synth.make_layer(code, 4096, 4096, 2, V=V, Q=Q, tag="ncfull%d" % code)
    x16 = synth.activations("ncfullx", 1, 4096)
    lay = q.upload_layer(host, dev)
    _say("new code full", synth.CODE_NAMES[code], V)
    y = _to_f64(q.gemv(lay, _f16_tensor(x16, dev)))
    torch.cuda.synchronize()
    _check_output(y, oracle.forward(host, x16))


def test_gemv_edge_cases(q, dev):
    import torch
    import dataclasses
    m, n = 512, 256
    host = synth.make_layer(synth.HYB, m, n, 2, tag="edge")
    x16 = synth.activations("edgex", 2, n)
    # no Hadamard at all (isolates the decoder), no signs, small blocks
    for kw in (dict(had_in=1, had_out=1), dict(sign_in=None, sign_out=None),
               dict(had_in=16, had_out=128), dict(had_in=64, had_out=512),
               dict(had_in=2, had_out=2), dict(had_in=4, had_out=8)):
        h2 = dataclasses.replace(host, **kw)
        lay = q.upload_layer(h2, dev)
        for b in (1, 2):     # the chunk transform in the workgroups, and the RHT kernel
            _say("gemv edge", kw, "b", b)
            y = q.gemv(lay, _f16_tensor(x16[:b], dev))
            torch.cuda.synchronize()
            _check_output(_to_f64(y), oracle.forward(h2, x16[:b]), (kw, b))
    # zero input gives exactly zero output
    lay = q.upload_layer(host, dev)
    z = q.gemv(lay, torch.zeros((1, n), dtype=torch.float16, device=dev))
    torch.cuda.synchronize()
    assert torch.count_nonzero(z).item() == 0
    # one workspace serves many calls, whatever it holds on entry: filled
    # with garbage (NaN bit patterns) first, the results stay right and equal
    ws = q.workspace(lay, 2, q.QDEC_OP_GEMV, dev)
    ws.fill_(0xFF)
    ref = oracle.forward(host, x16)
    xt = _f16_tensor(x16, dev)
    for b in (1, 2):
        ys = [q.gemv(lay, xt[:b], ws=ws).clone() for rep in range(5)]
        torch.cuda.synchronize()
        for yy in ys:
            _check_output(_to_f64(yy), ref[:b])
            assert torch.equal(yy, ys[0]), b                 # fixed summation order


def test_injected_launch_failure(q, dev):
    """qdec_debug_fail_launches(1): the next call returns QDEC_EHIP, names the
    hook in qdec_last_error and launches nothing (its output keeps a
    sentinel); the call after it runs normally and matches the oracle."""
    import ctypes
    import torch
    host = synth.make_layer(synth.HYB, 256, 512, 2, tag="inject")
    x16 = synth.activations("inject/x", 1, 512)
    lay = q.upload_layer(host, dev)
    xt = _f16_tensor(x16, dev)
    y = torch.full((1, 256), 7.0, dtype=torch.float16, device=dev)
    ws = q.workspace(lay, 1, q.QDEC_OP_GEMV, dev)
    torch.cuda.synchronize()
    _say("injected launch failure")
    assert q._lib.qdec_debug_fail_launches(1) == q.QDEC_OK
    try:
        st = q.raw_status("qdec_gemv", ctypes.byref(lay.desc()), xt.data_ptr(), y.data_ptr(), 1,
                          ws.data_ptr(), ws.numel(), None)
        msg = q._lib.qdec_last_error()
    finally:
        q._lib.qdec_debug_fail_launches(0)
    assert st == q.QDEC_EHIP
    assert b"injected" in msg
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))
    y2 = q.gemv(lay, xt, ws=ws, y=y)
    torch.cuda.synchronize()
    _check_output(_to_f64(y2), oracle.forward(host, x16))


def test_gemv_mixed_batches_one_workspace(q, dev):
    """One workspace sized for 8 columns serves calls of every batch in any
    order: on a 14336x4096 layer 8 columns take the batched MFMA path
    (8 * m * n >= 4e8) and 1-3 columns the fused GEMV, whose accumulator
    must stay zero across the others' scratch."""
    import torch
    m, n = 14336, 4096
    host = synth.make_layer(synth.HYB, m, n, 2, tag="mixws")
    lay = q.upload_layer(host, dev)
    ws = q.workspace(lay, 8, q.QDEC_OP_GEMV, dev)
    x16 = synth.activations("mixwsx", 8, n)
    xt = _f16_tensor(x16, dev)
    ref = oracle.forward(host, x16)
    for b in (8, 3, 1, 8, 2, 8, 1):
        _say("gemv mixed batches", b)
        y = _to_f64(q.gemv(lay, xt[:b], ws=ws))
        torch.cuda.synchronize()
        _check_output(y, ref[:b], b)


# qdec_gemv calls of several columns on large layers (NB * m * n >= 4e8, NB
# the batch rounded up to 2, 4 or 8) run the batched MFMA path with
# 16-column tiles: other codes, a half-TCQ layer (two row parts sharing the
# K-split slices) and the smallest batches that take the path.
ROUTED_CASES = [(synth.NUQ, 3, 0, 0, 4096, 14336, 8), (synth.VQ, 4, 0, 0, 4096, 14336, 7),
                (synth.HYB, 0, 5, 7168, 14336, 4096, 8), (synth.MAD1, 2, 0, 0, 28672, 4096, 3),
                (synth.HYB, 2, 0, 0, 14336, 4096, 5)]


@pytest.mark.parametrize("code,k,kv_b,m_a,m,n,b", ROUTED_CASES,
                         ids=["%s_k%d_%dx%d_b%d" % (synth.CODE_NAMES[c], k, m, n, b)
                              for c, k, _, _, m, n, b in ROUTED_CASES])
def test_gemv_routed_to_mfma_whole(q, dev, code, k, kv_b, m_a, m, n, b):
    import torch
    kw = dict(kv=6, kv_b=kv_b, m_a=m_a) if m_a else {}
    host = synth.make_layer(code, m, n, k, tag="routed%d_%d_%d" % (code, m, n), **kw)
    x16 = synth.activations("routedx%d" % n, b, n)
    _say("gemv routed", synth.CODE_NAMES[code], k, m, n, b, kw)
    lay = q.upload_layer(host, dev)
    ws = q.workspace(lay, b, q.QDEC_OP_GEMV, dev)
    y = _to_f64(q.gemv(lay, _f16_tensor(x16, dev), ws=ws))
    torch.cuda.synchronize()
    _check_output(y, oracle.forward(host, x16))


@pytest.mark.parametrize("m,had_out", [(1280, 256), (4096, 4096), (8192, 8192), (16384, 16384)])
def test_gemv_output_blocks(q, dev, m, had_out):
    """Output Hadamard blocks of 256 to 16384 rows (2 to 128 panels per block
    in the finisher's cross-panel transform), at one, three and eight batch
    columns (the finisher's workgroups of several columns in one XCD-major
    order), twice on one workspace (bit-identical results)."""
    import torch
    n = 256
    host = synth.make_layer(synth.HYB, m, n, 2, had_out=had_out, tag="ob%d" % m)
    lay = q.upload_layer(host, dev)
    for b in (1, 3, 8):
        _say("gemv output blocks", m, had_out, "b", b)
        x16 = synth.activations("obx%d" % b, b, n)
        ref = oracle.forward(host, x16)
        ws = q.workspace(lay, b, q.QDEC_OP_GEMV, dev)
        xt = _f16_tensor(x16, dev)
        ys = []
        for rep in range(2):
            y = q.gemv(lay, xt, ws=ws)
            torch.cuda.synchronize()
            _check_output(_to_f64(y), ref, (b, rep))
            ys.append(y.clone())
        assert torch.equal(ys[0], ys[1]), b


def _full_gemv_cases():
    cases = []
    for wname in ("hyb4096", "computed4096", "llama3_8b_layer", "llama3_8b_layer_fused", "down_nuq", "down_vq"):
        wl = synth.WORKLOADS[wname]
        for spec in wl.layers:
            for b in wl.batches:
                cases.append((wname, spec, b))
    return cases


@pytest.mark.parametrize("wname,spec,b", _full_gemv_cases(),
                         ids=["%s/%s/b%d" % (w, s.name, b) for w, s, b in _full_gemv_cases()])
def test_gemv_full_size_whole(q, dev, wname, spec, b):
    """Full-size layer in the launch configuration the bench times: every
    output of every batch column against the oracle's full forward pass
    (all output Hadamard blocks, all panels and input chunks)."""
    import torch
    _say("gemv full", wname, spec.name, b)
    host = spec.build(wname)
    x16 = synth.activations(wname + "/x", b, spec.n)
    lay = q.upload_layer(host, dev)
    y = _to_f64(q.gemv(lay, _f16_tensor(x16, dev)))
    torch.cuda.synchronize()
    ref = oracle.forward(host, x16)
    _check_output(y, ref, (wname, spec.name, b))


# Wide input chunks: 224 row panels make the GEMV pick 2048-column chunks at
# b = 1, 2 (1024 at b = 3), so each wave streams 32 tile columns through its
# prefetch ring; n = 5136 leaves a ragged 1040-column last chunk and a
# 16-point input Hadamard block.
WIDE_CASES = [(8192, 1, 3), (8192, 3, 3), (5136, 1, 2), (5136, 2, 2)]


@pytest.mark.parametrize("n,b,k", WIDE_CASES, ids=["n%d_b%d_k%d" % c for c in WIDE_CASES])
def test_gemv_wide_chunks_whole(q, dev, n, b, k):
    import torch
    m = 28672
    _say("gemv wide", m, n, b, k)
    host = synth.make_layer(synth.HYB, m, n, k, tag="wide%d_%d" % (n, k))
    x16 = synth.activations("widex%d" % n, b, n)
    lay = q.upload_layer(host, dev)
    y = _to_f64(q.gemv(lay, _f16_tensor(x16, dev)))
    torch.cuda.synchronize()
    _check_output(y, oracle.forward(host, x16), (n, b, k))


# ---------------------------------------------------------------------------
# GEMM (MFMA path)

@pytest.mark.parametrize("code,k,m,n,b", [
    (synth.HYB, 3, 256, 512, 64), (synth.HYB, 2, 384, 592, 5), (synth.HYB, 3, 128, 80, 70),
    (synth.MAD1, 2, 256, 256, 64), (synth.INST3, 4, 256, 256, 33), (synth.NUQ, 3, 256, 512, 64),
    (synth.VQ, 4, 256, 256, 64), (synth.HYB, 4, 1024, 1024, 64), (synth.NUQ, 2, 256, 512, 64),
    (synth.NUQ, 4, 384, 256, 40), (synth.VQ, 2, 256, 256, 64), (synth.VQ, 3, 128, 160, 64),
    (synth.MAD1, 4, 256, 256, 64), (synth.INST3, 2, 256, 512, 64), (synth.HYB, 2, 256, 256, 256),
    # 16-column batch tiles (batch <= 16): full, ragged and one-column tiles
    (synth.HYB, 3, 384, 592, 16), (synth.MAD1, 2, 256, 256, 1), (synth.INST3, 4, 256, 256, 12),
    (synth.NUQ, 3, 256, 512, 9), (synth.VQ, 4, 256, 256, 16), (synth.HYB, 4, 1024, 1040, 17)])
def test_gemm_small_matches_oracle(q, dev, code, k, m, n, b):
    import torch
    _say("gemm small", synth.CODE_NAMES[code], k, m, n, b)
    host = synth.make_layer(code, m, n, k, tag="gm%d_%d_%d_%d" % (code, k, m, n))
    x16 = synth.activations("gmx%d_%d" % (n, b), b, n)
    ref = oracle.forward(host, x16)
    lay = q.upload_layer(host, dev)
    ws = q.workspace(lay, b, q.QDEC_OP_GEMM, dev)
    xt = _f16_tensor(x16, dev)
    y = q.gemm(lay, xt, ws=ws)
    torch.cuda.synchronize()
    _check_output(_to_f64(y), ref)
    # the workspace accumulator is left zeroed: a second call agrees
    y2 = q.gemm(lay, xt, ws=ws)
    torch.cuda.synchronize()
    _check_output(_to_f64(y2), ref)


def test_gemm_two_k_halves_half_tcq_whole(q, dev):
    """A half-TCQ layer (rows [0, 4096) at kV = 5, [4096, 8192) at kV = 6)
    large enough for two K halves per workgroup: each part is launched with
    the whole layer's K split and halves, writing its rows of the shared
    slices.  Every output against the oracle."""
    import torch
    m, n, b = 8192, 1040, 64
    host = synth.make_layer(synth.HYB, m, n, 0, kv=5, kv_b=6, m_a=4096, tag="ksubhalf")
    x16 = synth.activations("ksubhalfx", b, n)
    _say("gemm two K halves, half-TCQ", m, n, b)
    lay = q.upload_layer(host, dev)
    y = _to_f64(q.gemm(lay, _f16_tensor(x16, dev)))
    torch.cuda.synchronize()
    _check_output(y, oracle.forward(host, x16))


@pytest.mark.parametrize("b", [64, 130])
def test_gemm_two_k_halves_whole(q, dev, b):
    """A layer large enough for the 16-wave GEMM (32 panel pairs per 64
    columns: two K halves per workgroup, added in LDS) with a ragged K of
    17 steps of 64 columns: the second split's second half has one live
    step, whose last tile column is the layer's last.  Every output of every
    batch column against the oracle."""
    import torch
    m, n = 8192, 1040
    host = synth.make_layer(synth.HYB, m, n, 3, tag="ksub")
    x16 = synth.activations("ksubx", b, n)
    _say("gemm two K halves", m, n, b)
    lay = q.upload_layer(host, dev)
    y = _to_f64(q.gemm(lay, _f16_tensor(x16, dev)))
    torch.cuda.synchronize()
    _check_output(y, oracle.forward(host, x16), b)


def test_gemm_full_size_whole(q, dev):
    """70B-class up-projection, X 64 x 8192 (the batch-64 workload as the
    bench times it): all 64 batch columns x all 28672 outputs (every output
    Hadamard block, every panel pair and K split) against the oracle."""
    import torch
    wl = synth.WORKLOADS["up70b_prefill"]
    spec = wl.layers[0]
    b = wl.batches[0]
    _say("gemm full", spec.m, spec.n, b)
    host = spec.build(wl.name)
    x16 = synth.activations(wl.name + "/x", b, spec.n)
    lay = q.upload_layer(host, dev)
    y = _to_f64(q.gemm(lay, _f16_tensor(x16, dev)))
    torch.cuda.synchronize()
    _check_output(y, oracle.forward(host, x16), "up70b b=64")


def test_graph_replays_match_eager(q, dev):
    """Calls captured into a HIP graph (as the bench replays them) and replayed
    several times, with eager work on the same buffers between the replays:
    every replay gives the eager result bit for bit: every path adds its K
    slices in a fixed order."""
    import torch
    m, n = 1024, 2048
    host = synth.make_layer(synth.HYB, m, n, 2, tag="graph")
    lay = q.upload_layer(host, dev)
    x16 = synth.activations("graphx", 64, n)
    xt = _f16_tensor(x16, dev)
    ref1 = oracle.forward(host, x16[:1])
    ref4 = oracle.forward(host, x16[:4])
    ws1 = q.workspace(lay, 1, q.QDEC_OP_GEMV, dev)
    ws4 = q.workspace(lay, 4, q.QDEC_OP_GEMV, dev)
    wsg = q.workspace(lay, 64, q.QDEC_OP_GEMM, dev)
    y1 = torch.empty((1, m), dtype=torch.float16, device=dev)
    y4 = torch.empty((4, m), dtype=torch.float16, device=dev)
    yg = torch.empty((64, m), dtype=torch.float16, device=dev)
    x1, x4 = xt[:1].contiguous(), xt[:4].contiguous()

    def calls():
        q.gemv(lay, x1, ws=ws1, y=y1)
        q.gemv(lay, x4, ws=ws4, y=y4)
        q.gemm(lay, xt, ws=wsg, y=yg)
    calls()                                   # eager first (also sets kernel attributes)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y1, y4, yg)]
    _check_output(_to_f64(y1), ref1)
    _check_output(_to_f64(y4), ref4)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        _say("graph replay", rep)
        for t in (y1, y4, yg):
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip((y1, y4, yg), eager):
            assert torch.equal(t, e), rep      # every path sums in a fixed order
        calls()                               # eager work between the replays
        torch.cuda.synchronize()
        for t, e in zip((y1, y4, yg), eager):
            assert torch.equal(t, e), rep
    del g


def test_graph_replays_routed_gemv(q, dev):
    """An 8-column qdec_gemv on a 14336x4096 layer (the batched MFMA path:
    input RHT, 16-column GEMM tiles, output RHT over the K-split slices)
    captured into a HIP graph: every replay equals the eager call bit for
    bit (fixed summation order), with an eager one-column call on the same
    workspace between the replays; both match the oracle."""
    import torch
    m, n, b = 14336, 4096, 8
    host = synth.make_layer(synth.HYB, m, n, 2, tag="graphrouted")
    lay = q.upload_layer(host, dev)
    x16 = synth.activations("graphroutedx", b, n)
    xt = _f16_tensor(x16, dev)
    ws = q.workspace(lay, b, q.QDEC_OP_GEMV, dev)
    y = torch.empty((b, m), dtype=torch.float16, device=dev)
    y1 = torch.empty((1, m), dtype=torch.float16, device=dev)
    x1 = xt[:1].contiguous()
    q.gemv(lay, xt, ws=ws, y=y)
    torch.cuda.synchronize()
    eager = y.clone()
    _check_output(_to_f64(eager), oracle.forward(host, x16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.gemv(lay, xt, ws=ws, y=y)
    for rep in range(3):
        _say("routed graph replay", rep)
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), rep
        q.gemv(lay, x1, ws=ws, y=y1)          # the fused GEMV on the same workspace
        torch.cuda.synchronize()
    del g
    _check_output(_to_f64(y1), oracle.forward(host, x16[:1]))


def test_gemm_agrees_with_gemv(q, dev):
    import torch
    host = synth.make_layer(synth.HYB, 512, 1024, 2, tag="gmgv")
    x16 = synth.activations("gmgvx", 8, 1024)
    lay = q.upload_layer(host, dev)
    xt = _f16_tensor(x16, dev)
    a = _to_f64(q.gemv(lay, xt))
    g = _to_f64(q.gemm(lay, xt))
    torch.cuda.synchronize()
    assert _rel(g, a) < REL_TOL


# ---------------------------------------------------------------------------
# Fractional widths (kV = 5, 7 at V = 2: 2.5 and 3.5 bits per weight) and
# half-TCQ (rows split at a panel boundary into two widths): decode, GEMV,
# GEMM.  Lanes of odd kV start mid-word, and the parts have their own tile
# arrays, so every case is checked on whole small layers and on a decode
# range that crosses the part boundary.
FRAC_CASES = [(synth.HYB, 5, 0, 0), (synth.HYB, 7, 0, 0), (synth.HYB, 5, 6, 128),
              (synth.HYB, 7, 4, 256), (synth.HYB, 4, 5, 128), (synth.HYB, 8, 7, 384),
              (synth.MAD1, 2, 3, 128), (synth.LUT, 4, 2, 256)]


@pytest.mark.parametrize("code,kv,kv_b,m_a", FRAC_CASES,
                         ids=["%s_kv%d_%d_ma%d" % (synth.CODE_NAMES[c], a, b_, ma) for c, a, b_, ma in FRAC_CASES])
def test_fractional_and_half_tcq(q, dev, code, kv, kv_b, m_a):
    import torch
    for (m, n) in [(384, 160), (512, 592), (1024, 1024)]:
        if m_a >= m:
            continue
        host = synth.make_layer(code, m, n, 0, kv=kv, kv_b=kv_b, m_a=m_a,
                                tag="fr%d_%d_%d_%d_%d" % (code, kv, kv_b, m_a, n))
        lay = q.upload_layer(host, dev)
        _say("frac decode", synth.CODE_NAMES[code], kv, kv_b, m_a, m, n)
        want = oracle.decode_tiles_storage(host, 0, host.n_tiles)
        out = torch.zeros((host.n_tiles, 256), dtype=torch.int16, device=dev)
        q.qdec_decode_tile(lay, 0, host.n_tiles, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), want)
        if m_a:
            ta = (m_a // 16) * (n // 16)
            first, cnt = ta - 10, 37
            out2 = torch.zeros((cnt, 256), dtype=torch.int16, device=dev)
            q.qdec_decode_tile(lay, first, cnt, out2)
            torch.cuda.synchronize()
            assert np.array_equal(out2.cpu().numpy().view(np.uint16), want[first:first + cnt])
        for b in (1, 3, 8):
            _say("frac gemv", b)
            x16 = synth.activations("frx%d_%d" % (b, n), b, n)
            y = q.gemv(lay, _f16_tensor(x16, dev))
            torch.cuda.synchronize()
            _check_output(_to_f64(y), oracle.forward(host, x16), (m, n, b))
        _say("frac gemm")
        x16 = synth.activations("frx70_%d" % n, 70, n)
        y = q.gemm(lay, _f16_tensor(x16, dev))
        torch.cuda.synchronize()
        _check_output(_to_f64(y), oracle.forward(host, x16), (m, n))


FRAC_FULL = [(4096, 4096, 5, 0, 0, 1), (4096, 4096, 7, 0, 0, 1), (4096, 4096, 5, 6, 2048, 1),
             (28672, 8192, 5, 6, 14336, 64)]


@pytest.mark.parametrize("m,n,kv,kv_b,m_a,b", FRAC_FULL,
                         ids=["%dx%d_kv%d_%d_b%d" % (m, n, a, b_, bb) for m, n, a, b_, ma, bb in FRAC_FULL])
def test_fractional_full_size_whole(q, dev, m, n, kv, kv_b, m_a, b):
    """Full-size fractional and half-TCQ layers in the launch configuration
    the bench times (GEMV at b = 1, GEMM at b = 64): every output against the
    oracle (both sides of the part boundary); the decode of every tile."""
    import torch
    had_in = 8192 if n == 8192 else None
    had_out = 4096 if m == 28672 else None
    host = synth.make_layer(synth.HYB, m, n, 0, kv=kv, kv_b=kv_b, m_a=m_a, had_in=had_in,
                            had_out=had_out, tag="frfull%d_%d_%d" % (m, kv, kv_b))
    x16 = synth.activations("frfullx%d" % n, b, n)
    lay = q.upload_layer(host, dev)
    _say("frac full", m, n, kv, kv_b, m_a, b)
    fn = q.gemv if b <= 8 else q.gemm
    y = _to_f64(fn(lay, _f16_tensor(x16, dev)))
    torch.cuda.synchronize()
    _check_output(y, oracle.forward(host, x16), (m, n, kv, kv_b, b))
    out = torch.empty((host.n_tiles, 256), dtype=torch.int16, device=dev)
    q.qdec_decode_tile(lay, 0, host.n_tiles, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = oracle.decode_tiles_storage(host, 0, host.n_tiles)
    bad = np.nonzero((got != want).any(1))[0]
    assert bad.size == 0, "first mismatching tiles %s" % bad[:8]


# ---------------------------------------------------------------------------
# qdec_gemv_group: several one-column products in one call (one MFMA launch
# per code and width among the layers' row parts, one finisher launch).

def _group_case(name, specs, n_by_layer=None):
    """specs: (code, m, n, k, extra make_layer keywords) per layer."""
    hosts, xs = [], []
    for i, (code, m, n, k, kw) in enumerate(specs):
        hosts.append(synth.make_layer(code, m, n, k, tag="grp_%s_%d" % (name, i), **kw))
        xs.append(synth.activations("grpx_%s_%d" % (name, i), 1, n))
    return hosts, xs


GROUP_CASES = {
    # three HYB layers of one width, ragged n (1040 = 2 x 512 + 16 columns:
    # the last column range holds one tile column) and small Hadamard blocks
    "hyb_ragged": [(synth.HYB, 384, 1040, 2, dict(had_out=128)), (synth.HYB, 1024, 1040, 2, {}),
                   (synth.HYB, 128, 1040, 2, dict(had_out=64))],
    # every code in one call: one launch per code and width
    "mixed_codes": [(synth.HYB, 512, 1024, 3, {}), (synth.VQ, 256, 1024, 4, {}),
                    (synth.NUQ, 384, 1024, 3, {}), (synth.MAD1, 256, 1024, 3, {}),
                    (synth.INST3, 128, 1024, 2, {}), (synth.HYB, 256, 1024, 2, dict(V=1, Q=6)),
                    (synth.LUT, 256, 1024, 2, {}), (synth.HYB, 384, 1024, 2, {})],
    # half-TCQ layers (two row parts of different widths) beside a plain one
    "half_tcq": [(synth.HYB, 1024, 2048, 0, dict(kv=5, kv_b=6, m_a=512)), (synth.HYB, 512, 2048, 2, {}),
                 (synth.MAD1, 768, 2048, 0, dict(kv=2, kv_b=3, m_a=256))],
    # inputs of different lengths in one launch
    "widths": [(synth.HYB, 256, 512, 2, {}), (synth.HYB, 640, 4096, 2, {}), (synth.HYB, 128, 2064, 2, {})],
    # input Hadamard blocks smaller than the row (1024-, 2048- and 4096-value
    # transforms whose upper stages are skipped) beside a tiny block
    "small_blocks": [(synth.HYB, 512, 4096, 2, dict(had_in=2048)), (synth.HYB, 256, 2048, 2, dict(had_in=1024)),
                     (synth.HYB, 384, 1024, 2, dict(had_in=8))],
    # one K range per workgroup (1024-column ranges of 256-column blocks)
    "range_blocks": [(synth.HYB, 8192, 4096, 2, dict(had_in=256))],
    # HYB tables of different sizes (Q = 6: 128 table copies; Q = 10, 11:
    # fewer): one launch per Q
    "table_sizes": [(synth.HYB, 256, 1024, 2, dict(Q=6)), (synth.HYB, 384, 2048, 2, dict(Q=10)),
                    (synth.HYB, 128, 4096, 2, dict(Q=11)), (synth.HYB, 256, 1024, 2, {})],
    # more units than workgroups (448 panels on 256 workgroups): some
    # workgroups walk two units, each unit's slice rows written once
    "several_units": [(synth.HYB, 28672, 4096, 2, {}), (synth.HYB, 28672, 4096, 2, {})],
    # the largest group, one code, width and Q: one launch whose eight layers
    # use every layer bound the kernels take as leading arguments
    "eight_layers": [(synth.HYB, 128 * (i + 1), 1024 if i % 2 else 2048, 2, {}) for i in range(8)],
}


@pytest.mark.parametrize("name", sorted(GROUP_CASES))
def test_gemv_group_matches_oracle(q, dev, name):
    import torch
    _say("gemv group", name)
    hosts, xs = _group_case(name, GROUP_CASES[name])
    lays = [q.upload_layer(h, dev) for h in hosts]
    xts = [_f16_tensor(x, dev) for x in xs]
    ws = torch.empty(q.qdec_gemv_group_workspace_bytes(lays), dtype=torch.uint8, device=dev)
    ws.fill_(0xFF)                          # contents on entry do not matter
    ys = q.gemv_group(lays, xts, ws=ws)
    torch.cuda.synchronize()
    first = [y.clone() for y in ys]
    for i, (h, x, y) in enumerate(zip(hosts, xs, ys)):
        _check_output(_to_f64(y), oracle.forward(h, x), (name, i))
    # again on the same workspace: bit-identical
    ys2 = q.gemv_group(lays, xts, ws=ws)
    torch.cuda.synchronize()
    for a, b in zip(first, ys2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("groups", [("q", "k", "v"), ("gate", "up")], ids=["qkv", "gate_up"])
def test_gemv_group_llama_full_size_whole(q, dev, groups):
    """The Llama-3-8B layer's same-input projections as the bench calls them:
    q, k, v (one x) and gate, up (one x) in one grouped call each, every
    output against the oracle."""
    import torch
    wl = synth.WORKLOADS["llama3_8b_layer"]
    specs = {s.name: s for s in wl.layers}
    hosts = [specs[g].build(wl.name) for g in groups]
    x16 = synth.activations(wl.name + "/x", 1, hosts[0].n)
    _say("gemv group full", groups)
    lays = [q.upload_layer(h, dev) for h in hosts]
    xt = _f16_tensor(x16, dev)
    ys = q.gemv_group(lays, [xt] * len(lays))
    torch.cuda.synchronize()
    for g, h, y in zip(groups, hosts, ys):
        _check_output(_to_f64(y), oracle.forward(h, x16), g)


# ---------------------------------------------------------------------------
# The encoder: codes bit-exact against the oracle's Viterbi (same fp32 path
# costs and tie rules), on layers of more tiles than the encoder's 256
# workgroups, for every state layout (kV = 2 .. 8) and code.
ENC_CASES = [(synth.HYB, 2, 4, 9, 0, 0), (synth.HYB, 2, 5, 9, 0, 0), (synth.HYB, 2, 6, 9, 0, 0),
             (synth.HYB, 2, 7, 9, 0, 0), (synth.HYB, 2, 8, 9, 0, 0), (synth.HYB, 1, 3, 6, 0, 0),
             (synth.MAD1, 1, 2, 9, 0, 0), (synth.MAD1, 1, 4, 9, 0, 0), (synth.INST3, 1, 3, 9, 0, 0),
             (synth.HYB, 2, 5, 9, 6, 128)]


@pytest.mark.parametrize("code,V,kv,Q,kv_b,m_a", ENC_CASES,
                         ids=["%s_V%d_kv%d_%d" % (synth.CODE_NAMES[c], v, k, kb) for c, v, k, qq, kb, ma in ENC_CASES])
def test_encode_matches_oracle(q, dev, code, V, kv, Q, kv_b, m_a):
    import torch
    m, n = 256, 288                      # 288 tiles: more than one per workgroup
    host = synth.make_layer(code, m, n, 0, V=V, Q=Q, kv=kv, kv_b=kv_b, m_a=m_a,
                            tag="enc%d_%d_%d_%d" % (code, V, kv, kv_b))
    rng = synth.rng_for("encw", code, kv)
    W = (host.scale * rng.standard_normal((m, n))).astype(np.float32)
    _say("encode", synth.CODE_NAMES[code], V, kv, kv_b, m_a)
    want, sse = oracle.encode_layer(host, W)
    lay = q.upload_layer(host, dev)
    got = q.encode(lay, torch.from_numpy(W).to(dev))
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "first differing code words %s of %d" % (bad[:8], got.size)
    # the codes decode (on the GPU) to a layer with the reported error
    lay2 = q.upload_layer(synth.with_codes(host, got), dev)
    out = torch.empty((host.n_tiles, 256), dtype=torch.int16, device=dev)
    q.qdec_decode_tile(lay2, 0, host.n_tiles, out)
    torch.cuda.synchronize()
    tiles = out.cpu().numpy().view(np.float16).astype(np.float64) * np.float32(host.scale)
    W2 = np.zeros((m, n))
    for i in range(host.n_tiles):
        R, C = _storage_coords(host, i)
        W2[R * 16:R * 16 + 16, C * 16:C * 16 + 16] = tiles[i].reshape(16, 16)
    assert abs(((W - W2) ** 2).sum() - sse) <= 1e-3 * sse


def _storage_coords(host, i):
    """Grid coordinates of storage index i (the part boundary of a
    half-TCQ layer included)."""
    tpr = host.n // 16
    ta = (host.m_a // 16) * tpr if host.m_a else host.n_tiles
    j = i if i < ta else i - ta
    R, C = (j >> 3) // tpr * 8 + (j & 7), (j >> 3) % tpr
    return (R if i < ta else R + host.m_a // 16), C
