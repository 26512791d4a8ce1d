"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/qdec.h declares, sizes workspaces, and rejects bad
arguments with a negative status before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "qdec.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qdec_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def q():
    import dequant_matmul_packed_amd as q
    return q


def test_header_functions_exported(q):
    names = _header_functions()
    assert set(names) == set(q.EXPORTS)
    lib = ctypes.CDLL(q.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(q):
    assert q._lib.qdec_abi_version() == q.QDEC_ABI_VERSION
    for st in (0, -1, -2, -3, -4, -5):
        assert q._status_string(st) not in ("", "unknown status")
    assert q._status_string(7) == "unknown status"


FAKE = 0x7F0000000000   # never dereferenced: every case below fails validation


def _layer(q, **kw):
    base = dict(code=q.QDEC_CODE_HYB, L=16, k=2, V=2, Q=9, m=256, n=128, codes=FAKE, lut=FAKE + 4096,
                group_scale=None, group=0, layer_scale=0.02, sign_in=None, sign_out=None,
                had_in=128, had_out=256)
    base.update(kw)
    return q.Layer(**base)


def test_workspace_sizes(q):
    """qdec_gemv's workspace: fp16 x' (b x n), then the fp32 K slices of the
    largest set any call of up to b columns writes, each part 256-byte
    aligned; nothing in it needs initialising."""
    lay = _layer(q)                        # 256 x 128
    # b = 1: x' 128 * 2 = 256 B.  Slices: the MFMA GEMV's ranges of 512
    # columns (one range: 1 x 256 rows x 4 B = 1024) and the dot-product
    # GEMV's chunks (256 columns: one chunk, 1024 B) -> 1024.
    gv = q.qdec_workspace_bytes(lay, 1, q.QDEC_OP_GEMV)
    assert gv == 256 + 1024
    # b = 8: x' 8 * 128 * 2 = 2048; the dot-product GEMV takes 64-column
    # chunks at b > 1 (two chunks: 2 x 8 x 256 x 4 = 16384 B)
    assert q.qdec_workspace_bytes(lay, 8, q.QDEC_OP_GEMV) == 2048 + 16384
    # a 4096 x 4096 layer at b = 1: x' 8192 B; 16 chunks of 256 columns
    # (16 x 4096 x 4 = 262144) cover the MFMA GEMV's 8 ranges of 512
    big = _layer(q, m=4096, n=4096, had_in=4096, had_out=4096)
    assert q.qdec_workspace_bytes(big, 1, q.QDEC_OP_GEMV) == 8192 + 262144
    # a workspace for a batch covers every smaller one
    for l in (lay, big, _layer(q, m=28672, n=4096, had_in=4096, had_out=4096)):
        sizes = [q.qdec_workspace_bytes(l, b, q.QDEC_OP_GEMV) for b in range(1, 9)]
        assert sizes == sorted(sizes)
    gm = q.qdec_workspace_bytes(lay, 64, q.QDEC_OP_GEMM)
    # X' (b x n fp16), then one fp32 b x m slice per K split (here 2: n/64)
    assert gm == 64 * 128 * 2 + 2 * 64 * 256 * 4
    # a half-TCQ layer needs the same workspace as one of a single width
    half = _layer(q, k=0, kv=5, m_a=128, kv_b=6)
    assert q.qdec_workspace_bytes(half, 1, q.QDEC_OP_GEMV) == gv
    assert q.qdec_workspace_bytes(half, 64, q.QDEC_OP_GEMM) == gm
    assert q.qdec_workspace_bytes(lay, 9, q.QDEC_OP_GEMV) == 0
    assert q.qdec_workspace_bytes(lay, 0, q.QDEC_OP_GEMM) == 0
    assert q.qdec_workspace_bytes(lay, 1, 99) == 0


def test_group_workspace_sizes(q):
    """qdec_gemv_group: one set of fp32 range slices per layer (m rows each,
    256-byte aligned), with one column range for the whole group."""
    # q, k, v of the Llama-8B layer: 48 panels of 128 rows; ranges of 1024
    # columns give 192 units (one round of 256 workgroups, 4 steps per
    # quarter); 4 slices per layer
    qq = _layer(q, m=4096, n=4096, had_in=4096, had_out=4096)
    kk = _layer(q, m=1024, n=4096, had_in=4096, had_out=1024)
    vv = _layer(q, m=1024, n=4096, had_in=4096, had_out=1024)
    assert q.qdec_gemv_group_workspace_bytes([qq, kk, vv]) == 4 * 4 * (4096 + 1024 + 1024)
    # gate and up: 224 panels, one range of 4096 columns (224 units)
    g = _layer(q, m=14336, n=4096, had_in=4096, had_out=2048)
    assert q.qdec_gemv_group_workspace_bytes([g, g]) == 2 * 14336 * 4
    # a bad layer, no layers, too many layers: 0
    assert q.qdec_gemv_group_workspace_bytes([qq, _layer(q, m=100)]) == 0
    assert q.qdec_gemv_group_workspace_bytes([]) == 0
    assert q.qdec_gemv_group_workspace_bytes([qq] * 9) == 0


BAD_LAYERS = [
    dict(m=100), dict(n=40), dict(m=0), dict(k=0), dict(k=9), dict(Q=0), dict(V=3), dict(L=12),
    dict(code=6, L=12, V=1), dict(code=6, L=16, V=2), dict(code=6, L=16, V=1, lut=None),
    dict(code=1, V=1, k=9),
    dict(had_in=3), dict(had_in=256), dict(had_out=512), dict(codes=FAKE + 8), dict(codes=None),
    dict(lut=None), dict(code=9), dict(code=4, L=3, k=3, V=1, group=128, group_scale=None),
    dict(code=4, L=3, k=3, V=1, group=24, group_scale=FAKE), dict(code=5, L=6, k=2, V=2),
    dict(code=2, V=2), dict(layer_scale=float("nan")),
    # bits per step and half-TCQ parts
    dict(kv=5), dict(k=0, kv=17), dict(k=0, kv=5, m_a=100, kv_b=6), dict(k=0, kv=5, m_a=256, kv_b=6),
    dict(kv_b=6), dict(k=0, kv=5, m_a=128, kv_b=0), dict(m_a=-128, kv_b=4),
    dict(code=4, L=3, k=0, kv=3, V=1, group=128, group_scale=FAKE),
    dict(code=5, L=4, k=2, V=2, m_a=128, kv_b=4),
]


@pytest.mark.parametrize("kw", BAD_LAYERS, ids=[str(k) for k in BAD_LAYERS])
def test_invalid_layers_rejected(q, kw):
    lay = _layer(q, **kw)
    d = ctypes.byref(lay.desc())
    assert q.qdec_workspace_bytes(lay, 1, q.QDEC_OP_GEMV) == 0
    ws = FAKE + (1 << 20)
    for fn in ("qdec_gemv", "qdec_gemm"):
        st = q.raw_status(fn, d, FAKE + (1 << 24), FAKE + (1 << 25), 1, ws, 1 << 20, None)
        assert st in (q.QDEC_EINVAL, q.QDEC_EUNSUPPORTED), (fn, st)
    assert q.raw_status("qdec_decode_tile", d, 0, 1, FAKE + (1 << 24), None) in (
        q.QDEC_EINVAL, q.QDEC_EUNSUPPORTED)


@pytest.mark.parametrize("kw", [dict(k=5), dict(Q=13), dict(k=0, kv=9), dict(k=0, kv=3),
                                dict(k=0, kv=5, m_a=128, kv_b=9), dict(code=2, V=1, k=0, kv=5),
                                dict(code=2, V=1, k=2, m_a=128, kv_b=6)])
def test_unsupported_but_valid(q, kw):
    lay = _layer(q, **kw)
    d = ctypes.byref(lay.desc())
    assert q.raw_status("qdec_decode_tile", d, 0, 1, FAKE + (1 << 24), None) == q.QDEC_EUNSUPPORTED


def test_call_argument_errors(q):
    lay = _layer(q)
    d = ctypes.byref(lay.desc())
    X, Y, WS = FAKE + (1 << 24), FAKE + (1 << 25), FAKE + (1 << 26)
    need = q.qdec_workspace_bytes(lay, 1, q.QDEC_OP_GEMV)
    E = q.QDEC_EINVAL
    assert q.raw_status("qdec_gemv", d, None, Y, 1, WS, need, None) == E
    assert q.raw_status("qdec_gemv", d, X, None, 1, WS, need, None) == E
    assert q.raw_status("qdec_gemv", d, X + 2, Y, 1, WS, need, None) == E         # misaligned x
    assert q.raw_status("qdec_gemv", d, X, Y, 0, WS, need, None) == E
    assert q.raw_status("qdec_gemv", d, X, Y, 9, WS, need, None) == q.QDEC_EUNSUPPORTED
    assert q.raw_status("qdec_gemv", d, X, X + 64, 1, WS, need, None) == E        # x and y overlap
    assert q.raw_status("qdec_gemv", d, X, Y, 1, None, need, None) == q.QDEC_EWORKSPACE
    assert q.raw_status("qdec_gemv", d, X, Y, 1, WS, need - 4, None) == q.QDEC_EWORKSPACE
    assert q.raw_status("qdec_gemv", d, X, Y, 1, WS + 16, need, None) == q.QDEC_EWORKSPACE
    assert q.raw_status("qdec_gemv", d, X, Y, 1, X, need, None) == E              # ws overlaps x
    assert q.raw_status("qdec_gemm", d, X, Y, 257, WS, 1 << 30, None) == q.QDEC_EUNSUPPORTED
    ntiles = (256 // 16) * (128 // 16)
    assert q.raw_status("qdec_decode_tile", d, -1, 1, Y, None) == E
    assert q.raw_status("qdec_decode_tile", d, ntiles - 1, 2, Y, None) == E
    assert q.raw_status("qdec_decode_tile", d, 0, 1, None, None) == E
    assert q.raw_status("qdec_decode_tile", d, 0, 0, None, None) == q.QDEC_OK    # nothing to do
    R = q.raw_status
    assert R("qdec_rht", X, 0, Y, 0, 1, 96, 64, None, 0, ctypes.c_float(1.0), None) == E  # block
    assert R("qdec_rht", X, 2, Y, 0, 1, 64, 64, None, 0, ctypes.c_float(1.0), None) == E  # dtype
    assert R("qdec_rht", X, 0, Y, 0, 1, 64, 64, None, 2, ctypes.c_float(1.0), None) == E  # mode
    assert R("qdec_rht", X, 0, X + 2, 0, 1, 64, 64, None, 0, ctypes.c_float(1.0), None) == E
    assert R("qdec_rht", X, 0, X, 1, 1, 64, 64, None, 0, ctypes.c_float(1.0), None) == E
    assert R("qdec_rht", X, 0, Y, 0, 1, 1 << 15, 1 << 15, None, 0, ctypes.c_float(1.0),
             None) == q.QDEC_EUNSUPPORTED


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="a valid call would launch on a real device")
def test_valid_call_without_device_reports_enodev(q):
    lay = _layer(q)
    d = ctypes.byref(lay.desc())
    need = q.qdec_workspace_bytes(lay, 1, q.QDEC_OP_GEMV)
    st = q.raw_status("qdec_gemv", d, FAKE + (1 << 24), FAKE + (1 << 25), 1, FAKE + (1 << 26), need, None)
    assert st == q.QDEC_ENODEV


def test_encode_workspace_and_argument_errors(q):
    lay = _layer(q)
    # one [256/V][1024] word array of backpointers per encoder workgroup (256)
    assert q.qdec_workspace_bytes(lay, 1, q.QDEC_OP_ENCODE) == 256 * 128 * 1024 * 4
    mad = _layer(q, code=q.QDEC_CODE_1MAD, V=1)
    assert q.qdec_workspace_bytes(mad, 1, q.QDEC_OP_ENCODE) == 256 * 256 * 1024 * 4
    assert q.qdec_workspace_bytes(lay, 2, q.QDEC_OP_ENCODE) == 0
    lut = _layer(q, code=q.QDEC_CODE_LUT, V=1)
    assert q.qdec_workspace_bytes(lut, 1, q.QDEC_OP_ENCODE) == 0
    d = ctypes.byref(lay.desc())
    W, C, WS = FAKE + (1 << 24), FAKE + (1 << 26), FAKE + (1 << 28)
    need = q.qdec_workspace_bytes(lay, 1, q.QDEC_OP_ENCODE)
    E = q.QDEC_EINVAL
    assert q.raw_status("qdec_encode", d, None, C, WS, need, None) == E
    assert q.raw_status("qdec_encode", d, W, None, WS, need, None) == E
    assert q.raw_status("qdec_encode", d, W + 2, C, WS, need, None) == E        # misaligned w
    assert q.raw_status("qdec_encode", d, W, C + 4, WS, need, None) == E        # misaligned codes
    assert q.raw_status("qdec_encode", d, W, W + 64, WS, need, None) == E       # codes overlap w
    assert q.raw_status("qdec_encode", d, W, C, None, need, None) == q.QDEC_EWORKSPACE
    assert q.raw_status("qdec_encode", d, W, C, WS, need - 4, None) == q.QDEC_EWORKSPACE
    assert q.raw_status("qdec_encode", d, W, C, WS + 16, need, None) == q.QDEC_EWORKSPACE
    assert q.raw_status("qdec_encode", d, W, C, W, need, None) == E             # ws overlaps w
    dl = ctypes.byref(lut.desc())
    assert q.raw_status("qdec_encode", dl, W, C, WS, need, None) == q.QDEC_EUNSUPPORTED
    for kw in BAD_LAYERS[:6]:
        bad = _layer(q, **kw)
        assert q.raw_status("qdec_encode", ctypes.byref(bad.desc()), W, C, WS, need, None) in (
            q.QDEC_EINVAL, q.QDEC_EUNSUPPORTED)


def test_group_call_errors_before_any_launch(q):
    """qdec_gemv_group rejects bad arguments on the host; with valid
    arguments and no device it returns ENODEV (nothing is dereferenced)."""
    import ctypes as C
    a = _layer(q, m=256, n=128)
    b = _layer(q, m=384, n=128, had_out=128)
    layers = [a, b]
    descs = [l.desc() for l in layers]
    lp = (C.c_void_p * 2)(*[C.addressof(d) for d in descs])
    X0, X1 = FAKE + (1 << 24), FAKE + (1 << 24) + 4096
    Y0, Y1 = FAKE + (1 << 25), FAKE + (1 << 25) + 4096
    WS = FAKE + (1 << 26)
    need = q.qdec_gemv_group_workspace_bytes(layers)
    assert need > 0
    xp = (C.c_void_p * 2)(X0, X1)
    yp = (C.c_void_p * 2)(Y0, Y1)
    E, EW = q.QDEC_EINVAL, q.QDEC_EWORKSPACE
    st = lambda *args: q.raw_status("qdec_gemv_group", *args)
    assert st(None, 2, xp, yp, WS, need, None) == E
    assert st(lp, 0, xp, yp, WS, need, None) == E
    assert st(lp, 9, xp, yp, WS, need, None) == q.QDEC_EUNSUPPORTED
    assert st(lp, 2, None, yp, WS, need, None) == E
    assert st(lp, 2, (C.c_void_p * 2)(X0 + 2, X1), yp, WS, need, None) == E        # misaligned x
    assert st(lp, 2, xp, (C.c_void_p * 2)(Y0, Y1 + 2), WS, need, None) == E        # misaligned y
    assert st(lp, 2, xp, (C.c_void_p * 2)(Y0, Y0 + 256), WS, need, None) == E      # outputs overlap
    assert st(lp, 2, xp, (C.c_void_p * 2)(X0, Y1), WS, need, None) == E            # output on an input
    assert st(lp, 2, xp, yp, WS, need - 256, None) == EW                          # too small
    assert st(lp, 2, xp, yp, WS + 16, need, None) == EW                           # misaligned
    assert st(lp, 2, xp, yp, None, need, None) == EW
    bad = [_layer(q, m=100).desc(), descs[1]]
    assert st((C.c_void_p * 2)(*[C.addressof(d) for d in bad]), 2, xp, yp, WS, need, None) == E
    # inputs may be shared (q, k and v read one x)
    assert st(lp, 2, (C.c_void_p * 2)(X0, X0), yp, WS, need, None) == q.QDEC_ENODEV
    assert st(lp, 2, xp, yp, WS, need, None) == q.QDEC_ENODEV


def test_noalloc_entry_point_rejects_before_any_launch(q):
    """qdec_gemv_noalloc: its static workspace is 8 MiB; a call whose
    qdec_gemv workspace would exceed it returns QDEC_EWORKSPACE, and bad
    descriptors or batches are rejected, all before touching a device."""
    assert q.qdec_noalloc_scratch_bytes() == 8 << 20
    big = _layer(q, m=128, n=1 << 20, had_in=16384, had_out=128)
    assert q.qdec_workspace_bytes(big, 8, q.QDEC_OP_GEMV) > q.qdec_noalloc_scratch_bytes()
    X, Y = FAKE + (1 << 24), FAKE + (1 << 25)
    st = lambda lay, b: q.raw_status("qdec_gemv_noalloc", ctypes.byref(lay.desc()), X, Y, b, None)
    assert st(big, 8) == q.QDEC_EWORKSPACE
    assert st(_layer(q, m=100), 1) == q.QDEC_EINVAL
    assert st(_layer(q), 0) == q.QDEC_EINVAL
    assert st(_layer(q), 9) == q.QDEC_EUNSUPPORTED
    assert st(_layer(q), 1) == q.QDEC_ENODEV          # valid: no device here


def test_header_abi_version_matches_binding(q):
    """The binding's copy of the header's ABI version."""
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "qdec.h")).read()
    assert int(re.search(r"#define QDEC_ABI_VERSION (\d+)u", hdr).group(1)) == q.QDEC_ABI_VERSION


def test_fail_launches_hook_arguments(q):
    """qdec_debug_fail_launches: a negative count is rejected; a pending
    injected failure is taken only by a call that reaches the launch stage,
    so argument errors (and, with no device, ENODEV) come first."""
    assert q._lib.qdec_debug_fail_launches(-1) == q.QDEC_EINVAL
    assert q._lib.qdec_debug_fail_launches(1) == q.QDEC_OK
    try:
        lay = _layer(q)
        d = ctypes.byref(lay.desc())
        need = q.qdec_workspace_bytes(lay, 1, q.QDEC_OP_GEMV)
        # an argument error wins over the pending failure
        assert q.raw_status("qdec_gemv", d, FAKE + 2, FAKE + (1 << 25), 1, FAKE + (1 << 26), need,
                            None) == q.QDEC_EINVAL
        if not _has_gpu():
            st = q.raw_status("qdec_gemv", d, FAKE + (1 << 24), FAKE + (1 << 25), 1, FAKE + (1 << 26), need,
                              None)
            assert st == q.QDEC_ENODEV
    finally:
        assert q._lib.qdec_debug_fail_launches(0) == q.QDEC_OK
