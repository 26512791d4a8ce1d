"""qdec_gemv_noalloc (the workspace in a static device array, for callers
that cannot allocate) against qdec_gemv with a caller workspace, through the
C ABI: bit-identical outputs (the same kernels and summation order) on two
calls in a row, the second with a smaller input, and the oracle's bar."""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _f16(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


def _f64(t):
    import torch
    return t.cpu().view(torch.int16).numpy().view(np.float16).astype(np.float64)


def _rel(y, ref):
    return max(np.linalg.norm(y[c] - ref[c]) / np.linalg.norm(ref[c]) for c in range(ref.shape[0]))


# (code, m, n, k, batch): the first call large (the MFMA GEMV at one column,
# or several columns), the second smaller
CALLS = [
    [(synth.HYB, 14336, 4096, 2, 1), (synth.HYB, 512, 1024, 2, 1)],
    [(synth.HYB, 4096, 4096, 2, 8), (synth.VQ, 1024, 2048, 4, 3)],
]


@pytest.mark.parametrize("pair", range(len(CALLS)))
def test_noalloc_matches_workspace_call(dev, pair):
    import torch
    import dequant_matmul_packed_amd as q
    assert q.qdec_noalloc_scratch_bytes() == 8 << 20
    for i, (code, m, n, k, b) in enumerate(CALLS[pair]):
        _say("noalloc", pair, i, synth.CODE_NAMES[code], m, n, k, b)
        host = synth.make_layer(code, m, n, k, tag="noalloc%d_%d" % (pair, i))
        x16 = synth.activations("noallocx%d_%d" % (pair, i), b, n)
        lay = q.upload_layer(host, dev)
        xt = _f16(x16, dev)
        y_ws = q.gemv(lay, xt)                            # caller workspace
        y_na = torch.empty((b, m), dtype=torch.float16, device=dev)
        q.qdec_gemv_noalloc(lay, xt, y_na, b)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), (pair, i)
        assert _rel(_f64(y_na), oracle.forward(host, x16)) < 2e-3


def test_noalloc_rejects_oversized_layers(dev):
    import dequant_matmul_packed_amd as q
    # 128 x 2^20 at 8 columns (x' alone is 16 MiB) needs more than the 8 MiB
    # scratch: the call returns QDEC_EWORKSPACE before any launch (the layer's
    # buffers are never read)
    lay = q.Layer(code=q.QDEC_CODE_HYB, L=16, k=2, V=2, Q=9, m=128, n=1 << 20, codes=0x7F0000000000,
                  lut=0x7F0000001000, layer_scale=0.02, had_in=16384, had_out=128)
    need = q.qdec_workspace_bytes(lay, 8, q.QDEC_OP_GEMV)
    assert need > q.qdec_noalloc_scratch_bytes()
    st = q.raw_status("qdec_gemv_noalloc", q.ctypes.byref(lay.desc()), 0x7F0000100000, 0x7F0000200000, 8, None)
    assert st == q.QDEC_EWORKSPACE
