"""Child process of tests/test_sanitizers.py: loads the library built with
host-side sanitizers (QDEC_SANITIZED_LIB) in place of the plain one and runs
the C-ABI tests of test_abi_cpu.py against it (descriptor validation,
workspace sizes, grouped and allocation-free calls, error statuses)."""
import ctypes
import inspect
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import dequant_matmul_packed_amd as q  # noqa: E402

san = ctypes.CDLL(os.environ["QDEC_SANITIZED_LIB"])
for name in q.EXPORTS:
    f, g = getattr(q._lib, name), getattr(san, name)
    g.argtypes, g.restype = f.argtypes, f.restype
q._lib = san

import test_abi_cpu as T  # noqa: E402

ran = 0
for name, fn in sorted(vars(T).items()):
    if not name.startswith("test_") or not callable(fn):
        continue
    params = list(inspect.signature(fn).parameters)
    if params == ["q"]:
        fn(q)
        ran += 1
    elif params == ["q", "kw"] and name == "test_invalid_layers_rejected":
        for kw in T.BAD_LAYERS:
            fn(q, kw)
            ran += 1
print("sanitized ABI checks passed: %d" % ran, flush=True)
