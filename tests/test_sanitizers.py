"""CPU AddressSanitizer and UndefinedBehaviorSanitizer runs (no GPU needed):

- the oracle (plain C) built with gcc -fsanitize=address,undefined, then the
  oracle pins run against that build in a child process;
- the library's host code (api.hip: descriptor validation, workspace sizing,
  call planning) built by hipcc with the host-side sanitizers only (the
  device code is compiled as usual), linked with the other objects of the
  library, then the C-ABI tests run against it in a child process.

Any sanitizer report aborts the child (-fno-sanitize-recover=all), and the
test fails.  Leak checking is off: the Python interpreter itself keeps
allocations until exit."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dequant_matmul_packed_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("san"))


def test_oracle_pins_under_asan_ubsan(workdir):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    lib = os.path.join(workdir, "liboracle_san.so")
    rc, out = _run([gcc, *SAN_FLAGS, "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                    os.path.join(ROOT, "oracle", "qdec_oracle.c"), "-o", lib, "-lm"])
    assert rc == 0, out
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run([gcc, "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD="%s:%s" % (asan, ubsan), QDEC_ORACLE_SANITIZED_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    # every pin except the exhaustive fp16 binades (16.7 million values each)
    rc, out = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", "not exhaustive_binades"],
                   env=env, timeout=900)
    assert rc == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_library_host_code_under_asan_ubsan(workdir):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    objs = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.endswith(".o") and f != "api.o") \
        if os.path.isdir(BUILD) else []
    if not objs:
        pytest.skip("the library's objects are not built (run __graft_entry__.build())")
    obj = os.path.join(workdir, "api_san.o")
    host = []
    for f in SAN_FLAGS:
        host += ["-Xarch_host", f]
    rc, out = _run([hipcc, "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", *host, "-Xarch_host", "-shared-libasan",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "api.hip"),
                    "-o", obj], timeout=900)
    assert rc == 0, out
    lib = os.path.join(workdir, "libqdec_san.so")
    rc, out = _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libasan",
                    "-fsanitize=address,undefined", "-o", lib, obj, *objs], timeout=900)
    assert rc == 0, out
    rt = subprocess.run([hipcc.replace("hipcc", "amdclang++") if os.path.exists(hipcc.replace("hipcc", "amdclang++"))
                         else "/opt/rocm/llvm/bin/clang++", "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not os.path.exists(rt):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not found:
            pytest.skip("clang's ASan runtime not found")
        rt = found[0]
    env = dict(os.environ, LD_PRELOAD=rt, QDEC_SANITIZED_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    script = os.path.join(ROOT, "tests", "sanitized_abi_child.py")
    rc, out = _run([sys.executable, script], env=env, timeout=900)
    assert rc == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "sanitized ABI checks passed" in out, out[-4000:]
