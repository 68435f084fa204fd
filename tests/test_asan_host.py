"""The host-side code of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The library's host objects -- argument validation and dispatch (abi.cpp),
the no-allocation entry point's host part (noalloc.hip), Pulsar's Max-IDF
selection (pulsar.cpp) and the rocBLAS wrapper (blas.cpp) -- are rebuilt
with AddressSanitizer and UndefinedBehaviorSanitizer (undefined behaviour
aborts) on their host pass and linked with the normal kernel objects.  The
ABI tests (every entry point's validation, the Pulsar selection against the
oracle, the RoPE frequencies) then run against that
build in a child Python process with the sanitizer runtime preloaded
(Python itself is not instrumented).  A planted overflow -- the Pulsar call
told that its output holds more rows than it does -- must be reported, so a
silently inactive sanitizer cannot pass.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_amd", "csrc")
HOST_SRCS = ("abi.cpp", "pulsar.cpp", "noalloc.hip", "blas.cpp")


def asan_runtime():
    from block_sparse_amd import build as B
    llvm = os.path.dirname(os.path.dirname(os.path.realpath(B.hipcc())))
    cands = sorted(glob.glob(os.path.join(llvm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    cands += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        pytest.fail("no clang AddressSanitizer runtime found next to hipcc")
    return cands[-1]


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    from block_sparse_amd import build as B
    objdir = B.OUT_DIR
    kernels = [os.path.join(objdir, os.path.basename(s) + ".o") for s in B.sources()
               if os.path.basename(s) not in HOST_SRCS]
    if not all(os.path.exists(o) for o in kernels):
        B.build()
    out = tmp_path_factory.mktemp("asan")
    objs = []
    for name in HOST_SRCS:
        obj = str(out / (name + ".o"))
        cmd = [B.hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}",
               *B.DEVICE_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, name), "-o", obj,
               "-Xarch_host", "-fsanitize=address,undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined",
               "-Xarch_host", "-fno-omit-frame-pointer"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        objs.append(obj)
    lib = str(out / "libstarattn_asan.so")
    cmd = [B.hipcc(), "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *objs, *kernels, "-o", lib,
           "-lrocblas", "-Xarch_host", "-fsanitize=address,undefined",
           "-Xarch_host", "-shared-libasan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return lib


def run_under_asan(lib, args, timeout=600):
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), STAR_ATTN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    return subprocess.run([sys.executable, *args], capture_output=True, text=True, env=env,
                          cwd=ROOT, timeout=timeout)


PLANTED = """
import ctypes, numpy as np
from block_sparse_amd import _lib
lib = _lib.load()
L, b = 4096, 1024
tok = np.random.default_rng(0).integers(0, 50000, L).astype(np.int32)
rows = np.zeros(16, dtype=np.int64)          # far fewer rows than the call is told
n = ctypes.c_int64(0)
st = np.zeros(4, np.int64); ln = np.zeros(4, np.int64)
P64 = ctypes.POINTER(ctypes.c_int64)
lib.star_pulsar_prefix(tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), L, b, 32, 64, 16,
                       rows.ctypes.data_as(P64), 100000, ctypes.byref(n),
                       st.ctypes.data_as(P64), ln.ctypes.data_as(P64), 4)
print("no report", n.value)
"""


def test_undefined_behaviour_checks_are_compiled_in(asan_lib):
    """The host objects carry UndefinedBehaviorSanitizer checks (their
    handlers are referenced by this build of the library), so the ABI tests
    below also run under them."""
    r = subprocess.run(["nm", "-D", "--undefined-only", asan_lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "__ubsan_handle_" in r.stdout
    assert "__asan_" in r.stdout


def test_sanitizer_catches_a_planted_overflow(asan_lib):
    r = run_under_asan(asan_lib, ["-c", PLANTED])
    assert r.returncode == 23 and "AddressSanitizer" in r.stderr, (r.returncode, r.stderr[-2000:])


def test_abi_host_tests_under_asan(asan_lib):
    r = run_under_asan(asan_lib, ["-m", "pytest", "-q", "-p", "no:cacheprovider",
                                  os.path.join("tests", "test_abi_host.py")])
    assert "AddressSanitizer" not in r.stderr + r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
