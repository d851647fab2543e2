"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer.

Two instrumented builds, made here in a temporary directory:
  - the oracle, built by gcc with -fsanitize=address,undefined, under which
    the oracle's own test files (its pins, the format variants, the
    chunk-parallel driver) run;
  - the HIP library with its host code instrumented (hipcc, each
    -fsanitize= after -Xarch_host; the device code is unchanged), under which
    the host-side tests run: stream parsing, structural validation of
    corrupt streams, codebook building and argument checks.
Each run is a child pytest with the sanitizer runtime preloaded; any report
fails it (UBSan does not recover, and ASan aborts). A planted over-read
checks that the instrumentation is live: validating a stream whose buffer
is shorter than the size passed must be reported by ASan."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _gcc_asan():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _env(preload, **extra):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": preload, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "PYTHONPATH": ROOT})
    env.update(extra)
    return env


def _run(args, env, timeout=900):
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    import oracle
    from lossless_bf16_tensor_amd import build as hip_build
    d = tmp_path_factory.mktemp("san")
    olib = oracle.build(sanitize=True, out=str(d / "liboracle_san.so"))
    hlib = hip_build.build(sanitize=True, out=str(d / "libuzip_san.so"))
    return olib, hlib


def test_oracle_under_asan_ubsan(san_libs):
    olib, _ = san_libs
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    tests = [t for t in tests if not t.endswith("test_oracle_mutants.py")]   # rebuilds plain copies
    r = _run(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu and not slow",
              *tests, os.path.join(ROOT, "tests", "test_cpu_parallel.py")],
             _env(_gcc_asan(), UZIP_ORACLE_LIB=olib))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_host_library_under_asan_ubsan(san_libs):
    _, hlib = san_libs
    rt = _clang_asan()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    r = _run(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_host_abi.py")],
             _env(rt, UZIP_LIB=hlib))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


PLANTED = r"""
import ctypes, numpy as np, oracle
from lossless_bf16_tensor_amd import uzip
x = np.arange(64, dtype=np.uint16) * 512
ocb = oracle.calibrate(x)
cb = uzip.codebook_from_hist(ocb.hist)
s = oracle.encode(x, 64, ocb.dec)
libc = ctypes.CDLL(None)
libc.malloc.restype = ctypes.c_void_p
p = libc.malloc(300)
ctypes.memmove(p, s.tobytes()[:300], 300)
uzip.lib().uzip_validate_host(ctypes.c_void_p(p), s.size, ctypes.byref(cb))
"""


def test_planted_over_read_is_reported(san_libs):
    _, hlib = san_libs
    rt = _clang_asan()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    r = _run(["-c", PLANTED], _env(rt, UZIP_LIB=hlib), timeout=300)
    assert r.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in r.stderr
