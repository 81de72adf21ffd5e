"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/piattn_oracle.c) is built with gcc
  -fsanitize=address,undefined and the oracle pin tests run against it.
* The library is built with its host code instrumented the same way (device
  code unchanged, the sanitizer flags go to the host pass only) and the
  C-ABI rejection tests run against it: argument validation, kernel
  selection and the error paths, with fake device addresses that nothing
  dereferences.

Each run is a child process with the sanitizer runtime preloaded; a report
aborts it (halt on error), so a clean exit means no report.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_context_piattn_amd", "csrc")
sys.path.insert(0, ROOT)
from sparse_long_context_piattn_amd.build import SOURCES  # noqa: E402  (the library's own source list)
SAN_OPTS = "detect_leaks=0:halt_on_error=1:abort_on_error=0"


def _gcc_runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def _run(cmd, env, timeout):
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    with tempfile.TemporaryDirectory(prefix="piattn_san_") as tmp:
        lib = os.path.join(tmp, "liboracle_san.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                               "-fno-omit-frame-pointer", "-o", lib, os.path.join(ROOT, "oracle", "piattn_oracle.c"),
                               "-lm"])
        env = dict(os.environ, PIATTN_ORACLE_LIB=lib, LD_PRELOAD=asan + " " + ubsan, ASAN_OPTIONS=SAN_OPTS,
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
        out = _run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_oracle_pins.py")], env, 1500)
        assert " passed" in out


def test_c_abi_validation_under_asan_and_ubsan():
    asan = _clang_asan_runtime()
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not asan or not os.path.exists(hipcc):
        pytest.skip("hipcc or clang's ASan runtime not installed")
    with tempfile.TemporaryDirectory(prefix="piattn_san_") as tmp:
        procs, objs = [], []
        for s in SOURCES:
            obj = os.path.join(tmp, s + ".o")
            cmd = [hipcc, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", obj, "-O1", "-g", "-std=c++17", "-fPIC",
                   "--offload-arch=gfx950", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                   "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
            objs.append(obj)
        for p in procs:
            out, _ = p.communicate()
            assert p.returncode == 0, out
        lib = os.path.join(tmp, "libpiattn_hostsan.so")
        subprocess.check_call([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", lib] + objs +
                              ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"])
        runner = ("import sys; sys.path.insert(0, %r); import pytest; "
                  "from sparse_long_context_piattn_amd import binding; binding.LIB_PATH = %r; "
                  "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', %r]))"
                  % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi_cpu.py")))
        env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS=SAN_OPTS,
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        out = _run([sys.executable, "-c", runner], env, 900)
        assert " passed" in out
