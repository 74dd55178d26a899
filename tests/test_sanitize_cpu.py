"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs of the two pieces
of C that run on the CPU: the fp64 oracle (built with gcc) and the C ABI's
host layer (its hipcc host pass instrumented, the kernels linked in
uninstrumented).  Each driver under tests/sanitize/ walks its code's paths
that need no GPU and exits 0 only when every call did what it should; a
sanitizer report aborts it with a non-zero status."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:] + r.stderr[-4000:]
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_asan")
    _run([gcc, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", os.path.join(ROOT, "oracle", "gdn_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm", "-pthread"])
    r = _run([exe], env=SAN_ENV)
    assert "oracle driver: ok" in r.stdout


def test_abi_host_layer_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from linear_attention_delta_amd import build
    hipcc = build.HIPCC
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(hipcc) or not os.path.exists(clang):
        pytest.skip("no ROCm toolchain")
    kernels = [s for s in build.SOURCES if s.endswith(".hip")]
    objs = [os.path.join(build.BUILD_DIR, s + ".o") for s in kernels]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    flags = [f for f in build.COMMON if f not in ("-O3", "-fPIC")]
    api = str(tmp_path / "gdn_api_san.o")
    # the sanitizer options apply to the host pass only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([hipcc] + flags + ["-O1", "-g", "-x", "hip"] + san +
         ["-c", os.path.join(build.CSRC, "gdn_api.cpp"), "-o", api])
    nm = shutil.which("nm")
    if nm:  # the host pass really is instrumented
        syms = _run([nm, api]).stdout
        assert "__asan_" in syms and "__ubsan_" in syms
    drv = str(tmp_path / "abi_driver.o")
    _run([clang, "-O1", "-g", "-std=c++17", "-I" + build.INCLUDE, "-fsanitize=address,undefined",
          "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_asan")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(clang)), "..", "lib")
    _run([clang, "-fsanitize=address,undefined", drv, api] + objs +
         ["-L" + rocm_lib, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe])
    r = _run([exe], env=SAN_ENV)
    assert "abi driver: ok" in r.stdout
