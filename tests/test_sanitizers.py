"""CPU sanitizer builds (no GPU): AddressSanitizer + UndefinedBehaviorSanitizer.

* The fp64 oracle (oracle/wide_oracle.c, gcc) driven by tests/sanitize/
  oracle_driver.c: every entry point on small inputs, row subsets, empty
  inputs and rejected arguments.
* The host side of libwide.so (csrc/wide_api.cpp: validation, workspace
  layout, dispatch), compiled for the host only and linked against stand-in
  launchers (tests/sanitize/host_driver.cpp) that write every byte the real
  kernels write into exact-size host buffers, plus C callers passing enum
  values outside their enumerators (tests/sanitize/c_caller.c).
The sanitizers abort on the first error (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "group_sparse_ffn_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas",
          os.path.join(ROOT, "oracle", "wide_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
          "-o", exe, "-lm"])
    out = _run([exe], env=ENV)
    assert "ok" in out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_host_validation_under_asan_ubsan(tmp_path):
    obj = str(tmp_path / "c_caller.o")
    exe = str(tmp_path / "host_san")
    _run([CLANG, "-c", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", f"-I{INCLUDE}", os.path.join(SAN, "c_caller.c"), "-o", obj])
    # host-only compile of the HIP source; each sanitizer flag applies to the host pass
    _run([HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "wide_api.cpp"),
          os.path.join(SAN, "host_driver.cpp"), "-x", "none", obj, "-o", exe])
    out = _run([exe], env=ENV)
    assert "host sanitizer driver: ok" in out
