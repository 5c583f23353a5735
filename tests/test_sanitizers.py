"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer builds (CPU only).

* The fp64 oracle (oracle/oracle.c) is compiled with gcc and both sanitizers,
  together with a driver (tests/sanitize/oracle_check.c) that calls every
  exported oracle function on small inputs in each input format and with
  rejected arguments; leaks are checked too.
* The library's host code (attn_api.hip: validation, library-owned buffers,
  the kernel-timing session) is compiled with both sanitizers on its host
  side only, linked with the library's other objects as built for gfx950, and
  driven by tests/sanitize/abi_check.cpp through every entry point's
  rejection paths (no GPU is touched).

Each run must exit 0 with no sanitizer report.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "exact_attention_28_amd")
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-pthread", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          os.path.join(SAN, "oracle_check.c"), os.path.join(ROOT, "oracle", "oracle.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV)
    assert "ok" in r.stdout and "ERROR" not in r.stderr and "runtime error" not in r.stderr


def test_library_host_code_under_asan_ubsan(tmp_path):
    if shutil.which("hipcc") is None or not os.path.exists(CLANG):
        pytest.skip("ROCm toolchain not available")
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.hip.o")))
    if len(objs) < 2:
        from exact_attention_28_amd import build
        build.build()
        objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.hip.o")))
    kernels = [o for o in objs if not o.endswith("attn_api.hip.o")]
    api = str(tmp_path / "attn_api_san.o")
    # sanitizers on the host side of the compilation only
    _run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-omit-frame-pointer",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
          "-c", os.path.join(PKG, "csrc", "attn_api.hip"), "-o", api])
    drv = str(tmp_path / "abi_check.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
          "-I", "/opt/rocm/include", "-c", os.path.join(SAN, "abi_check.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_check")
    _run([CLANG, "-fsanitize=address,undefined", drv, api, *kernels, "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=ENV)
    assert "ok" in r.stdout and "ERROR" not in r.stderr and "runtime error" not in r.stderr
