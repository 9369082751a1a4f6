"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle's C code (oracle/kda_oracle.c), built with gcc and both
  sanitizers (leak checking on), runs every export through
  tests/sanitize/oracle_driver.c: odd sizes, T = 0, column subsets, several
  thread counts.
- The C ABI layer (kda_api.cpp), its host code built with both sanitizers and
  linked with the kernels' objects of the regular build, runs through
  tests/sanitize/abi_driver.c: size queries at extreme sizes and every entry
  point's rejected arguments.  That driver never reaches a device call and
  refuses to run where a GPU is visible.
"""
import glob
import os
import shutil
import subprocess

import pytest

from chunked_gated_delta_12_amd import build as kbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
LLVM = "/opt/rocm/llvm/bin"


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-Wall", "-Wextra", os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm", "-lpthread", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = _run([exe], env=env)
    assert "oracle driver: ok" in res.stdout


def test_abi_host_code_under_asan_ubsan(tmp_path):
    if os.path.exists("/dev/kfd"):
        pytest.skip("host-only check: runs where no GPU is visible")
    try:
        hipcc = kbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    objs = [p for p in glob.glob(os.path.join(kbuild.BUILD_DIR, "*.hip.o")) if "peaks" not in p]
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if len(objs) < len(kbuild.SOURCES) - 1 or not rt or not os.path.exists(os.path.join(LLVM, "clang")):
        pytest.skip("needs the regular build's objects and the clang sanitizer runtime")
    api = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libkda_san.so")
    exe = str(tmp_path / "abi_driver")
    # host-only sanitizers: every -fsanitize on the hipcc line sits behind -Xarch_host
    _run([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={kbuild.ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"),
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-omit-frame-pointer",
          "-c", os.path.join(kbuild.CSRC, "kda_api.cpp"), "-o", api])
    _run([os.path.join(LLVM, "clang++"), "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan",
          "-o", lib, api] + sorted(objs) + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    _run([os.path.join(LLVM, "clang"), "-std=c11", "-g", "-O1", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-shared-libasan", "-I", os.path.join(ROOT, "include"),
          os.path.join(SAN, "abi_driver.c"), "-L", str(tmp_path), "-lkda_san",
          f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{os.path.dirname(rt[0])}", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = _run([exe], env=env)
    assert "abi driver: ok" in res.stdout
