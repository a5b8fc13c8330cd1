"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer: api.cpp is
compiled again with both sanitizers for the host side only, linked with the library's device
objects from the regular build, and driven by tests/host_abi_driver.cpp through the argument
checks, size and workspace arithmetic, the k-split plan scan and the descriptor checks. None
of those calls reaches a GPU, so this runs on the CPU. Needs the regular build (_build/)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "host_sanitized")
CSRC = os.path.join(ROOT, "transformer_encoder_remove_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
# host-side sanitizer flags, each behind -Xarch_host so that no device code is instrumented
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_abi_under_asan_and_ubsan():
    objs = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD)
                  if f.endswith(".hip.o")) if os.path.isdir(BUILD) else []
    if not objs or not os.path.exists(CLANGXX):
        pytest.skip("needs the regular build's device objects and the ROCm clang")
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "api.cpp.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
          "-I", CSRC, "-I", INCLUDE, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o])
    lib = os.path.join(OUT, "libtel_hostsan.so")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "lib")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_o, *objs, "-o", lib,
          "-L", rocm_lib, f"-Wl,-rpath,{rocm_lib}", "-lrocprofiler-sdk-roctx"])
    exe = os.path.join(OUT, "host_abi_driver")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", INCLUDE,
          os.path.join(ROOT, "tests", "host_abi_driver.cpp"), lib, f"-Wl,-rpath,{OUT}",
          "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "host ABI checks passed" in r.stdout, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
