"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

`tests/sanitize/abi_check.cpp` drives every validation path of the C ABI
(sizes up to 2^62, misaligned and null pointers, unknown enum values, the
workspace arithmetic).  It is linked against `api.cpp` compiled with host-side
sanitizers (device code is compiled as usual and never runs: every call is
rejected, or is a no-op, before the library touches a GPU).  Any
out-of-bounds access, leak, signed overflow, invalid enum load or other
undefined behaviour aborts the program and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_memory_relation_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{out}"
    return out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not installed")
def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE, "-I", CSRC,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    # host code of the ABI with sanitizers (each flag for the host pass only)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([HIPCC, *common, *host_san, "-c", os.path.join(CSRC, "api.cpp"), "-o", "api.o"], tmp_path)
    # the kernels, unchanged (linked, never launched)
    for src in ("kernels", "wide", "proj"):
        _run([HIPCC, *common, "-c", os.path.join(CSRC, src + ".hip"), "-o", src + ".o"], tmp_path)
    # the check program and the link, host only
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    _run([CLANG, "-std=c++17", "-g", "-I", INCLUDE, *san, "-c", os.path.join(ROOT, "tests", "sanitize",
                                                                             "abi_check.cpp"), "-o", "drv.o"],
         tmp_path)
    _run([CLANG, *san, "drv.o", "api.o", "kernels.o", "wide.o", "proj.o", "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", "abi_check"], tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([os.path.join(tmp_path, "abi_check")], cwd=tmp_path, capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0 and "OK: 0 failure(s)" in r.stdout, r.stdout + r.stderr
