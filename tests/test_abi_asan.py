"""The host-side C-ABI layer under AddressSanitizer.

ra_abi.cpp (argument validation, range and overlap checks, the segment
tables) is built for the CPU alone with AddressSanitizer, its kernel
launchers replaced by counting stand-ins (tests/abi_stubs.cpp), and the ABI
tests (tests/test_abi.py) run against that build in a subprocess with the
sanitizer runtime preloaded. Any invalid memory access in the validation
code fails the run; the stand-ins also let the tests check that rejected
calls reach no launcher.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_attention_ra_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")


def _asan_runtime():
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not found")
def test_abi_layer_under_address_sanitizer(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("AddressSanitizer runtime not found")
    lib = str(tmp_path / "libra_asan.so")
    cmd = [CLANG, "-x", "c++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "ra_abi.cpp"), os.path.join(ROOT, "tests", "abi_stubs.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["RA_TEST_ABI_LIB"] = lib
    # the tests that call the library (the others exercise the Python binding)
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not binding and not variants and not ring_drivers"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    # every selected test ran, the launch counting one included
    assert " passed" in out and "skipped" not in out, out[-2000:]
