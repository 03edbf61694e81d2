"""The ABI tests again, against a host build of the ABI layer (flh_api.cpp) under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The layer is compiled with g++ (it holds no device code), with the kernel launchers
replaced by stubs (tests/abi_host_stubs.cpp), and tests/test_abi.py runs in a child
process that preloads the sanitizer runtimes and loads that build through
FLH_LIBRARY.  A sanitizer report fails the child, and so this test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not found")
    lib = str(tmp_path / "libflh_sanitized.so")
    build = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
             "-I", os.path.join(ROOT, "entropy_block_sparse_amd", "csrc"), "-I", os.path.join(ROCM, "include"),
             os.path.join(ROOT, "entropy_block_sparse_amd", "csrc", "flh_api.cpp"),
             os.path.join(ROOT, "tests", "abi_host_stubs.cpp"),
             "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", lib]
    res = subprocess.run(build, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ)
    env.update({"FLH_LIBRARY": lib, "LD_PRELOAD": f"{asan}:{ubsan}",
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert "passed" in res.stdout
