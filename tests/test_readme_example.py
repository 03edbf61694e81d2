"""The C example in README.md compiles against include/flh.h (syntax and types only; CPU)."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_readme_c_example_compiles(tmp_path):
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```c\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    src = tmp_path / "example.cpp"
    src.write_text(blocks[0])
    res = subprocess.run(["g++", "-std=c++17", "-fsyntax-only", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), str(src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
