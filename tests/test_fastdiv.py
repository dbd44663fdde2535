"""The GEMM splits its work with divisions by launch-time constants written
as a multiply-high, an add and a shift (gptq_bit_weight_amd/csrc/
q4_fastdiv.h). The header is plain C++ on the host side, so this builds
tests/fastdiv_check.cpp with the host compiler and compares the divider with
the hardware division over more than ten million (numerator, divisor) pairs
(no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fast_division_matches_hardware_division(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    exe = tmp_path / "fastdiv_check"
    cmd = [cxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "gptq_bit_weight_amd", "csrc"),
           os.path.join(ROOT, "tests", "fastdiv_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:]
    assert r.stdout.strip() == "ok"
