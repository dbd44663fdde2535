"""The C ABI from plain C (no GPU needed): tests/abi_client.c includes
include/q4.h as C99, references every declared call and links libq4.so;
building it checks that the header is valid C and that every call is
exported with C linkage, and running it exercises the host-only calls."""
import os
import shutil
import subprocess

import pytest

import gptq_bit_weight_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_client_builds_links_and_runs(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = q4.load_library()
    libdir = os.path.dirname(lib._name)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = tmp_path / "abi_client"
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_client.c"), "-L", libdir, "-lq4",
           "-Wl,-rpath," + libdir, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = libdir + os.pathsep + os.path.join(rocm, "lib") + os.pathsep + env.get("LD_LIBRARY_PATH", "")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"check {r.returncode} failed: {r.stderr[-2000:]}"
    assert r.stdout.strip() == "ok"
