"""The boundary from plain C: tests/abi_check.c is compiled by the C
compiler against include/muon.h (C99, warnings as errors) and linked to
libmuon.so; it runs the calls that need no GPU.  Shows the header is valid C
and the library usable without Python or torch."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "newton_schulz_09_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client(tmp_path):
    lib = os.path.join(LIBDIR, "libmuon.so")
    if not os.path.exists(lib):
        pytest.skip("libmuon.so is not built")
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_check.c"), "-o", str(exe), "-L", LIBDIR, "-lmuon", "-lm",
           f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
