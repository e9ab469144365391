"""The library's host code (argument validation, launch planning, workspace
and pointer-table carving; csrc/api.hip) built for the CPU with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through every
planning entry point at the workloads' shapes and at the largest accepted
ones (16384 x 16384, 16 x 2^20, more than 128 matrices, more than 8 shapes).
The kernel launchers are replaced by stubs (tests/host_check/launch_stubs.cpp)
that check each launch's workspace ranges, grid and pointer-table indices in
64-bit arithmetic instead of launching.  A second run registers every
workspace 256 bytes short and must be caught."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
SOURCES = [os.path.join(ROOT, "newton_schulz_09_amd", "csrc", "api.hip"),
           os.path.join(ROOT, "tests", "host_check", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "host_check", "driver.cpp")]


@pytest.fixture(scope="module")
def host_check(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc is not available")
    d = tmp_path_factory.mktemp("host_check")
    objs = []
    for src in SOURCES:
        obj = str(d / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g", *SAN,
               "-fno-sanitize-recover=all", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(d / "host_check")
    r = subprocess.run([HIPCC, *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)


def test_planning_is_clean_under_sanitizers(host_check):
    r = _run(host_check)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host check ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_stubs_catch_a_workspace_too_small(host_check):
    r = _run(host_check, "shrink")
    assert r.returncode != 0
    assert "host check failed" in r.stderr
