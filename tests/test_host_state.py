"""Host-side state machine and planners, compiled with g++ under
AddressSanitizer/UBSan and run on the CPU (no HIP involved)."""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "kv_cache_management_amd", "csrc")


def test_host_state_cpp(tmp_path):
    exe = str(tmp_path / "test_host_state")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(HERE, "host", "test_host_state.cpp"), os.path.join(CSRC, "host_state.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", LD_PRELOAD="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
