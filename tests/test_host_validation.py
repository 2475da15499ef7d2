"""Host validation of the C ABI on the CPU, through host-built cache objects.

Builds tests/cpu/host_validation.cpp with the host C++ compiler against the
library's own headers (the cache objects are plain host structs) and links it
to libkvattn.so: every refused call returns its status and leaves the
lengths' host mirror unchanged; a call that passes validation but cannot
reach a device enqueues nothing and changes nothing.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "kv_cached_causal_amd")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_refused_calls_leave_the_cache_unchanged(tmp_path):
    exe = tmp_path / "host_validation"
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", f"-I{ROOT}/include", f"-I{LIB_DIR}/csrc",
           os.path.join(ROOT, "tests", "cpu", "host_validation.cpp"), f"-L{LIB_DIR}", "-lkvattn",
           f"-Wl,-rpath,{LIB_DIR}", "-Wl,-rpath-link,/opt/rocm/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert " 0 failed" in run.stdout
