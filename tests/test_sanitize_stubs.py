"""The CPU sanitizer harness (tests/sanitize/) builds the C-ABI host layer
with stand-ins for the kernel launchers.  This test builds the same sources
without the sanitizers and loads the result with every symbol resolved, so
that a launcher whose signature changes fails here (the sanitizer run itself
is a separate, slower script)."""
import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_layer_links_against_the_stand_in_launchers(tmp_path):
    out = tmp_path / "libua_host_stubs.so"
    cmd = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "paged_varlen_flashattention_amd", "csrc"), "-O0", "-fPIC", "-shared",
           os.path.join(ROOT, "paged_varlen_flashattention_amd", "csrc", "ua_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    lib = ctypes.CDLL(str(out), mode=os.RTLD_NOW)       # every symbol resolved at load
    assert lib.ua_abi_version() > 0
