"""The host-only half of the C ABI (argument checks, planners, tile map;
csrc/host_abi.hpp) built on the CPU with the address and undefined-behaviour
sanitizers and driven over ordinary, edge and hostile inputs
(tests/sanitize/host_abi_checks.cpp). Any overflow, out-of-bounds access or
other undefined operation aborts the driver; the driver also checks that
every plan's tile map is a bijection onto its tile grid."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tile_partitioned_dense_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_abi_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "host_abi_checks.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert "runtime error" not in r.stderr, r.stderr
