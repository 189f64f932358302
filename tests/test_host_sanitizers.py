"""The host Lloyd-Max solver (csrc/tq_codebook.cpp) built with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, CPU only) and run over
a grid of (d, bits) by tests/host_asan_driver.cpp: no memory or UB report,
finite strictly increasing centroids, the uniform grid at d = 3."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "kv_cache_vector_rht_amd", "csrc", "tq_codebook.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_codebook_solver_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "asan_driver"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", os.path.join(HERE, "host_asan_driver.cpp"), SRC, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert r.stdout.strip().endswith("ok")
