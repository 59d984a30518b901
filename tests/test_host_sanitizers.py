"""The library's host code (calibration, save/load, host unpack, error paths)
built with AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: a C++
driver (tests/native/host_sanitize.cpp) links calib.cpp and api.cpp with the
two device-table entry points stubbed and exercises every host call; any
sanitizer report aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compression_sq_compress_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{CSRC}", os.path.join(ROOT, "tests", "native", "host_sanitize.cpp"),
           os.path.join(CSRC, "calib.cpp"), os.path.join(CSRC, "api.cpp"),
           "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, str(tmp_path / "c.sqcal")], capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failures" in r.stdout
