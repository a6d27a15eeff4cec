"""The library's host-only C++ (the schedule lowering and verifier, the cost
model, the calibration-file parser) built with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer and driven by tests/sanitize_driver.cpp:
every lowering for p = 2..16 and every topology proven, randomly mutated
schedules verified without crashing (dropped transfers rejected), the model
evaluated everywhere, and 4000 corrupted calibration files parsed or
refused cleanly."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "all_reduce_reduction_amd", "csrc")


@pytest.mark.slow
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "sanitize_driver")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize_driver.cpp"),
           os.path.join(CSRC, "schedule.cpp"), os.path.join(CSRC, "select.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, str(tmp_path / "model.json")], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "lowered" in r.stdout
    print(r.stdout)
