"""Host-side sanitizer run of the argument validation (CPU).

The validation layer (csrc/validate.cpp) is pure C++ and runs before
anything is enqueued, so it can be exercised without a GPU: it is built here
with AddressSanitizer and UndefinedBehaviorSanitizer together with a seeded
fuzz driver (tests/native/validate_fuzz.cpp) that throws edge and random
descriptors, batch sizes and configurations at both checkers, then packs
small matrices into a few hundred bytes and checks the buffer-overlap rule
against a row-by-row brute force on every call.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_validation_under_asan_ubsan(tmp_path):
    exe = tmp_path / "validate_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", f"-I{ROOT}/include", f"-I{ROOT}/muon_newton_schulz_update_amd/csrc",
           f"{ROOT}/tests/native/validate_fuzz.cpp", f"{ROOT}/muon_newton_schulz_update_amd/csrc/validate.cpp",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in (r.stderr or "").lower() and "cannot find" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    lines = run.stdout.splitlines()
    assert any(l.startswith("overlap ") for l in lines), run.stdout   # the overlap rule's fuzz ran and agreed
    assert lines and lines[-1].startswith("ok "), run.stdout
