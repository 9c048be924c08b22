"""Host allocator under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds csrc/allocator.cpp with tests/allocator_driver.cpp (randomised append
plans with shared prefixes, copy on write, exhaustion and error paths, full
release) and runs it; any sanitizer report or failed check fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_allocator_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "allocator_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "online_softmax_paged_amd", "csrc", "allocator.cpp"),
           os.path.join(ROOT, "tests", "allocator_driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: another library may be preloaded into every process
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    plans = dict(kv.split("=") for kv in r.stdout.split()[1:])
    # the scenarios reached both outcomes and made copies on write
    assert int(plans["plans"]) > 100 and int(plans["refused"]) > 10 and int(plans["copies"]) > 10
