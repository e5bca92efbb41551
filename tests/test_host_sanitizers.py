"""The host half of libplsh (plsh_host.cpp: sampler, table builder,
validator, work counts, error reporting) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/host_sanitize_main.cpp; no GPU and no HIP runtime involved."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "approximate_long_context_amd", "csrc")


def test_host_half_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(HERE, "host_sanitize_main.cpp"), os.path.join(CSRC, "plsh_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr and "unrecognized" in r.stderr:
        pytest.skip("this g++ has no sanitizer runtime")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if run.returncode != 0 and "runtime does not come first" in run.stderr:
        pytest.skip("another preloaded library precedes the sanitizer runtime in this environment")
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr
    assert "host checks passed" in run.stdout
