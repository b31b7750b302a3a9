"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, no OpenMP), every function driven
on small inputs by tests/oracle_sanitize_main.c: no out-of-bounds access, use after free, leak or undefined
behaviour.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    flags = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-Wall", "-Wno-unknown-pragmas",
                           "-Wno-unused-function"] + flags +
                          [os.path.join(HERE, "oracle_sanitize_main.c"), "-o", str(exe), "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle calls done: 0 0 0" in r.stdout
