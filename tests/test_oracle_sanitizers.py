"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and driven through every entry point by
tests/sanitize_oracle_main.c on exactly sized heap buffers: no out-of-bounds
access, leak or undefined arithmetic, plus a few results the definition fixes.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-Wall", "-Wextra", "-Werror",
           "-o", str(exe), os.path.join(HERE, "sanitize_oracle_main.c"), os.path.join(ROOT, "oracle", "attention.c"),
           "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, f"sanitized oracle run failed ({res.returncode}):\n{res.stderr[-4000:]}"
    assert "oracle sanitizer run ok" in res.stdout
