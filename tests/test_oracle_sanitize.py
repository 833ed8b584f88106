"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/oracle_sanitize_driver.c calls every entry point of oracle/attn_oracle.c
on small inputs (both masks, one and three threads, full and sampled entry
points, an empty call); built with gcc -fsanitize=address,undefined and
-fno-sanitize-recover, any out-of-bounds access, use after free, leak or
undefined arithmetic ends the run with a report and a nonzero status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-pthread", "-o", str(exe),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), os.path.join(ROOT, "oracle", "attn_oracle.c"),
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in (r.stderr or ""):
        pytest.skip(f"sanitizer runtime unavailable: {r.stderr[-300:]}")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok" in run.stdout
