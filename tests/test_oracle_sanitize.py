"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/oracle_sanitize.c calls every oracle entry point on tiny layers (fp32, fp16 and int4
weights; ReLU, ReGLU and dReLU; a router) with each array in a heap block of exactly its contract
size, so any out-of-bounds access, use of freed memory, leak or undefined operation is reported,
and checks identities that hold for any values (no mask == all-ones mask, additivity over a split
of the active set, router weights summing to one).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "ffn_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip("the sanitizer runtimes are not installed: " + r.stderr.strip()[:200])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle sanitizer run: OK" in run.stdout
    assert "runtime error" not in run.stderr and "Sanitizer" not in run.stderr, run.stderr
