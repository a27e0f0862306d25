"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
tests/oracle_sanitize_driver.c exercises every input mode and argument error of
oracle/kda_oracle.c, compiled with gcc -fsanitize=address,undefined and
-fno-sanitize-recover, so any invalid access or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
