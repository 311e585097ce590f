"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a C
driver (tests/oracle_sanitize.c) runs every oracle function at the shapes
and edge cases of the pins (zero, spike, tiny, +-3e38, all-negative and tied
blocks; random code bytes; exact top-k ties, k = 1 and k = E; an all-zero
mixer token) in a gcc build with -fsanitize=address,undefined and
float-cast-overflow, aborting on the first report."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_clean_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all", "-o", exe,
           os.path.join(HERE, "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "ds4moe_oracle.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitize driver: ok" in r.stdout
