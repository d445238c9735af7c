"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU):
tests/native/oracle_sanitize_driver.c is linked with oracle/nsa_oracle.c,
both instrumented, and run over shapes that reach the oracle's edge cases
(see the driver's header).  A memory error or undefined operation makes the
sanitizers abort with a report; the test requires a clean run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "tests", "native", "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "nsa_oracle.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
