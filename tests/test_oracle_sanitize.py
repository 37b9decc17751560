"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host
only) and driven over small problems that reach every branch of its indexing
(oracle/sanitize_driver.c): no memory error, no undefined behaviour, every call returns 0
with finite outputs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_is_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    src = [os.path.join(ROOT, "oracle", f) for f in ("ssm_oracle.c", "sanitize_driver.c")]
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "oracle"), *src, "-o", exe, "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert "0 failures" in r.stdout
