"""The C oracle (oracle/m3_oracle.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven over several shapes, with and without
a carried state and a final state, on 1 and 3 threads
(tests/oracle_sanitize_main.c).  Any out-of-bounds access, use after free,
leak or undefined behaviour fails the test, as does a thread-count
dependence of the results."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    exe = tmp_path / "oracle_sanitized"
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "m3_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_main.c"),
           "-o", str(exe), "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"sanitized oracle failed:\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "ok" in r.stdout
