"""The CPU oracle under the host AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/oracle_sanitized_driver.c calls every oracle entry on seeded inputs of ragged sizes (every
weight format, FP6 activations, a padded row stride) and checks a few round trips; here it is
linked with oracle/mx_oracle.c, both built by gcc with -fsanitize=address,undefined, and run.
Any out-of-bounds access, use of freed memory or undefined arithmetic ends the run with a
sanitizer report and a non-zero status.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    build = subprocess.run(
        ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall",
         os.path.join(ROOT, "tests", "oracle_sanitized_driver.c"),
         os.path.join(ROOT, "oracle", "mx_oracle.c"), "-lm", "-o", exe],
        capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("the sanitizer runtimes are not installed: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout[-1000:], run.stderr[-4000:])
    assert "oracle sanitized run ok" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
