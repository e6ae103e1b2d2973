"""The C oracle under the host address and undefined-behaviour sanitizers: a driver
calls every exported function (odd and power-of-two lengths, row subsets, both
convolution modes, the backward, the rejected arguments) in a gcc build with
-fsanitize=address,undefined; any sanitizer report or unexpected return fails."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off",
           os.path.join(ROOT, "oracle", "hyena_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=120)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "0 unexpected results" in r.stdout
