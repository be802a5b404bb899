"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

``oracle/sanitize_driver.c`` calls every oracle entry point on small inputs --
valid calls, edge shapes and every refusal -- with buffers of exactly the
needed size; built with the sanitizers, any out-of-bounds access or undefined
behaviour in the oracle aborts the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    src = [os.path.join(ROOT, "oracle", "dcconv_oracle.c"), os.path.join(ROOT, "oracle", "sanitize_driver.c")]
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", str(exe), *src, "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "ok" in r.stdout
