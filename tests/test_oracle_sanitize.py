"""The oracle built with gcc under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only), driven through every entry point on small inputs by oracle_sanitize_main.c:
no out-of-bounds access, leak or undefined operation in the checker the parity tests
trust."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-Wall", "-Wno-unknown-pragmas",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(HERE, "oracle_sanitize_main.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "oracle sanitizer run ok" in res.stdout
