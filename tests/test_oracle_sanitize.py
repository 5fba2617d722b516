"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): tests/sanitize/oracle_driver.c drives every oracle entry point on
small seeded inputs, edge cases and argument checks included, in a binary
built with gcc -fsanitize=address,undefined.  Any out-of-bounds access,
leak, signed overflow or other undefined behaviour fails the run."""
import os
import shutil
import subprocess

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-fast-math", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(REPO, "oracle", "ssm_oracle.c"), os.path.join(REPO, "tests", "sanitize", "oracle_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "oracle sanitizer driver ok" in r.stdout
