"""The CPU oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer:
oracle/sanitize_check.c drives every entry point on packed rows holding the
varlen edge cases (empty sequences, one token, a sequence longer than the
backward's checkpoint block, an empty row).  Any out-of-bounds access, use of
freed memory, leak or undefined behaviour aborts the program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    src = [os.path.join(ROOT, "oracle", "gdn_oracle.c"), os.path.join(ROOT, "oracle", "sanitize_check.c")]
    # no OpenMP: its runtime's thread pools are not what is under test here
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe, *src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    proc = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert proc.stdout.count("checksum=") == 3, proc.stdout
    assert "runtime error" not in proc.stderr, proc.stderr
