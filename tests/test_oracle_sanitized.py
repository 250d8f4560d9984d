"""The CPU oracle under AddressSanitizer and UBSan (no GPU).

tests/sanitize/zco_fuzz.c round-trips seeded tensors through the oracle
(coded and raw streams) and decodes damaged copies from exact-size heap
buffers; a read past a buffer or undefined arithmetic ends the run with a
sanitizer report.  The decoder must validate every offset before it reads.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_decoder_under_sanitizers(tmp_path):
    exe = tmp_path / "zco_fuzz"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "tests", "sanitize", "zco_fuzz.c"),
           os.path.join(ROOT, "oracle", "zco.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok:")
