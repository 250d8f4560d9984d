"""The library's host plan code under AddressSanitizer and UBSan (no GPU).

tests/sanitize/plan_layout_fuzz.cpp builds plan layouts (segment geometry,
kernel item lists, workspace carve-up) with the library's own header,
lossless_bf16_exponent_zc_amd/csrc/zc_plan_layout.h, for seeded random segment
lists including empty segments, segments of 2^32 - 1 values and 256 segments,
and checks them against the stream format's closed forms and the kernels'
indexing; any out-of-bounds access, overflow or failed check ends the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_layout_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_layout_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Werror",
           "-I", os.path.join(ROOT, "lossless_bf16_exponent_zc_amd", "csrc"),
           os.path.join(ROOT, "tests", "sanitize", "plan_layout_fuzz.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=900, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok:")
