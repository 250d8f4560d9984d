"""Host-side checks of bench.py: the one-GPU guard, the parsing of the
committed counter summaries, and the issue-roofline arithmetic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_valu_peak_matches_the_fp32_vector_peak():
    # 157.3 TFLOP/s = lane operations x 2 (FMA) x 2 (packed)
    assert bench.VALU_PEAK * 4 == pytest.approx(157.3e12, rel=1e-3)


def test_committed_summaries_parse():
    for path, tag in ((bench.TRAFFIC_FILE, "traffic"), (bench.ISSUE_FILE, "valu")):
        lines = [l.split() for l in open(path) if l.startswith(tag + " ")]
        assert lines, f"{path}: no '{tag}' lines"
        for f in lines:
            assert len(f) == 4 and f[1] in bench.KERNEL_SOURCES, f
            assert int(f[2]) > 0 and len(f[3]) == 16 and int(f[3], 16) >= 0, f


def test_stale_summary_gives_none_and_current_one_counts(tmp_path, monkeypatch):
    k = "zc_decode"
    p = tmp_path / "issue.txt"
    p.write_text(f"valu {k} 1000000 {'0' * 16}\n")
    monkeypatch.setattr(bench, "ISSUE_FILE", str(p))
    assert bench.measured_valu(k) is None and bench.issue_roofline(k, 1e-5) is None
    p.write_text(f"valu {k} 1000000 {bench.sources_hash(k)}\n")
    r = bench.issue_roofline(k, 1e-5)
    assert r["valu_instructions"] == 1000000
    assert r["frac"] == pytest.approx(1e6 * 64 / 1e-5 / bench.VALU_PEAK, abs=1e-4)
    assert r["bound"] == "alu" and r["launch_us"] == 10.0


def test_source_hash_ignores_comments_but_not_code():
    src = 'int a = 1;  // one\n/* two\n   lines */ int b = a + 2;\nasm volatile("" ::"s"(a));\n'
    assert bench.code_text(src) == 'int a = 1; int b = a + 2; asm volatile("" ::"s"(a));'
    assert bench.code_text(src.replace("// one", "// first value")) == bench.code_text(src)
    assert bench.code_text(src.replace("a + 2", "a + 3")) != bench.code_text(src)
