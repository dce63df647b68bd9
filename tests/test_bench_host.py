"""bench.py's host logic on the CPU: the kernel-source hash that ties the
committed counter runs to the sources ignores comments but not code, the
committed traffic figure matches the current sources, and a multi-GPU
request exits with a message instead of running."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_of_drops_comments_only():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "// not a comment";\n'
    assert bench.code_of(src) == 'int a = 1; const char* s = "// not a comment";'
    assert bench.code_of("x  =\n\n y;") == "x = y;"


def test_hash_ignores_comment_edits_and_sees_code(tmp_path, monkeypatch):
    files = []
    for p in bench.KERNEL_SOURCES:
        q = tmp_path / os.path.basename(p)
        q.write_text(open(p, encoding="utf-8").read(), encoding="utf-8")
        files.append(str(q))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", files)
    h0 = bench.kernel_source_hash()
    with open(files[0], "a", encoding="utf-8") as f:
        f.write("\n// a remark\n/* and another */\n")
    assert bench.kernel_source_hash() == h0
    with open(files[0], "a", encoding="utf-8") as f:
        f.write("static int unused_probe_symbol;\n")
    assert bench.kernel_source_hash() != h0


def test_committed_traffic_is_plausible():
    """When the counter runs in profiles/ were taken on the current attention
    sources, the traffic figure the bench line carries lies just above the
    algorithmic KV bytes (no byte fetched twice)."""
    import pytest

    t = bench.measured_traffic(bench.kernel_source_hash(), "decode_b16_16k_e4m3_p128")
    if t is None:
        pytest.skip("counters not yet retaken on the current attention sources")
    assert 134_217_728 < t < 1.05 * 134_217_728


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
