"""CPU checks of bench.py's command-line contract that need no GPU: the build runs on one GPU, so any
other --gpus value ends the run with a message and a failing status before a device is touched, and
the traffic records it reads are keyed by the current kernel sources."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                         text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert line["n_gpus_requested"] == n and "one GPU" in line["error"]


def test_traffic_records_parse():
    """Every record of the committed counter summary names a workload, a call, a split count, a source
    hash and a positive byte count; records whose hash matches the sources are found by the lookup."""
    sys.path.insert(0, ROOT)
    import bench

    text = open(bench.COUNTERS_FILE).read()
    recs = json.loads(text.split("```json", 1)[1].split("```", 1)[0])["records"]
    assert recs
    sha = bench.sources_sha()
    for r in recs:
        assert r["traffic_bytes_per_call"] > 0 and len(r["source_sha"]) == 16
        got = bench.recorded_traffic(r["workload"], r["call"], r["n_splits"], cold=True)
        assert got == (r["traffic_bytes_per_call"] if r["source_sha"] == sha else None)
        assert bench.recorded_traffic(r["workload"], r["call"], r["n_splits"], cold=False) is None


def test_source_hash_follows_code_not_comments(tmp_path):
    """The records' key hashes the code only: a comment or blank-line edit keeps it, a code edit changes it."""
    sys.path.insert(0, ROOT)
    import bench

    code = "int f(int a) {\n  return a + 1;\n}\n"
    a = tmp_path / "a.hip"
    a.write_text(code)
    b = tmp_path / "b.hip"
    b.write_text("// header\n/* a block\n   comment */\nint f(int a) {   \n\n  return a + 1;  // one more\n}\n")
    c = tmp_path / "c.hip"
    c.write_text(code.replace("a + 1", "a + 2"))
    assert bench.sources_sha([str(a)]) == bench.sources_sha([str(b)])
    assert bench.sources_sha([str(a)]) != bench.sources_sha([str(c)])
