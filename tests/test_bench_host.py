"""Host-side checks of bench.py (no GPU): the recorded HBM traffic belongs
to the current kernel sources, and the one-GPU contract is enforced."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_record_matches_the_kernel_sources():
    # profiles/hbm_traffic.txt stores a checksum of each path's sources next
    # to its counter figures; a source change that did not retake the
    # counters leaves roofline.traffic null in every bench line
    for path in ("prefill", "decode"):
        t = bench.measured_traffic(path)
        assert t is not None, f"hbm_traffic.txt has no line for the current {path} sources"
        assert t["bytes_per_call"] == t["fetch_bytes"] + t["write_bytes"]


def test_source_checksum_ignores_comments_only(tmp_path, monkeypatch):
    import shutil
    for f in set(bench.KERNEL_SOURCES["prefill"]):
        shutil.copy(os.path.join(bench.CSRC, f), tmp_path / f)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    a = bench.sources_sha256("prefill")
    src = tmp_path / "fa_fwd.hip"
    src.write_text(src.read_text() + "\n// a comment\n/* and a block\n comment */\n")
    assert bench.sources_sha256("prefill") == a
    src.write_text(src.read_text() + "\nstatic int fa_unused_for_checksum;\n")
    assert bench.sources_sha256("prefill") != a


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
