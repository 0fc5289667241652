"""bench.py's host-side contract (no GPU): one GPU only, and the attention
traffic record is used only for the source it was taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    """The roofline's `traffic` comes from the committed FETCH_SIZE /
    WRITE_SIZE record only while attention.hip hashes to the source those
    passes measured; for any other source it is null, never a stale number."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert rec["bytes_per_launch"] > 0
    same = tmp_path / "same.hip"
    same.write_bytes(open(bench.ATTN_SRC, "rb").read())
    monkeypatch.setattr(bench, "ATTN_SRC", str(same))
    want = rec["bytes_per_launch"] if rec["attention_source_sha256_16"] == bench.source_hash(str(same)) else None
    assert bench.recorded_traffic() == want
    other = tmp_path / "other.hip"
    other.write_bytes(open(bench.ATTN_SRC, "rb").read() + b"// changed\n")
    monkeypatch.setattr(bench, "ATTN_SRC", str(other))
    assert bench.recorded_traffic() is None
