"""Host-side checks of the benchmark script (no GPU): the one-GPU rule and
the traffic figure read from the committed counter summary."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_summary_parses():
    """The counter summary names the bytes per call and the sha256 of the
    decode sources; the figure is used only while the sources match."""
    text = open(bench.TRAFFIC_PROFILE).read()
    vals = dict(line.split(" = ", 1) for line in text.splitlines() if " = " in line)
    assert int(vals["traffic_bytes_per_launch"]) > 0
    assert len(vals["decode_source_sha256"].strip()) == 64
    t = bench.measured_traffic()
    assert t is None or t == int(vals["traffic_bytes_per_launch"])


def test_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    text = open(bench.TRAFFIC_PROFILE).read().replace("decode_source_sha256 = ", "decode_source_sha256 = 0")
    fake = tmp_path / "summary.md"
    fake.write_text(text)
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(fake))
    assert bench.measured_traffic() is None
