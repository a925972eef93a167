"""Host logic of bench.py: the one-GPU refusal, percentiles, and the SHA-keyed traffic lookup."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_percentile_interpolates():
    v = [1.0, 2.0, 3.0, 4.0, 5.0]
    assert bench.percentile(v, 50) == 3.0
    assert bench.percentile(v, 10) == pytest.approx(1.4)
    assert bench.percentile(v, 90) == pytest.approx(4.6)
    assert bench.percentile([7.0], 90) == 7.0


def _write(path, text):
    with open(path, "w") as f:
        f.write(text)


def test_traffic_counts_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    # two "sources" under a fake root; the digest covers both, in order
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "k.hip").write_text("kernel v1")
    (tmp_path / "h.h").write_text("header v1")
    digest = hashlib.sha256(b"kernel v1" + b"header v1").hexdigest()
    assert bench.source_digest("k.hip,h.h") == digest
    assert bench.source_digest("k.hip,missing.h") is None
    table = tmp_path / "traffic.md"
    _write(table, f"prose line\n    traffic quantize bytes_per_launch=123 source=k.hip,h.h sha256={digest}\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(table))
    assert bench.measured_traffic("quantize") == 123
    assert bench.measured_traffic("dequantize") is None
    # a changed header voids the figure, like a changed kernel file
    (tmp_path / "h.h").write_text("header v2")
    assert bench.measured_traffic("quantize") is None
