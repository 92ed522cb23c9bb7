"""Host-side logic of bench.py: the counter table lookup behind roofline.traffic."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _table(tmp_path, digest):
    p = tmp_path / "t.md"
    p.write_text("fetch_scale: 2.0\nwrite_scale: 1.0\n\n"
                 "| kernel | workload | family | digest | FETCH_SIZE KiB | WRITE_SIZE KiB | n | bytes |\n"
                 "|---|---|---|---|---|---|---|---|\n"
                 f"| stream_bwd | 5 | stream | {digest} | 100.0 | 50.0 | 3 | x |\n")
    return str(p)


def test_traffic_scaled_when_sources_match(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_TABLE", _table(tmp_path, bench.source_digest("stream")))
    assert bench.measured_traffic("stream_bwd", 5) == (100.0 * 2.0 + 50.0) * 1024.0
    assert bench.measured_traffic("stream_bwd", 2) is None
    assert bench.measured_traffic("stream_fwd", 5) is None


def test_traffic_null_when_sources_changed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_TABLE", _table(tmp_path, "0000000000000000"))
    assert bench.measured_traffic("stream_bwd", 5) is None


def test_committed_table_parses():
    # every row of the committed table names a known kernel and family
    with open(bench.TRAFFIC_TABLE) as f:
        rows = [l for l in f if l.startswith("| ") and l.split("|")[1].strip() in bench.KERNEL_FAMILY]
    assert len(rows) >= 6
    for l in rows:
        c = [x.strip() for x in l.strip().strip("|").split("|")]
        assert bench.KERNEL_FAMILY[c[0]] == c[2]
