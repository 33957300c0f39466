"""Host-side logic of bench.py (no GPU): the one-GPU guard and the rule that counter-derived
HBM traffic is reported only while the kernel sources it was measured on are unchanged."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_traffic_is_kept_only_for_unchanged_sources(tmp_path):
    good = bench.source_digest(bench.KERNEL_SOURCES["prefill"])
    rec = {"kernels": {
        "prefill": {"source_sha256": good, "hbm_bytes_per_launch": 123.0},
        "decode": {"source_sha256": "0" * 64, "hbm_bytes_per_launch": 456.0},
        "unknown": {"source_sha256": good, "hbm_bytes_per_launch": 789.0},
    }}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    assert bench.load_traffic(str(p)) == {"prefill": 123.0}


def test_digest_covers_every_listed_source(tmp_path, monkeypatch):
    # a one-byte change in any listed file changes the digest
    src = tmp_path / "root"
    for rel in set(bench.KERNEL_SOURCES["prefill"] + bench.KERNEL_SOURCES["decode"]):
        d = src / os.path.dirname(rel)
        d.mkdir(parents=True, exist_ok=True)
        (src / rel).write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(src))
    for kind, paths in bench.KERNEL_SOURCES.items():
        before = bench.source_digest(paths)
        for rel in paths:
            f = src / rel
            data = f.read_bytes()
            f.write_bytes(data + b" ")
            assert bench.source_digest(paths) != before, (kind, rel)
            f.write_bytes(data)
        assert bench.source_digest(paths) == before


def test_missing_or_broken_traffic_file_gives_nothing(tmp_path):
    assert bench.load_traffic(str(tmp_path / "absent.json")) == {}
    p = tmp_path / "broken.json"
    p.write_text("{not json")
    assert bench.load_traffic(str(p)) == {}
