"""bench.py: its host-side logic (no GPU): the one-GPU guard and the rule that counter-derived
HBM traffic is reported only while the kernel sources it was measured on are unchanged; and,
on the GPU, the shape of its JSON line."""
import json
import os
import subprocess
import sys

import pytest

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


@pytest.mark.gpu
def test_bench_line_contract():
    """A short bench.py run on the GPU prints exactly one JSON line with the fields the
    benchmark contract names, a positive rate consistent with its step time, and roofline
    entries whose fractions are achieved / peak."""
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "2",
                        "--no-long", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["dtype"] == "bf16"
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["value"] > 0 and abs(d["value"] - 16384 / (d["prefill"]["ms"] * 1e-3)) <= 1e-6 * d["value"]
    assert abs(d["ms_per_step"] - d["prefill"]["ms"] - d["decode"]["ms"]) < 1e-9
    for rk in ("roofline", "roofline_decode"):
        rl = d[rk]
        assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
        assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-12 and 0 < rl["frac"] < 1
    assert "workload" in d["config"]
