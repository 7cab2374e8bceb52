"""Host logic of bench.py (no GPU): the one-GPU guard, the binding-roof arithmetic and the
rule that committed counter totals apply only to the source they were measured on."""
import hashlib
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
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_roofline_picks_the_binding_roof():
    # 1 TFLOP and 1 GB in 1 ms: MFMA time at 2.5 PF = 0.4 ms > HBM time at 8 TB/s = 0.125 ms
    r = bench.roofline("k", 1e12, 1e9, 1.0, 2500.0, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1000.0)
    assert r["frac"] == pytest.approx(0.4)
    assert r["hbm_frac"] == pytest.approx(1000.0 / 8000.0)
    assert r["hbm_frac_measured"] is None
    # 0.1 TFLOP and 4 GB in 1 ms: HBM time 0.5 ms > MFMA time 0.04 ms
    r = bench.roofline("k", 1e11, 4e9, 1.0, 2500.0, 6e9)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0)
    assert r["frac"] == pytest.approx(0.5)
    assert r["mfma_frac"] == pytest.approx(100.0 / 2500.0)
    assert r["traffic"] == 6e9
    assert r["hbm_frac_measured"] == pytest.approx(6000.0 / 8000.0)


def test_measured_traffic_follows_the_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// kernel v1\n")
    summary = tmp_path / "k_traffic.json"

    def write_summary(text, workload="top2_bf16", nbytes=123.0):
        digest = hashlib.sha256(text.encode()).hexdigest()
        summary.write_text(json.dumps({"workload": workload, "source_sha256": digest,
                                       "bytes_per_launch": nbytes}))

    monkeypatch.setitem(bench.TRAFFIC, "k", (str(summary), [str(src)]))
    assert bench.measured_traffic("k", "top2_bf16") is None  # no summary yet
    write_summary("// kernel v1\n")
    assert bench.measured_traffic("k", "top2_bf16") == 123.0
    assert bench.measured_traffic("k", "switch_bf16") is None  # another workload
    src.write_text("// kernel v2\n")  # the kernel changed after the counters were taken
    assert bench.measured_traffic("k", "top2_bf16") is None


def test_committed_traffic_summaries_are_well_formed():
    for kernel, (path, sources) in bench.TRAFFIC.items():
        t = json.load(open(path))
        assert t["kernel"] == kernel and t["workload"] == "top2_bf16"
        assert t["bytes_per_launch"] > 0 and len(t["source_sha256"]) == 64
        assert all(os.path.exists(p) for p in sources)
