"""Host-side logic of bench.py (no GPU): the one-GPU guard, the kernel-source
hash that guards recorded HBM traffic, and the counter summary format."""
import csv
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


def test_sources_hash_is_stable_and_covers_the_kernels():
    h1, h2 = bench.sources_hash(), bench.sources_hash()
    assert h1 == h2 and len(h1) == 16
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, f)), f
    assert any(f.endswith("attn_bwd.hip") for f in bench.KERNEL_SOURCES)


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, val) in enumerate(rows):
            w.writerow([i, name, counter, val])


def test_counter_summary_scales_by_the_copy_and_sums_an_entry_points_kernels(tmp_path):
    gib_kib = float(1 << 20)
    # the copy reads half its bytes in FETCH_SIZE units and writes all of them
    fetch = [("__amd_rocclr_copyBuffer", gib_kib / 2), ("__amd_rocclr_copyBuffer", 3.0),
             ("void splitkv::attn_bwd_dkdv_kernel<128>(...)", 100.0),
             ("void splitkv::attn_bwd_dkdv_kernel<128>(...)", 300.0),
             ("void splitkv::attn_bwd_dq_kernel<128>(...)", 50.0),
             ("void splitkv::block_range_kernel(...)", 1.0),
             ("void splitkv::attn_fwd_bf16_kernel<128, unsigned short>(...)", 10.0)]
    write = [("__amd_rocclr_copyBuffer", gib_kib), ("void splitkv::attn_bwd_dq_kernel<128>(...)", 8.0)]
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", write)
    text = bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"), "weak8", "cmd")
    rec = json.loads([l for l in text.splitlines() if l.startswith("traffic-json: ")][0][14:])
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    bwd = rec["per_launch_bytes"]["splitkv_attn_bwd"]
    # mean per dispatch of each kernel of the call, summed, in bytes, times the factor
    assert bwd["fetch"] == round((200.0 + 50.0 + 1.0) * 1024 * 2.0)
    assert bwd["write"] == round(8.0 * 1024)
    fwd = rec["per_launch_bytes"]["splitkv_attn_fwd"]
    assert fwd["fetch"] == round((1.0 + 10.0) * 1024 * 2.0)
    assert rec["sources_sha256"] == bench.sources_hash()


def test_recorded_traffic_is_used_only_with_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"workload": "weak8", "sources_sha256": "0" * 16, "per_launch_bytes": {}}
    (prof / "x_traffic.md").write_text("traffic-json: " + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_hash", lambda: "1" * 16)
    assert bench.load_traffic("weak8") is None
    monkeypatch.setattr(bench, "sources_hash", lambda: "0" * 16)
    assert bench.load_traffic("weak8") == rec
    assert bench.load_traffic("strong8") is None
