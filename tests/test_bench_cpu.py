"""Host-side checks of the measurement plumbing (CPU only): the benchmark's
one-GPU guard, the counter-to-bytes scaling of the profile summaries, and the
rule that a summary taken on another version of a kernel's source is not used.
"""
import csv
import json
import os
import re
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from compressed_attention_fwht_amd import profsummary  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_scaling_by_the_copy_calibration(tmp_path):
    """A copy of N bytes that FETCH_SIZE reports as N/2 KiB*1024 and WRITE_SIZE
    as N: the kernel's counters are scaled by 2 and 1, averaged over its
    dispatches; the small copies of the run are ignored."""
    n = 1 << 28
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", n / 2 / 1024), ("__amd_rocclr_copyBuffer", n / 2 / 1024),
        ("__amd_rocclr_copyBuffer", 3.0),                       # a small copy: not calibration
        ("void kvq::demo_kernel<1>(int)", 1000.0), ("void kvq::demo_kernel<1>(int)", 1200.0)])
    _counter_csv(write, "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", n / 1024),
        ("void kvq::demo_kernel<1>(int)", 500.0), ("void kvq::demo_kernel<1>(int)", 500.0)])
    out = tmp_path / "t.md"
    args = types.SimpleNamespace(fetch=str(fetch), write=str(write), kernel="demo_kernel",
                                 source="rotate.hip", copy_bytes=n, algorithmic_bytes=1_000_000,
                                 title="t", cmd_fetch="f", cmd_write="w", out=str(out))
    profsummary.traffic(args)
    d = json.loads(re.search(r"```json\n(.*?)\n```", out.read_text(), re.S).group(1))
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["fetch_bytes_per_launch"] == round(1100.0 * 1024 * 2)
    assert d["write_bytes_per_launch"] == round(500.0 * 1024)
    assert d["traffic_bytes_per_launch"] == round(1100.0 * 2048 + 500.0 * 1024)
    assert d["traffic_over_algorithmic"] == pytest.approx(
        (1100.0 * 2048 + 500.0 * 1024) / 1_000_000, abs=1e-3)
    assert len(d["source_sha256"]) == 64


def test_stale_profile_is_not_used(monkeypatch):
    """bench.profiled_traffic reports no traffic for a summary whose recorded
    source hash differs from the source as it stands."""
    sys.path.insert(0, ROOT)
    import bench
    names = [f for f in os.listdir(bench.PROFILES) if f.startswith("encode_mfma_kernel")]
    assert names, "the encode kernel's counter summary is committed"
    monkeypatch.setattr(bench, "source_sha", lambda name: "0" * 64)
    traffic, fn = bench.profiled_traffic("encode_mfma_kernel", "encode.hip")
    assert traffic is None and fn == names[0]
    monkeypatch.setattr(bench, "PROFILES", os.path.join(ROOT, "no-such-folder"))
    assert bench.profiled_traffic("encode_mfma_kernel", "encode.hip") == (None, None)
