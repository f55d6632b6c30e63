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
    assert list(d["sources_sha256"]) == ["rotate.hip"]
    assert len(d["sources_sha256"]["rotate.hip"]) == 64


def test_traffic_sums_the_kernels_of_one_call(tmp_path):
    """Several kernel names: the per-launch bytes are the sum of each kernel's
    mean per dispatch (one launch of each per call), every source hashed."""
    n = 1 << 28
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", n / 1024), ("void kvq::prep_kernel<16>()", 100.0),
        ("void kvq::chunk_kernel<16>()", 2000.0), ("void kvq::chunk_kernel<16>()", 2200.0),
        ("void kvq::merge_kernel()", 10.0)])
    _counter_csv(write, "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", n / 1024), ("void kvq::prep_kernel<16>()", 50.0),
        ("void kvq::chunk_kernel<16>()", 30.0), ("void kvq::merge_kernel()", 4.0)])
    out = tmp_path / "t.md"
    args = types.SimpleNamespace(fetch=str(fetch), write=str(write),
                                 kernel="prep_kernel;chunk_kernel;merge_kernel",
                                 source="attend.hip;attend_rc.hip", copy_bytes=n,
                                 algorithmic_bytes=0, title="t", cmd_fetch="f", cmd_write="w",
                                 out=str(out))
    profsummary.traffic(args)
    d = json.loads(re.search(r"```json\n(.*?)\n```", out.read_text(), re.S).group(1))
    assert d["fetch_bytes_per_launch"] == round((100.0 + 2100.0 + 10.0) * 1024)
    assert d["write_bytes_per_launch"] == round((50.0 + 30.0 + 4.0) * 1024)
    assert d["dispatches"]["fetch_run"] == [1, 2, 1]
    assert set(d["sources_sha256"]) == {"attend.hip", "attend_rc.hip"}


def test_stale_profile_is_not_used(monkeypatch, tmp_path):
    """bench.profiled_traffic reports no traffic for a summary whose recorded
    hash of any of its sources differs from that source as it stands."""
    sys.path.insert(0, ROOT)
    import bench
    shas = {s: bench.source_sha(s) for s in bench.DECODE_SOURCES}
    (tmp_path / "d.md").write_text("# t\n\n```json\n" + json.dumps(
        {"traffic_bytes_per_launch": 123, "sources_sha256": shas}) + "\n```\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.profiled_traffic("d.md", bench.DECODE_SOURCES) == (123, "d.md")
    real = bench.source_sha
    monkeypatch.setattr(bench, "source_sha",
                        lambda name: "0" * 64 if name == "attend_common.h" else real(name))
    assert bench.profiled_traffic("d.md", bench.DECODE_SOURCES) == (None, "d.md")
    assert bench.profiled_traffic("missing.md", bench.DECODE_SOURCES) == (None, None)


def test_committed_headline_summaries_name_their_sources():
    """The counter summaries the bench line reads exist and hash the sources
    the bench checks them against."""
    import bench
    for fname, sources in ((bench.DECODE_TRAFFIC, bench.DECODE_SOURCES),
                           (bench.ENCODE_TRAFFIC, bench.ENCODE_SOURCES)):
        path = os.path.join(bench.PROFILES, fname)
        if not os.path.exists(path):
            pytest.skip(f"{fname} not taken yet")
        d = json.loads(re.search(r"```json\n(.*?)\n```", open(path).read(), re.S).group(1))
        assert set(d["sources_sha256"]) == set(sources)


def test_coverage_summary_names_instances(tmp_path):
    """The coverage summary keeps a kernel's template arguments, drops its
    parameter list and leaves out kernels that are not the library's."""
    assert profsummary._instance("void kvq::attn_rc_kernel<64>(unsigned char const*, int)") == \
        "attn_rc_kernel<64>"
    assert profsummary._instance("kvq::pack_codebooks_kernel(float const*, long)") == \
        "pack_codebooks_kernel"
    assert profsummary._instance("void kvq::k<1, std::array<int, 2> >(int)") == \
        "k<1, std::array<int, 2> >"
    assert profsummary._instance("void at::native::reduce_kernel<512, 1>(int)") is None
    csv_path = tmp_path / "s.csv"
    csv_path.write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void kvq::a<1>(int)",3,1,1,1,1,1,0\n'
        '"void kvq::a<1>(int, float)",2,1,1,1,1,1,0\n'
        '"__amd_rocclr_copyBuffer",9,1,1,1,1,1,0\n')
    out = tmp_path / "cov.md"
    profsummary.main(["coverage", str(csv_path), "--title", "t", "--cmd", "c", "--out", str(out)])
    text = out.read_text()
    assert "1 kernel instances launched." in text and "| `a<1>` | 5 |" in text
    assert "rocclr" not in text
