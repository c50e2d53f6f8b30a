"""Host logic of bench.py: the roofline bound and fraction, the staleness rule
of the committed traffic counters.  No GPU."""
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_roofline_takes_the_slowest_floor():
    # 8 GB in 2 ms at the 8 TB/s peak: 1 ms of HBM floor, 0.5 of MFMA
    r = bench.roofline("k", 2.0, 8e9, 1.25e15 * 1e-3)
    assert r["bound"] == "hbm"
    assert r["achieved"] == pytest.approx(4000.0)
    assert r["frac"] == pytest.approx(0.5)
    # the same bytes with four times the flops: the matrix cores bind
    r = bench.roofline("k", 2.0, 8e9, 5e12)
    assert r["bound"] == "mfma"
    assert r["frac"] == pytest.approx(5e12 / 2e-3 / 1e12 / bench.BF16_PEAK_TFLOPS)
    # vector ALU operations above both floors
    ops = bench.VALU_PEAK_TOPS * 1e12 * 3e-3
    r = bench.roofline("k", 4.0, 8e9, 1e12, ops_per_launch=ops)
    assert r["bound"] == "alu"
    assert r["frac"] == pytest.approx(0.75)


def test_code_hash_ignores_comments_and_spacing(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) {  /* body */\n  return x + 1;  // one\n}\n")
    b.write_text("int f(int x) {\n\n    return x + 1;\n}\n/* other\n   words */\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench._code_only(str(a)) == bench._code_only(str(b))
    assert bench._code_only(str(a)) != bench._code_only(str(c))


def test_traffic_is_null_once_the_kernel_source_differs(tmp_path, monkeypatch):
    rec = {"kernel_src_sha": bench.kernel_src_sha("gemm_mfma"),
           "bytes_per_launch": 123.0}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "traffic_file", lambda kind, leg: str(f))
    assert bench.traffic_entry("gemm_mfma", "x") == 123.0
    rec["kernel_src_sha"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.traffic_entry("gemm_mfma", "x") is None
    monkeypatch.setattr(bench, "traffic_file", lambda kind, leg: str(tmp_path / "none"))
    assert bench.traffic_entry("gemm_mfma", "x") is None
