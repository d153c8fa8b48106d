"""Host-side checks of bench.py: algorithmic byte counts and the rocprofv3 summary parsers."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("name,total,full", [
    # per-step bytes without the new token's store: score (r + 4 per token and KV head), selected K+V (4d per
    # row and KV head), indices written and read, q + out + block table; full-KV the same over every position
    ("llama8b_32k", 287_703_040, 2_147_876_864),
    ("llama8b_128k", 370_540_544, 4_295_360_512),
    ("hybrid_64k", 1_262_622_720, 13_087_414_272),
    ("mla_128k", 159_711_232, 1_210_253_312),
])
def test_step_bytes(name, total, full):
    w = WORKLOADS[name]
    seq = [w.seq_len] * w.batch
    t, parts = bench.step_bytes(w, seq, True)
    assert t - parts["store"] == total
    assert bench.step_bytes(w, seq, False)[0] == full


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_counter_summary_scales_by_probe(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    fetch, write = tmp_path / "f", tmp_path / "w"
    # the probe reads 1 GiB but the counter reports 0.5 GiB: factor 2
    _write(str(fetch / "host" / "1_counter_collection.csv"), hdr, [
        [1, "void jssa::select_stream<2, 16>(jssa::SelectArgs)", "FETCH_SIZE", 1000.0],
        [1, "void jssa::select_stream<2, 16>(jssa::SelectArgs)", "FETCH_SIZE", 500.0],
        [2, "void jssa::select_stream<2, 16>(jssa::SelectArgs)", "FETCH_SIZE", 1500.0],
        [3, "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>", "FETCH_SIZE", 512.0 * 1024]])
    _write(str(write / "host" / "1_counter_collection.csv"), hdr, [
        [1, "void jssa::select_stream<2, 16>(jssa::SelectArgs)", "WRITE_SIZE", 100.0],
        [3, "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>", "WRITE_SIZE", 1024.0 * 1024]])
    r = bench.summarize_counters(str(fetch), str(write), "llama8b_128k", 10_000, "cmd")
    assert r["fetch_kib_per_dispatch"] == 1500.0 and r["write_kib_per_dispatch"] == 100.0
    assert r["scale_fetch"] == 2.0 and r["scale_write"] == 1.0
    assert r["hbm_bytes_per_dispatch"] == int(1500 * 1024 * 2 + 100 * 1024)
    json.dumps(r)


def test_trace_summary(tmp_path):
    _write(str(tmp_path / "h" / "1_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [["a", 2, 2000, 1000, 10.0, 900, 1100, 1], ["b", 1, 8000, 8000, 40.0, 8000, 8000, 0],
            ["void jssa::select_stream<2, 16>(jssa::SelectArgs)", 2, 10000, 5000, 50.0, 4000, 6000, 1]])
    txt = bench.summarize_trace(str(tmp_path), "rocprofv3 ...")
    lines = txt.splitlines()
    assert "select_stream" in lines[6] and "5.00" in lines[6]
    assert "other kernels" in lines[-1] and lines[-1].split("|")[2].strip() == "3"


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    """The counters are keyed to the stream's code: a comment or blank-line edit keeps the key, a code edit
    changes it."""
    csrc = tmp_path / "long_context_decode_amd" / "csrc"
    csrc.mkdir(parents=True)
    f = csrc / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f.write_text("int a = 1;  // one\n/* block\n comment */ int b = 2;\n")
    h0 = bench._src_hash("k.hip")
    f.write_text("// new header\n\nint a = 1;  // changed words\n/* other */ int b = 2;\n\n")
    assert bench._src_hash("k.hip") == h0
    f.write_text("int a = 1;\nint b = 3;\n")
    assert bench._src_hash("k.hip") != h0
