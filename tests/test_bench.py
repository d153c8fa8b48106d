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


def test_counter_summary_derives_request_size_from_probe(tmp_path):
    """Three passes: the probe's 1 GiB read fixes the bytes of a full L2 read request (here 128, with none
    counted as 128-byte 'bubbles': the FETCH_SIZE definition would count them as 64); 32-byte requests count
    32; writes follow the WRITE_SIZE definition; busy and conflict percentages follow the rocprofv3
    definitions (256 CUs, 1024 SIMDs)."""
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    st = "void jssa::select_stream<2, 16, 0>(jssa::SelectArgs)"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    rd, wr, sq = tmp_path / "r", tmp_path / "w", tmp_path / "s"
    _write(str(rd / "h" / "1_counter_collection.csv"), hdr, [
        [1, st, "TCC_EA0_RDREQ_sum", 600.0], [1, st, "TCC_EA0_RDREQ_sum", 400.0],      # two instances, one dispatch
        [1, st, "TCC_EA0_RDREQ_32B_sum", 10.0], [1, st, "TCC_BUBBLE_sum", 0.0],
        [2, st, "TCC_EA0_RDREQ_sum", 1000.0], [2, st, "TCC_EA0_RDREQ_32B_sum", 10.0], [2, st, "TCC_BUBBLE_sum", 0.0],
        [3, neg, "TCC_EA0_RDREQ_sum", float(2 ** 30 // 128)], [3, neg, "TCC_EA0_RDREQ_32B_sum", 0.0],
        [3, neg, "TCC_BUBBLE_sum", 0.0]])
    _write(str(wr / "h" / "1_counter_collection.csv"), hdr, [
        [1, st, "TCC_EA0_WRREQ_sum", 100.0], [1, st, "TCC_EA0_WRREQ_64B_sum", 50.0],
        [1, st, "TCC_HIT_sum", 30.0], [1, st, "TCC_MISS_sum", 70.0],
        [3, neg, "TCC_EA0_WRREQ_sum", float(2 ** 30 // 64)], [3, neg, "TCC_EA0_WRREQ_64B_sum", float(2 ** 30 // 64)],
        [3, neg, "TCC_HIT_sum", 0.0], [3, neg, "TCC_MISS_sum", 1.0]])
    _write(str(sq / "h" / "1_counter_collection.csv"), hdr, [
        [1, st, "GRBM_GUI_ACTIVE", 1000.0], [1, st, "GRBM_GUI_ACTIVE", 990.0],   # per-XCD instances: max
        [1, st, "SQ_ACTIVE_INST_VALU", 64000.0],
        [1, st, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0], [1, st, "SQ_LDS_BANK_CONFLICT", 2560.0],
        [1, st, "SQ_INSTS_LDS", 5.0], [1, st, "SQ_WAVES", 7.0], [1, st, "SQ_BUSY_CU_CYCLES", 1.0],
        # one summed row per dispatch (rocprofv3's own CSV): the per-XCD cycles are the row / 8
        [3, neg, "GRBM_GUI_ACTIVE", 8000.0], [3, neg, "SQ_ACTIVE_INST_VALU", 25600.0],
        [3, neg, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0], [3, neg, "SQ_LDS_BANK_CONFLICT", 0.0],
        [3, neg, "SQ_INSTS_LDS", 0.0], [3, neg, "SQ_WAVES", 1.0]])
    r = bench.summarize_counters(str(rd), str(wr), str(sq), "llama8b_128k", {"select_stream": 254_080}, "cmd")
    assert r["probe"]["bytes_per_read_request"] == 128.0
    assert r["probe"]["fetch_size_definition_bytes"] == 2 ** 30 // 2
    assert r["probe"]["write_size_definition_bytes"] == 2 ** 30
    k = r["kernels"]["select_stream"]
    assert k["read_bytes"] == 10 * 32 + 990 * 128 and k["write_bytes"] == 50 * 32 + 50 * 64
    assert k["hbm_bytes_per_dispatch"] == k["read_bytes"] + k["write_bytes"]
    assert k["l2_hit_rate"] == 0.3 and k["dispatches"] == 2
    assert k["valu_busy_pct"] == 25.0 and k["mfma_busy_pct"] == 0.0 and k["lds_bank_conflict_pct"] == 1.0
    assert k["traffic_over_algorithmic"] == round((k["read_bytes"] + k["write_bytes"]) / 254_080, 4)
    n = r["kernels"][bench.PROBE_KERNEL]
    assert n["gui_active_cycles"] == 1000 and n["valu_busy_pct"] == 10.0
    json.dumps(r)
    assert "select_stream" in bench.counters_markdown(r)


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
