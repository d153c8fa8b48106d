#!/usr/bin/env python
"""Benchmark of the JSSA decode attention stage on one MI355X.

A step is one decode step of the whole batch through the library's C ABI:
for a single-layer workload one jssa_decode call (store the new token's
projected key, select = qhat + sampled threshold, FP8 score stream over every
cached token, exact top-B, then gather-free attention with the split-K
merge); for the hybrid stack all of its layers in order (sliding-window layers
through jssa_full_decode, global layers through jssa_decode, each with its own
basis).  The default workload is the Llama-3.1-8B-shaped layer at 128K,
batch 8.  Inputs are synthetic and seeded; each basis M comes from the
library's own calibration (jssa_calib_moments + jssa_basis) on synthetic
calibration sequences.  Everything is resident in HBM before the timed region;
cache replicas are rotated when one step's bytes would fit in the 256 MB
Infinity Cache.

Also measured: the same steps captured in HIP graphs, the dense full-KV decode
on the same caches (speedup), each stage alone with HIP events (roofline of
the dominant kernel) and the CPU oracle on a bounded sample (cpu_baseline).
Prints one JSON line.

Two helper modes turn rocprofv3 output into the short summaries kept under
profiles/:
  --summarize-trace DIR   kernel-trace statistics -> markdown table
  --summarize-counters READ_DIR WRITE_DIR SQ_DIR   three counter passes
      (HBM reads, HBM writes, SQ busy/LDS counters) per dispatch of each hot
      kernel, scaled by the same counters on the 1 GiB elementwise probe
      (--copy-probe) -> JSON read back by this script, plus a markdown table
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _early_cpu_threads(argv):
    """--cpu-threads N has to reach the OpenBLAS and OpenMP pools before numpy and torch load them: a limit set
    later is not honoured by every pool on every host."""
    for i, a in enumerate(argv):
        v = a.split("=", 1)[1] if a.startswith("--cpu-threads=") else (
            argv[i + 1] if a == "--cpu-threads" and i + 1 < len(argv) else None)
        if v is not None and v.isdigit() and int(v) > 0:
            for name in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
                os.environ[name] = v


if __name__ == "__main__":
    _early_cpu_threads(sys.argv[1:])

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
STREAM_KERNEL = "select_stream"
PROBE_KERNEL = "neg_kernel"           # torch's elementwise negation kernel: the 1 GiB probe
PROBE_BYTES = 1 << 30                 # fp32 neg over 2^28 elements: 1 GiB read, 1 GiB written
STREAM_SOURCES = ("select.hip", "common.h", "kernels.h")
METRIC = "decode attn-stage steps/s @128K; HBM GB/s vs peak; speedup vs full-KV decode"


def counters_path(workload):
    return os.path.join(ROOT, "profiles", f"counters_{workload}.json")


def _code_lines(text: str):
    """The source's code without comments and blank lines (a comment edit leaves the hash alone)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    for line in text.splitlines():
        line = line.split("//", 1)[0].rstrip()
        if line:
            yield line


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_decode_amd", "csrc", n)) as f:
            for line in _code_lines(f.read()):
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- algorithmic bytes

SCALE_BYTES = {"fp32": 4, "e8m0": 1, "none": 0, "bf16": 0}
KEY_BYTES = {"fp32": 1, "e8m0": 1, "none": 1, "bf16": 2}        # bytes per scoring dim


def layer_bytes(w, seq_lens, mode, scale_format="fp32"):
    """Bytes one layer must move per step.  mode: 'sparse' (JSSA), 'full' (all positions), 'window'."""
    S, d, hkv, hq, B = w.score_dims, w.head_dim, w.num_kv_heads, w.num_q_heads, w.budget
    row = d * 2 if w.kind == "mla" else 2 * d * 2    # one latent row (K = V) / one K + V pair per KV head
    io = w.batch * hq * (d + w.v_dim) * 2 + w.batch * w.pages_per_seq * 4
    if mode == "full":
        return {"kv": sum(n * hkv * row for n in seq_lens), "q_out_table": io}
    if mode == "window":      # only the window's pages of the block table are read
        io_w = w.batch * hq * (d + w.v_dim) * 2 + w.batch * (-(-w.window // w.page_size)) * 4
        return {"kv": sum(min(n, w.window) * hkv * row for n in seq_lens), "q_out_table": io_w}
    sb = SCALE_BYTES[scale_format]
    S = S * KEY_BYTES[scale_format]
    return {"score": sum(n * hkv * (S + sb) for n in seq_lens),
            "selected_kv": sum(min(B, n) * hkv * row for n in seq_lens),
            "indices": w.batch * hkv * B * 4 * 2,
            "q_out_table": io,
            "store": w.batch * hkv * (d * 2 + S + sb)}


def step_bytes(w, seq_lens, sparse=True, scale_format="fp32"):
    """Sum over the step's layers, with the per-part breakdown."""
    parts = {}
    for l in range(w.num_layers if w.window else 1):
        if w.window and l in w.window_layers():
            p = {"window_" + k: v for k, v in layer_bytes(w, seq_lens, "window").items()}
        else:
            p = layer_bytes(w, seq_lens, "sparse" if sparse else "full", scale_format)
        for k, v in p.items():
            parts[k] = parts.get(k, 0) + v
    return sum(parts.values()), parts


def mla_attend_flops(w, seq_lens, sparse=True):
    """2 * Hq * (576 + 512) flops per attended row and sequence."""
    n = sum(min(w.budget, s) if sparse else s for s in seq_lens)
    return 2 * w.num_q_heads * (w.head_dim + w.v_dim) * n


# ----------------------------------------------------------------------------- setup

def calibrate_gqa(L, w, layer, device):
    import torch
    from synth import make_gqa_calibration
    shape = L.shape_for(w)
    qc, kc = make_gqa_calibration(w, layer, device=device)
    T = qc.shape[0]
    gq = torch.zeros((w.num_kv_heads, w.head_dim, w.head_dim), dtype=torch.float32, device=device)
    gk = torch.zeros_like(gq)
    ws = torch.empty(L.calib_workspace_bytes(shape, T), dtype=torch.uint8, device=device)
    L.jssa_calib_moments(shape, qc, kc, gq, gk, ws)
    return torch.from_numpy(L.jssa_basis(shape, gq.cpu().numpy(), gk.cpu().numpy())).to(device)


def calibrate_mla(L, w, device):
    import torch
    from synth import make_mla_calibration
    shape = L.shape_for(w)
    gq = torch.zeros((1, w.latent_dim, w.latent_dim), dtype=torch.float32, device=device)
    gk = torch.zeros_like(gq)
    ws = torch.empty(L.calib_workspace_bytes(shape, 2048), dtype=torch.uint8, device=device)
    for qc, lat in make_mla_calibration(w, device=device, chunk=2048):
        L.jssa_calib_moments(shape, qc, lat, gq, gk, ws)
    return torch.from_numpy(L.jssa_basis(shape, gq.cpu().numpy(), gk.cpu().numpy())[0]).to(device)


def bulk_store(L, w, shape, keys_flat, block_table, seq_lens, M, kp, ks):
    """Store every cached position (rows gathered in logical order, 128K tokens per call)."""
    import torch
    P = w.page_size
    bt = block_table.long()
    for b in range(w.batch):
        n = int(seq_lens[b])
        for t0 in range(0, n, 1 << 17):
            t = torch.arange(t0, min(n, t0 + (1 << 17)), device=keys_flat.device)
            slots = (bt[b, t // P] * P + t % P).to(torch.int32)
            L.jssa_store(shape, keys_flat[slots.long()].contiguous(), slots, M, kp, ks, check_slots=False)


def new_token(w, keys_flat, block_table, seq_lens):
    """Key and slot of position N-1 of every sequence (the token being decoded)."""
    import torch
    P = w.page_size
    bt = block_table.long()
    last = seq_lens.long() - 1
    slot = (bt[torch.arange(w.batch, device=bt.device), last // P] * P + last % P).to(torch.int32)
    return keys_flat[slot.long()].contiguous(), slot


class Layer:
    """Device state of one layer: inputs, caches and (global layers) basis + scoring cache."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def setup(w, device, replicas, scale_format="fp32"):
    """Returns (shape, layers of every replica, block_table, seq_lens, generated case)."""
    import torch
    import long_context_decode_amd as L
    from synth import make_gqa_case, make_mla_case

    shape = L.shape_for(w, scale_format=L.SCALE_FORMATS[scale_format])
    if w.kind == "mla":
        M = calibrate_mla(L, w, device)
        case = make_mla_case(w, device=device)
        kp, ks = L.alloc_scoring_cache(shape, case.latent.shape[0], device)
        flat = case.latent.view(-1, w.head_dim)
        bulk_store(L, w, shape, flat, case.block_table, case.seq_lens, M, kp, ks)
        k_new, slot_new = new_token(w, flat, case.block_table, case.seq_lens)
        base = [Layer(window=0, q=case.q, kc=case.latent, vc=None, M=M, kp=kp, ks=ks, k_new=k_new,
                      slot_new=slot_new)]
    else:
        case = make_gqa_case(w, device=device, layers=list(range(w.num_layers if w.window else 1)))
        base = []
        for l, lay in sorted(case.layers.items()):
            if w.window and l in w.window_layers():
                base.append(Layer(window=w.window, q=lay.q, kc=lay.k_cache, vc=lay.v_cache))
                continue
            M = calibrate_gqa(L, w, l, device)
            kp, ks = L.alloc_scoring_cache(shape, lay.k_cache.shape[0], device)
            flat = lay.k_cache.view(-1, w.num_kv_heads, w.head_dim)
            bulk_store(L, w, shape, flat, case.block_table, case.seq_lens, M, kp, ks)
            k_new, slot_new = new_token(w, flat, case.block_table, case.seq_lens)
            base.append(Layer(window=0, q=lay.q, kc=lay.k_cache, vc=lay.v_cache, M=M, kp=kp, ks=ks,
                              k_new=k_new, slot_new=slot_new))
    reps = [base]
    for _ in range(replicas - 1):
        reps.append([Layer(**{k: (v.clone() if k in ("kc", "vc", "kp", "ks") and v is not None else v)
                              for k, v in lay.__dict__.items()}) for lay in base])
    torch.cuda.synchronize()
    return shape, reps, case.block_table.to(device), case.seq_lens.to(device), case


# ----------------------------------------------------------------------------- timing

def _quantiles(xs):
    s = sorted(xs)

    def q(p):
        return s[min(len(s) - 1, max(0, int(round(p * (len(s) - 1)))))]
    return q(0.5), q(0.1), q(0.9)


def time_steps(fn, steps, warmup, n_rep, blocks=5):
    """K steps in one timed region (events at block boundaries, no sync inside), bracketed by
    synchronisations.  Returns (mean ms/step, block median, p10, p90, host wall ms/step)."""
    import torch
    for i in range(warmup):
        fn(i % n_rep)
    torch.cuda.synchronize()
    blocks = max(1, min(blocks, steps))
    bounds = [round(i * steps / blocks) for i in range(blocks + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    t0 = time.perf_counter()
    ev[0].record()
    for k in range(blocks):
        for i in range(bounds[k], bounds[k + 1]):
            fn(i % n_rep)
        ev[k + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per_block = [ev[k].elapsed_time(ev[k + 1]) / (bounds[k + 1] - bounds[k]) for k in range(blocks)]
    med, p10, p90 = _quantiles(per_block)
    return ev[0].elapsed_time(ev[-1]) / steps, med, p10, p90, wall


def time_graph(fn, steps, warmup, n_rep):
    """The same step captured once per replica in a HIP graph; the graphs replayed back to back."""
    import torch
    graphs = []
    for r in range(n_rep):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(r)
        graphs.append(g)
    total, med, p10, p90, _ = time_steps(lambda r: graphs[r].replay(), steps, warmup, n_rep)
    return total, med, p10, p90


def time_graph_multi(fn, steps, warmup, n_rep, per_graph=8):
    """per_graph consecutive steps (rotating the replicas) captured in one HIP graph, as a serving loop
    captures a whole model step; the graph replayed back to back.  Returns ms per step."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i % n_rep)
    replays = max(1, steps // per_graph)
    for _ in range(max(1, warmup // per_graph)):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * per_graph)


def time_stages(stage_fns, steps, n_rep):
    """Average duration of each stage: `steps` back-to-back launches of that stage alone (rotating the
    replicas) between two HIP events on the current stream, the stream every library call launches on.
    A kernel that runs longer than the host needs to issue the next call is timed exactly (the launches
    queue up with no idle gap); shorter ones read high by the host's launch interval."""
    import torch
    res = {}
    for name, fn in stage_fns.items():
        for i in range(2):
            fn(i % n_rep)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            fn(i % n_rep)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    return res


def time_stages_graph(stage_fns, n_rep, launches=60, replays=4):
    """Average duration of each stage on the GPU: `launches` launches of that stage alone (rotating over
    n_rep units) captured in one HIP graph, replayed `replays` times between two HIP events on the current
    stream (the graph runs on it).  No host launch interval enters, so short kernels are timed too; the
    figure includes the gap between consecutive kernels of a graph."""
    import torch
    res = {}
    for name, fn in stage_fns.items():
        for i in range(2):
            fn(i % n_rep)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(launches):
                fn(i % n_rep)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / (launches * replays)
        del g
    return res


# ----------------------------------------------------------------------------- CPU oracle

def _host_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count()


def cpu_baseline(w, case, n_seqs, min_seconds=10.0, max_passes=5):
    """The oracle (as is) on host cores: store of the first layer's cache (untimed), then passes of select +
    attend over n_seqs sequences, every KV head, repeated until about min_seconds have run; the median pass,
    scaled to the batch, is one step."""
    import numpy as np
    import torch
    from oracle import calibrate as ocal
    from oracle import gqa as ogqa
    from oracle import mla as omla
    from synth import bf16_bits, make_gqa_calibration, make_mla_calibration

    bt = case.block_table
    jobs = []                                   # one closure per sequence: the timed oracle work
    if w.kind == "mla":
        chunks = ((ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(l)))
                  for q, l in make_mla_calibration(w, chunk=512))
        m32 = omla.calibrate(chunks, w.latent_dim, w.rank)[0].astype(np.float32)
        q = bf16_bits(case.q)
        for b in range(n_seqs):
            n = int(case.seq_lens[b])
            t = torch.arange(n, device=case.latent.device)
            rows = bf16_bits(case.latent[bt[b].long()[t // w.page_size], t % w.page_size])
            codes, scale = omla.store(rows, m32)
            jobs.append(lambda q=q[b], rows=rows, codes=codes, scale=scale: omla.decode_step(
                q, rows, m32, w.budget, w.sm_scale, codes=codes, scale=scale))
    else:
        qc, kc = make_gqa_calibration(w, 0, device="cpu")
        m32 = ocal.calibrate(ocal.bf16_to_f64(bf16_bits(qc)), ocal.bf16_to_f64(bf16_bits(kc)), w.group,
                             w.rank).astype(np.float32)
        lay = case.layers[0]
        q = bf16_bits(lay.q)
        for b in range(n_seqs):
            n = int(case.seq_lens[b])
            t = torch.arange(n, device=lay.k_cache.device)
            pg = bt[b].long()[t // w.page_size]
            kr = bf16_bits(lay.k_cache[pg, t % w.page_size])
            vr = bf16_bits(lay.v_cache[pg, t % w.page_size])
            codes, scale = ogqa.store(kr, m32)
            jobs.append(lambda q=q[b], kr=kr, vr=vr, codes=codes, scale=scale: ogqa.decode_step(
                q, kr, vr, m32, w.budget, w.sm_scale, codes=codes, scale=scale))
    passes = []
    while len(passes) < max_passes and (sum(passes) < min_seconds or len(passes) < 1):
        t0 = time.perf_counter()
        for job in jobs:
            job()
        passes.append(time.perf_counter() - t0)
    per_step = sorted(passes)[len(passes) // 2] * w.batch / n_seqs
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except Exception:  # pragma: no cover
        pass
    return {"value": round(1.0 / per_step, 4), "unit": "steps/s", "cores": int(_host_threads()), "kind": "oracle",
            "sample": f"{len(passes)} passes of select + attend (fp64 NumPy, every KV head) over {n_seqs} of "
                      f"{w.batch} sequences of one layer (store untimed), {sum(passes):.1f} s in all; median "
                      f"pass scaled x{w.batch / n_seqs:g} to one step; host {cpu}"}


# ----------------------------------------------------------------------------- counters

def traffic_for(workload):
    """HBM bytes per dispatch of the score-stream kernel from committed rocprofv3 counters, if they were
    taken on the current kernel source."""
    path = counters_path(workload)
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    if c.get("source_hash") != _src_hash(*STREAM_SOURCES):
        return None
    k = c.get("kernels", {}).get(STREAM_KERNEL)
    return None if k is None else k.get("hbm_bytes_per_dispatch")


def _rows(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


# rocprofv3 counter passes (one run each; at most 4 TCC, 8 SQ and 2 GRBM counters per pass)
COUNTER_PASSES = {
    "read": ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum"],
    "write": ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_HIT_sum", "TCC_MISS_sum"],
    "sq": ["SQ_WAVES", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES",
           "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"],
}
HOT_KERNELS = ("store_kernel", "select_prologue", "select_stream", "select_finish", "attend_kernel", "merge_kernel",
               "mla_sparse_kernel", "mla_dense_kernel", "decode_fused_kernel", "gather_kernel", PROBE_KERNEL)
CU_NUM, SIMD_NUM = 256, 1024


def _kernel_group(name):
    """The library kernel (or the probe) a dispatch belongs to; the sparse and dense GQA attention and the
    merge of each are told apart by their template arguments."""
    for k in HOT_KERNELS:
        if k in name:
            if k == "attend_kernel":
                return "attend_kernel (dense)" if re.search(r"attend_kernel<\d+, \d+, true>|Lb1E", name) else \
                    "attend_kernel (sparse)"
            return k
    return None


# counters with one instance per XCD that the rocprofv3 derived metrics reduce with max (the elapsed cycles
# of the dispatch); the others are summed over their instances.  rocprofv3's CSV holds one row per (dispatch,
# counter) with the instances already summed, so such a row is divided by the XCD count (on this GPU the 1 GiB
# probe's GRBM_GUI_ACTIVE row reads 8 x 2.4 GHz x its traced duration); rows given per instance take the max.
MAX_OVER_INSTANCES = ("GRBM_GUI_ACTIVE",)
XCD_NUM = 8


def _per_dispatch(d):
    """{kernel group: {counter: mean over the group's dispatches of the counter within a dispatch (summed over
    its instances, or reduced with max for MAX_OVER_INSTANCES)}}."""
    acc = {}
    for r in _rows(d, "counter_collection.csv"):
        g = _kernel_group(r.get("Kernel_Name", ""))
        if g is None:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        name, v = r["Counter_Name"], float(r["Counter_Value"])
        acc.setdefault(g, {}).setdefault(name, {}).setdefault(key, []).append(v)
    out = {}
    for g, cs in acc.items():
        red = {}
        for c, per in cs.items():
            if c in MAX_OVER_INSTANCES:
                vals = [v[0] / XCD_NUM if len(v) == 1 else max(v) for v in per.values()]
            else:
                vals = [sum(v) for v in per.values()]
            red[c] = sum(vals) / len(vals)
        out[g] = red
        out[g]["dispatches"] = max(len(v) for v in cs.values())
    return out


def summarize_counters(read_dir, write_dir, sq_dir, workload, alg_bytes, command):
    """Per hot kernel and dispatch: HBM bytes read and written, L2 hit rate, VALU busy, MFMA busy and LDS
    bank-conflict time, from the three counter passes.  Bytes read: the L2's 32-byte requests count 32 B and
    its other read requests the size that makes the probe's known read (1 GiB) come out, derived from the
    probe's own counters; bytes written: the WRITE_SIZE definition (32- and 64-byte requests), checked on the
    probe's 1 GiB write."""
    rd, wr, sq = _per_dispatch(read_dir), _per_dispatch(write_dir), _per_dispatch(sq_dir)
    pr, pw = rd[PROBE_KERNEL], wr[PROBE_KERNEL]
    full = pr["TCC_EA0_RDREQ_sum"] - pr["TCC_EA0_RDREQ_32B_sum"]
    bytes_per_req = (PROBE_BYTES - 32.0 * pr["TCC_EA0_RDREQ_32B_sum"]) / full
    fetch_def = (pr["TCC_BUBBLE_sum"] * 128 + (pr["TCC_EA0_RDREQ_sum"] - pr["TCC_BUBBLE_sum"] -
                                                pr["TCC_EA0_RDREQ_32B_sum"]) * 64 + pr["TCC_EA0_RDREQ_32B_sum"] * 32)

    def wbytes(c):
        return (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"]) * 32 + c["TCC_EA0_WRREQ_64B_sum"] * 64

    kernels = {}
    for g in sorted(set(rd) | set(wr) | set(sq)):
        k = {}
        if g in rd:
            c = rd[g]
            k["read_bytes"] = int(32 * c["TCC_EA0_RDREQ_32B_sum"] +
                                  bytes_per_req * (c["TCC_EA0_RDREQ_sum"] - c["TCC_EA0_RDREQ_32B_sum"]))
            k["read_requests"] = int(c["TCC_EA0_RDREQ_sum"])
            k["read_128b_bubble"] = int(c["TCC_BUBBLE_sum"])
        if g in wr:
            c = wr[g]
            k["write_bytes"] = int(wbytes(c))
            hm = c["TCC_HIT_sum"] + c["TCC_MISS_sum"]
            k["l2_hit_rate"] = round(c["TCC_HIT_sum"] / hm, 4) if hm else None
        if "read_bytes" in k and "write_bytes" in k:
            k["hbm_bytes_per_dispatch"] = k["read_bytes"] + k["write_bytes"]
        if g in sq:
            c = sq[g]
            gui = c["GRBM_GUI_ACTIVE"]
            k["gui_active_cycles"] = int(gui)
            k["valu_busy_pct"] = round(100.0 * c["SQ_ACTIVE_INST_VALU"] / CU_NUM / gui, 2) if gui else None
            k["mfma_busy_pct"] = round(100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMD_NUM), 2) if gui else None
            k["lds_bank_conflict_pct"] = round(100.0 * c["SQ_LDS_BANK_CONFLICT"] / gui / CU_NUM, 3) if gui else None
            k["lds_instructions"] = int(c["SQ_INSTS_LDS"])
            k["waves"] = int(c["SQ_WAVES"])
        k["dispatches"] = max(x[g]["dispatches"] for x in (rd, wr, sq) if g in x)
        if g in alg_bytes:
            k["algorithmic_bytes_per_dispatch"] = alg_bytes[g]
            if "hbm_bytes_per_dispatch" in k:
                k["traffic_over_algorithmic"] = round(k["hbm_bytes_per_dispatch"] / alg_bytes[g], 4)
        kernels[g] = k
    return {"workload": workload, "source_hash": _src_hash(*STREAM_SOURCES),
            "probe": {"kernel": PROBE_KERNEL, "bytes_read": PROBE_BYTES, "bytes_written": PROBE_BYTES,
                      "read_requests": int(pr["TCC_EA0_RDREQ_sum"]), "read_32b": int(pr["TCC_EA0_RDREQ_32B_sum"]),
                      "read_128b_bubble": int(pr["TCC_BUBBLE_sum"]),
                      "bytes_per_read_request": round(bytes_per_req, 2),
                      "fetch_size_definition_bytes": int(fetch_def),
                      "write_size_definition_bytes": int(wbytes(pw))},
            "kernels": kernels, "command": command}


def counters_markdown(c):
    lines = [f"# rocprofv3 counters, {c['workload']}", "", f"Command: `{c['command']}`", "",
             f"Probe (torch neg over 1 GiB): {c['probe']['read_requests']} L2 read requests for 2^30 bytes = "
             f"{c['probe']['bytes_per_read_request']} bytes per request ({c['probe']['read_128b_bubble']} counted "
             f"as 128-byte); the FETCH_SIZE definition gives {c['probe']['fetch_size_definition_bytes']} bytes. "
             f"WRITE_SIZE definition: {c['probe']['write_size_definition_bytes']} bytes for the 2^30 written.", "",
             "| kernel | dispatches | HBM read MB | HBM write MB | traffic / algorithmic | L2 hit | VALU busy % | "
             "MFMA busy % | LDS bank conflict % |", "|---|---|---|---|---|---|---|---|---|"]
    for g, k in c["kernels"].items():
        f = lambda x, d=1: "" if x is None else (f"{x / 1e6:.{d}f}" if isinstance(x, int) else f"{x}")  # noqa: E731
        lines.append(f"| `{g}` | {k.get('dispatches')} | {f(k.get('read_bytes'), 2)} | {f(k.get('write_bytes'), 2)} | "
                     f"{k.get('traffic_over_algorithmic', '')} | {k.get('l2_hit_rate', '')} | "
                     f"{k.get('valu_busy_pct', '')} | {k.get('mfma_busy_pct', '')} | {k.get('lds_bank_conflict_pct', '')} |")
    return "\n".join(lines) + "\n"


def summarize_trace(d, command):
    """Markdown table of the library's kernels (and the probe); everything else the run launched (synthetic
    data generation, torch copies, calibration set-up) is folded into one line."""
    rows = _rows(d, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    other = [0, 0.0, 0.0]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("|", "/")
        if "jssa::" not in name and PROBE_KERNEL not in name:
            other[0] += int(r["Calls"])
            other[1] += float(r["TotalDurationNs"])
            other[2] += float(r["Percentage"])
            continue
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    if other[0]:
        lines.append(f"| other kernels (set-up: data generation, copies) | {other[0]} | "
                     f"{other[1] / other[0] / 1e3:.2f} | | | {other[2]:.2f} |")
    return "\n".join(lines) + "\n"


# ----------------------------------------------------------------------------- recall sweep

def recall_sweep(name, ranks, n_seqs, query_shift=0):
    """Top-B recall of the FP8 projected-score selection against the exact top-B of qbar . k (fp32 scores
    from plain torch on the GPU), for several ranks and three bases per KV head: the joint basis M*
    (jssa_calib_moments + jssa_basis), the top-r eigenvectors of the key moments alone (jssa_basis with the
    key moments on both sides) and a random orthonormal basis; and the joint basis over BF16 projected keys.
    Also reports the planted needles found."""
    import numpy as np
    import torch
    import long_context_decode_amd as L
    from synth import WORKLOADS, make_gqa_calibration, make_gqa_case
    from synth.workloads import haar_orthogonal

    w = WORKLOADS[name].scaled(batch=n_seqs, query_shift=query_shift)
    dev = torch.device("cuda:0")
    case = make_gqa_case(w, device=dev, layers=[0])
    lay = case.layers[0]
    bt, sl = case.block_table.to(dev), case.seq_lens.to(dev)
    qc, kc = make_gqa_calibration(w, 0, device=dev)
    # exact top-B per (sequence, KV head) from fp32 scores qbar . k
    P, N, G = w.page_size, w.seq_len, w.group
    t = torch.arange(N, device=dev)
    exact = []
    for b in range(w.batch):
        keys = lay.k_cache[bt[b].long()[t // P], t % P].float()                      # [N, Hkv, d]
        qbar = lay.q[b].float().view(w.num_kv_heads, G, w.head_dim).mean(1)         # [Hkv, d]
        s = torch.einsum("nhd,hd->hn", keys, qbar)
        exact.append(torch.topk(s, w.budget, dim=1).indices)                         # [Hkv, B]
    needles = {k: torch.as_tensor(v, device=dev) for k, v in lay.needles.items()}
    rows = []
    for r in ranks:
        # ranks below the kernels' 16-dim pieces: the first r rows of the rank-16 basis (rows are in
        # descending eigenvalue order), zero-padded to 16 rows.  The zero rows add nothing to a score
        # and leave each token's scale (max |y|) unchanged, so the selection is that of rank r.
        rk = max(r, 16)
        shape = L.shape_for(w.scaled(rank=rk))
        T = qc.shape[0]
        gq = torch.zeros((w.num_kv_heads, w.head_dim, w.head_dim), dtype=torch.float32, device=dev)
        gk = torch.zeros_like(gq)
        L.jssa_calib_moments(shape, qc, kc, gq, gk,
                             torch.empty(L.calib_workspace_bytes(shape, T), dtype=torch.uint8, device=dev))
        gq_h, gk_h = gq.cpu().numpy(), gk.cpu().numpy()
        bases = {
            "joint M*": L.jssa_basis(shape, gq_h, gk_h),
            "keys only": L.jssa_basis(shape, gk_h, gk_h),
            "random": np.stack([haar_orthogonal(w.head_dim, 1000 + 7 * h + r)[:, :rk].T
                                for h in range(w.num_kv_heads)]).astype(np.float32),
        }
        for m in bases.values():
            m[:, r:, :] = 0.0
        # the FP8 cache for every basis, and the joint basis over BF16 keys (the README's non-FP8 option)
        variants = [(bname, m, L.SCALE_FP32) for bname, m in bases.items()]
        variants.append(("joint M*, BF16 keys", bases["joint M*"], L.KEYS_BF16))
        for bname, m, fmt in variants:
            shp = L.shape_for(w.scaled(rank=rk), scale_format=fmt)
            M = torch.from_numpy(np.ascontiguousarray(m)).to(dev)
            kp, ks = L.alloc_scoring_cache(shp, lay.k_cache.shape[0], dev)
            bulk_store(L, w, shp, lay.k_cache.view(-1, w.num_kv_heads, w.head_dim), bt, sl, M, kp, ks)
            idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=dev)
            L.jssa_select(shp, lay.q, M, kp, ks, bt, sl, idx, L.alloc_workspace(shp, dev))
            hits, found, total_n = 0, 0, 0
            for b in range(w.batch):
                for h in range(w.num_kv_heads):
                    sel = idx[b, h].long()
                    hits += int(torch.isin(sel, exact[b][h]).sum())
                    nd = needles[(b, h)]
                    found += int(torch.isin(nd, sel).sum())
                    total_n += len(nd)
            rows.append({"rank": r, "basis": bname,
                         "topB_recall": round(hits / (w.batch * w.num_kv_heads * w.budget), 4),
                         "needle_recall": round(found / max(total_n, 1), 4)})
            print(f"[recall] r={r} {bname}: {rows[-1]}", file=sys.stderr, flush=True)
            del kp, ks
    return {"workload": w.name, "sequences": w.batch, "seq_len": w.seq_len, "budget": w.budget,
            "query_shift": query_shift, "scoring_cache": "fp8 e4m3fn + fp32 scale", "rows": rows}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_128k",
                    help="llama8b_128k (default), llama8b_32k, hybrid_64k, mla_128k, tiny, tiny_mla")
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas rotated per step (0: automatic)")
    ap.add_argument("--cpu-seqs", type=int, default=-1,
                    help="sequences per CPU-oracle pass (0: skip; default the whole batch on the default workload)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU oracle's BLAS/OpenMP pools (0: all the host offers)")
    ap.add_argument("--no-graph", action="store_true",
                    help="no HIP graphs at all: skip the graph timing of the step and time each stage from "
                         "host-launched calls (for counter collection)")
    ap.add_argument("--scale-format", default="fp32", choices=["fp32", "e8m0", "none", "bf16"],
                    help="scoring-cache format: FP8 with an fp32 scale per token (default), with a one-byte power of two, "
                         "with no scale, or BF16 projected keys")
    ap.add_argument("--decode-path", default="auto", choices=["auto", "split", "fused"],
                    help="jssa_decode's path: the library's choice, the five-launch split path, or the single launch")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one elementwise kernel over 1 GiB (reference for counter scaling)")
    ap.add_argument("--recall-sweep", action="store_true",
                    help="top-B recall vs rank for the joint, key-only and random bases (prints one JSON line)")
    ap.add_argument("--ranks", default="4,8,16,32,48,64")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("READ_DIR", "WRITE_DIR", "SQ_DIR"),
                    help="rocprofv3 counter passes (COUNTER_PASSES) -> profiles/counters_<workload>.json / .md")
    ap.add_argument("--command", default="", help="profiling command recorded in a summary")
    ap.add_argument("--out", help="summary output file")
    args = ap.parse_args()

    if args.summarize_trace or args.summarize_counters:
        if args.summarize_trace:
            txt = summarize_trace(args.summarize_trace, args.command)
            if args.out:
                with open(args.out, "w") as f:
                    f.write(txt)
            else:
                print(txt)
            return
        from synth import WORKLOADS
        w = WORKLOADS[args.workload]
        lb = layer_bytes(w, [w.seq_len] * w.batch, "sparse")
        alg = {STREAM_KERNEL: lb["score"],
               "attend_kernel (sparse)": lb["selected_kv"] + lb["indices"] // 2,
               "mla_sparse_kernel": lb["selected_kv"] + lb["indices"] // 2}
        c = summarize_counters(*args.summarize_counters, args.workload, alg, args.command)
        with open(counters_path(args.workload), "w") as f:
            f.write(json.dumps(c, indent=1) + "\n")
        with open(counters_path(args.workload)[:-5] + ".md", "w") as f:
            f.write(counters_markdown(c))
        print(counters_markdown(c))
        return

    if args.recall_sweep:
        from synth import WORKLOADS
        w = args.workload if args.workload != "llama8b_128k" else "llama8b_32k"
        ranks = [int(x) for x in args.ranks.split(",")]
        # queries sharing the keys' leading directions, then queries whose energy sits half a basis away
        res = [recall_sweep(w, ranks, 4, shift) for shift in (0, WORKLOADS[w].head_dim // 2)]
        print(json.dumps(res), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the JSSA decode path runs per GPU and has no multi-GPU mode here "
              "(batch and KV heads would shard with no exchange inside the attention stage)", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_decode_amd as L
    from synth import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seq = [w.seq_len] * w.batch
    total_bytes, parts = step_bytes(w, seq, True, args.scale_format)
    full_bytes, _ = step_bytes(w, seq, False)
    n_rep = args.replicas or (1 if total_bytes > (1 << 30) else 3)

    t_setup = time.perf_counter()
    shape, reps, bt, sl, case = setup(w, dev, n_rep, args.scale_format)
    print(f"[bench] {w.name}: setup {time.perf_counter() - t_setup:.1f} s, {n_rep} replica(s)", file=sys.stderr,
          flush=True)
    ws = L.alloc_workspace(shape, dev)
    idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.num_q_heads, w.v_dim), dtype=torch.bfloat16, device=dev)
    modes = {"auto": L.SELECT_AUTO, "split": L.SELECT_SPLIT, "fused": L.SELECT_FUSED}
    single = L.decode_single_launch(L.shape_for(w, scale_format=L.SCALE_FORMATS[args.scale_format],
                                                select_mode=modes[args.decode_path]))

    def run_layer(lay, sparse, mode=modes[args.decode_path]):
        if lay.window or not sparse:
            L.jssa_full_decode(shape, lay.q, lay.kc, lay.vc, bt, sl, lay.window, w.sm_scale, out, ws)
        else:
            dshape = L.shape_for(w, scale_format=L.SCALE_FORMATS[args.scale_format], select_mode=mode)
            L.jssa_decode(dshape, lay.q, lay.k_new, lay.slot_new, lay.M, lay.kp, lay.ks, lay.kc, lay.vc, bt, sl,
                          idx, w.sm_scale, out, ws)

    def step(r):
        for lay in reps[r]:
            run_layer(lay, True)

    def full(r):
        for lay in reps[r]:
            run_layer(lay, False)

    ms, med, p10, p90, wall_ms = time_steps(step, args.steps, args.warmup, n_rep)
    print(f"[bench] eager {ms:.4f} ms/step", file=sys.stderr, flush=True)
    graph = None
    if not args.no_graph:
        g_ms, g_med, g_p10, g_p90 = time_graph(step, args.steps, args.warmup, n_rep)
        graph = {"ms_per_step": round(g_ms, 5), "block_median_ms": round(g_med, 5), "p10_ms": round(g_p10, 5),
                 "p90_ms": round(g_p90, 5), "steps_per_s": round(1e3 / g_ms, 2)}
        print(f"[bench] graph {g_ms:.4f} ms/step", file=sys.stderr, flush=True)
        gm_ms = time_graph_multi(step, args.steps, args.warmup, n_rep)
        graph["eight_steps_per_graph_ms_per_step"] = round(gm_ms, 5)
        print(f"[bench] graph of 8 steps {gm_ms:.4f} ms/step", file=sys.stderr, flush=True)
    ms_full, _, _, _, _ = time_steps(full, max(10, args.steps // 10), max(2, args.warmup // 4), n_rep)
    print(f"[bench] full-KV {ms_full:.4f} ms/step", file=sys.stderr, flush=True)
    paths = None
    if single:                                  # the same step through the five-launch split path
        def split_step(r):
            for lay in reps[r]:
                run_layer(lay, True, L.SELECT_SPLIT)
        ms_split = time_steps(split_step, args.steps, args.warmup, n_rep)[0]
        paths = {"single_launch_ms": round(ms, 5), "split_ms": round(ms_split, 5),
                 "ratio": round(ms_split / ms, 3)}
        print(f"[bench] split path {ms_split:.4f} ms/step", file=sys.stderr, flush=True)

    # stages of the sparse layers, rotating over (replica, layer) so that no launch finds the previous
    # launch's bytes in the Infinity Cache (and the whole of a window layer, if any)
    units = [(r, i) for r in range(n_rep) for i, lay in enumerate(reps[r]) if not lay.window]

    def lay_of(k):
        r, i = units[k % len(units)]
        return reps[r][i]

    def sel(stage):
        return lambda r: L.jssa_select(shape, lay_of(r).q, lay_of(r).M, lay_of(r).kp, lay_of(r).ks, bt, sl, idx, ws,
                                       stages=stage)

    stages = {
        "store": lambda r: L.jssa_store(shape, lay_of(r).k_new, lay_of(r).slot_new, lay_of(r).M, lay_of(r).kp,
                                        lay_of(r).ks, check_slots=False),
        "select_prologue": sel(L.STAGE_PROLOGUE),
        "select_stream": sel(L.STAGE_STREAM),
        "select_finish": sel(L.STAGE_FINISH),
        "attend": lambda r: L.jssa_attend(shape, lay_of(r).q, lay_of(r).kc, lay_of(r).vc, bt, sl, idx, w.sm_scale,
                                          out, ws),
        # the gather-then-attend baseline over the same selection (staging copy + dense attention)
        "gather_attend": lambda r: L.jssa_gather_attend(shape, lay_of(r).q, lay_of(r).kc, lay_of(r).vc, bt, sl, idx,
                                                        w.sm_scale, out, ws),
    }
    win = [(r, i) for r in range(n_rep) for i, lay in enumerate(reps[r]) if lay.window]
    if win:
        stages["window_layer"] = lambda k: run_layer(reps[win[k % len(win)][0]][win[k % len(win)][1]], True)
    n_units = max(len(units), len(win))
    for i in range(3):
        for f in stages.values():
            f(i)
    stage_ms = time_stages(stages, args.steps, n_units) if args.no_graph else time_stages_graph(stages, n_units)

    # achievable-bandwidth probe: torch's elementwise negation over 1 GiB (1 GiB read + 1 GiB written);
    # with --copy-probe it runs once more alone, as the reference dispatch for counter scaling
    src = torch.empty(PROBE_BYTES // 4, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    probe_ms = time_stages({"probe": lambda r: torch.neg(src, out=dst)}, 10, 1)["probe"]
    if args.copy_probe:
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
    del src, dst

    lb = layer_bytes(w, seq, "sparse", args.scale_format)
    stream_bytes = lb["score"]
    achieved = stream_bytes / (stage_ms["select_stream"] * 1e-3) / 1e9
    # the dominant kernel alone (the score stream); the whole step's figure is step_roofline
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_for(w.name) if args.scale_format == "fp32" else None,
                "kernel": "select_stream (FP8 score stream + candidate compaction; dominant kernel only)",
                "bytes_per_launch": stream_bytes, "avg_launch_ms": round(stage_ms["select_stream"], 5)}
    step_gbps = total_bytes / (ms * 1e-3) / 1e9
    step_roofline = {"bound": "hbm", "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(step_gbps / HBM_PEAK_GBPS, 4), "bytes_per_step": total_bytes,
                     "ms_per_step": round(ms, 5),
                     "what": "whole step: store + select (prologue, stream, finish) + attend + merge, all layers"}

    extra = {}
    if w.kind == "mla":
        fl = mla_attend_flops(w, seq, True)
        att_s = stage_ms["attend"] * 1e-3
        extra["mla_attend"] = {"flops": fl, "tflops": round(fl / att_s / 1e12, 1),
                               "mfma_bf16_frac": round(fl / att_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                               "gbps": round((lb["selected_kv"] + lb["q_out_table"]) / att_s / 1e9, 1)}
        ffl = mla_attend_flops(w, seq, False)
        extra["mla_full"] = {"flops": ffl, "tflops": round(ffl / (ms_full * 1e-3) / 1e12, 1),
                             "mfma_bf16_frac": round(ffl / (ms_full * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}

    n_cpu = args.cpu_seqs if args.cpu_seqs >= 0 else (w.batch if w.name == "llama8b_128k" and
                                                       args.scale_format == "fp32" else 0)
    cpu = None
    if n_cpu > 0 and not w.window:
        if args.cpu_threads > 0:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=args.cpu_threads):
                cpu = cpu_baseline(w, case, min(n_cpu, w.batch))
        else:
            cpu = cpu_baseline(w, case, min(n_cpu, w.batch))

    cfg = {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
           "head_dim": w.head_dim, "seq_len": w.seq_len, "page_size": w.page_size, "rank": w.rank,
           "budget": w.budget, "kv_dtype": "bf16",
           "scoring_cache": {"fp32": "fp8 e4m3fn + fp32 scale per token", "e8m0": "fp8 e4m3fn + e8m0 scale byte",
                             "none": "fp8 e4m3fn, no scale", "bf16": "bf16 projected keys, no scale"}[args.scale_format],
           "replicas": n_rep,
           "decode_path": "single launch per layer" if single else "split (prologue, stream, finish, attend, merge)"}
    if w.window:
        cfg.update(layers=w.num_layers, window=w.window, window_layers=list(w.window_layers()))
    res = {
        "metric": METRIC,
        "value": round(1e3 / ms, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded anisotropic keys/queries, 1% planted needles, random page permutation)",
        "config": cfg,
        "roofline": roofline,
        "step_roofline": step_roofline,
        "cpu_baseline": cpu,
        "hbm_gbps": round(total_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": total_bytes,
        "bytes_breakdown": parts,
        "block_median_ms": round(med, 5), "p10_ms": round(p10, 5), "p90_ms": round(p90, 5),
        "graph": graph,
        "decode_paths": paths,
        "hbm_copy_probe_gbps": round(2 * PROBE_BYTES / (probe_ms * 1e-3) / 1e9, 1),
        "full_kv_ms_per_step": round(ms_full, 4),
        "full_kv_gbps": round(full_bytes / (ms_full * 1e-3) / 1e9, 1),
        "speedup_vs_full_kv": round(ms_full / ms, 3),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "gather_free_vs_gather": {
            "attend_ms": round(stage_ms["attend"], 5), "gather_then_attend_ms": round(stage_ms["gather_attend"], 5),
            "ratio": round(stage_ms["gather_attend"] / stage_ms["attend"], 3)},
        "host_wall_ms_per_step": round(wall_ms, 5),
        **extra,
        "context": "pages' own figure: up to 6.43x end-to-end over full KV at 128K on one NVIDIA B200 "
                   "(MLA model, vLLM); not a target",
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
