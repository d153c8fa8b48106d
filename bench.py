#!/usr/bin/env python
"""Benchmark of one JSSA decode step on one MI355X.

A step is one jssa_decode call over the whole batch of one layer: store the
new token's projected key, select (qhat + sampled threshold, FP8 score stream
over every cached token, exact top-B) and gather-free attention with the
split-K merge.  The workload (default: the Llama-3.1-8B-shaped layer at 128K,
batch 8) is synthetic and seeded; its basis M comes from the library's own
calibration (jssa_calib_moments + jssa_basis) on synthetic calibration
sequences.  Inputs are resident in HBM before the timed region; three cache
replicas are rotated so the 256 MB Infinity Cache cannot serve a step from
the previous one.  Also timed: the dense full-KV decode on the same caches
(speedup), each stage alone with HIP events (roofline of the dominant
kernel), and the CPU oracle on a bounded sample (cpu_baseline).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "counters_select_stream_llama8b_128k.json")


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_decode_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, seq_lens, sparse=True):
    """Bytes the method itself must move per step (roofline)."""
    S = w.score_dims
    d, hkv, hq, B = w.head_dim, w.num_kv_heads, w.num_q_heads, w.budget
    io = 2 * w.batch * hq * d * 2 + w.batch * w.pages_per_seq * 4
    if not sparse:
        return sum(n * hkv * 2 * d * 2 for n in seq_lens) + io, {}
    score = sum(n * hkv * (S + 4) for n in seq_lens)
    kv = sum(min(B, n) * hkv * 2 * d * 2 for n in seq_lens)
    idx = w.batch * hkv * B * 4 * 2
    store = w.batch * hkv * (d * 2 + S + 4)
    parts = dict(score=score, selected_kv=kv, indices=idx, q_out_table=io, store=store)
    return sum(parts.values()), parts


def setup(w, device, replicas):
    import numpy as np
    import torch

    import long_context_decode_amd as L
    from synth import make_gqa_calibration, make_gqa_case

    shape = L.shape_for(w)
    # calibration with the library: moments on the GPU, eigenvectors on the host
    qc, kc = make_gqa_calibration(w, 0, device=device)
    T = qc.shape[0]
    gq = torch.zeros((w.num_kv_heads, w.head_dim, w.head_dim), dtype=torch.float32, device=device)
    gk = torch.zeros_like(gq)
    cws = torch.empty(L.calib_workspace_bytes(shape, T), dtype=torch.uint8, device=device)
    L.jssa_calib_moments(shape, qc, kc, gq, gk, cws)
    M = torch.from_numpy(L.jssa_basis(shape, gq.cpu().numpy(), gk.cpu().numpy())).to(device)
    del qc, kc, cws
    case = make_gqa_case(w, device=device, layers=[0])
    lay = case.layers[0]
    n_pages = lay.k_cache.shape[0]
    kp, ks = L.alloc_scoring_cache(shape, n_pages, device)
    # bulk store of every cached position
    P = w.page_size
    bt = case.block_table.long()
    flat_k = lay.k_cache.view(-1, w.num_kv_heads, w.head_dim)
    for b in range(w.batch):
        n = int(case.seq_lens[b])
        for t0 in range(0, n, 1 << 17):
            t = torch.arange(t0, min(n, t0 + (1 << 17)), device=device)
            slots = (bt[b, t // P] * P + t % P).to(torch.int32)
            L.jssa_store(shape, flat_k[slots.long()].contiguous(), slots, M, kp, ks, check_slots=False)
    last = case.seq_lens.long() - 1
    slot_new = (bt[torch.arange(w.batch, device=device), last // P] * P + last % P).to(torch.int32)
    k_new = flat_k[slot_new.long()].contiguous()
    reps = [(kp, ks, lay.k_cache, lay.v_cache)]
    for _ in range(replicas - 1):
        reps.append(tuple(x.clone() for x in reps[0]))
    torch.cuda.synchronize()
    return shape, M, case, reps, k_new, slot_new, case.block_table.to(device), case.seq_lens.to(device)


def time_steps(fn, steps, warmup, n_rep):
    import torch
    for i in range(warmup):
        fn(i % n_rep)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(i % n_rep)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall * 1e3 / steps


def time_stages(stage_fns, steps, n_rep):
    """Average duration of each stage, each bracketed by its own HIP events on the current stream."""
    import torch
    names = list(stage_fns)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
          for _ in range(steps)]
    for i in range(steps):
        for j, n in enumerate(names):
            ev[i][j][0].record()
            stage_fns[n](i % n_rep)
            ev[i][j][1].record()
    torch.cuda.synchronize()
    return {n: sum(ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)) / steps
            for j, n in enumerate(names)}


def cpu_baseline(w, case, n_seqs):
    """The oracle (as is) on host cores: select + attend for n_seqs sequences, all KV heads, scaled to a step."""
    import numpy as np
    import torch
    from oracle import calibrate as ocal
    from oracle import gqa as ogqa
    from synth import bf16_bits, make_gqa_calibration

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    qc, kc = make_gqa_calibration(w, 0, device="cpu")
    m32 = ocal.calibrate(ocal.bf16_to_f64(bf16_bits(qc)), ocal.bf16_to_f64(bf16_bits(kc)), w.group,
                         w.rank).astype(np.float32)
    lay = case.layers[0]
    bt = case.block_table.cpu().numpy()
    q = bf16_bits(lay.q)
    elapsed = 0.0
    for b in range(n_seqs):
        n = int(case.seq_lens[b])
        t = torch.arange(n, device=lay.k_cache.device)
        pg = case.block_table[b].long()[t // w.page_size]
        kr = bf16_bits(lay.k_cache[pg, t % w.page_size])
        vr = bf16_bits(lay.v_cache[pg, t % w.page_size])
        codes, scale = ogqa.store(kr, m32)                       # cache construction: not timed
        t0 = time.perf_counter()
        ogqa.decode_step(q[b], kr, vr, m32, w.budget, w.sm_scale, codes=codes, scale=scale)
        elapsed += time.perf_counter() - t0
    per_step = elapsed * w.batch / n_seqs
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_seqs} of {w.batch} sequences x {w.num_kv_heads} KV heads (score + top-B + attend, "
                      f"fp64 NumPy), {elapsed:.1f} s, scaled x{w.batch / n_seqs:g} to one step"}


def traffic_for(launch_bytes):
    """HBM bytes per dispatch from committed rocprofv3 counters, if they were taken on the current kernel."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    if c.get("source_hash") != _src_hash("select.hip", "common.h"):
        return None
    return c.get("hbm_bytes_per_dispatch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_128k")
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--cpu-seqs", type=int, default=6, help="sequences in the CPU-oracle sample (0: skip)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device copy (reference kernel for counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the JSSA decode path is per-GPU and this build has no multi-GPU mode "
              "(batch and KV heads would shard with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_decode_amd as L
    from synth import WORKLOADS

    w = WORKLOADS[args.workload]
    if w.kind != "gqa" or w.window:
        print(f"workload {w.name}: bench times single-layer GQA workloads", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    shape, M, case, reps, k_new, slot_new, bt, sl = setup(w, dev, args.replicas)
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    q = case.layers[0].q
    seq = [int(x) for x in case.seq_lens.cpu()]
    ws = L.alloc_workspace(shape, dev)
    idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    n_rep = len(reps)

    def step(r):
        kp, ks, kc, vc = reps[r]
        L.jssa_decode(shape, q, k_new, slot_new, M, kp, ks, kc, vc, bt, sl, idx, w.sm_scale, out, ws)

    def full(r):
        _, _, kc, vc = reps[r]
        L.jssa_full_decode(shape, q, kc, vc, bt, sl, 0, w.sm_scale, out, ws)

    ms, wall_ms = time_steps(step, args.steps, args.warmup, n_rep)
    ms_full, _ = time_steps(full, max(10, args.steps // 10), max(2, args.warmup // 4), n_rep)

    stages = {
        "store": lambda r: L.jssa_store(shape, k_new, slot_new, M, reps[r][0], reps[r][1], check_slots=False),
        "select_prologue": lambda r: L.jssa_select(shape, q, M, reps[r][0], reps[r][1], bt, sl, idx, ws,
                                                   stages=L.STAGE_PROLOGUE),
        "select_stream": lambda r: L.jssa_select(shape, q, M, reps[r][0], reps[r][1], bt, sl, idx, ws,
                                                 stages=L.STAGE_STREAM),
        "select_finish": lambda r: L.jssa_select(shape, q, M, reps[r][0], reps[r][1], bt, sl, idx, ws,
                                                 stages=L.STAGE_FINISH),
        "attend": lambda r: L.jssa_attend(shape, q, reps[r][2], reps[r][3], bt, sl, idx, w.sm_scale, out, ws),
    }
    for i in range(3):
        for f in stages.values():
            f(i % n_rep)
    stage_ms = time_stages(stages, args.steps, n_rep)

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    total_bytes, parts = algorithmic_bytes(w, seq, True)
    full_bytes, _ = algorithmic_bytes(w, seq, False)
    stream_bytes = parts["score"]
    achieved = stream_bytes / (stage_ms["select_stream"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_for(stream_bytes),
                "kernel": "select_stream (FP8 score stream + candidate compaction)",
                "bytes_per_launch": stream_bytes, "avg_launch_ms": round(stage_ms["select_stream"], 5)}

    cpu = None
    if args.cpu_seqs > 0:
        cpu = cpu_baseline(w, case, min(args.cpu_seqs, w.batch))

    res = {
        "metric": "decode attn-stage steps/s @128K; HBM GB/s vs peak; speedup vs full-KV decode",
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
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "seq_len": w.seq_len,
                   "page_size": w.page_size, "rank": w.rank, "budget": w.budget, "kv_dtype": "bf16",
                   "scoring_cache": "fp8 e4m3fn + fp32 scale", "replicas": n_rep},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_gbps": round(total_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": total_bytes,
        "bytes_breakdown": parts,
        "full_kv_ms_per_step": round(ms_full, 4),
        "full_kv_gbps": round(full_bytes / (ms_full * 1e-3) / 1e9, 1),
        "speedup_vs_full_kv": round(ms_full / ms, 3),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "host_wall_ms_per_step": round(wall_ms, 5),
        "context": "pages' own figure: up to 6.43x end-to-end over full KV at 128K on one NVIDIA B200 "
                   "(MLA model, vLLM); not a target",
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
