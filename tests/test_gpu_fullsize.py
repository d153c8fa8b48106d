"""Parity at the benchmark workloads' full sizes, in the launch configuration bench.py times.

Each case builds the whole workload on the GPU (synthetic generator), stores every
cached position with jssa_store, runs one jssa_decode step (which stores the new
token again) and the dense jssa_full_decode baseline through the C ABI with the
workload's own shape (so the same split and chunk plans), then checks every
(sequence, KV head) pair against the oracle, each pair in full (pairs in a thread
pool on the host: the oracle is plain NumPy and releases the GIL in its array work):

* store: the GPU codes and scales of every position of the pair against the
  oracle's (code distance <= 1, <= 0.1 % of codes differ; scales <= 1e-5 relative);
* select: the GPU's top-B set against the oracle's top-B on the GPU's own codes
  (equal sizes; differences only within 1e-5 |tau| of the B-th score);
* attend / dense: the pair's query heads against fp64 attention over the GPU's set
  and over all positions (or the window).

The basis M is the oracle's own calibration of the layer (an input to both sides).
"""
import concurrent.futures as cf
import functools
import os

import numpy as np
import pytest
import torch

import long_context_decode_amd as L
from oracle import calibrate as ocal
from oracle import gqa as ogqa
from oracle import mla as omla
from synth import WORKLOADS, bf16_bits, make_gqa_calibration, make_gqa_case, make_mla_calibration, make_mla_case
from util import check_attention, check_codes, check_selection

pytestmark = pytest.mark.gpu
DEV = "cuda"


@functools.lru_cache(maxsize=None)
def _gqa_basis(name, layer):
    w = WORKLOADS[name]
    q, k = make_gqa_calibration(w, layer)
    return ocal.calibrate(ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(k)), w.group,
                          w.rank).astype(np.float32)


@functools.lru_cache(maxsize=None)
def _mla_basis(name):
    w = WORKLOADS[name]
    chunks = ((ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(l)))
              for q, l in make_mla_calibration(w, chunk=1024))
    return omla.calibrate(chunks, w.latent_dim, w.rank)[0].astype(np.float32)


def _bulk_store(w, shape, flat, bt, sl, M, kp, ks):
    P = w.page_size
    btl = bt.long()
    for b in range(w.batch):
        n = int(sl[b])
        for t0 in range(0, n, 1 << 17):
            t = torch.arange(t0, min(n, t0 + (1 << 17)), device=DEV)
            slots = (btl[b, t // P] * P + t % P).to(torch.int32)
            L.jssa_store(shape, flat[slots.long()].contiguous(), slots, M, kp, ks, check_slots=False)


def _logical(cache, bt_row, n, P):
    """Rows of positions 0..n-1 of one sequence from a paged cache [pages, P, ...] (on the GPU)."""
    t = torch.arange(n, device=cache.device)
    return cache[bt_row.long()[t // P], t % P]


def _pair_codes(kp, ks, bt_row, n, P, h):
    """GPU codes [n, S] (BF16 keys: [n, 2S] bytes) and scales [n] (None without a scale array) of KV head h
    of one sequence from the piece-major scoring cache."""
    npg = -(-n // P)
    pages = bt_row.long()[:npg]
    c = kp[pages, h]                                  # [npg, pieces, P, 16]
    c = c.permute(0, 2, 1, 3).reshape(npg * P, -1)[:n]
    s = None if ks is None else ks[pages, h].reshape(-1)[:n].cpu().numpy()
    return c.cpu().numpy(), s


def _run_gqa(name, layer, window_layer, fmt="fp32", full=True):
    w = WORKLOADS[name]
    shape = L.shape_for(w, scale_format=L.SCALE_FORMATS[fmt])
    case = make_gqa_case(w, device=DEV, layers=[layer])
    lay = case.layers[layer]
    bt, sl = case.block_table, case.seq_lens
    out_f = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lse_f = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    ws = L.alloc_workspace(shape)
    window = w.window if window_layer else 0
    if full:
        L.jssa_full_decode(shape, lay.q, lay.k_cache, lay.v_cache, bt, sl, window, w.sm_scale, out_f, ws, lse_f)
    res = dict(w=w, case=case, lay=lay, out_f=out_f.float().cpu().numpy(), lse_f=lse_f.cpu().numpy())
    if window_layer:
        return res
    m32 = _gqa_basis(name, layer)
    M = torch.from_numpy(m32).to(DEV)
    kp, ks = L.alloc_scoring_cache(shape, lay.k_cache.shape[0], DEV)
    flat = lay.k_cache.view(-1, w.num_kv_heads, w.head_dim)
    _bulk_store(w, shape, flat, bt, sl, M, kp, ks)
    P = w.page_size
    last = sl.long() - 1
    slot_new = (bt.long()[torch.arange(w.batch, device=DEV), last // P] * P + last % P).to(torch.int32)
    k_new = flat[slot_new.long()].contiguous()
    idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV)
    out = torch.empty_like(out_f)
    lse = torch.empty_like(lse_f)
    L.jssa_decode(shape, lay.q, k_new, slot_new, M, kp, ks, lay.k_cache, lay.v_cache, bt, sl, idx, w.sm_scale, out,
                  ws, lse)
    torch.cuda.synchronize()
    res.update(m32=m32, kp=kp, ks=ks, idx=idx.cpu().numpy(), out=out.float().cpu().numpy(), lse=lse.cpu().numpy())
    return res


def _pairs(w):
    return [(0, 0), (w.batch // 2, w.num_kv_heads - 1), (w.batch - 1, w.num_kv_heads // 2)]


def _all_pairs(w):
    return [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]


def _pool_run(fn, items, workers=None):
    """fn over items in host threads; the first failure is re-raised with its item."""
    workers = workers or min(16, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {ex.submit(fn, it): it for it in items}
        for f in cf.as_completed(futs):
            try:
                f.result()
            except Exception as e:  # noqa: BLE001
                raise AssertionError(f"case {futs[f]}: {e}") from e


def _host_rows(cache, bt_row, n, P):
    """bf16 bits of positions 0..n-1 of one sequence, all KV heads: [n, Hkv, d] (or [n, 576] for MLA)."""
    return bf16_bits(_logical(cache, bt_row, n, P))


def _check_gqa_pair(w, r, q, rows_k, rows_v, codes_all, scales_all, b, h, window=None):
    """Every check of one (sequence, KV head) pair of a global layer (window None) or a window layer."""
    G = w.group
    rk, rv = rows_k[b][:, h], rows_v[b][:, h]
    n = rk.shape[0]
    if window is not None:
        sel_w = ogqa.window_indices(n, window)
        for g in range(G):
            j = h * G + g
            o, l = ogqa.attend(q[b, j], rk[sel_w], rv[sel_w], w.sm_scale)
            check_attention(r["out_f"][b, j], o)
            assert abs(r["lse_f"][b, j] - l) <= 1e-3
        return
    codes, scale = codes_all[b][:, h], scales_all[b][:, h]
    oc, os_ = ogqa.store(rk[:, None, :], r["m32"][h:h + 1])
    check_codes(codes, oc[:, 0])
    assert np.all(np.abs(scale.astype(np.float64) - os_[:, 0]) <= 1e-5 * np.abs(os_[:, 0]))
    qhat = ogqa.project_query(q[b], r["m32"], G)[h]
    sc = ogqa.scores(qhat, codes, scale)
    oidx, tau = ogqa.select_topb(sc, w.budget)
    check_selection(r["idx"][b, h], oidx, sc, tau)
    sel = r["idx"][b, h][r["idx"][b, h] >= 0]
    for g in range(G):
        j = h * G + g
        o, l = ogqa.attend(q[b, j], rk[sel], rv[sel], w.sm_scale)
        check_attention(r["out"][b, j], o)
        assert abs(r["lse"][b, j] - l) <= 1e-3
        if "out_f" in r:
            o, l = ogqa.attend(q[b, j], rk, rv, w.sm_scale)
            check_attention(r["out_f"][b, j], o)
            assert abs(r["lse_f"][b, j] - l) <= 1e-3


def _host_layer(w, case, lay, r=None):
    """Per sequence: K and V rows of every KV head and, for a global layer, the GPU's codes and scales."""
    P = w.page_size
    rows_k, rows_v, codes, scales = [], [], [], []
    for b in range(w.batch):
        n = int(case.seq_lens[b])
        rows_k.append(_host_rows(lay.k_cache, case.block_table[b], n, P))
        rows_v.append(_host_rows(lay.v_cache, case.block_table[b], n, P))
        if r is not None and "kp" in r:
            ch = [_pair_codes(r["kp"], r["ks"], case.block_table[b], n, P, h) for h in range(w.num_kv_heads)]
            codes.append(np.stack([c for c, _ in ch], 1))
            scales.append(np.stack([s for _, s in ch], 1))
    return rows_k, rows_v, codes, scales


@pytest.mark.parametrize("name,layer", [("llama8b_128k", 0), ("llama8b_32k", 0)])
def test_fullsize_gqa_decode_step(name, layer):
    """The layer at its benchmark shape and launch plan: bulk store, one decode step (new token stored inside
    it) and the dense baseline; every (sequence, KV head) pair checked in full against the oracle."""
    r = _run_gqa(name, layer, window_layer=False)
    w, case, lay = r["w"], r["case"], r["lay"]
    q = bf16_bits(lay.q)
    rows_k, rows_v, codes, scales = _host_layer(w, case, lay, r)
    _pool_run(lambda bh: _check_gqa_pair(w, r, q, rows_k, rows_v, codes, scales, *bh), _all_pairs(w))
    del r
    torch.cuda.empty_cache()


def test_fullsize_hybrid_stack_step():
    """The 6-layer hybrid stack as one benchmark step at its full shape: the sliding-window layers through
    jssa_full_decode, the global layers through jssa_decode (each with its own basis, the new token stored
    inside the step), back to back on one stream; then every (sequence, KV head) pair of every layer against
    the oracle (window layers: fp64 attention over the window; global layers: codes, selection on the GPU's
    codes, attention over the GPU's set)."""
    name = "hybrid_64k"
    w = WORKLOADS[name]
    shape = L.shape_for(w)
    case = make_gqa_case(w, device=DEV, layers=list(range(w.num_layers)))
    bt, sl, P = case.block_table, case.seq_lens, w.page_size
    ws = L.alloc_workspace(shape)
    last = sl.long() - 1
    res = {}
    for l in range(w.num_layers):                         # the caches and scoring caches first
        lay = case.layers[l]
        if l in w.window_layers():
            res[l] = dict(window=True)
            continue
        m32 = _gqa_basis(name, l)
        M = torch.from_numpy(m32).to(DEV)
        kp, ks = L.alloc_scoring_cache(shape, lay.k_cache.shape[0], DEV)
        flat = lay.k_cache.view(-1, w.num_kv_heads, w.head_dim)
        _bulk_store(w, shape, flat, bt, sl, M, kp, ks)
        slot_new = (bt.long()[torch.arange(w.batch, device=DEV), last // P] * P + last % P).to(torch.int32)
        res[l] = dict(window=False, m32=m32, M=M, kp=kp, ks=ks, slot_new=slot_new,
                      k_new=flat[slot_new.long()].contiguous())
    torch.cuda.synchronize()
    outs = {}
    for l in range(w.num_layers):                         # the step: all layers back to back
        lay, st = case.layers[l], res[l]
        out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
        if st["window"]:
            L.jssa_full_decode(shape, lay.q, lay.k_cache, lay.v_cache, bt, sl, w.window, w.sm_scale, out, ws, lse)
            outs[l] = (out, lse, None)
        else:
            idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV)
            L.jssa_decode(shape, lay.q, st["k_new"], st["slot_new"], st["M"], st["kp"], st["ks"], lay.k_cache,
                          lay.v_cache, bt, sl, idx, w.sm_scale, out, ws, lse)
            outs[l] = (out, lse, idx)
    torch.cuda.synchronize()
    for l in range(w.num_layers):
        lay, st = case.layers[l], res[l]
        out, lse, idx = outs[l]
        r = dict(w=w, m32=st.get("m32"), kp=st.get("kp"), ks=st.get("ks"))
        q = bf16_bits(lay.q)
        if st["window"]:
            r.update(out_f=out.float().cpu().numpy(), lse_f=lse.cpu().numpy())
            rows_k, rows_v, _, _ = _host_layer(w, case, lay)
            _pool_run(lambda bh: _check_gqa_pair(w, r, q, rows_k, rows_v, None, None, *bh, window=w.window),
                      _all_pairs(w))
        else:
            r.update(out=out.float().cpu().numpy(), lse=lse.cpu().numpy(), idx=idx.cpu().numpy())
            rows_k, rows_v, codes, scales = _host_layer(w, case, lay, r)
            _pool_run(lambda bh: _check_gqa_pair(w, r, q, rows_k, rows_v, codes, scales, *bh), _all_pairs(w))
        del rows_k, rows_v
    del res, outs, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["e8m0", "none", "bf16"])
def test_fullsize_scale_formats(fmt):
    """The 128K layer at its benchmark shape with the other scoring-cache formats: bulk store, one decode step
    (new token stored inside it); on two (sequence, KV head) pairs the selection against the oracle's top-B on
    the GPU's own codes and the attention against fp64 attention over the GPU's set."""
    r = _run_gqa("llama8b_128k", 0, window_layer=False, fmt=fmt, full=False)
    w, case, lay = r["w"], r["case"], r["lay"]
    q = bf16_bits(lay.q)
    G, P = w.group, w.page_size
    for b, h in _pairs(w)[:2]:
        n = int(case.seq_lens[b])
        rk = bf16_bits(_logical(lay.k_cache, case.block_table[b], n, P)[:, h])
        rv = bf16_bits(_logical(lay.v_cache, case.block_table[b], n, P)[:, h])
        codes, scale = _pair_codes(r["kp"], r["ks"], case.block_table[b], n, P, h)
        qhat = ogqa.project_query(q[b], r["m32"], G)[h]
        sc = ogqa.scores(qhat, codes, scale, fmt)
        oidx, tau = ogqa.select_topb(sc, w.budget)
        check_selection(r["idx"][b, h], oidx, sc, tau)
        sel = r["idx"][b, h][r["idx"][b, h] >= 0]
        for g in range(G):
            j = h * G + g
            o, l = ogqa.attend(q[b, j], rk[sel], rv[sel], w.sm_scale)
            check_attention(r["out"][b, j], o)
            assert abs(r["lse"][b, j] - l) <= 1e-3
    del r
    torch.cuda.empty_cache()


def test_fullsize_mla_decode_step():
    name = "mla_128k"
    w = WORKLOADS[name]
    shape = L.shape_for(w)
    case = make_mla_case(w, device=DEV)
    bt, sl, P = case.block_table, case.seq_lens, w.page_size
    m32 = _mla_basis(name)
    M = torch.from_numpy(m32).to(DEV)
    kp, ks = L.alloc_scoring_cache(shape, case.latent.shape[0], DEV)
    flat = case.latent.view(-1, w.head_dim)
    _bulk_store(w, shape, flat, bt, sl, M, kp, ks)
    last = sl.long() - 1
    slot_new = (bt.long()[torch.arange(w.batch, device=DEV), last // P] * P + last % P).to(torch.int32)
    k_new = flat[slot_new.long()].contiguous()
    ws = L.alloc_workspace(shape)
    idx = torch.empty((w.batch, 1, w.budget), dtype=torch.int32, device=DEV)
    out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    out_f, lse_f = torch.empty_like(out), torch.empty_like(lse)
    L.jssa_decode(shape, case.q, k_new, slot_new, M, kp, ks, case.latent, None, bt, sl, idx, w.sm_scale, out, ws, lse)
    L.jssa_full_decode(shape, case.q, case.latent, None, bt, sl, 0, w.sm_scale, out_f, ws, lse_f)
    torch.cuda.synchronize()
    gidx, got, glse = idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    gotf, glsef = out_f.float().cpu().numpy(), lse_f.cpu().numpy()
    q = bf16_bits(case.q)
    host = []
    for b in range(w.batch):
        n = int(sl[b])
        host.append((_host_rows(case.latent, bt[b], n, P), *_pair_codes(kp, ks, bt[b], n, P, 0)))

    def check(b):                                      # every sequence, in host threads
        rows, codes, scale = host[b]
        oc, os_ = omla.store(rows, m32)
        check_codes(codes, oc)
        assert np.all(np.abs(scale.astype(np.float64) - os_) <= 1e-5 * np.abs(os_))
        qhat = omla.project_query(q[b], m32)
        sc = ogqa.scores(qhat, codes, scale)
        oidx, tau = ogqa.select_topb(sc, w.budget)
        check_selection(gidx[b, 0], oidx, sc, tau)
        o, l = omla.attend(q[b], rows[gidx[b, 0][gidx[b, 0] >= 0]], w.sm_scale)
        check_attention(got[b], o)
        assert np.all(np.abs(glse[b] - l) <= 1e-3)
        o, l = omla.attend(q[b], rows, w.sm_scale)
        check_attention(gotf[b], o)
        assert np.all(np.abs(glsef[b] - l) <= 1e-3)

    _pool_run(check, list(range(w.batch)), workers=4)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["e8m0", "bf16"])
def test_fullsize_mla_scale_formats(fmt):
    """The 128K MLA layer at its benchmark shape with the one-byte scale and with BF16 keys: bulk store, one
    decode step; on two sequences the selection against the oracle's top-B on the GPU's own codes and the
    attention against fp64 attention over the GPU's set."""
    name = "mla_128k"
    w = WORKLOADS[name]
    shape = L.shape_for(w, scale_format=L.SCALE_FORMATS[fmt])
    case = make_mla_case(w, device=DEV)
    bt, sl, P = case.block_table, case.seq_lens, w.page_size
    m32 = _mla_basis(name)
    M = torch.from_numpy(m32).to(DEV)
    kp, ks = L.alloc_scoring_cache(shape, case.latent.shape[0], DEV)
    flat = case.latent.view(-1, w.head_dim)
    _bulk_store(w, shape, flat, bt, sl, M, kp, ks)
    last = sl.long() - 1
    slot_new = (bt.long()[torch.arange(w.batch, device=DEV), last // P] * P + last % P).to(torch.int32)
    k_new = flat[slot_new.long()].contiguous()
    idx = torch.empty((w.batch, 1, w.budget), dtype=torch.int32, device=DEV)
    out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    L.jssa_decode(shape, case.q, k_new, slot_new, M, kp, ks, case.latent, None, bt, sl, idx, w.sm_scale, out,
                  L.alloc_workspace(shape), lse)
    torch.cuda.synchronize()
    gidx, got, glse = idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    q = bf16_bits(case.q)
    for b in (0, w.batch - 1):
        n = int(sl[b])
        rows = bf16_bits(_logical(case.latent, bt[b], n, P))
        codes, scale = _pair_codes(kp, ks, bt[b], n, P, 0)
        sc = ogqa.scores(omla.project_query(q[b], m32), codes, scale, fmt)
        oidx, tau = ogqa.select_topb(sc, w.budget)
        check_selection(gidx[b, 0], oidx, sc, tau)
        o, l = omla.attend(q[b], rows[gidx[b, 0][gidx[b, 0] >= 0]], w.sm_scale)
        check_attention(got[b], o)
        assert np.all(np.abs(glse[b] - l) <= 1e-3)
    torch.cuda.empty_cache()
