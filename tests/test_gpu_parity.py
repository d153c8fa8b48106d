"""GPU parity of every stage of the HIP path against the CPU oracle.

Stage-wise: each GPU stage is fed the oracle's output of the previous stage
(never the other way round), and compared with the oracle on the same input:
  store   codes within 1 ulp on <= 0.1% of entries, scales within 1e-5 relative;
  select  equal sets except tokens whose oracle score is within 1e-5 |tau| of
          the B-th score (tau, on the same codes);
  attend  bf16 output within max-abs 2e-2 and mean-abs 2e-3 of fp64 attention
          over the same set; lse within 1e-3.
"""
import functools

import numpy as np
import pytest
import torch

from oracle import calibrate as ocal
from oracle import fp8
from oracle import gqa as ogqa
from oracle import mla as omla
from synth import WORKLOADS, bf16_bits, make_gqa_calibration, make_gqa_case, make_mla_calibration, make_mla_case
from synth.workloads import population_basis

from util import (CodeTally, check_attention, check_codes, check_scores, check_selection, pack_kp, slots_for,
                  unpack_kp)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import long_context_decode_amd as L

DEV = "cuda"


def _w(base, **kw):
    return WORKLOADS[base].scaled(**kw) if kw else WORKLOADS[base]


# GQA cases: (name, workload, ragged)
GQA_CASES = {
    "tiny": (_w("tiny"), False),
    "mid_sampled": (_w("tiny", name="mid", model="test", batch=3, seq_len=40000, budget=512), True),
    "d256_r48": (_w("hybrid_64k", name="h", model="test", batch=2, num_kv_heads=4, num_q_heads=8, seq_len=20000,
                    calib_seqs=2, calib_len=1024), True),
    "short_ctx": (_w("tiny", name="short", model="test", batch=2, seq_len=300, budget=512), True),
    "page32_g8": (_w("tiny", name="p32", model="test", batch=2, num_q_heads=16, num_kv_heads=2, page_size=32,
                     seq_len=9000, budget=1000), True),
    # the largest budget (4096): the sampled threshold aims at 6144 candidates, under 2B
    "max_budget": (_w("tiny", name="maxb", model="test", batch=2, seq_len=40000, budget=4096), True),
    # 12325, 12288 and 12251 tokens: sampled threshold above the 12288-token candidate capacity, every
    # token a candidate at and below it
    "cap_edge": (_w("tiny", name="capedge", model="test", batch=3, seq_len=12325, budget=1024), True),
}


@functools.lru_cache(maxsize=None)
def _basis(w):
    q, k = make_gqa_calibration(w, 0)
    m = ocal.calibrate(ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(k)), w.group, w.rank)
    return m.astype(np.float32)


@functools.lru_cache(maxsize=None)
def _gqa(name):
    """Case data + oracle store on every sequence (logical rows and codes)."""
    w, ragged = GQA_CASES[name]
    case = make_gqa_case(w, ragged=ragged)
    lay = case.layers[0]
    m32 = _basis(w)
    bt = case.block_table.numpy()
    sl = case.seq_lens.numpy()
    kc, vc = bf16_bits(lay.k_cache), bf16_bits(lay.v_cache)
    rows_k = [ogqa.logical_rows(kc, bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    rows_v = [ogqa.logical_rows(vc, bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    stored = [ogqa.store(rk, m32) for rk in rows_k]
    return w, case, m32, rows_k, rows_v, stored


def _upload(w, case, m32, stored):
    shape = L.shape_for(w)
    n_pages = case.layers[0].k_cache.shape[0]
    kp, ks = pack_kp([c for c, _ in stored], [s for _, s in stored], case.block_table.numpy(), w.page_size,
                     n_pages, case.seq_lens.numpy())
    return shape, torch.from_numpy(kp).to(DEV), torch.from_numpy(ks).to(DEV), torch.from_numpy(m32).to(DEV)


# ----------------------------------------------------------------------------- FP8 conversions on gfx950

def test_hw_fp8_encode_matches_oracle_on_every_code_and_midpoint():
    """M = [I_r | 0], rows led by 448: the scale is exactly 1, so codes = E4M3FN(k) for every finite
    code value and every midpoint between neighbours (all exact in bf16)."""
    d, r = 128, 32
    vals = fp8.decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    pool = np.concatenate([vals, -vals, mids, -mids])
    rows = []
    for i in range(0, len(pool), r - 1):
        row = np.zeros(d)
        chunk = pool[i:i + r - 1]
        row[0] = 448.0
        row[1:1 + len(chunk)] = chunk
        rows.append(row)
    k = torch.tensor(np.array(rows)[:, None, :], dtype=torch.bfloat16)
    T = k.shape[0]
    m = np.zeros((1, r, d), np.float32)
    m[0, :, :r] = np.eye(r)
    page = 16
    n_pages = -(-T // page)
    shape = L.make_shape(0, 1, 1, 1, d, page, n_pages, r, 16)
    kp, ks = L.alloc_scoring_cache(shape, n_pages, DEV)
    slot = torch.arange(T, dtype=torch.int32, device=DEV)
    L.jssa_store(shape, k.to(DEV), slot, torch.from_numpy(m).to(DEV), kp, ks)
    codes, scales = unpack_kp(kp.cpu().numpy(), ks.cpu().numpy(), np.arange(n_pages), T, page)
    ref_codes, ref_scales = ogqa.store(bf16_bits(k), m)
    assert np.all(scales == 1.0)
    assert np.array_equal(fp8.signed_magnitude(codes), fp8.signed_magnitude(ref_codes))


def test_hw_fp8_decode_exact_on_every_code():
    """Scores with qhat = e_3 and unit scales are exactly dec(code_3): checks the hardware decode of all codes."""
    d, r, page = 128, 16, 16
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    T = len(codes)
    n_pages = -(-T // page)
    logical = np.zeros((T, 1, r), np.uint8)
    logical[:, 0, 3] = codes
    logical[:, 0, 7] = 0x38                                     # other elements do not matter
    kp, ks = pack_kp([logical], [np.ones((T, 1), np.float32)], np.arange(n_pages)[None], page, n_pages, [T])
    m = np.zeros((1, r, d), np.float32)
    m[0, :, :r] = np.eye(r)
    q = torch.zeros((1, 1, d), dtype=torch.bfloat16)
    q[0, 0, 3] = 1.0
    shape = L.make_shape(0, 1, 1, 1, d, page, n_pages, r, 16)
    scores = torch.full((1, 1, n_pages * page), np.nan, dtype=torch.float32, device=DEV)
    idx = torch.empty((1, 1, 16), dtype=torch.int32, device=DEV)
    L.jssa_select(shape, q.to(DEV), torch.from_numpy(m).to(DEV), torch.from_numpy(kp).to(DEV),
                  torch.from_numpy(ks).to(DEV), torch.arange(n_pages, dtype=torch.int32, device=DEV)[None],
                  torch.tensor([T], dtype=torch.int32, device=DEV), idx, L.alloc_workspace(shape), scores)
    got = scores.cpu().numpy()[0, 0, :T].astype(np.float64)
    ref = fp8.decode(codes)
    ref = np.where(ref == 0, 0.0, ref)
    assert np.array_equal(got, ref)
    # top-16 of the decoded values, lowest position first among equal values
    want, _ = ogqa.select_topb(ref, 16)
    assert np.array_equal(idx.cpu().numpy()[0, 0], want)


# ----------------------------------------------------------------------------- store

@pytest.mark.parametrize("name", ["tiny", "d256_r48", "page32_g8"])
def test_store_parity(name):
    w, case, m32, rows_k, _, stored = _gqa(name)
    shape = L.shape_for(w)
    n_pages = case.layers[0].k_cache.shape[0]
    kp, ks = L.alloc_scoring_cache(shape, n_pages, DEV)
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    slots, who = slots_for(bt, sl, w.page_size)
    k_new = torch.from_numpy(np.concatenate(rows_k).view(np.int16)).view(torch.bfloat16)
    L.jssa_store(shape, k_new.to(DEV), torch.from_numpy(slots).to(DEV), torch.from_numpy(m32).to(DEV), kp, ks)
    kp_h, ks_h = kp.cpu().numpy(), ks.cpu().numpy()
    fracs = []
    for b in range(w.batch):
        c, s = unpack_kp(kp_h, ks_h, bt[b], int(sl[b]), w.page_size)
        fracs.append(check_codes(c, stored[b][0]))
        rel = np.abs(s.astype(np.float64) - stored[b][1]) / np.maximum(stored[b][1], 1e-30)
        assert rel.max() <= 1e-5
    print(f"{name}: differing codes {max(fracs):.2e}")


def test_store_skips_negative_slots_and_zero_rows():
    w = _w("tiny")
    shape = L.shape_for(w)
    kp, ks = L.alloc_scoring_cache(shape, 4, DEV)
    kp.fill_(0xAB)
    ks.fill_(7.0)
    k_new = torch.zeros((3, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    slot = torch.tensor([5, -1, 17], dtype=torch.int32, device=DEV)
    m = torch.from_numpy(_basis(w)).to(DEV)
    L.jssa_store(shape, k_new, slot, m, kp, ks)
    c, s = unpack_kp(kp.cpu().numpy(), ks.cpu().numpy(), np.arange(4), 64, w.page_size)
    assert np.all(c[5] == 0) and np.all(s[5] == 0) and np.all(c[17] == 0) and np.all(s[17] == 0)
    untouched = [t for t in range(64) if t not in (5, 17)]
    assert np.all(c[untouched] == 0xAB) and np.all(s[untouched] == 7.0)


def test_store_of_no_tokens_changes_nothing():
    """T = 0: the call succeeds and launches nothing; the scoring cache and its scales keep their bytes."""
    w = _w("tiny")
    shape = L.shape_for(w)
    kp, ks = L.alloc_scoring_cache(shape, 4, DEV)
    kp.fill_(0xAB)
    ks.fill_(7.0)
    k_new = torch.zeros((0, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    slot = torch.zeros((0,), dtype=torch.int32, device=DEV)
    L.jssa_store(shape, k_new, slot, torch.from_numpy(_basis(w)).to(DEV), kp, ks)
    torch.cuda.synchronize()
    assert bool((kp == 0xAB).all()) and bool((ks == 7.0).all())


# ----------------------------------------------------------------------------- select

def _run_select(name, mode=0):
    w, case, m32, rows_k, _, stored = _gqa(name)
    shape, kp, ks, M = _upload(w, case, m32, stored)
    shape.select_mode = mode
    maxn = shape.max_pages_per_seq * shape.page_size
    scores = torch.zeros((w.batch, w.num_kv_heads, maxn), dtype=torch.float32, device=DEV)
    idx = torch.full((w.batch, w.num_kv_heads, w.budget), -7, dtype=torch.int32, device=DEV)
    L.jssa_select(shape, case.layers[0].q.to(DEV), M, kp, ks, case.block_table.to(DEV), case.seq_lens.to(DEV), idx,
                  L.alloc_workspace(shape), scores)
    return w, case, m32, stored, idx.cpu().numpy(), scores.cpu().numpy()


@pytest.mark.parametrize("name", list(GQA_CASES))
@pytest.mark.parametrize("mode", [0, 1])
def test_select_parity(name, mode):
    w, case, m32, stored, gidx, gsc = _run_select(name, mode)
    q = bf16_bits(case.layers[0].q)
    exempt, worst = 0, 0.0
    for b in range(w.batch):
        n = int(case.seq_lens[b])
        qhat = ogqa.project_query(q[b], m32, w.group)
        for h in range(w.num_kv_heads):
            s = ogqa.scores(qhat[h], stored[b][0][:, h], stored[b][1][:, h])
            oidx, tau = ogqa.select_topb(s, w.budget)
            if n == 0:
                assert np.all(gidx[b, h] == -1)
                continue
            exempt += check_selection(gidx[b, h], oidx, s, tau)
            err = check_scores(gsc[b, h, :n], qhat[h], stored[b][0][:, h], stored[b][1][:, h], s)
            worst = max(worst, err / abs(tau))
    print(f"{name} mode {mode}: exempt {exempt}, max score err / |tau| {worst:.2e} (reported)")


def test_select_needles_and_determinism():
    w, case, m32, stored, gidx, _ = _run_select("mid_sampled")
    for (b, h), pos in case.layers[0].needles.items():
        assert set(pos.tolist()) <= set(gidx[b, h].tolist())
    _, _, _, _, gidx2, _ = _run_select("mid_sampled")
    assert np.array_equal(gidx, gidx2)


# ----------------------------------------------------------------------------- attend

@pytest.mark.parametrize("name", ["tiny", "mid_sampled", "d256_r48", "short_ctx", "page32_g8", "max_budget",
                                  "cap_edge"])
def test_attend_parity(name):
    w, case, m32, rows_k, rows_v, stored = _gqa(name)
    q = bf16_bits(case.layers[0].q)
    B = w.budget
    idx = np.full((w.batch, w.num_kv_heads, B), -1, np.int32)
    for b in range(w.batch):
        qhat = ogqa.project_query(q[b], m32, w.group)
        for h in range(w.num_kv_heads):
            s = ogqa.scores(qhat[h], stored[b][0][:, h], stored[b][1][:, h])
            idx[b, h], _ = ogqa.select_topb(s, B)
    shape = L.shape_for(w)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    lay = case.layers[0]
    L.jssa_attend(shape, lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV), case.block_table.to(DEV),
                  case.seq_lens.to(DEV), torch.from_numpy(idx).to(DEV), w.sm_scale, out, L.alloc_workspace(shape), lse)
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    errs = []
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            j0 = h * w.group
            o, l = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:, h], rows_v[b][:, h], idx[b, h], w.sm_scale)
            errs.append(check_attention(got[b, j0:j0 + w.group], o))
            fin = np.isfinite(l)
            assert np.array_equal(np.isfinite(glse[b, j0:j0 + w.group]), fin)
            assert np.all(np.abs(glse[b, j0:j0 + w.group][fin] - l[fin]) <= 1e-3)
    print(f"{name}: max abs {max(e[0] for e in errs):.2e}, mean abs {max(e[1] for e in errs):.2e}")


@pytest.mark.parametrize("name,window", [("tiny", 0), ("tiny", 1024), ("d256_r48", 0), ("d256_r48", 1000),
                                         ("short_ctx", 100), ("page32_g8", 0),
                                         ("short_ctx", 1),       # a single position
                                         ("short_ctx", 5000)])   # wider than every sequence: all positions
def test_full_decode_parity(name, window):
    w, case, m32, rows_k, rows_v, _ = _gqa(name)
    q = bf16_bits(case.layers[0].q)
    shape = L.shape_for(w)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    lay = case.layers[0]
    L.jssa_full_decode(shape, lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV), case.block_table.to(DEV),
                       case.seq_lens.to(DEV), window, w.sm_scale, out, L.alloc_workspace(shape), lse)
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(w.batch):
        n = int(case.seq_lens[b])
        sel = ogqa.window_indices(n, window)
        for h in range(w.num_kv_heads):
            j0 = h * w.group
            o, l = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:, h], rows_v[b][:, h], sel, w.sm_scale)
            check_attention(got[b, j0:j0 + w.group], o)
            assert np.all(np.abs(glse[b, j0:j0 + w.group] - l) <= 1e-3)


@pytest.mark.parametrize("kw,window", [
    # 129 pages of 16 at batch 8 and 8 KV heads: the 2048-token window takes 8 splits, the whole capacity 5
    (dict(batch=8, num_q_heads=32, num_kv_heads=8, seq_len=2064, budget=256), 2048),
    # 257 pages at batch 4, G = 1: 16 splits for the 4096-token window against 9
    (dict(batch=4, num_q_heads=8, num_kv_heads=8, seq_len=4112, budget=1), 4096),
])
def test_full_decode_window_plan_beyond_full_plan(kw, window):
    """A sliding window whose split plan has more splits than the whole-capacity plan (the workspace's
    partials are sized for the larger one): every query head against fp64 attention over the window."""
    w = _w("tiny", name="winsplit", model="test", **kw)
    case = make_gqa_case(w)
    lay = case.layers[0]
    shape = L.shape_for(w)
    assert L.attend_splits(shape, False, window)[0] > L.attend_splits(shape, False, 0)[0]
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    kc, vc = bf16_bits(lay.k_cache), bf16_bits(lay.v_cache)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    L.jssa_full_decode(shape, lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV), case.block_table.to(DEV),
                       case.seq_lens.to(DEV), window, w.sm_scale, out, L.alloc_workspace(shape), lse)
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    q = bf16_bits(lay.q)
    for b in range(w.batch):
        n = int(sl[b])
        rk = ogqa.logical_rows(kc, bt[b], n, w.page_size)
        rv = ogqa.logical_rows(vc, bt[b], n, w.page_size)
        sel = ogqa.window_indices(n, window)
        for h in range(w.num_kv_heads):
            j0 = h * w.group
            o, l = ogqa.attend_group(q[b, j0:j0 + w.group], rk[:, h], rv[:, h], sel, w.sm_scale)
            check_attention(got[b, j0:j0 + w.group], o)
            assert np.all(np.abs(glse[b, j0:j0 + w.group] - l) <= 1e-3)


# ----------------------------------------------------------------------------- one decode step

def test_decode_step_stores_new_token_then_selects_and_attends():
    """Cache of positions < N-1 from the oracle; jssa_decode stores position N-1 itself."""
    w, case, m32, rows_k, rows_v, stored = _gqa("mid_sampled")
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    prev = [(c.copy(), s.copy()) for c, s in stored]
    for b in range(w.batch):                      # blank the newest token in what we upload
        prev[b][0][-1] = 0
        prev[b][1][-1] = 0
    shape, kp, ks, M = _upload(w, case, m32, prev)
    new_slot = np.array([bt[b, (sl[b] - 1) // w.page_size] * w.page_size + (sl[b] - 1) % w.page_size
                         for b in range(w.batch)], np.int32)
    k_new = torch.from_numpy(np.stack([rows_k[b][-1] for b in range(w.batch)]).view(np.int16)).view(torch.bfloat16)
    idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lay = case.layers[0]
    L.jssa_decode(shape, lay.q.to(DEV), k_new.to(DEV), torch.from_numpy(new_slot).to(DEV), M, kp, ks,
                  lay.k_cache.to(DEV), lay.v_cache.to(DEV), case.block_table.to(DEV), case.seq_lens.to(DEV), idx,
                  w.sm_scale, out, L.alloc_workspace(shape))
    kp_h, ks_h = kp.cpu().numpy(), ks.cpu().numpy()
    gidx, got = idx.cpu().numpy(), out.float().cpu().numpy()
    q = bf16_bits(lay.q)
    tally = CodeTally()
    for b in range(w.batch):
        n = int(sl[b])
        c, s = unpack_kp(kp_h, ks_h, bt[b], n, w.page_size)
        tally.add(c[-1:], stored[b][0][-1:])                         # the row jssa_decode stored
        qhat = ogqa.project_query(q[b], m32, w.group)
        for h in range(w.num_kv_heads):
            # oracle scores on exactly the codes the GPU selected from (the new row may differ by one ulp)
            codes_b = stored[b][0][:, h].copy()
            scale_b = stored[b][1][:, h].copy()
            codes_b[-1], scale_b[-1] = c[-1, h], s[-1, h]
            sc = ogqa.scores(qhat[h], codes_b, scale_b)
            oidx, tau = ogqa.select_topb(sc, w.budget)
            check_selection(gidx[b, h], oidx, sc, tau)
            j0 = h * w.group
            o, _ = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:, h], rows_v[b][:, h], gidx[b, h], w.sm_scale)
            check_attention(got[b, j0:j0 + w.group], o)
    tally.check()


# ----------------------------------------------------------------------------- MLA store + select

MLA_CASES = {
    "tiny_mla": _w("tiny_mla"),
    "mla_sampled": _w("tiny_mla", name="mla_mid", model="test", batch=2, seq_len=40000, budget=1024),
    "mla_max_budget": _w("tiny_mla", name="mla_maxb", model="test", batch=2, seq_len=40000, budget=4096),
}


@functools.lru_cache(maxsize=None)
def _mla(name):
    w = MLA_CASES[name]
    case = make_mla_case(w, ragged=True)
    m32 = population_basis(w, 0, 0).astype(np.float32)
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    lat = bf16_bits(case.latent)
    rows = [ogqa.logical_rows(lat, bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    stored = [omla.store(r, m32) for r in rows]
    return w, case, m32, rows, stored


@pytest.mark.parametrize("name", list(MLA_CASES))
def test_mla_store_parity(name):
    w, case, m32, rows, stored = _mla(name)
    shape = L.shape_for(w)
    kp, ks = L.alloc_scoring_cache(shape, case.latent.shape[0], DEV)
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    slots, _ = slots_for(bt, sl, w.page_size)
    k_new = torch.from_numpy(np.concatenate(rows).view(np.int16)).view(torch.bfloat16)
    L.jssa_store(shape, k_new.to(DEV), torch.from_numpy(slots).to(DEV), torch.from_numpy(m32).to(DEV), kp, ks)
    kp_h, ks_h = kp.cpu().numpy(), ks.cpu().numpy()
    for b in range(w.batch):
        c, s = unpack_kp(kp_h, ks_h, bt[b], int(sl[b]), w.page_size)
        check_codes(c[:, 0], stored[b][0])
        assert np.max(np.abs(s[:, 0].astype(np.float64) - stored[b][1]) / stored[b][1]) <= 1e-5


@pytest.mark.parametrize("name", list(MLA_CASES))
@pytest.mark.parametrize("mode", [0, 1])
def test_mla_select_parity(name, mode):
    w, case, m32, rows, stored = _mla(name)
    shape = L.shape_for(w, select_mode=mode)
    kp, ks = pack_kp([c[:, None, :] for c, _ in stored], [s[:, None] for _, s in stored], case.block_table.numpy(),
                     w.page_size, case.latent.shape[0], case.seq_lens.numpy())
    maxn = shape.max_pages_per_seq * w.page_size
    scores = torch.zeros((w.batch, 1, maxn), dtype=torch.float32, device=DEV)
    idx = torch.empty((w.batch, 1, w.budget), dtype=torch.int32, device=DEV)
    L.jssa_select(shape, case.q.to(DEV), torch.from_numpy(m32).to(DEV), torch.from_numpy(kp).to(DEV),
                  torch.from_numpy(ks).to(DEV), case.block_table.to(DEV), case.seq_lens.to(DEV), idx,
                  L.alloc_workspace(shape), scores)
    gidx, gsc = idx.cpu().numpy(), scores.cpu().numpy()
    q = bf16_bits(case.q)
    for b in range(w.batch):
        n = int(case.seq_lens[b])
        qhat = omla.project_query(q[b], m32)
        s = ogqa.scores(qhat, stored[b][0], stored[b][1])
        oidx, tau = ogqa.select_topb(s, w.budget)
        check_selection(gidx[b, 0], oidx, s, tau)
        err = check_scores(gsc[b, 0, :n], qhat, stored[b][0], stored[b][1], s)
        print(f"{name} mode {mode} b{b}: max score err / |tau| {err / abs(tau):.2e} (reported)")


# ----------------------------------------------------------------------------- calibration

@pytest.mark.parametrize("name", ["tiny", "d256_r48"])
def test_calibration_moments_and_basis(name):
    w, _ = GQA_CASES[name]
    q, k = make_gqa_calibration(w, 0)
    shape = L.shape_for(w)
    T = q.shape[0]
    gq = torch.zeros((w.num_kv_heads, w.head_dim, w.head_dim), dtype=torch.float32, device=DEV)
    gk = torch.zeros_like(gq)
    ws = torch.empty(L.calib_workspace_bytes(shape, T // 2), dtype=torch.uint8, device=DEV)
    for c0 in (0, T // 2):                       # two chunks accumulate
        L.jssa_calib_moments(shape, q[c0:c0 + T // 2].to(DEV).contiguous(), k[c0:c0 + T // 2].to(DEV).contiguous(),
                             gq, gk, ws)
    q64, k64 = ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(k))
    oq, ok = ocal.moments_per_head(q64, k64, w.group)
    gq_h, gk_h = gq.cpu().numpy().astype(np.float64) / T, gk.cpu().numpy().astype(np.float64) / T
    for got, ref in ((gq_h, oq), (gk_h, ok)):
        assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
    m = L.jssa_basis(shape, gq.cpu().numpy(), gk.cpu().numpy())
    for h in range(w.num_kv_heads):
        mo = ocal.basis(oq[h], ok[h], w.rank)
        mh = m[h].astype(np.float64)
        assert abs(ocal.l_marg(mh.T @ mh, oq[h], ok[h]) - ocal.l_marg(mo.T @ mo, oq[h], ok[h])) < 1e-5


# ----------------------------------------------------------------------------- edge cases

def test_empty_sequence_selects_nothing_and_attends_to_zero():
    w, case, m32, rows_k, rows_v, stored = _gqa("short_ctx")
    shape, kp, ks, M = _upload(w, case, m32, stored)
    sl = case.seq_lens.clone()
    sl[1] = 0
    lay = case.layers[0]
    idx = torch.full((w.batch, w.num_kv_heads, w.budget), 5, dtype=torch.int32, device=DEV)
    ws = L.alloc_workspace(shape)
    L.jssa_select(shape, lay.q.to(DEV), M, kp, ks, case.block_table.to(DEV), sl.to(DEV), idx, ws)
    gidx = idx.cpu().numpy()
    assert np.all(gidx[1] == -1)
    assert np.all(gidx[0, :, :int(sl[0])] >= 0) and np.all(gidx[0, :, int(sl[0]):] == -1)
    for fn in ("sparse", "dense"):
        out = torch.full((w.batch, w.num_q_heads, w.head_dim), 3.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.zeros((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
        if fn == "sparse":
            L.jssa_attend(shape, lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV), case.block_table.to(DEV),
                          sl.to(DEV), idx, w.sm_scale, out, ws, lse)
        else:
            L.jssa_full_decode(shape, lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV),
                               case.block_table.to(DEV), sl.to(DEV), 0, w.sm_scale, out, ws, lse)
        o = out.float().cpu().numpy()
        assert np.all(o[1] == 0) and np.all(np.isneginf(lse.cpu().numpy()[1]))
        assert np.all(np.isfinite(lse.cpu().numpy()[0]))


def test_budget_one_and_all_equal_scores():
    """B = 1 and a sequence whose projected keys are all identical: every score ties, position 0 wins."""
    w = _w("tiny", name="ties", model="test", budget=1, seq_len=20000)
    shape = L.shape_for(w)
    n_pages = w.pages_per_seq
    codes = np.full((w.seq_len, w.num_kv_heads, w.rank), 0x38, np.uint8)
    scales = np.ones((w.seq_len, w.num_kv_heads), np.float32)
    bt = np.random.default_rng(1).permutation(n_pages).astype(np.int32)[None]
    kp, ks = pack_kp([codes], [scales], bt, w.page_size, n_pages, [w.seq_len])
    q = torch.randn((1, w.num_q_heads, w.head_dim)).to(torch.bfloat16)
    M = torch.from_numpy(_basis(WORKLOADS["tiny"])).to(DEV)
    for mode in (0, 1):
        shape.select_mode = mode
        idx = torch.empty((1, w.num_kv_heads, 1), dtype=torch.int32, device=DEV)
        L.jssa_select(shape, q.to(DEV), M, torch.from_numpy(kp).to(DEV), torch.from_numpy(ks).to(DEV),
                      torch.from_numpy(bt).to(DEV), torch.tensor([w.seq_len], dtype=torch.int32, device=DEV), idx,
                      L.alloc_workspace(shape))
        assert np.all(idx.cpu().numpy() == 0)


# ----------------------------------------------------------------------------- MLA attention (MFMA)

@pytest.mark.parametrize("name", list(MLA_CASES))
def test_mla_attend_parity(name):
    w, case, m32, rows, stored = _mla(name)
    q = bf16_bits(case.q)
    idx = np.full((w.batch, 1, w.budget), -1, np.int32)
    for b in range(w.batch):
        qhat = omla.project_query(q[b], m32)
        s = ogqa.scores(qhat, stored[b][0], stored[b][1])
        idx[b, 0], _ = ogqa.select_topb(s, w.budget)
    shape = L.shape_for(w)
    out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    L.jssa_attend(shape, case.q.to(DEV), case.latent.to(DEV), None, case.block_table.to(DEV), case.seq_lens.to(DEV),
                  torch.from_numpy(idx).to(DEV), w.sm_scale, out, L.alloc_workspace(shape), lse)
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(w.batch):
        sel = idx[b, 0][idx[b, 0] >= 0]
        o, l = omla.attend(q[b], rows[b][sel], w.sm_scale)
        err = check_attention(got[b], o)
        assert np.all(np.abs(glse[b] - l) <= 1e-3), np.abs(glse[b] - l).max()
        print(f"{name} b{b}: max abs {err[0]:.2e} mean abs {err[1]:.2e}")


def test_mla_decode_step():
    w, case, m32, rows, stored = _mla("mla_sampled")
    shape = L.shape_for(w)
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    prev = [(c.copy(), s.copy()) for c, s in stored]
    for b in range(w.batch):
        prev[b][0][-1] = 0
        prev[b][1][-1] = 0
    kp, ks = pack_kp([c[:, None, :] for c, _ in prev], [s[:, None] for _, s in prev], bt, w.page_size,
                     case.latent.shape[0], sl)
    kp, ks = torch.from_numpy(kp).to(DEV), torch.from_numpy(ks).to(DEV)
    new_slot = np.array([bt[b, (sl[b] - 1) // w.page_size] * w.page_size + (sl[b] - 1) % w.page_size
                         for b in range(w.batch)], np.int32)
    k_new = torch.from_numpy(np.stack([rows[b][-1] for b in range(w.batch)]).view(np.int16)).view(torch.bfloat16)
    idx = torch.empty((w.batch, 1, w.budget), dtype=torch.int32, device=DEV)
    out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
    L.jssa_decode(shape, case.q.to(DEV), k_new.to(DEV), torch.from_numpy(new_slot).to(DEV),
                  torch.from_numpy(m32).to(DEV), kp, ks, case.latent.to(DEV), None, case.block_table.to(DEV),
                  case.seq_lens.to(DEV), idx, w.sm_scale, out, L.alloc_workspace(shape))
    kp_h, ks_h = kp.cpu().numpy(), ks.cpu().numpy()
    gidx, got = idx.cpu().numpy(), out.float().cpu().numpy()
    q = bf16_bits(case.q)
    tally = CodeTally()
    for b in range(w.batch):
        n = int(sl[b])
        c, s = unpack_kp(kp_h, ks_h, bt[b], n, w.page_size)
        tally.add(c[-1:, 0], stored[b][0][-1:])
        codes_b, scale_b = stored[b][0].copy(), stored[b][1].copy()
        codes_b[-1], scale_b[-1] = c[-1, 0], s[-1, 0]
        qhat = omla.project_query(q[b], m32)
        sc = ogqa.scores(qhat, codes_b, scale_b)
        oidx, tau = ogqa.select_topb(sc, w.budget)
        check_selection(gidx[b, 0], oidx, sc, tau)
        sel = gidx[b, 0][gidx[b, 0] >= 0]
        o, _ = omla.attend(q[b], rows[b][sel], w.sm_scale)
        check_attention(got[b], o)
    tally.check()


@pytest.mark.parametrize("name,window", [("tiny_mla", 0), ("mla_sampled", 0), ("mla_sampled", 1000), ("tiny_mla", 1)])
def test_mla_full_decode_parity(name, window):
    """Dense MLA baseline (all positions, or the last `window`) on the matrix cores."""
    w, case, m32, rows, stored = _mla(name)
    q = bf16_bits(case.q)
    shape = L.shape_for(w)
    out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    L.jssa_full_decode(shape, case.q.to(DEV), case.latent.to(DEV), None, case.block_table.to(DEV),
                       case.seq_lens.to(DEV), window, w.sm_scale, out, L.alloc_workspace(shape), lse)
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(w.batch):
        sel = ogqa.window_indices(int(case.seq_lens[b]), window)
        o, l = omla.attend(q[b], rows[b][sel], w.sm_scale)
        check_attention(got[b], o)
        assert np.all(np.abs(glse[b] - l) <= 1e-3), np.abs(glse[b] - l).max()


def test_mla_calibration_moments_and_basis():
    """MLA: moments over the head-mean query's latent part and the cached latents, then the host basis."""
    w = MLA_CASES["tiny_mla"]
    shape = L.shape_for(w)
    gq = torch.zeros((1, 512, 512), dtype=torch.float32, device=DEV)
    gk = torch.zeros_like(gq)
    chunks = list(make_mla_calibration(w, chunk=256))
    ws = torch.empty(L.calib_workspace_bytes(shape, 256), dtype=torch.uint8, device=DEV)
    T = 0
    for qc, lat in chunks:
        L.jssa_calib_moments(shape, qc.to(DEV), lat.to(DEV), gq, gk, ws)
        T += qc.shape[0]
    q64 = [(ocal.bf16_to_f64(bf16_bits(qc)), ocal.bf16_to_f64(bf16_bits(lat))) for qc, lat in chunks]
    sq = sum(q.mean(axis=1)[:, :512].T @ q.mean(axis=1)[:, :512] for q, _ in q64) / T
    sk = sum(r[:, :512].T @ r[:, :512] for _, r in q64) / T
    gq_h, gk_h = gq.cpu().numpy()[0].astype(np.float64) / T, gk.cpu().numpy()[0].astype(np.float64) / T
    for got, ref in ((gq_h, sq), (gk_h, sk)):
        assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()
    m = L.jssa_basis(shape, gq.cpu().numpy(), gk.cpu().numpy())[0].astype(np.float64)
    mo = omla.calibrate(iter(q64), 512, w.rank)[0]
    assert abs(ocal.l_marg(m.T @ m, sq, sk) - ocal.l_marg(mo.T @ mo, sq, sk)) < 1e-5


def test_graph_replay_matches_eager():
    """One decode step captured in a HIP graph replays bit-identically to the eager call, replay after replay."""
    w, case, m32, rows_k, rows_v, stored = _gqa("mid_sampled")
    shape, kp, ks, M = _upload(w, case, m32, stored)
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    new_slot = torch.from_numpy(np.array([bt[b, (sl[b] - 1) // w.page_size] * w.page_size + (sl[b] - 1) % w.page_size
                                          for b in range(w.batch)], np.int32)).to(DEV)
    k_new = torch.from_numpy(np.stack([rows_k[b][-1] for b in range(w.batch)]).view(np.int16)).view(torch.bfloat16)
    k_new = k_new.to(DEV)
    lay = case.layers[0]
    q, kc, vc = lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV)
    btd, sld = case.block_table.to(DEV), case.seq_lens.to(DEV)
    ws = L.alloc_workspace(shape)
    idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)

    def step():
        L.jssa_decode(shape, q, k_new, new_slot, M, kp, ks, kc, vc, btd, sld, idx, w.sm_scale, out, ws, lse)

    step()
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        idx.fill_(-7)
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), rep
        assert torch.equal(out.view(torch.int16), ref[1].view(torch.int16)), rep
        assert torch.equal(lse, ref[2]), rep
        step()                                    # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0])


def test_hybrid_stack_layers_in_sequence():
    """A 4-layer sliding-window / global stack run back to back like one step: window layers through
    jssa_full_decode, global layers through jssa_decode with their own basis M (per layer, per KV head)."""
    w = _w("hybrid_64k", name="hyb", model="test", batch=2, num_q_heads=8, num_kv_heads=4, seq_len=6000,
           budget=512, num_layers=4, window=512, calib_seqs=2, calib_len=1024)
    case = make_gqa_case(w, ragged=True)
    shape = L.shape_for(w)
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    btd, sld = case.block_table.to(DEV), case.seq_lens.to(DEV)
    ws = L.alloc_workspace(shape)
    new_slot = np.array([bt[b, (sl[b] - 1) // w.page_size] * w.page_size + (sl[b] - 1) % w.page_size
                         for b in range(w.batch)], np.int32)
    host, dev_out = {}, {}
    for l, lay in sorted(case.layers.items()):
        kc, vc = bf16_bits(lay.k_cache), bf16_bits(lay.v_cache)
        rows_k = [ogqa.logical_rows(kc, bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
        rows_v = [ogqa.logical_rows(vc, bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
        out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
        if l in w.window_layers():
            L.jssa_full_decode(shape, lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV), btd, sld, w.window,
                               w.sm_scale, out, ws)
            host[l] = (rows_k, rows_v, None, None)
            dev_out[l] = (out, None, None, None)
            continue
        q, k = make_gqa_calibration(w, l)
        m32 = ocal.calibrate(ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(k)), w.group,
                             w.rank).astype(np.float32)
        stored = [ogqa.store(rk, m32) for rk in rows_k]
        prev = [(c.copy(), s.copy()) for c, s in stored]
        for b in range(w.batch):                  # the newest token is stored by jssa_decode itself
            prev[b][0][-1] = 0
            prev[b][1][-1] = 0
        kp, ks = pack_kp([c for c, _ in prev], [s for _, s in prev], bt, w.page_size, lay.k_cache.shape[0], sl)
        kp, ks = torch.from_numpy(kp).to(DEV), torch.from_numpy(ks).to(DEV)
        k_new = torch.from_numpy(np.stack([rows_k[b][-1] for b in range(w.batch)]).view(np.int16)).view(torch.bfloat16)
        idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV)
        L.jssa_decode(shape, lay.q.to(DEV), k_new.to(DEV), torch.from_numpy(new_slot).to(DEV),
                      torch.from_numpy(m32).to(DEV), kp, ks, lay.k_cache.to(DEV), lay.v_cache.to(DEV), btd, sld, idx,
                      w.sm_scale, out, ws)
        host[l] = (rows_k, rows_v, m32, stored)
        dev_out[l] = (out, idx, kp, ks)
    torch.cuda.synchronize()
    tally = CodeTally()
    for l, lay in sorted(case.layers.items()):
        rows_k, rows_v, m32, stored = host[l]
        out, idx, kp, ks = dev_out[l]
        got = out.float().cpu().numpy()
        q = bf16_bits(lay.q)
        if m32 is None:
            for b in range(w.batch):
                sel = ogqa.window_indices(int(sl[b]), w.window)
                for h in range(w.num_kv_heads):
                    j0 = h * w.group
                    o, _ = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:, h], rows_v[b][:, h], sel, w.sm_scale)
                    check_attention(got[b, j0:j0 + w.group], o)
            continue
        kp_h, ks_h, gidx = kp.cpu().numpy(), ks.cpu().numpy(), idx.cpu().numpy()
        for b in range(w.batch):
            n = int(sl[b])
            c, s = unpack_kp(kp_h, ks_h, bt[b], n, w.page_size)
            tally.add(c[-1], stored[b][0][-1])
            qbar_hat = ogqa.project_query(q[b], m32, w.group)
            for h in range(w.num_kv_heads):
                sc = ogqa.scores(qbar_hat[h], c[:, h], s[:, h])
                oidx, tau = ogqa.select_topb(sc, w.budget)
                check_selection(gidx[b, h], oidx, sc, tau)
                j0 = h * w.group
                o, _ = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:, h], rows_v[b][:, h], gidx[b, h],
                                         w.sm_scale)
                check_attention(got[b, j0:j0 + w.group], o)
    tally.check()


# ----------------------------------------------------------------------------- gather-then-attend

@pytest.mark.parametrize("name", ["mid_sampled", "d256_r48", "short_ctx", "page32_g8"])
def test_gather_attend_parity(name):
    """Staged (gathered) rows + dense attention give the indexed attention's result."""
    w, case, m32, rows_k, rows_v, stored = _gqa(name)
    shape, kp, ks, M = _upload(w, case, m32, stored)
    lay = case.layers[0]
    btd, sld = case.block_table.to(DEV), case.seq_lens.to(DEV)
    ws = L.alloc_workspace(shape)
    idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV)
    L.jssa_select(shape, lay.q.to(DEV), M, kp, ks, btd, sld, idx, ws)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    L.jssa_gather_attend(shape, lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV), btd, sld, idx, w.sm_scale,
                         out, ws, lse)
    gidx, got, glse = idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    q = bf16_bits(lay.q)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            j0 = h * w.group
            o, l = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:, h], rows_v[b][:, h], gidx[b, h], w.sm_scale)
            check_attention(got[b, j0:j0 + w.group], o)
            assert np.all(np.abs(glse[b, j0:j0 + w.group] - l) <= 1e-3)


def test_gather_attend_parity_mla():
    w, case, m32, rows, stored = _mla("mla_sampled")
    q = bf16_bits(case.q)
    idx = np.full((w.batch, 1, w.budget), -1, np.int32)
    for b in range(w.batch):
        s = ogqa.scores(omla.project_query(q[b], m32), stored[b][0], stored[b][1])
        idx[b, 0], _ = ogqa.select_topb(s, w.budget)
    shape = L.shape_for(w)
    out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    L.jssa_gather_attend(shape, case.q.to(DEV), case.latent.to(DEV), None, case.block_table.to(DEV),
                         case.seq_lens.to(DEV), torch.from_numpy(idx).to(DEV), w.sm_scale, out,
                         L.alloc_workspace(shape), lse)
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(w.batch):
        o, l = omla.attend(q[b], rows[b][idx[b, 0][idx[b, 0] >= 0]], w.sm_scale)
        check_attention(got[b], o)
        assert np.all(np.abs(glse[b] - l) <= 1e-3)


def _nan_first_page(cache, bt):
    """The cache with one NaN page in front and the block table moved past it: physical slot 0 then
    belongs to no sequence and holds NaN."""
    pad = torch.full((1,) + tuple(cache.shape[1:]), float("nan"), dtype=cache.dtype)
    return torch.cat([pad, cache]), bt + 1


def test_nan_in_unused_slot_zero_does_not_reach_the_output():
    """A partial batch (past a sequence's end) reads its missing positions at slot 0 with weight 0;
    whatever slot 0 holds must add nothing: indexed, dense, windowed and gathered, GQA and MLA."""
    w, case, m32, rows_k, rows_v, stored = _gqa("short_ctx")
    lay = case.layers[0]
    kc, bt = _nan_first_page(lay.k_cache, case.block_table)
    vc, _ = _nan_first_page(lay.v_cache, case.block_table)
    q = bf16_bits(lay.q)
    idx = np.full((w.batch, w.num_kv_heads, w.budget), -1, np.int32)
    for b in range(w.batch):
        qhat = ogqa.project_query(q[b], m32, w.group)
        for h in range(w.num_kv_heads):
            s = ogqa.scores(qhat[h], stored[b][0][:, h], stored[b][1][:, h])
            idx[b, h], _ = ogqa.select_topb(s, w.budget)
    shape = L.shape_for(w)
    ws = L.alloc_workspace(shape)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    qd, kd, vd, btd, sld = lay.q.to(DEV), kc.to(DEV), vc.to(DEV), bt.to(DEV), case.seq_lens.to(DEV)
    idxd = torch.from_numpy(idx).to(DEV)

    def check(sets):
        got = out.float().cpu().numpy()
        assert np.isfinite(got).all()
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                j0 = h * w.group
                o, _ = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:, h], rows_v[b][:, h], sets(b, h),
                                         w.sm_scale)
                check_attention(got[b, j0:j0 + w.group], o)

    L.jssa_attend(shape, qd, kd, vd, btd, sld, idxd, w.sm_scale, out, ws)
    check(lambda b, h: idx[b, h])
    L.jssa_gather_attend(shape, qd, kd, vd, btd, sld, idxd, w.sm_scale, out, ws)
    check(lambda b, h: idx[b, h])
    for window in (0, 100):
        L.jssa_full_decode(shape, qd, kd, vd, btd, sld, window, w.sm_scale, out, ws)
        check(lambda b, h: ogqa.window_indices(int(case.seq_lens[b]), window))

    w, case, m32, rows, stored = _mla("tiny_mla")
    lat, bt = _nan_first_page(case.latent, case.block_table)
    q = bf16_bits(case.q)
    idx = np.full((w.batch, 1, w.budget), -1, np.int32)
    for b in range(w.batch):
        s = ogqa.scores(omla.project_query(q[b], m32), stored[b][0], stored[b][1])
        idx[b, 0], _ = ogqa.select_topb(s, w.budget)
    shape = L.shape_for(w)
    ws = L.alloc_workspace(shape)
    out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
    qd, ld, btd, sld = case.q.to(DEV), lat.to(DEV), bt.to(DEV), case.seq_lens.to(DEV)

    def check_mla(sets):
        got = out.float().cpu().numpy()
        assert np.isfinite(got).all()
        for b in range(w.batch):
            o, _ = omla.attend(q[b], rows[b][sets(b)], w.sm_scale)
            check_attention(got[b], o)

    L.jssa_attend(shape, qd, ld, None, btd, sld, torch.from_numpy(idx).to(DEV), w.sm_scale, out, ws)
    check_mla(lambda b: idx[b, 0][idx[b, 0] >= 0])
    for window in (0, 100):
        L.jssa_full_decode(shape, qd, ld, None, btd, sld, window, w.sm_scale, out, ws)
        check_mla(lambda b: ogqa.window_indices(int(case.seq_lens[b]), window))


def _spoil(idx, n, marks):
    """Overwrite entries of an index list with positions outside [0, n): the attend kernels must skip them."""
    bad = idx.copy()
    for i, kind in marks:
        bad[i] = {"neg": -1, "end": n, "far": n + 12345, "huge": 2 ** 30}[kind]
    return bad


def test_listed_positions_outside_the_sequence_are_skipped():
    """Entries outside [0, N) of an index list (negative, N and beyond) are skipped wherever they fall: at the
    first row of a tile or batch, and as a whole split of the MLA kernel, whose rows are then all missing.
    The result is attention over the valid entries."""
    w, case, m32, rows_k, rows_v, stored = _gqa("mid_sampled")
    lay = case.layers[0]
    q = bf16_bits(lay.q)
    sl = case.seq_lens.numpy()
    idx = np.full((w.batch, w.num_kv_heads, w.budget), -1, np.int32)
    for b in range(w.batch):
        qhat = ogqa.project_query(q[b], m32, w.group)
        for h in range(w.num_kv_heads):
            s = ogqa.scores(qhat[h], stored[b][0][:, h], stored[b][1][:, h])
            sel, _ = ogqa.select_topb(s, w.budget)
            idx[b, h] = _spoil(sel, int(sl[b]), [(0, "neg"), (64, "end"), (65, "far"), (128, "huge"),
                                                 (255, "neg")] + [(i, "neg") for i in range(256, 320)])
    shape = L.shape_for(w)
    ws = L.alloc_workspace(shape)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    args = (shape, lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV), case.block_table.to(DEV),
            case.seq_lens.to(DEV), torch.from_numpy(idx).to(DEV), w.sm_scale, out, ws)
    for fn in (L.jssa_attend, L.jssa_gather_attend):
        fn(*args)
        got = out.float().cpu().numpy()
        assert np.isfinite(got).all()
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                j0 = h * w.group
                ok = idx[b, h][(idx[b, h] >= 0) & (idx[b, h] < int(sl[b]))]
                o, _ = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:, h], rows_v[b][:, h], ok, w.sm_scale)
                check_attention(got[b, j0:j0 + w.group], o)

    for name in ("mla_sampled", "mla_max_budget"):
        w, case, m32, rows, stored = _mla(name)
        q = bf16_bits(case.q)
        sl = case.seq_lens.numpy()
        shape = L.shape_for(w)
        splits, _ = L.attend_splits(shape, True)
        span = -(-min(w.budget, int(sl.max())) // splits)      # rows per split, about
        idx = np.full((w.batch, 1, w.budget), -1, np.int32)
        for b in range(w.batch):
            s = ogqa.scores(omla.project_query(q[b], m32), stored[b][0], stored[b][1])
            sel, _ = ogqa.select_topb(s, w.budget)
            marks = [(0, "neg"), (32, "end"), (33, "far"), (96, "huge")]
            marks += [(i, "neg") for i in range(2 * span, min(4 * span, w.budget))]   # whole splits
            idx[b, 0] = _spoil(sel, int(sl[b]), marks)
        out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
        L.jssa_attend(shape, case.q.to(DEV), case.latent.to(DEV), None, case.block_table.to(DEV),
                      case.seq_lens.to(DEV), torch.from_numpy(idx).to(DEV), w.sm_scale, out,
                      L.alloc_workspace(shape), lse)
        got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
        assert np.isfinite(got).all()
        for b in range(w.batch):
            ok = idx[b, 0][(idx[b, 0] >= 0) & (idx[b, 0] < int(sl[b]))]
            o, lref = omla.attend(q[b], rows[b][ok], w.sm_scale)
            check_attention(got[b], o)
            assert np.all(np.abs(glse[b] - lref) <= 1e-3), np.abs(glse[b] - lref).max()
