"""GPU parity of the single-launch decode path (select_mode FUSED).

For short sequences jssa_decode can run the whole step (qhat, the new token's
store, exact scoring of every position, top-B, attention) in one launch per
layer.  Each case runs one jssa_decode step through the split path (SPLIT) and
through the single launch (FUSED) from the same scoring cache and compares:

* the stored new token: identical bytes (both follow jssa_store's arithmetic);
* the index lists: identical (the same keys and the same tie rule);
* the outputs and lse: within the attention tolerance of each other, and each
  path against the oracle (the selection against the oracle's top-B on the
  GPU's own codes, the attention against fp64 attention over the GPU's set).

AUTO must give FUSED's bits where the shape allows the single launch, and FUSED
must refuse a shape it does not cover.
"""
import functools

import numpy as np
import pytest
import torch

import long_context_decode_amd as L
from oracle import calibrate as ocal
from oracle import gqa as ogqa
from synth import WORKLOADS, bf16_bits, make_gqa_calibration, make_gqa_case
from util import check_attention, check_selection

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _w(**kw):
    return WORKLOADS["tiny"].scaled(model="fused", **kw)


CASES = {
    # the tiny workload's shape, three ragged sequences
    "tiny_b3": _w(name="f1", batch=3),
    # capacity at the limit (12288 tokens), B = 1024, ragged
    "cap_12k": _w(name="f2", batch=2, seq_len=12288, budget=1024),
    # d = 256, G = 2, r = 48 (the hybrid layers' head shape)
    "d256_r48": _w(name="f3", batch=2, num_q_heads=4, num_kv_heads=2, head_dim=256, rank=48, seq_len=6000,
                   budget=512),
    # G = 1, page 64, r = 64, B = 2048
    "g1_p64_r64": _w(name="f4", batch=2, num_q_heads=4, num_kv_heads=4, page_size=64, rank=64, seq_len=5000,
                     budget=2048),
    # every sequence shorter than B: all positions selected
    "short": _w(name="f5", batch=2, seq_len=300, budget=512),
    # r = 16, page 32, G = 4
    "r16_p32": _w(name="f6", batch=2, page_size=32, rank=16, seq_len=3000, budget=128),
}


@functools.lru_cache(maxsize=None)
def _case(name):
    w = CASES[name]
    q, k = make_gqa_calibration(w, 0)
    m32 = ocal.calibrate(ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(k)), w.group,
                         w.rank).astype(np.float32)
    case = make_gqa_case(w, ragged=True)
    lay = case.layers[0]
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    rows_k = [ogqa.logical_rows(bf16_bits(lay.k_cache), bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    rows_v = [ogqa.logical_rows(bf16_bits(lay.v_cache), bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    return w, case, m32, rows_k, rows_v


def _stored_cache(w, shape, case, M):
    """The scoring cache with every position but each sequence's last one stored by jssa_store."""
    lay = case.layers[0]
    kp, ks = L.alloc_scoring_cache(shape, lay.k_cache.shape[0], DEV)
    P = w.page_size
    bt = case.block_table.to(DEV).long()
    flat = lay.k_cache.view(lay.k_cache.shape[0] * P, *lay.k_cache.shape[2:]).to(DEV)
    for b in range(w.batch):
        n = int(case.seq_lens[b]) - 1
        if n <= 0:
            continue
        t = torch.arange(n, device=DEV)
        slots = (bt[b, t // P] * P + t % P).to(torch.int32)
        L.jssa_store(shape, flat[slots.long()].contiguous(), slots, M, kp, ks)
    torch.cuda.synchronize()
    return kp, ks


def _decode(w, case, m32, rows_k, fmt, mode, seq_lens=None):
    """One jssa_decode step in `mode`: (idx, out, lse, kp, ks) on the host."""
    sfmt = L.SCALE_FORMATS[fmt]
    shape = L.shape_for(w, scale_format=sfmt, select_mode=mode)
    M = torch.from_numpy(m32).to(DEV)
    lay = case.layers[0]
    kp, ks = _stored_cache(w, L.shape_for(w, scale_format=sfmt), case, M)
    bt = case.block_table.numpy()
    sl = case.seq_lens.numpy() if seq_lens is None else seq_lens
    new_slot = np.array([bt[b, (sl[b] - 1) // w.page_size] * w.page_size + (sl[b] - 1) % w.page_size
                         if sl[b] > 0 else -1 for b in range(w.batch)], np.int32)
    k_new = torch.from_numpy(np.stack([rows_k[b][int(case.seq_lens[b]) - 1] for b in range(w.batch)])
                             .view(np.int16)).view(torch.bfloat16)
    ws = L.alloc_workspace(shape)
    idx = torch.full((w.batch, w.num_kv_heads, w.budget), 7, dtype=torch.int32, device=DEV)
    out = torch.full((w.batch, w.num_q_heads, w.head_dim), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    L.jssa_decode(shape, lay.q.to(DEV), k_new.to(DEV), torch.from_numpy(new_slot).to(DEV), M, kp, ks,
                  lay.k_cache.to(DEV), lay.v_cache.to(DEV), case.block_table.to(DEV),
                  torch.from_numpy(np.ascontiguousarray(sl, np.int32)).to(DEV), idx, w.sm_scale, out, ws, lse)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy(), kp.cpu().numpy(),
            None if ks is None else ks.cpu().numpy())


def _unpack(kp, ks, bt_row, n, P, h):
    t = np.arange(n)
    pg, sl = bt_row[t // P], t % P
    c = kp[pg, h, :, sl, :].reshape(n, -1)
    return c, (None if ks is None else ks[pg, h, sl])


def _check_oracle(w, case, m32, rows_k, rows_v, fmt, res, seq_lens=None):
    gidx, got, lse, kp_h, ks_h = res
    bt = case.block_table.numpy()
    sl = case.seq_lens.numpy() if seq_lens is None else seq_lens
    q = bf16_bits(case.layers[0].q)
    for b in range(w.batch):
        n = int(sl[b])
        if n == 0:
            assert np.all(gidx[b] == -1)
            assert np.all(got[b] == 0.0) and np.all(np.isneginf(lse[b]))
            continue
        qhat = ogqa.project_query(q[b], m32, w.group)
        for h in range(w.num_kv_heads):
            gc, gs = _unpack(kp_h, ks_h, bt[b], n, w.page_size, h)
            sc = ogqa.scores(qhat[h], gc, gs, fmt)
            oidx, tau = ogqa.select_topb(sc, w.budget)
            check_selection(gidx[b, h], oidx, sc, tau)
            j0 = h * w.group
            o, ol = ogqa.attend_group(q[b, j0:j0 + w.group], rows_k[b][:n, h], rows_v[b][:n, h], gidx[b, h],
                                      w.sm_scale)
            check_attention(got[b, j0:j0 + w.group], o)
            assert np.max(np.abs(lse[b, j0:j0 + w.group] - ol)) <= 1e-3


def _compare(split, fused):
    si, so, sls, skp, sks = split
    fi, fo, fls, fkp, fks = fused
    assert np.array_equal(skp, fkp), "stored scoring cache differs"
    assert (sks is None and fks is None) or np.array_equal(sks, fks), "stored scales differ"
    assert np.array_equal(si, fi), "index lists differ"
    check_attention(fo, so.astype(np.float64))
    fin = np.isfinite(sls)
    assert np.array_equal(fin, np.isfinite(fls))
    assert np.max(np.abs(fls[fin] - sls[fin]), initial=0.0) <= 1e-4


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_split_and_oracle(name):
    w, case, m32, rows_k, rows_v = _case(name)
    split = _decode(w, case, m32, rows_k, "fp32", L.SELECT_SPLIT)
    fused = _decode(w, case, m32, rows_k, "fp32", L.SELECT_FUSED)
    _compare(split, fused)
    _check_oracle(w, case, m32, rows_k, rows_v, "fp32", fused)


@pytest.mark.parametrize("fmt", ["e8m0", "none", "bf16"])
def test_fused_scale_formats(fmt):
    w, case, m32, rows_k, rows_v = _case("tiny_b3")
    split = _decode(w, case, m32, rows_k, fmt, L.SELECT_SPLIT)
    fused = _decode(w, case, m32, rows_k, fmt, L.SELECT_FUSED)
    _compare(split, fused)
    _check_oracle(w, case, m32, rows_k, rows_v, fmt, fused)


def test_fused_empty_sequence_and_auto():
    """An empty sequence (seq_len 0, no new token): -1 indices, zero output, lse -inf; AUTO = FUSED bits."""
    w, case, m32, rows_k, rows_v = _case("tiny_b3")
    sl = case.seq_lens.numpy().copy()
    sl[1] = 0
    fused = _decode(w, case, m32, rows_k, "fp32", L.SELECT_FUSED, seq_lens=sl)
    split = _decode(w, case, m32, rows_k, "fp32", L.SELECT_SPLIT, seq_lens=sl)
    _compare(split, fused)
    _check_oracle(w, case, m32, rows_k, rows_v, "fp32", fused, seq_lens=sl)
    assert L.decode_single_launch(L.shape_for(w))                 # AUTO takes the single launch here
    auto = _decode(w, case, m32, rows_k, "fp32", L.SELECT_AUTO, seq_lens=sl)
    for a, f in zip(auto, fused):
        assert (a is None and f is None) or np.array_equal(a, f, equal_nan=True)


def test_fused_refuses_uncovered_shapes():
    """FUSED on a shape it does not cover returns JSSA_ERR_UNSUPPORTED before any launch."""
    base = CASES["tiny_b3"]
    for w in (base.scaled(seq_len=12289),                     # capacity above the LDS key array
              base.scaled(num_q_heads=16, num_kv_heads=2),      # G * d = 1024
              base.scaled(rank=80)):                          # r > 64
        shape = L.shape_for(w, select_mode=L.SELECT_FUSED)
        kp, ks = L.alloc_scoring_cache(shape, 1, DEV)
        t = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device=DEV)
        ws = L.alloc_workspace(shape)
        with pytest.raises(L.JSSAError) as err:
            L.jssa_decode(shape, t(w.batch, w.num_q_heads, w.head_dim), None, None,
                          t(w.num_kv_heads, w.rank, w.head_dim, dt=torch.float32), kp, ks,
                          t(1, w.page_size, w.num_kv_heads, w.head_dim), t(1, w.page_size, w.num_kv_heads, w.head_dim),
                          torch.zeros((w.batch, w.pages_per_seq), dtype=torch.int32, device=DEV),
                          torch.zeros((w.batch,), dtype=torch.int32, device=DEV),
                          torch.zeros((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV),
                          w.sm_scale, t(w.batch, w.num_q_heads, w.head_dim), ws)
        assert err.value.status == -3                        # JSSA_ERR_UNSUPPORTED


def test_select_treats_split_and_fused_as_auto():
    """jssa_select has no single-launch variant: SPLIT and FUSED select exactly as AUTO does."""
    w, case, m32, rows_k, rows_v = _case("cap_12k")
    M = torch.from_numpy(m32).to(DEV)
    kp, ks = _stored_cache(w, L.shape_for(w), case, M)
    got = {}
    for mode in (L.SELECT_AUTO, L.SELECT_SPLIT, L.SELECT_FUSED):
        shape = L.shape_for(w, select_mode=mode)
        idx = torch.full((w.batch, w.num_kv_heads, w.budget), 7, dtype=torch.int32, device=DEV)
        L.jssa_select(shape, case.layers[0].q.to(DEV), M, kp, ks, case.block_table.to(DEV), case.seq_lens.to(DEV),
                      idx, L.alloc_workspace(shape))
        torch.cuda.synchronize()
        got[mode] = idx.cpu().numpy()
    assert np.array_equal(got[L.SELECT_AUTO], got[L.SELECT_SPLIT])
    assert np.array_equal(got[L.SELECT_AUTO], got[L.SELECT_FUSED])


def _sweep_cases():
    """A seeded sample of small shapes the single launch covers: d, G, page, r, B (odd ones too) and N."""
    rng = np.random.default_rng(7)
    out = []
    for i in range(10):
        d = int(rng.choice([128, 256]))
        g = int(rng.choice([1, 2, 4] if d == 128 else [1, 2]))
        hkv = int(rng.choice([1, 2, 3]))
        page = int(rng.choice([16, 32, 64]))
        r = int(rng.choice([16, 32, 48, 64]))
        budget = int(rng.choice([1, 17, 256, 1000]))
        seq = int(rng.integers(200, 6000))
        out.append(_w(name=f"s{i}", batch=2, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, page_size=page,
                      rank=r, budget=budget, seq_len=seq, calib_seqs=1, calib_len=512))
    return out


@pytest.mark.parametrize("w", _sweep_cases(), ids=lambda w: w.name)
def test_fused_equals_split_sweep(w):
    q, k = make_gqa_calibration(w, 0)
    m32 = ocal.calibrate(ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(k)), w.group,
                         w.rank).astype(np.float32)
    case = make_gqa_case(w, ragged=True)
    lay = case.layers[0]
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    rows_k = [ogqa.logical_rows(bf16_bits(lay.k_cache), bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    rows_v = [ogqa.logical_rows(bf16_bits(lay.v_cache), bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    assert L.decode_single_launch(L.shape_for(w))
    split = _decode(w, case, m32, rows_k, "fp32", L.SELECT_SPLIT)
    fused = _decode(w, case, m32, rows_k, "fp32", L.SELECT_FUSED)
    _compare(split, fused)
    _check_oracle(w, case, m32, rows_k, rows_v, "fp32", fused)


def test_fused_graph_replay_matches_eager():
    """The single launch captured in a HIP graph replays bit-identically to the eager call, with eager work
    between the replays (the new token is stored each time: the same bytes)."""
    w, case, m32, rows_k, rows_v = _case("tiny_b3")
    shape = L.shape_for(w, select_mode=L.SELECT_FUSED)
    M = torch.from_numpy(m32).to(DEV)
    kp, ks = _stored_cache(w, shape, case, M)
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    new_slot = torch.tensor([bt[b, (sl[b] - 1) // w.page_size] * w.page_size + (sl[b] - 1) % w.page_size
                             for b in range(w.batch)], dtype=torch.int32, device=DEV)
    k_new = torch.from_numpy(np.stack([rows_k[b][int(sl[b]) - 1] for b in range(w.batch)]).view(np.int16)) \
        .view(torch.bfloat16).to(DEV)
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
    ref = (idx.clone(), out.clone(), lse.clone(), kp.clone())
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
        assert torch.equal(kp, ref[3]), rep
        step()                                    # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0])
