"""GPU parity of the split decode path over a seeded sweep of shapes (one jssa_decode step each).

Sequences of 13K-20K tokens, so that the sampled threshold, the score stream and the finish
all run; budgets of 1, 17, 256 and 1000; 1 to 3 KV heads, G up to 8, d = 128 and 256, pages
of 16, 32 and 64, r from 16 to 64.  The new token is stored inside the step.  Each step is
checked against the oracle: the selection against the oracle's top-B on the GPU's own codes
and scales, the attention against fp64 attention over the GPU's set (lse included).
"""
import numpy as np
import pytest

import long_context_decode_amd as L
from oracle import calibrate as ocal
from oracle import gqa as ogqa
from synth import WORKLOADS, bf16_bits, make_gqa_calibration, make_gqa_case
from test_gpu_fused import _check_oracle, _decode
from util import check_attention, check_selection

pytestmark = pytest.mark.gpu


def _sweep_cases():
    rng = np.random.default_rng(11)
    out = []
    for i in range(8):
        d = int(rng.choice([128, 256]))
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 3]))
        page = int(rng.choice([16, 32, 64]))
        r = int(rng.choice([16, 32, 48, 64]))
        budget = int(rng.choice([1, 17, 256, 1000]))
        seq = int(rng.integers(13000, 20000))
        out.append(WORKLOADS["tiny"].scaled(name=f"p{i}", model="sweep", batch=2, num_q_heads=g * hkv,
                                            num_kv_heads=hkv, head_dim=d, page_size=page, rank=r, budget=budget,
                                            seq_len=seq, calib_seqs=1, calib_len=512))
    return out


@pytest.mark.parametrize("w", _sweep_cases(), ids=lambda w: w.name)
def test_split_decode_sweep_against_oracle(w):
    q, k = make_gqa_calibration(w, 0)
    m32 = ocal.calibrate(ocal.bf16_to_f64(bf16_bits(q)), ocal.bf16_to_f64(bf16_bits(k)), w.group,
                         w.rank).astype(np.float32)
    case = make_gqa_case(w, ragged=True)
    lay = case.layers[0]
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    rows_k = [ogqa.logical_rows(bf16_bits(lay.k_cache), bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    rows_v = [ogqa.logical_rows(bf16_bits(lay.v_cache), bt[b], int(sl[b]), w.page_size) for b in range(w.batch)]
    assert not L.decode_single_launch(L.shape_for(w))          # capacity above the single launch's
    res = _decode(w, case, m32, rows_k, "fp32", L.SELECT_AUTO)
    _check_oracle(w, case, m32, rows_k, rows_v, "fp32", res)


def _mla_cases():
    rng = np.random.default_rng(13)
    out = []
    for i in range(5):
        out.append(WORKLOADS["tiny_mla"].scaled(
            name=f"m{i}", model="sweep_mla", num_q_heads=int(rng.choice([32, 64, 96, 128])),
            page_size=int(rng.choice([16, 32, 64])), budget=int(rng.choice([1, 17, 512, 2048])),
            seq_len=int(rng.integers(13000, 20000))))
    return out


@pytest.mark.parametrize("w", _mla_cases(), ids=lambda w: w.name)
def test_mla_decode_sweep_against_oracle(w):
    """MLA decode steps (head counts 32-128, pages 16-64, odd budgets): store the new latent row, select,
    attend on the matrix cores; selection and attention against the oracle."""
    import torch
    from oracle import mla as omla
    from synth import make_mla_case
    from synth.workloads import population_basis
    dev = "cuda"
    shape = L.shape_for(w)
    case = make_mla_case(w, ragged=True)
    m32 = population_basis(w, 0, 0).astype(np.float32)
    M = torch.from_numpy(m32).to(dev)
    P = w.page_size
    bt, sl = case.block_table.numpy(), case.seq_lens.numpy()
    kp, ks = L.alloc_scoring_cache(shape, case.latent.shape[0], dev)
    flat = case.latent.view(-1, w.head_dim).to(dev)
    btd = case.block_table.to(dev).long()
    for b in range(w.batch):                                    # every position but the last
        t = torch.arange(int(sl[b]) - 1, device=dev)
        slots = (btd[b, t // P] * P + t % P).to(torch.int32)
        L.jssa_store(shape, flat[slots.long()].contiguous(), slots, M, kp, ks)
    last = [int(bt[b, (sl[b] - 1) // P]) * P + int(sl[b] - 1) % P for b in range(w.batch)]
    k_new = flat[torch.tensor(last, device=dev).long()].contiguous()
    idx = torch.empty((w.batch, 1, w.budget), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    L.jssa_decode(shape, case.q.to(dev), k_new, torch.tensor(last, dtype=torch.int32, device=dev), M, kp, ks,
                  case.latent.to(dev), None, case.block_table.to(dev), case.seq_lens.to(dev), idx, w.sm_scale, out,
                  L.alloc_workspace(shape), lse)
    torch.cuda.synchronize()
    kp_h, ks_h = kp.cpu().numpy(), ks.cpu().numpy()
    gidx, got, gl = idx.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    q = bf16_bits(case.q)
    lat = bf16_bits(case.latent)
    for b in range(w.batch):
        n = int(sl[b])
        t = np.arange(n)
        pg, so = bt[b, t // P], t % P
        codes, scale = kp_h[pg, 0, :, so, :].reshape(n, -1), ks_h[pg, 0, so]
        sc = ogqa.scores(omla.project_query(q[b], m32), codes, scale)
        oidx, tau = ogqa.select_topb(sc, w.budget)
        check_selection(gidx[b, 0], oidx, sc, tau)
        rows = ogqa.logical_rows(lat, bt[b], n, P)
        sel = gidx[b, 0][gidx[b, 0] >= 0]
        o, ol = omla.attend(q[b], rows[sel], w.sm_scale)
        check_attention(got[b], o)
        assert np.max(np.abs(gl[b] - ol)) <= 1e-3
