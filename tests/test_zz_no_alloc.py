"""jssa_attend_noalloc (the entry point for callers that cannot allocate) against jssa_attend: the same
kernels and split plan, so identical outputs, and within the attention tolerance of the fp64 oracle over
the same index sets.  Two calls in a row, the second with a smaller input (fewer sequences, shorter
ones); the shared scratch array keeps the first call's contents, which the second must not depend on."""
import numpy as np
import pytest
import torch

import long_context_decode_amd as L
from oracle import gqa as ogqa
from oracle import mla as omla
from synth import WORKLOADS, bf16_bits, make_gqa_case, make_mla_case
from util import check_attention

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _indices(w, seq_lens, seed):
    """A valid index list per (sequence, KV head): min(N, B) distinct positions < N, ascending, -1 padded."""
    rng = np.random.default_rng(seed)
    idx = np.full((w.batch, w.num_kv_heads, w.budget), -1, np.int32)
    for b in range(w.batch):
        n = int(seq_lens[b])
        for h in range(w.num_kv_heads):
            k = min(n, w.budget)
            idx[b, h, :k] = np.sort(rng.choice(n, size=k, replace=False))
    return idx


def _gqa_call(w, seed):
    case = make_gqa_case(w, ragged=True)
    lay = case.layers[0]
    shape = L.shape_for(w)
    sl = case.seq_lens.numpy()
    idx = _indices(w, sl, seed)
    args = (lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV), case.block_table.to(DEV), case.seq_lens.to(DEV),
            torch.from_numpy(idx).to(DEV))
    out_a = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lse_a = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    out_n, lse_n = torch.empty_like(out_a), torch.empty_like(lse_a)
    L.jssa_attend(shape, *args, w.sm_scale, out_a, L.alloc_workspace(shape), lse_a)
    L.jssa_attend_noalloc(shape, *args, w.sm_scale, out_n, lse_n)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_n), "outputs differ from jssa_attend"
    assert torch.equal(lse_a, lse_n), "lse differs from jssa_attend"
    got = out_n.float().cpu().numpy()
    glse = lse_n.cpu().numpy()
    q = bf16_bits(lay.q)
    kc, vc = bf16_bits(lay.k_cache), bf16_bits(lay.v_cache)
    bt = case.block_table.numpy()
    for b in range(w.batch):
        n = int(sl[b])
        rk = ogqa.logical_rows(kc, bt[b], n, w.page_size)
        rv = ogqa.logical_rows(vc, bt[b], n, w.page_size)
        for h in range(w.num_kv_heads):
            j0 = h * w.group
            o, l = ogqa.attend_group(q[b, j0:j0 + w.group], rk[:, h], rv[:, h], idx[b, h], w.sm_scale)
            check_attention(got[b, j0:j0 + w.group], o)
            assert np.max(np.abs(glse[b, j0:j0 + w.group] - l)) <= 1e-3


def test_noalloc_attend_gqa_two_calls():
    base = WORKLOADS["tiny"]
    _gqa_call(base.scaled(name="na1", model="test", batch=3, num_q_heads=8, num_kv_heads=2, seq_len=20000,
                          budget=1024), 1)
    _gqa_call(base.scaled(name="na2", model="test", batch=2, num_q_heads=8, num_kv_heads=2, seq_len=3000,
                          budget=512), 2)


def _mla_call(w, seed):
    case = make_mla_case(w, ragged=True, needles=False)
    shape = L.shape_for(w)
    sl = case.seq_lens.numpy()
    idx = _indices(w, sl, seed)
    args = (case.q.to(DEV), case.latent.to(DEV), None, case.block_table.to(DEV), case.seq_lens.to(DEV),
            torch.from_numpy(idx).to(DEV))
    out_a = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse_a = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    out_n, lse_n = torch.empty_like(out_a), torch.empty_like(lse_a)
    L.jssa_attend(shape, *args, w.sm_scale, out_a, L.alloc_workspace(shape), lse_a)
    L.jssa_attend_noalloc(shape, *args, w.sm_scale, out_n, lse_n)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_n), "outputs differ from jssa_attend"
    assert torch.equal(lse_a, lse_n), "lse differs from jssa_attend"
    got = out_n.float().cpu().numpy()
    q = bf16_bits(case.q)
    lat = bf16_bits(case.latent)
    bt = case.block_table.numpy()
    for b in range(w.batch):
        n = int(sl[b])
        rows = ogqa.logical_rows(lat, bt[b], n, w.page_size)
        sel = idx[b, 0][idx[b, 0] >= 0]
        o, _ = omla.attend(q[b], rows[sel], w.sm_scale)
        check_attention(got[b], o)


def test_noalloc_attend_mla_two_calls():
    base = WORKLOADS["tiny_mla"]
    _mla_call(base.scaled(name="nm1", model="test", batch=2, seq_len=6000, budget=2048), 3)
    _mla_call(base.scaled(name="nm2", model="test", batch=1, seq_len=1500, budget=256), 4)
