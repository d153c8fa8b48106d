"""GPU: no result depends on what the caller's workspace held before a call, nor on other calls.

The workspace that jssa_workspace_bytes sizes is caller memory with no initialisation requirement
(include/jssa.h, conventions), so every call must write whatever it later reads back: candidate
regions and their counts, the projected query and threshold, split-K partials, staged rows.  Each
path below runs twice on the same inputs, once on a workspace of 0xFF bytes (NaN floats, all-ones
words, -1 ints) and once on zeros, and everything it writes (indices, bf16 output, lse, the scoring
cache it stores into) must be bit-identical.  Two decode steps overlapping on two streams must also
write what serial calls write.  Parity with the oracle is checked elsewhere; this file checks
independence from the workspace's prior contents and from concurrent calls.
"""
import numpy as np
import pytest
import torch

from test_gpu_parity import DEV, _gqa, _mla, _upload
from util import pack_kp

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import long_context_decode_amd as L


def _ws(shape, byte):
    ws = L.alloc_workspace(shape)
    ws.fill_(byte)
    return ws


def _same(run):
    a, b = run(0xFF), run(0x00)
    torch.cuda.synchronize()
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


@pytest.mark.parametrize("name", ["tiny", "mid_sampled", "cap_edge", "d256_r48"])
def test_gqa_paths_do_not_read_stale_workspace(name):
    """jssa_select, jssa_attend, jssa_decode (with the new token's store), jssa_full_decode (all
    positions and a window) and jssa_gather_attend on a 0xFF-filled and a zeroed workspace."""
    w, case, m32, rows_k, rows_v, stored = _gqa(name)
    lay = case.layers[0]
    q, kc, vc = lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV)
    bt, sl = case.block_table.to(DEV), case.seq_lens.to(DEV)
    btn, sln = case.block_table.numpy(), case.seq_lens.numpy()
    new_slot = torch.from_numpy(np.array([btn[b, (sln[b] - 1) // w.page_size] * w.page_size
                                          + (sln[b] - 1) % w.page_size for b in range(w.batch)], np.int32)).to(DEV)
    k_new = torch.from_numpy(np.stack([rows_k[b][-1] for b in range(w.batch)]).view(np.int16)).view(
        torch.bfloat16).to(DEV)

    def outs():
        return (torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV),
                torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV),
                torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV))

    def select_attend(byte):
        shape, kp, ks, M = _upload(w, case, m32, stored)
        idx, out, lse = outs()
        L.jssa_select(shape, q, M, kp, ks, bt, sl, idx, _ws(shape, byte))
        L.jssa_attend(shape, q, kc, vc, bt, sl, idx, w.sm_scale, out, _ws(shape, byte), lse)
        return idx, out, lse

    def decode(byte):
        shape, kp, ks, M = _upload(w, case, m32, stored)
        idx, out, lse = outs()
        L.jssa_decode(shape, q, k_new, new_slot, M, kp, ks, kc, vc, bt, sl, idx, w.sm_scale, out,
                      _ws(shape, byte), lse)
        return idx, out, lse, kp, ks

    def dense(byte):
        shape = L.shape_for(w)
        res = []
        for window in (0, 1000):
            _, out, lse = outs()
            L.jssa_full_decode(shape, q, kc, vc, bt, sl, window, w.sm_scale, out, _ws(shape, byte), lse)
            res += [out, lse]
        return tuple(res)

    def gather(byte):
        shape, kp, ks, M = _upload(w, case, m32, stored)
        idx, out, lse = outs()
        L.jssa_select(shape, q, M, kp, ks, bt, sl, idx, _ws(shape, 0))
        L.jssa_gather_attend(shape, q, kc, vc, bt, sl, idx, w.sm_scale, out, _ws(shape, byte), lse)
        return out, lse

    for run in (select_attend, decode, dense, gather):
        _same(run)


@pytest.mark.parametrize("name", ["tiny_mla", "mla_sampled"])
def test_mla_paths_do_not_read_stale_workspace(name):
    """MLA: jssa_decode (store, select, sparse attend on the matrix cores) and jssa_full_decode on a
    0xFF-filled and a zeroed workspace."""
    w, case, m32, rows, stored = _mla(name)
    btn, sln = case.block_table.numpy(), case.seq_lens.numpy()
    bt, sl = case.block_table.to(DEV), case.seq_lens.to(DEV)
    q, lat, M = case.q.to(DEV), case.latent.to(DEV), torch.from_numpy(m32).to(DEV)
    new_slot = torch.from_numpy(np.array([btn[b, (sln[b] - 1) // w.page_size] * w.page_size
                                          + (sln[b] - 1) % w.page_size for b in range(w.batch)], np.int32)).to(DEV)
    k_new = torch.from_numpy(np.stack([rows[b][-1] for b in range(w.batch)]).view(np.int16)).view(
        torch.bfloat16).to(DEV)

    def decode(byte):
        shape = L.shape_for(w)
        kp, ks = pack_kp([c[:, None, :] for c, _ in stored], [s[:, None] for _, s in stored], btn, w.page_size,
                         case.latent.shape[0], sln)
        kp, ks = torch.from_numpy(kp).to(DEV), torch.from_numpy(ks).to(DEV)
        idx = torch.empty((w.batch, 1, w.budget), dtype=torch.int32, device=DEV)
        out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
        L.jssa_decode(shape, q, k_new, new_slot, M, kp, ks, lat, None, bt, sl, idx, w.sm_scale, out,
                      _ws(shape, byte), lse)
        return idx, out, lse, kp, ks

    def dense(byte):
        shape = L.shape_for(w)
        out = torch.empty((w.batch, w.num_q_heads, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
        L.jssa_full_decode(shape, q, lat, None, bt, sl, 0, w.sm_scale, out, _ws(shape, byte), lse)
        return out, lse

    for run in (decode, dense):
        _same(run)


def test_concurrent_calls_on_two_streams_match_serial_calls():
    """The library keeps no state between calls (include/jssa.h, conventions), so two decode steps
    on two streams, each with its own workspace, outputs and scoring cache, overlapping on the GPU,
    write exactly what the same calls write one after the other.  Both streams keep the default
    priority."""
    w, case, m32, rows_k, rows_v, stored = _gqa("mid_sampled")
    lay = case.layers[0]
    q, kc, vc = lay.q.to(DEV), lay.k_cache.to(DEV), lay.v_cache.to(DEV)
    bt, sl = case.block_table.to(DEV), case.seq_lens.to(DEV)
    btn, sln = case.block_table.numpy(), case.seq_lens.numpy()
    new_slot = torch.from_numpy(np.array([btn[b, (sln[b] - 1) // w.page_size] * w.page_size
                                          + (sln[b] - 1) % w.page_size for b in range(w.batch)], np.int32)).to(DEV)
    k_new = torch.from_numpy(np.stack([rows_k[b][-1] for b in range(w.batch)]).view(np.int16)).view(
        torch.bfloat16).to(DEV)

    def prepare():
        shape, kp, ks, M = _upload(w, case, m32, stored)
        idx = torch.empty((w.batch, w.num_kv_heads, w.budget), dtype=torch.int32, device=DEV)
        out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
        return dict(shape=shape, kp=kp, ks=ks, M=M, idx=idx, out=out, ws=_ws(shape, 0xFF))

    def step(r, reps=4):
        for _ in range(reps):          # repeated steps: the same token stored again, the same result
            L.jssa_decode(r["shape"], q, k_new, new_slot, r["M"], r["kp"], r["ks"], kc, vc, bt, sl, r["idx"],
                          w.sm_scale, r["out"], r["ws"])

    serial = prepare()
    step(serial)
    torch.cuda.synchronize()
    a, b = prepare(), prepare()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        step(a)
    with torch.cuda.stream(s2):
        step(b)
    torch.cuda.synchronize()
    for r in (a, b):
        for key in ("idx", "out", "kp", "ks"):
            assert torch.equal(r[key].contiguous().view(torch.uint8), serial[key].contiguous().view(torch.uint8)), key
