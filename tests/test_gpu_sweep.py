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
