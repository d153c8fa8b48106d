"""Pins for the oracle's store / score / select / attend and its MLA variant — CPU only."""
import numpy as np
import pytest
import torch

from oracle import calibrate as cal
from oracle import fp8, gqa, mla
from synth import WORKLOADS, make_gqa_case, make_gqa_calibration, make_mla_case, bf16_bits
from synth.workloads import haar_orthogonal


def _bf16(x):
    return bf16_bits(torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16))


# ----------------------------------------------------------------------------- store

def test_store_recovers_coefficients_in_row_space():
    """k = M^T c lies in the row space of an orthonormal M, so M k = c: decoded codes * scale ~ c."""
    rng = np.random.default_rng(0)
    d, r, hkv = 128, 32, 3
    m = np.stack([haar_orthogonal(d, 10 + h)[:r] for h in range(hkv)]).astype(np.float32)
    c = rng.standard_normal((50, hkv, r))
    k = np.einsum("hrd,thr->thd", m.astype(np.float64), c)
    k_u16 = _bf16(k)
    codes, scale = gqa.store(k_u16, m)
    assert codes.shape == (50, hkv, r) and scale.shape == (50, hkv) and scale.dtype == np.float32
    y = np.einsum("hrd,thd->thr", m.astype(np.float64), cal.bf16_to_f64(k_u16))
    rec = fp8.decode(codes) * scale[..., None].astype(np.float64)
    # within half an FP8 ulp of the projection, which is itself within bf16 rounding of c
    tol = np.maximum(np.abs(y) * 2.0 ** -4, scale[..., None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(rec - y) <= tol)
    assert np.abs(y - c).max() < 0.05
    # the largest entry of every row lands exactly on +-448
    amax_code = np.take_along_axis(codes, np.argmax(np.abs(y), -1)[..., None], -1)[..., 0]
    assert np.all((amax_code == 0x7E) | (amax_code == 0xFE))


def test_store_identity_basis_exact_codes():
    """M = [I_r | 0] and a row whose first entry is 448: scale is exactly 1, codes are enc(k)."""
    d, r = 128, 32
    m = np.zeros((1, r, d), np.float32)
    m[0, :, :r] = np.eye(r)
    vals = fp8.decode(np.arange(0, 0x7F, dtype=np.uint8))           # every finite positive code
    mids = (vals[:-1] + vals[1:]) / 2                                # every midpoint (exact in bf16)
    pool = np.concatenate([vals, -vals, mids, -mids])
    rows = []
    for i in range(0, len(pool), r - 1):
        row = np.zeros(d)
        chunk = pool[i:i + r - 1]
        row[0] = 448.0
        row[1:1 + len(chunk)] = chunk
        rows.append(row)
    k = np.array(rows)[:, None, :]
    k_u16 = _bf16(k)
    assert np.array_equal(cal.bf16_to_f64(k_u16), k)                 # all exactly representable
    codes, scale = gqa.store(k_u16, m)
    assert np.all(scale == 1.0)
    # compared on the number line: an exact-zero projection may carry either sign
    assert np.array_equal(fp8.signed_magnitude(codes[:, 0, :]), fp8.signed_magnitude(fp8.encode(k[:, 0, :r])))


def test_store_zero_row():
    codes, scale = gqa.store(np.zeros((2, 1, 128), np.uint16), np.eye(128, dtype=np.float32)[None, :32])
    assert np.all(scale == 0) and np.all(codes == 0)


# ----------------------------------------------------------------------------- score

def test_scores_identity_basis_within_fp8_bound():
    """r = d, M = I: s^ = scale * qbar.dec(codes) is within the FP8 rounding bound of qbar.k."""
    rng = np.random.default_rng(1)
    d, n = 64, 500
    m = np.eye(d, dtype=np.float32)[None]
    k_u16 = _bf16(rng.standard_normal((n, 1, d)))
    q_u16 = _bf16(rng.standard_normal((4, d)))
    codes, scale = gqa.store(k_u16, m)
    qhat = gqa.project_query(q_u16, m, 4)[0]
    s_hat = gqa.scores(qhat, codes[:, 0], scale[:, 0])
    k = cal.bf16_to_f64(k_u16)[:, 0]
    exact = k @ qhat
    bound = (np.abs(qhat)[None, :] * np.maximum(np.abs(k) * 2.0 ** -4, scale[:, 0, None] * 2.0 ** -10)).sum(1)
    assert np.all(np.abs(s_hat - exact) <= bound * 1.0001)
    assert np.corrcoef(s_hat, exact)[0, 1] > 0.999


def test_scores_negative_zero_canonical():
    s = gqa.scores(np.array([1.0, -1.0]), np.array([[0x38, 0x38], [0x80, 0x00]], np.uint8),
                   np.array([1.0, 1.0], np.float32))
    assert s[0] == 0.0 and not np.signbit(s[0]) and s[1] == 0.0 and not np.signbit(s[1])


# ----------------------------------------------------------------------------- select

def _brute_topb(s, b):
    """Independent route: python sort of (score, position) pairs."""
    pairs = sorted(range(len(s)), key=lambda t: (-s[t], t))[:b]
    return sorted(pairs)


def _argpartition_topb(s, b):
    """Second route: argpartition, then repair ties at the threshold by position."""
    n = len(s)
    k = min(b, n)
    if k == n:
        return list(range(n))
    part = np.argpartition(-s, k - 1)[:k]
    tau = s[part].min()
    above = np.nonzero(s > tau)[0]
    ties = np.nonzero(s == tau)[0]
    return sorted(list(above) + list(ties[:k - len(above)]))


@pytest.mark.parametrize("n,b,levels", [(1, 4, 0), (37, 8, 0), (500, 64, 0), (4096, 256, 0),
                                        (3000, 300, 7), (4096, 256, 3), (100, 100, 0), (99, 100, 2)])
def test_select_matches_two_brute_force_routes(n, b, levels):
    rng = np.random.default_rng(n * 7 + b)
    s = rng.standard_normal(n)
    if levels:
        s = np.round(s * levels) / levels          # heavy ties
    idx, tau = gqa.select_topb(s, b)
    k = min(b, n)
    assert idx.shape == (b,) and np.all(idx[k:] == -1)
    assert list(idx[:k]) == _brute_topb(s, b)
    assert list(idx[:k]) == _argpartition_topb(s, b)
    assert np.all(np.diff(idx[:k]) > 0)
    assert tau == sorted(s, reverse=True)[k - 1]


def test_select_budget_at_least_n_selects_all_and_empty():
    idx, _ = gqa.select_topb(np.array([3.0, -1.0, 2.0]), 5)
    assert list(idx) == [0, 1, 2, -1, -1]
    idx, tau = gqa.select_topb(np.zeros(0), 3)
    assert list(idx) == [-1, -1, -1] and np.isnan(tau)


def test_select_tie_lowest_position_wins():
    s = np.array([1.0, 5.0, 2.0, 2.0, 2.0, 0.0, 2.0])
    idx, tau = gqa.select_topb(s, 3)
    assert list(idx) == [1, 2, 3] and tau == 2.0


# ----------------------------------------------------------------------------- attend

def _sdpa64(q, k, v, sm):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q)[None, None, None], torch.as_tensor(k)[None, None],
        torch.as_tensor(v)[None, None], scale=sm)
    return out[0, 0, 0].numpy()


def test_attend_full_set_matches_sdpa_fp64():
    rng = np.random.default_rng(2)
    n, d = 300, 128
    q_u16, k_u16, v_u16 = _bf16(rng.standard_normal(d) * 3), _bf16(rng.standard_normal((n, d))), \
        _bf16(rng.standard_normal((n, d)))
    o, lse = gqa.attend(q_u16, k_u16, v_u16, 0.0883883)
    ref = _sdpa64(cal.bf16_to_f64(q_u16), cal.bf16_to_f64(k_u16), cal.bf16_to_f64(v_u16), 0.0883883)
    assert np.abs(o - ref).max() < 1e-12
    x = 0.0883883 * cal.bf16_to_f64(k_u16) @ cal.bf16_to_f64(q_u16)
    assert abs(lse - np.log(np.exp(x).sum())) < 1e-10


def test_attend_single_row_permutation_and_empty():
    rng = np.random.default_rng(3)
    k_u16, v_u16 = _bf16(rng.standard_normal((20, 64))), _bf16(rng.standard_normal((20, 64)))
    q_u16 = _bf16(rng.standard_normal(64))
    o, lse = gqa.attend(q_u16, k_u16[5:6], v_u16[5:6], 0.125)
    assert np.array_equal(o, cal.bf16_to_f64(v_u16[5]))
    assert abs(lse - 0.125 * cal.bf16_to_f64(k_u16[5]) @ cal.bf16_to_f64(q_u16)) < 1e-12
    perm = rng.permutation(20)
    o1, l1 = gqa.attend(q_u16, k_u16, v_u16, 0.125)
    o2, l2 = gqa.attend(q_u16, k_u16[perm], v_u16[perm], 0.125)
    assert np.abs(o1 - o2).max() < 1e-12 and abs(l1 - l2) < 1e-12
    o, lse = gqa.attend(q_u16, k_u16[:0], v_u16[:0], 0.125)
    assert np.all(o == 0) and lse == -np.inf


def test_lse_merge_of_halves_equals_whole():
    rng = np.random.default_rng(4)
    k_u16, v_u16 = _bf16(rng.standard_normal((64, 32))), _bf16(rng.standard_normal((64, 32)))
    q_u16 = _bf16(rng.standard_normal(32) * 2)
    o, lse = gqa.attend(q_u16, k_u16, v_u16, 0.3)
    oa, la = gqa.attend(q_u16, k_u16[:23], v_u16[:23], 0.3)
    ob, lb = gqa.attend(q_u16, k_u16[23:], v_u16[23:], 0.3)
    mx = max(la, lb)
    wa, wb = np.exp(la - mx), np.exp(lb - mx)
    assert np.abs((wa * oa + wb * ob) / (wa + wb) - o).max() < 1e-12
    assert abs(mx + np.log(wa + wb) - lse) < 1e-12


def test_attend_group_uses_the_kv_heads_own_set():
    rng = np.random.default_rng(5)
    n, d, G = 40, 16, 3
    k_u16, v_u16 = _bf16(rng.standard_normal((n, d))), _bf16(rng.standard_normal((n, d)))
    q_u16 = _bf16(rng.standard_normal((G, d)))
    idx = np.array([3, 7, 8, 30, -1, -1], np.int32)
    o, lse = gqa.attend_group(q_u16, k_u16, v_u16, idx, 0.25)
    for g in range(G):
        og, lg = gqa.attend(q_u16[g], k_u16[[3, 7, 8, 30]], v_u16[[3, 7, 8, 30]], 0.25)
        assert np.array_equal(o[g], og) and lse[g] == lg


def test_window_indices():
    assert list(gqa.window_indices(10, 0)) == list(range(10))
    assert list(gqa.window_indices(10, 4)) == [6, 7, 8, 9]
    assert list(gqa.window_indices(3, 4)) == [0, 1, 2]


# ----------------------------------------------------------------------------- pipeline

@pytest.fixture(scope="module")
def tiny_step():
    w = WORKLOADS["tiny"]
    qc, kc = make_gqa_calibration(w, 0)
    m = cal.calibrate(cal.bf16_to_f64(bf16_bits(qc)), cal.bf16_to_f64(bf16_bits(kc)), w.group, w.rank)
    case = make_gqa_case(w)
    lay = case.layers[0]
    bt = case.block_table.numpy()
    n = int(case.seq_lens[0])
    k_rows = gqa.logical_rows(bf16_bits(lay.k_cache), bt[0], n, w.page_size)
    v_rows = gqa.logical_rows(bf16_bits(lay.v_cache), bt[0], n, w.page_size)
    res = gqa.decode_step(bf16_bits(lay.q)[0], k_rows, v_rows, m.astype(np.float32), w.budget, w.sm_scale)
    return w, case, m, k_rows, v_rows, res


def test_every_needle_selected(tiny_step):
    w, case, _, _, _, res = tiny_step
    for h in range(w.num_kv_heads):
        pos = case.layers[0].needles[(0, h)]
        assert len(pos) == w.seq_len // 100
        assert set(pos.tolist()) <= set(res["idx"][h].tolist())


def test_block_table_permutation_does_not_change_logical_result(tiny_step):
    w, case, m, k_rows, v_rows, res = tiny_step
    lay = case.layers[0]
    bt = case.block_table.numpy()
    rng = np.random.default_rng(9)
    perm = rng.permutation(bt.max() + 1)              # move every physical page elsewhere
    kc = bf16_bits(lay.k_cache)
    kc2 = np.empty_like(kc)
    kc2[perm] = kc
    bt2 = perm[bt]
    k2 = gqa.logical_rows(kc2, bt2[0], w.seq_len, w.page_size)
    assert np.array_equal(k2, k_rows)
    res2 = gqa.decode_step(bf16_bits(lay.q)[0], k2, v_rows, m.astype(np.float32), w.budget, w.sm_scale)
    assert np.array_equal(res2["idx"], res["idx"]) and np.array_equal(res2["out"], res["out"])


def test_sparse_step_close_to_dense(tiny_step):
    """Reported, not a parity claim (accuracy vs full KV is parity unpinned)."""
    w, case, m, k_rows, v_rows, res = tiny_step
    q_u16 = bf16_bits(case.layers[0].q)[0]
    G = w.group
    errs = []
    for j in range(w.num_q_heads):
        h = j // G
        o_dense, _ = gqa.attend(q_u16[j], k_rows[:, h], v_rows[:, h], w.sm_scale)
        errs.append(np.linalg.norm(res["out"][j] - o_dense) / np.linalg.norm(o_dense))
    assert np.median(errs) < 0.5


# ----------------------------------------------------------------------------- MLA

def test_mla_scoring_basis_is_orthonormal_block_diagonal():
    rng = np.random.default_rng(6)
    m = haar_orthogonal(512, 5)[:64].astype(np.float32)
    rows = rng.standard_normal((10, 576))
    y = mla.scoring_rows(rows, m, 512)
    m_ext = np.zeros((128, 576))
    m_ext[:64, :512] = m
    m_ext[64:, 512:] = np.eye(64)
    assert np.abs(m_ext @ m_ext.T - np.eye(128)).max() < 1e-6
    assert np.abs(y - rows @ m_ext.T).max() < 1e-12


def test_mla_reduces_to_gqa_with_one_kv_head():
    """MLA store/project == GQA store/project with Hkv = 1, G = Hq and basis blockdiag(M, I_64)."""
    w = WORKLOADS["tiny_mla"]
    case = make_mla_case(w)
    m = haar_orthogonal(512, 6)[:64].astype(np.float32)
    m_ext = np.zeros((1, 128, 576), np.float32)
    m_ext[0, :64, :512] = m
    m_ext[0, 64:, 512:] = np.eye(64)
    rows = gqa.logical_rows(bf16_bits(case.latent), case.block_table.numpy()[0], 1000, w.page_size)
    c1, s1 = mla.store(rows, m)
    c2, s2 = gqa.store(rows[:, None, :], m_ext)
    assert np.array_equal(c1, c2[:, 0]) and np.array_equal(s1, s2[:, 0])
    q = bf16_bits(case.q)[0]
    assert np.allclose(mla.project_query(q, m), gqa.project_query(q, m_ext, w.num_q_heads)[0], atol=1e-12)


def test_mla_attend_matches_sdpa_and_needles_selected():
    w = WORKLOADS["tiny_mla"]
    case = make_mla_case(w)
    from synth.workloads import population_basis
    m = population_basis(w, 0, 0).astype(np.float32)
    bt = case.block_table.numpy()
    n = int(case.seq_lens[1])
    rows = gqa.logical_rows(bf16_bits(case.latent), bt[1], n, w.page_size)
    q = bf16_bits(case.q)[1]
    res = mla.decode_step(q, rows, m, w.budget, w.sm_scale)
    assert set(case.needles[1].tolist()) <= set(res["idx"].tolist())
    sel = res["idx"][res["idx"] >= 0]
    kv = torch.as_tensor(cal.bf16_to_f64(rows[sel]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(cal.bf16_to_f64(q))[None, :, None], kv[None, None], kv[None, None, :, :512],
        scale=w.sm_scale)[0, :, 0].numpy()
    assert np.abs(res["out"] - ref).max() < 1e-12


# ----------------------------------------------------------------------------- scoring-cache scale formats

def test_e8m0_decode_matches_the_microscaling_definition():
    """E8M0 value 2^(E - 127): E = 127 is 1, 0 is 2^-127, 254 is 2^127 (OCP microscaling formats spec)."""
    assert gqa.e8m0_decode(np.array([127]))[0] == 1.0
    assert gqa.e8m0_decode(np.array([0]))[0] == 2.0 ** -127
    assert gqa.e8m0_decode(np.array([254]))[0] == 2.0 ** 127
    assert gqa.e8m0_decode(np.array([130]))[0] == 8.0


def test_e8m0_scale_is_the_smallest_power_of_two_keeping_rows_in_range():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((4000, 32)) * np.exp(rng.uniform(-20, 20, (4000, 1)))
    y[0] = 0.0
    codes, stored = gqa.quantise_rows(y, "e8m0")
    mult = gqa.e8m0_decode(stored)
    s32 = (np.abs(y).max(axis=1) / 448.0).astype(np.float32).astype(np.float64)
    nz = s32 > 0
    # smallest power of two >= the fp32 scale: 2^e >= s > 2^(e-1)
    assert np.all(mult[nz] >= s32[nz]) and np.all(mult[nz] / 2 < s32[nz])
    assert np.all(codes[0] == 0) and stored[0] == 0
    # dividing by a power of two is exact: the codes are those of y * 2^-e
    assert np.array_equal(codes[nz], fp8.encode(y[nz] / mult[nz, None]))
    # the scaled rows stay in range: |y| / 2^e <= 448
    assert np.all(np.abs(y[nz]) / mult[nz, None] <= 448.0)


def test_e8m0_equals_fp32_when_the_scale_is_a_power_of_two():
    y = np.zeros((3, 16))
    y[:, 0] = [448.0 * 0.25, 448.0 * 8.0, 448.0 * 2.0 ** -20]
    y[:, 1] = [1.0, -3.0, 2.0 ** -21]
    c32, s32 = gqa.quantise_rows(y, "fp32")
    c8, s8 = gqa.quantise_rows(y, "e8m0")
    assert np.array_equal(c32, c8)
    assert np.array_equal(s32.astype(np.float64), gqa.e8m0_decode(s8))
    assert np.array_equal(gqa.scores(np.ones(16), c32, s32, "fp32"), gqa.scores(np.ones(16), c8, s8, "e8m0"))


def test_unscaled_format_stores_the_projection_itself():
    rng = np.random.default_rng(6)
    y = rng.standard_normal((100, 32)) * 50.0
    y[0, 0] = 1000.0                                    # beyond the E4M3FN range: saturates to 448
    codes, stored = gqa.quantise_rows(y, "none")
    assert stored is None
    assert np.array_equal(codes, fp8.encode(y))
    assert fp8.decode(codes[:1, :1])[0, 0] == 448.0
    q = rng.standard_normal(32)
    assert np.allclose(gqa.scores(q, codes, None, "none"), fp8.decode(codes) @ q, rtol=0, atol=0)


def _normal_bf16_patterns():
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e = (u >> 7) & 0xFF
    return u[(e >= 1) & (e <= 254)]


def test_bf16_rounding_round_trips_every_normal_value_and_zero():
    u = _normal_bf16_patterns()
    assert np.array_equal(cal.f64_to_bf16(cal.bf16_to_f64(u)), u)
    assert cal.f64_to_bf16(np.array([0.0]))[0] == 0 and cal.f64_to_bf16(np.array([-0.0]))[0] == 0x8000


def test_bf16_rounding_is_nearest_with_ties_to_even():
    u = _normal_bf16_patterns()
    u = u[(u & 0x7F) != 0x7F]                           # neighbour u + 1 in the same binade
    lo, hi = cal.bf16_to_f64(u), cal.bf16_to_f64(u + 1)
    mid = (lo + hi) / 2                                  # exact in fp64
    even = np.where((u & 1) == 0, u, u + 1)
    assert np.array_equal(cal.f64_to_bf16(mid), even)
    step = (hi - lo) * 2.0 ** -20                        # toward hi (signed: negative values grow downward)
    assert np.array_equal(cal.f64_to_bf16(mid - step), u)
    assert np.array_equal(cal.f64_to_bf16(mid + step), u + 1)
    # a binade's last value and the next power of two
    assert cal.f64_to_bf16(np.array([1.0 + 255 / 256 * 1.0]))[0] == 0x4000      # 1.99609375 -> 2.0 (tie to even)
    with pytest.raises(ValueError):
        cal.f64_to_bf16(np.array([1e39]))


def test_bf16_format_stores_the_rounded_projection_and_scores_it():
    rng = np.random.default_rng(7)
    y = rng.standard_normal((50, 32)) * np.exp(rng.uniform(-10, 10, (50, 1)))
    codes, stored = gqa.quantise_rows(y, "bf16")
    assert stored is None and codes.dtype == np.uint8 and codes.shape == (50, 64)
    h = cal.f64_to_bf16(y)
    assert np.array_equal(codes[:, 0::2], (h & 0xFF).astype(np.uint8))          # little-endian bytes
    assert np.array_equal(codes[:, 1::2], (h >> 8).astype(np.uint8))
    assert np.all(np.abs(gqa.decode_keys(codes, "bf16") - y) <= np.abs(y) * 2.0 ** -8)   # half an ulp of 8 bits
    q = rng.standard_normal(32)
    assert np.array_equal(gqa.scores(q, codes, None, "bf16"), cal.bf16_to_f64(h) @ q)


@pytest.mark.parametrize("fmt", ["e8m0", "none", "bf16"])
def test_scale_formats_keep_the_needles(fmt):
    """Every planted needle is still selected with the coarser scoring caches."""
    from synth import WORKLOADS, make_gqa_case, make_gqa_calibration, bf16_bits
    w = WORKLOADS["tiny"]
    q, k = make_gqa_calibration(w, 0)
    m32 = cal.calibrate(cal.bf16_to_f64(bf16_bits(q)), cal.bf16_to_f64(bf16_bits(k)), w.group, w.rank).astype(np.float32)
    case = make_gqa_case(w)
    lay = case.layers[0]
    bt, n = case.block_table.numpy(), int(case.seq_lens[0])
    kr = gqa.logical_rows(bf16_bits(lay.k_cache), bt[0], n, w.page_size)
    vr = gqa.logical_rows(bf16_bits(lay.v_cache), bt[0], n, w.page_size)
    r = gqa.decode_step(bf16_bits(lay.q)[0], kr, vr, m32, w.budget, w.sm_scale, fmt=fmt)
    for h in range(w.num_kv_heads):
        assert set(lay.needles[(0, h)]) <= set(r["idx"][h])
