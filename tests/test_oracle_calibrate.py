"""Pins for the oracle's calibration (Eq. 1-5) — CPU only."""
import numpy as np
import pytest

from oracle import calibrate as cal
from oracle import gqa
from synth import WORKLOADS, make_gqa_calibration, bf16_bits
from synth.workloads import haar_orthogonal, key_spectrum, query_spectrum, query_amplitude


def _rand_spd(d, rng, decay=1.0):
    u = haar_orthogonal(d, int(rng.integers(1 << 30)))
    lam = np.arange(1, d + 1, dtype=np.float64) ** -decay * rng.uniform(0.5, 1.5, d)
    return (u * lam) @ u.T


def _haar_projector(d, r, rng):
    u = haar_orthogonal(d, int(rng.integers(1 << 30)))
    return u[:, :r] @ u[:, :r].T


@pytest.fixture(scope="module")
def tiny_moments():
    w = WORKLOADS["tiny"]
    q, k = make_gqa_calibration(w, 0)
    q64 = cal.bf16_to_f64(bf16_bits(q))
    k64 = cal.bf16_to_f64(bf16_bits(k))
    gq, gk = cal.moments_per_head(q64, k64, w.group)
    return w, q64, k64, gq, gk


def test_bf16_decode_exact():
    x = np.array([1.0, -2.5, 3.140625, 2.0 ** -100, 0.0, -0.0], dtype=np.float32)
    u16 = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(cal.bf16_to_f64(u16), x.astype(np.float64))


def test_group_mean_contiguous_groups():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((8, 5))
    m = cal.group_mean(q, 4)
    # heads 0..3 -> KV head 0, 4..7 -> KV head 1; G=1 is the identity
    assert np.allclose(m[0], sum(q[i] for i in range(4)) / 4, atol=1e-15)
    assert np.allclose(m[1], sum(q[i] for i in range(4, 8)) / 4, atol=1e-15)
    assert np.array_equal(cal.group_mean(q, 1), q)


def test_second_moments_match_population(tiny_moments):
    """Sample second moments vs the generator's closed-form population moments."""
    w, _, _, gq, gk = tiny_moments
    d, G = w.head_dim, w.group
    for h in range(w.num_kv_heads):
        from synth.workloads import _haar_cached, P_BASIS
        u = _haar_cached(w.model, 0, h, d, P_BASIS)
        pop_k = (u * key_spectrum(d) ** 2) @ u.T
        cq = query_amplitude(d, d)
        pop_q = (u * (cq ** 2 / G) * query_spectrum(d) ** 2) @ u.T
        T = w.calib_seqs * w.calib_len
        for g_hat, pop in ((gk[h], pop_k), (gq[h], pop_q)):
            rel = np.linalg.norm(g_hat - pop) / np.linalg.norm(pop)
            # Gaussian sample second moment: E|S - Sigma|_F^2 = (tr(Sigma)^2 + |Sigma|_F^2) / T
            expect = np.sqrt((np.trace(pop) ** 2 + np.linalg.norm(pop) ** 2) / T) / np.linalg.norm(pop)
            assert 0.5 * expect < rel < 1.5 * expect, (rel, expect)


def test_streamed_moments_equal_batch(tiny_moments):
    w, q, k, gq, gk = tiny_moments
    chunks = [(q[i:i + 300], k[i:i + 300]) for i in range(0, q.shape[0], 300)]
    sq, sk = cal.moments_streamed(chunks, w.group)
    assert np.allclose(sq, gq, rtol=1e-12, atol=1e-14)
    assert np.allclose(sk, gk, rtol=1e-12, atol=1e-14)


def test_basis_orthonormal_and_sign_rule(tiny_moments):
    w, _, _, gq, gk = tiny_moments
    for h in range(w.num_kv_heads):
        m = cal.basis(gq[h], gk[h], w.rank)
        assert m.shape == (w.rank, w.head_dim)
        assert np.abs(m @ m.T - np.eye(w.rank)).max() < 1e-12
        m32 = m.astype(np.float32).astype(np.float64)
        assert np.abs(m32 @ m32.T - np.eye(w.rank)).max() < 1e-6
        for row in m:
            assert row[np.argmax(np.abs(row))] > 0
        assert abs(np.trace(cal.unit_trace(gq[h])) - 1) < 1e-12


def test_ky_fan_closed_form_and_optimality(tiny_moments):
    """Eq. 5: L_marg(M*) equals the sum of the trailing eigenvalues and beats any other rank-r projector."""
    w, _, _, gq, gk = tiny_moments
    rng = np.random.default_rng(3)
    d, r = w.head_dim, w.rank
    for h in range(w.num_kv_heads):
        a = cal.joint_matrix(gq[h], gk[h])
        lam = np.sort(np.linalg.eigvalsh(a))[::-1]
        m = cal.basis(gq[h], gk[h], r)
        best = cal.l_marg(cal.projector(m), gq[h], gk[h])
        assert abs(best - lam[r:].sum()) < 1e-12
        assert abs(lam.sum() - 2.0) < 1e-12          # two unit-trace matrices
        for _ in range(200):
            assert cal.l_marg(_haar_projector(d, r, rng), gq[h], gk[h]) >= best - 1e-12
        from synth.workloads import _haar_cached, P_BASIS
        u = _haar_cached(w.model, 0, h, d, P_BASIS)
        pu = u[:, :r] @ u[:, :r].T
        assert cal.l_marg(pu, gq[h], gk[h]) >= best - 1e-12
        # the calibrated subspace is close to the generator's leading directions
        captured = np.linalg.norm(m @ u[:, :r]) ** 2 / r
        assert captured > 0.8, captured


def test_eq4_bound_on_many_projectors(tiny_moments):
    w, _, _, gq, gk = tiny_moments
    rng = np.random.default_rng(4)
    d, r = w.head_dim, w.rank
    projs = [cal.projector(cal.basis(gq[0], gk[0], r))] + [_haar_projector(d, r, rng) for _ in range(100)]
    for p in projs:
        assert cal.l_sel(p, gq[0], gk[0]) <= 0.25 * cal.l_marg(p, gq[0], gk[0]) ** 2 + 1e-14
    for _ in range(50):                                     # random SPD pairs, random ranks
        dd = int(rng.integers(4, 24))
        rr = int(rng.integers(1, dd))
        a, b = _rand_spd(dd, rng), _rand_spd(dd, rng, 0.5)
        p = _haar_projector(dd, rr, rng)
        assert cal.l_sel(p, a, b) >= -1e-14
        assert cal.l_sel(p, a, b) <= 0.25 * cal.l_marg(p, a, b) ** 2 + 1e-14


def test_eq4_equality_case():
    """A = B = u u^T with u orthogonal to range(P): L_sel = 1 = (1/4) * 2^2."""
    d, r = 10, 3
    u = haar_orthogonal(d, 11)
    p = u[:, :r] @ u[:, :r].T
    v = u[:, r + 2]
    a = np.outer(v, v)
    assert abs(cal.l_sel(p, a, a) - 1.0) < 1e-12
    assert abs(cal.l_marg(p, a, a) - 2.0) < 1e-12


def test_eq2_score_error_identity(tiny_moments):
    """s - s^ = qbar^T (I - P) k with s^ = (M qbar).(M k) from the oracle's projected query."""
    w, _, _, gq, gk = tiny_moments
    rng = np.random.default_rng(5)
    m = np.stack([cal.basis(gq[h], gk[h], w.rank) for h in range(w.num_kv_heads)]).astype(np.float32)
    q = rng.standard_normal((w.num_q_heads, w.head_dim)).astype(np.float32)
    q_u16 = (q.view(np.uint32) >> 16).astype(np.uint16)
    qhat = gqa.project_query(q_u16, m, w.group)
    q64 = cal.bf16_to_f64(q_u16)
    for h in range(w.num_kv_heads):
        qbar = q64[h * w.group:(h + 1) * w.group].mean(0)
        mh = m[h].astype(np.float64)
        p = mh.T @ mh
        for _ in range(20):
            k = rng.standard_normal(w.head_dim)
            s_hat = qhat[h] @ (mh @ k)
            s = qbar @ k
            assert abs((s - s_hat) - qbar @ (np.eye(w.head_dim) - p) @ k) < 1e-12
    # r = d with M = I reproduces the exact score qbar . k
    eye = np.stack([np.eye(w.head_dim, dtype=np.float32)] * w.num_kv_heads)
    qh = gqa.project_query(q_u16, eye, w.group)
    assert np.allclose(qh[1], q64[w.group:2 * w.group].mean(0), atol=1e-15)


# ----------------------------------------------------------------------------- uncentred moments (reading R3)

def test_second_moment_is_uncentred_on_a_hand_example():
    """Rows (1, 2) and (3, 4): (1/2)[[1+9, 2+12], [2+12, 4+16]] = [[5, 7], [7, 10]].  A centred covariance
    would be [[1, 1], [1, 1]] (mean (2, 3) removed), so centring anywhere in the chain fails this."""
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert np.array_equal(cal.second_moment(x), np.array([[5.0, 7.0], [7.0, 10.0]]))
    # the per-head moments over a contiguous group: heads 0, 1 -> KV head 0 with qbar = (1, 2) then (3, 4);
    # keys of KV head 0 are the same rows, so both moments are [[5, 7], [7, 10]]
    q = np.array([[[0.0, 2.0], [2.0, 2.0]], [[3.0, 5.0], [3.0, 3.0]]])        # [T=2, Hq=2, d=2]
    k = x[:, None, :]                                                          # [T=2, Hkv=1, d=2]
    gq, gk = cal.moments_per_head(q, k, 2)
    assert np.array_equal(gq[0], [[5.0, 7.0], [7.0, 10.0]])
    assert np.array_equal(gk[0], [[5.0, 7.0], [7.0, 10.0]])
    sq, sk = cal.moments_streamed([(q[:1], k[:1]), (q[1:], k[1:])], 2)
    assert np.array_equal(sq, gq) and np.array_equal(sk, gk)
    # Eq. 3-5 normalisation: each moment divided by its own trace (15), then added
    a = cal.joint_matrix(gq[0], np.diag([2.0, 2.0]))
    assert np.allclose(a, np.array([[5.0, 7.0], [7.0, 10.0]]) / 15.0 + np.diag([0.5, 0.5]), atol=1e-15)


def test_second_moments_keep_the_mean():
    """A population with a large mean: the uncentred moment is Sigma + mu mu^T, not Sigma."""
    rng = np.random.default_rng(21)
    d, T = 6, 200000
    mu = np.array([3.0, -2.0, 1.0, 0.0, 0.5, 4.0])
    x = rng.standard_normal((T, d)) * 0.5 + mu
    g = cal.second_moment(x)
    pop = 0.25 * np.eye(d) + np.outer(mu, mu)
    assert np.abs(g - pop).max() < 0.05
    assert np.abs(g - 0.25 * np.eye(d)).max() > 10.0


# ----------------------------------------------------------------------------- MLA calibration

def _mla_hand_chunks():
    """latent 2, rope 1, two heads: q rows [t, Hq=2, 3], cached rows [t, 3]."""
    q = np.array([[[1.0, 1.0, 9.0], [1.0, 3.0, -7.0]],       # head mean latent (1, 2)
                  [[2.0, 4.0, 5.0], [4.0, 4.0, 5.0]]])        # head mean latent (3, 4)
    rows = np.array([[1.0, 2.0, 100.0], [3.0, 4.0, -100.0]])  # latent (1, 2), (3, 4); RoPE dim ignored
    return q, rows


def test_mla_moments_hand_example():
    """Head mean of the latent part of the query and the latent part of the cached rows, uncentred, divided by
    the token count; the RoPE dims take no part (they are not projected)."""
    from oracle import mla as omla
    q, rows = _mla_hand_chunks()
    want = np.array([[5.0, 7.0], [7.0, 10.0]])
    gq, gk = omla.moments([(q, rows)], latent=2)
    assert np.array_equal(gq, want) and np.array_equal(gk, want)
    # streamed over chunks: the same; changing the RoPE dims changes nothing
    q2, rows2 = q.copy(), rows.copy()
    q2[..., 2] = 1e3
    rows2[:, 2] = -1e3
    gq2, gk2 = omla.moments([(q2[:1], rows2[:1]), (q2[1:], rows2[1:])], latent=2)
    assert np.array_equal(gq2, want) and np.array_equal(gk2, want)
    # the basis is Eq. 5 on those moments: rank 1 of [[5,7],[7,10]]/15 * 2 = the top eigenvector
    m = omla.calibrate([(q, rows)], latent=2, r=1)
    lam, vec = np.linalg.eigh(want)
    v = vec[:, -1] * np.sign(vec[np.argmax(np.abs(vec[:, -1])), -1])
    assert m.shape == (1, 1, 2)
    assert np.allclose(m[0, 0], v, atol=1e-14)


@pytest.fixture(scope="module")
def mla_moments():
    """The tiny MLA workload's calibration set (1024 tokens, 128 heads, 512 + 64 dims) in fp64."""
    from oracle import mla as omla
    from synth import make_mla_calibration
    w = WORKLOADS["tiny_mla"]
    chunks = [(cal.bf16_to_f64(bf16_bits(q)), cal.bf16_to_f64(bf16_bits(l)))
              for q, l in make_mla_calibration(w, chunk=512)]
    gq, gk = omla.moments(chunks, w.latent_dim)
    return w, chunks, gq, gk


def test_mla_moments_match_population(mla_moments):
    """Cached latents c = U diag(i^-0.8) z: E[c c^T] = U diag(i^-1.6) U^T; the head mean of Hq independent
    query heads amp U diag(i^-0.5) z': E = (amp^2 / Hq) U diag(i^-1) U^T.  Sample deviation as in the GQA pin."""
    import math
    from synth.workloads import _haar_cached, P_BASIS
    w, _, gq, gk = mla_moments
    dl, dr = w.latent_dim, w.rope_dim
    u = _haar_cached(w.model, 0, 0, dl, P_BASIS)
    tot = float(np.sum(np.arange(1, dl + 1, dtype=np.float64) ** -2.6) +
                np.sum(np.arange(1, dr + 1, dtype=np.float64) ** -2.6))
    amp = math.sqrt((128 + dr) / tot)
    pop_k = (u * key_spectrum(dl) ** 2) @ u.T
    pop_q = (u * (amp ** 2 / w.num_q_heads) * query_spectrum(dl) ** 2) @ u.T
    T = w.calib_seqs * w.calib_len
    for g_hat, pop in ((gk, pop_k), (gq, pop_q)):
        rel = np.linalg.norm(g_hat - pop) / np.linalg.norm(pop)
        expect = np.sqrt((np.trace(pop) ** 2 + np.linalg.norm(pop) ** 2) / T) / np.linalg.norm(pop)
        assert 0.5 * expect < rel < 1.5 * expect, (rel, expect)


def test_mla_basis_orthonormal_ky_fan_and_eq4(mla_moments):
    """The MLA basis: orthonormal rows (also in fp32), L_marg equal to the sum of the discarded eigenvalues of
    the normalised moment sum and no larger than that of 200 Haar-random rank-r projectors, Eq. 4 on its
    projector, and the same basis from any chunking of the calibration set."""
    from oracle import mla as omla
    w, chunks, gq, gk = mla_moments
    dl, r = w.latent_dim, w.rank
    m = omla.calibrate(iter(chunks), dl, r)[0]
    assert m.shape == (r, dl)
    assert np.abs(m @ m.T - np.eye(r)).max() < 1e-12
    m32 = m.astype(np.float32).astype(np.float64)
    assert np.abs(m32 @ m32.T - np.eye(r)).max() < 1e-6
    lam = np.sort(np.linalg.eigvalsh(cal.joint_matrix(gq, gk)))[::-1]
    p = cal.projector(m)
    best = cal.l_marg(p, gq, gk)
    assert abs(best - lam[r:].sum()) < 1e-12
    rng = np.random.default_rng(8)
    for _ in range(200):
        assert cal.l_marg(_haar_projector(dl, r, rng), gq, gk) >= best - 1e-12
    assert cal.l_sel(p, gq, gk) <= 0.25 * best ** 2 + 1e-14
    # one chunk of 1024 against two of 512
    q_all = np.concatenate([c[0] for c in chunks])
    r_all = np.concatenate([c[1] for c in chunks])
    m_one = omla.calibrate([(q_all, r_all)], dl, r)[0]
    assert np.abs(np.abs(np.sum(m_one * m, axis=1)) - 1.0).max() < 1e-9
