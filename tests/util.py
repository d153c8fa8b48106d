"""Test helpers: layout conversion between the oracle's logical arrays and the
library's paged projected scoring cache, tolerance checks, and a few builders.

The paged layout is the one documented in include/jssa.h:
  kp[page][h][i // 16][slot][i % 16], kp_scale[page][h][slot].
"""
from __future__ import annotations

import numpy as np

from oracle import fp8



def pack_kp(codes, scales, block_table, page, n_pages, seq_lens):
    """codes[b] [N_b, Hkv, S] uint8, scales[b] [N_b, Hkv] f32 -> (kp, ks) numpy in the paged layout."""
    hkv, s = codes[0].shape[1], codes[0].shape[2]
    kp = np.zeros((n_pages, hkv, s // 16, page, 16), np.uint8)
    ks = np.zeros((n_pages, hkv, page), np.float32)
    for b, n in enumerate(seq_lens):
        t = np.arange(int(n))
        pg, sl = block_table[b, t // page], t % page
        kp[pg, :, :, sl, :] = codes[b].reshape(len(t), hkv, s // 16, 16)
        ks[pg, :, sl] = scales[b]
    return kp, ks


def unpack_kp(kp, ks, block_row, n, page):
    """Paged (kp, ks) numpy -> logical codes [n, Hkv, S], scales [n, Hkv] of one sequence."""
    t = np.arange(int(n))
    pg, sl = block_row[t // page], t % page
    c = kp[pg, :, :, sl, :]
    return c.reshape(len(t), kp.shape[1], -1), ks[pg, :, sl]


def check_codes(gpu_codes, orc_codes, max_frac=1e-3):
    """FP8 store parity: <= 1 ulp everywhere, differing on <= max_frac of entries. Returns the differing fraction."""
    d = np.abs(fp8.signed_magnitude(gpu_codes) - fp8.signed_magnitude(orc_codes))
    assert d.max(initial=0) <= 1, f"code distance {d.max()} ulp"
    frac = float((d > 0).mean()) if d.size else 0.0
    assert frac <= max_frac, f"{frac:.2e} of codes differ"
    return frac


class CodeTally:
    """FP8 store parity counted over every code a test compares: each entry within 1 ulp (signed-magnitude
    distance), and the differing entries at most max_frac (0.1 %) of all entries compared in the test, not
    of one row (a row of 32 codes cannot express 0.1 %)."""

    def __init__(self):
        self.diff = 0
        self.total = 0

    def add(self, gpu_codes, orc_codes):
        d = np.abs(fp8.signed_magnitude(gpu_codes) - fp8.signed_magnitude(orc_codes))
        assert d.max(initial=0) <= 1, f"code distance {d.max()} ulp"
        self.diff += int((d > 0).sum())
        self.total += int(d.size)

    def check(self, max_frac=1e-3):
        assert self.total > 0
        assert self.diff <= max_frac * self.total, f"{self.diff} of {self.total} codes differ"
        return self.diff


def check_selection(gpu_idx, orc_idx, orc_scores, tau, rel=1e-5):
    """Selected sets equal except tokens whose oracle score is within rel*|tau| of the B-th score.

    gpu_idx / orc_idx: [B] int (-1 padded). Returns the number of exempt tokens."""
    g = gpu_idx[gpu_idx >= 0]
    o = orc_idx[orc_idx >= 0]
    assert len(g) == len(o), f"set sizes {len(g)} vs {len(o)}"
    assert len(np.unique(g)) == len(g), "duplicate positions"
    assert np.all(np.diff(g) > 0), "positions not ascending"
    assert np.all(gpu_idx[len(g):] == -1), "padding not -1"
    diff = np.setxor1d(g, o)
    for t in diff:
        assert abs(orc_scores[t] - tau) <= rel * abs(tau), \
            f"token {t}: score {orc_scores[t]!r} vs tau {tau!r} (rel {abs(orc_scores[t] - tau) / abs(tau):.2e})"
    return len(diff)


U32 = 2.0 ** -24


def score_error_bound(qhat, codes, scale):
    """A-priori bound on |s_gpu - s_oracle| per token for the kernel's fp32 arithmetic.

    The GPU rounds qhat (computed in fp64) to fp32 once (relative u), sums
    qhat_i * dec_i in four FMA chains of S/4 terms, adds the chains pairwise
    (two more roundings) and multiplies by the fp32 scale (one rounding):
      |ds| <= scale * gamma_(S/4 + 3) * sum_i |qhat_i dec_i| + u |s|,
    gamma_n = n u / (1 - n u), u = 2^-24.  dec and scale are exact on both sides."""
    S = codes.shape[-1]
    n = S // 4 + 3
    gamma = n * U32 / (1 - n * U32)
    dec = fp8.decode(codes)
    sc = np.asarray(scale, np.float32).astype(np.float64)
    terms = np.abs(dec) @ np.abs(qhat)
    s = sc * (dec @ qhat)
    return sc * gamma * terms + U32 * np.abs(s)


def check_scores(gpu_scores, qhat, codes, scale, ref):
    """GPU fp32 scores within the a-priori bound of the fp64 oracle scores; returns max |err|."""
    err = np.abs(np.asarray(gpu_scores, np.float64) - ref)
    bound = score_error_bound(qhat, codes, scale)
    bad = np.nonzero(err > bound * 1.0001)[0]
    assert len(bad) == 0, f"{len(bad)} scores outside the bound, e.g. t={bad[0]} err {err[bad[0]]:.3e} " \
                          f"bound {bound[bad[0]]:.3e}"
    return float(err.max(initial=0.0))


def check_attention(got, ref, max_abs=2e-2, mean_abs=2e-3):
    err = np.abs(np.asarray(got, np.float64) - ref)
    assert err.max(initial=0) <= max_abs, f"max abs err {err.max():.3e}"
    assert err.mean() <= mean_abs, f"mean abs err {err.mean():.3e}"
    return float(err.max(initial=0)), float(err.mean())


def slots_for(block_table, seq_lens, page):
    """Physical slot of every position of every sequence, concatenated, and the (b, t) of each."""
    out, who = [], []
    for b, n in enumerate(seq_lens):
        t = np.arange(int(n))
        out.append(block_table[b, t // page] * page + t % page)
        who.append(np.stack([np.full(len(t), b), t], 1))
    return np.concatenate(out).astype(np.int32), np.concatenate(who)
