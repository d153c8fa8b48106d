"""JSSA on an MLA layer — oracle (test infrastructure).

The summary page (§3.4 Projected Scoring Cache) gives the MLA scoring
representation as 64 latent + 64 RoPE dimensions (128 in all); the README page
(§2 Calibration) gives the MLA basis shape [1, r, kv_lora_rank] and (the
DeepGEMM patch note in §1 Install) says the score is the plain sum over heads.

Readings (listed in the design doc):
  * the latent part of each cached row [c (512); k_pe (64)] is projected by M
    (r x 512); the 64 RoPE dims pass through unprojected, i.e. the scoring basis
    is blockdiag(M, I_64);
  * the plain head sum equals Hq times the head mean, so the ranking is the
    same; the mean is used (Hkv = 1, G = Hq);
  * one fp32 scale per token over all 128 scoring dims;
  * attention: keys are the full 576-dim rows, values their first 512 dims
    (output [Hq, 512]); the value up-projection is outside this step.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .calibrate import bf16_to_f64, second_moment, basis
from .gqa import quantise_rows, scores, select_topb  # noqa: F401  (same score/select definition)


def scoring_rows(rows64: np.ndarray, m32: np.ndarray, latent: int) -> np.ndarray:
    """[c; k_pe] (fp64, [T, latent+rope]) -> [M c ; k_pe] (fp64, [T, r+rope])."""
    m = np.asarray(m32, dtype=np.float32).astype(np.float64)
    return np.concatenate([rows64[:, :latent] @ m.T, rows64[:, latent:]], axis=1)


def store(rows_u16: np.ndarray, m32: np.ndarray, latent: int = 512, fmt: str = "fp32") -> Tuple[np.ndarray, np.ndarray]:
    """rows [T, 576] bf16 bits -> codes uint8 [T, r+rope], stored scales [T] (see gqa.quantise_rows)."""
    return quantise_rows(scoring_rows(bf16_to_f64(rows_u16), m32, latent), fmt)


def project_query(q_u16: np.ndarray, m32: np.ndarray, latent: int = 512) -> np.ndarray:
    """q [Hq, 576] -> qhat [r+rope] = [M qbar[:latent]; qbar[latent:]] with qbar the head mean."""
    qbar = bf16_to_f64(q_u16).mean(axis=0)
    return scoring_rows(qbar[None, :], m32, latent)[0]


def attend(q_u16: np.ndarray, rows_u16: np.ndarray, sm: float, latent: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """All heads over the selected latent rows: q [Hq, 576], rows [n, 576] -> (o [Hq, latent], lse [Hq])."""
    q = bf16_to_f64(q_u16)
    kv = bf16_to_f64(rows_u16)
    hq = q.shape[0]
    if kv.shape[0] == 0:
        return np.zeros((hq, latent)), np.full(hq, -np.inf)
    x = sm * (q @ kv.T)                           # [Hq, n]
    mx = x.max(axis=1, keepdims=True)
    e = np.exp(x - mx)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ kv[:, :latent]) / l
    return o, (mx + np.log(l))[:, 0]


def moments(q_chunks, latent: int) -> Tuple[np.ndarray, np.ndarray]:
    """(G_Qbar, G_K) [latent, latent] from an iterator of (q [t, Hq, latent+rope], rows [t, latent+rope]) fp64
    chunks: the uncentred second moments (1/T) sum x x^T of the head-mean query's latent part and of the cached
    latents c (the RoPE dims are not projected, so they take no part)."""
    sq = sk = None
    n = 0
    for q, rows in q_chunks:
        qbar = q.mean(axis=1)[:, :latent]
        c = rows[:, :latent]
        aq = qbar.T @ qbar
        ak = c.T @ c
        sq = aq if sq is None else sq + aq
        sk = ak if sk is None else sk + ak
        n += q.shape[0]
    return sq / n, sk / n


def calibrate(q_chunks, latent: int, r: int) -> np.ndarray:
    """Basis M [1, r, latent]: the moments above, each unit-trace normalised, then Eq. 5 (summary page,
    Theoretical Foundation; README page §2 Calibration gives the MLA basis shape [1, r, kv_lora_rank])."""
    gq, gk = moments(q_chunks, latent)
    return basis(gq, gk, r)[None]


def decode_step(q_u16: np.ndarray, rows_u16: np.ndarray, m32: np.ndarray, budget: int, sm: float,
                latent: int = 512, codes: np.ndarray = None, scale: np.ndarray = None):
    """One sequence: q [Hq, 576], rows [N, 576] (logical order), m32 [r, latent]."""
    if codes is None:
        codes, scale = store(rows_u16, m32, latent)
    qhat = project_query(q_u16, m32, latent)
    sc = scores(qhat, codes, scale)
    idx, tau = select_topb(sc, budget)
    o, lse = attend(q_u16, rows_u16[idx[idx >= 0]], sm, latent)
    return dict(codes=codes, scale=scale, qhat=qhat, scores=sc, idx=idx, tau=tau, out=o, lse=lse)


__all__ = ["store", "project_query", "attend", "moments", "calibrate", "decode_step", "scoring_rows",
           "second_moment"]
