"""Joint query-key subspace calibration — oracle (test infrastructure).

Follows the paper summary page, "Theoretical Foundation" (Eq. 1-5) and §3.2
"Joint Query-Key Subspace", and the README page's paper-to-code map / §2
"Calibration": per (layer, KV head), accumulate the second moments of the
calibration group-mean queries and of the keys, normalise each to unit trace,
add them, and take the top-r eigenvectors of the sum as the rows of M.

Readings (the pages leave these open):
  * second moments are uncentred averages (1/T) sum x x^T;
  * group g of KV head h is query heads [h*G, (h+1)*G) (contiguous GQA groups);
  * eigenvectors are returned as rows in descending eigenvalue order, each
    sign-normalised so that its largest-magnitude entry is positive (first
    such coordinate on ties).  The projector P = M^T M does not depend on this.
All arithmetic in fp64.
"""
from __future__ import annotations

from typing import Iterable, Tuple

import numpy as np


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64, exactly (bf16 is the top half of fp32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), round to nearest, ties to even, in one step.

    bf16 keeps 8 significant bits of the fp64 value: the 45 low bits of the fp64
    significand are rounded away (ties to the even bit 45), then the result, now
    exactly representable in fp32, gives its top 16 bits.  Valid for the normal
    bf16 range (|x| >= 2^-126) and zero; larger magnitudes than bf16's maximum
    and subnormal results do not occur for projected keys and are rejected."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    r = rounded.view(np.float64)
    a = np.abs(r)
    if np.any((a != 0) & ((a < 2.0 ** -126) | ~np.isfinite(a) | (a > 3.3895313892515355e38))):
        raise ValueError("f64_to_bf16: value outside the normal bf16 range")
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def group_mean(q: np.ndarray, group: int) -> np.ndarray:
    """q [..., Hq, d] -> mean over each contiguous group of G query heads [..., Hq/G, d]
    (summary page, Theoretical Foundation: the mean query of the heads of a KV head)."""
    sh = q.shape
    return q.reshape(sh[:-2] + (sh[-2] // group, group, sh[-1])).mean(axis=-2)


def second_moment(x: np.ndarray) -> np.ndarray:
    """(1/T) sum_t x_t x_t^T for x [T, d]."""
    return (x.T @ x) / x.shape[0]


def unit_trace(g: np.ndarray) -> np.ndarray:
    return g / np.trace(g)


def moments_per_head(q_cal: np.ndarray, k_cal: np.ndarray, group: int) -> Tuple[np.ndarray, np.ndarray]:
    """q_cal [T, Hq, d], k_cal [T, Hkv, d] (fp64) -> (G_Qbar [Hkv,d,d], G_K [Hkv,d,d])."""
    qbar = group_mean(q_cal, group)
    hkv = k_cal.shape[1]
    gq = np.stack([second_moment(qbar[:, h]) for h in range(hkv)])
    gk = np.stack([second_moment(k_cal[:, h]) for h in range(hkv)])
    return gq, gk


def moments_streamed(chunks: Iterable[Tuple[np.ndarray, np.ndarray]], group: int):
    """Same as moments_per_head over an iterator of (q [t,Hq,d], k [t,Hkv,d]) chunks."""
    sq = sk = None
    n = 0
    for q, k in chunks:
        qbar = group_mean(q, group)
        aq = np.einsum("thi,thj->hij", qbar, qbar)
        ak = np.einsum("thi,thj->hij", k, k)
        sq = aq if sq is None else sq + aq
        sk = ak if sk is None else sk + ak
        n += q.shape[0]
    return sq / n, sk / n


def joint_matrix(gq: np.ndarray, gk: np.ndarray) -> np.ndarray:
    """G~_Qbar + G~_K, each unit-trace normalised (Eq. 3-5)."""
    return unit_trace(gq) + unit_trace(gk)


def sign_normalise(rows: np.ndarray) -> np.ndarray:
    out = rows.copy()
    for i in range(out.shape[0]):
        j = int(np.argmax(np.abs(out[i])))
        if out[i, j] < 0:
            out[i] = -out[i]
    return out


def top_eig_rows(a: np.ndarray, r: int) -> Tuple[np.ndarray, np.ndarray]:
    """(M [r, d], eigenvalues of a in descending order) — TopEig_r(a)^T of Eq. 5."""
    lam, vec = np.linalg.eigh(a)            # ascending
    order = np.argsort(-lam, kind="stable")
    lam = lam[order]
    vec = vec[:, order]
    return sign_normalise(vec[:, :r].T), lam


def basis(gq: np.ndarray, gk: np.ndarray, r: int) -> np.ndarray:
    """M* = TopEig_r(G~_Qbar + G~_K)^T for one (layer, KV head) (Eq. 5), fp64 [r, d]."""
    m, _ = top_eig_rows(joint_matrix(gq, gk), r)
    return m


def calibrate(q_cal: np.ndarray, k_cal: np.ndarray, group: int, r: int) -> np.ndarray:
    """Per-KV-head bases M [Hkv, r, d] (fp64) from calibration queries/keys (fp64)."""
    gq, gk = moments_per_head(q_cal, k_cal, group)
    return np.stack([basis(gq[h], gk[h], r) for h in range(gq.shape[0])])


def projector(m: np.ndarray) -> np.ndarray:
    """P = M^T M (summary page, Theoretical Foundation)."""
    return m.T @ m


def l_sel(p: np.ndarray, gq: np.ndarray, gk: np.ndarray) -> float:
    """Exact selection objective tr((I-P) G~_Qbar (I-P) G~_K) (Eq. 3)."""
    i_p = np.eye(p.shape[0]) - p
    return float(np.trace(i_p @ unit_trace(gq) @ i_p @ unit_trace(gk)))


def l_marg(p: np.ndarray, gq: np.ndarray, gk: np.ndarray) -> float:
    """Marginal objective tr((I-P)(G~_Qbar + G~_K)) (Eq. 4)."""
    i_p = np.eye(p.shape[0]) - p
    return float(np.trace(i_p @ joint_matrix(gq, gk)))
