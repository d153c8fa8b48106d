"""JSSA GQA decode step — oracle (test infrastructure).

Step by step, in the order of the paper summary page, §3.1 Overview, in fp64:

  store    K_proj = K M^T kept in FP8 (§3.4 Projected Scoring Cache; README
           §4 "FP8 projected-key cache"), one fp32 scale per (token, KV head)
  project  qbar = mean of the G query heads of KV head h, qhat = M qbar
           (Theoretical Foundation, Eq. 1; §3.1 step 1)
  score    s^ = qbar^T P k = qhat . (M k), here against the FP8 codes
           (Eq. 1; §3.1 step 2)
  select   the B highest-scoring positions per KV head (§3.1 step 2)
  attend   exact softmax attention of every full-dimensional query head of the
           group over the group's selected positions (§3.1 step 3, §3.3)

Readings where the pages are silent (each listed in the design doc):
  * scale = fp32(max_i |y_i| / 448); codes = RNE-saturating E4M3FN of y_i/scale
    (a zero row stores scale 0 and zero codes);
  * scoring-cache variants (README §4 "Notes": r bytes per token and KV head):
    "e8m0" stores the scale as one byte E with value 2^(E-127), E - 127 =
    ceil(log2 of the fp32 scale above), codes of y_i / 2^(E-127); "none"
    stores no scale, codes of y_i themselves (saturating); "bf16" is the
    README's non-FP8 option (jssa_fp8_projk off: BF16 projected keys), y_i
    rounded to bf16, 2 bytes per element, no scale;
  * the score is scale * sum_i qhat_i dec(code_i) and -0 counts as +0;
  * order by (score descending, position ascending): on a tie at the B-th score
    the lowest position wins; output positions ascending, padded with -1;
  * N <= B selects every position; no forced sink or local window;
  * attention logits x = sm * q.k with sm given; an empty set gives o = 0 and
    lse = -inf.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import fp8
from .calibrate import bf16_to_f64, f64_to_bf16, group_mean


# ------------------------------------------------------------------ paged views

def logical_rows(cache: np.ndarray, block_row: np.ndarray, n: int, page: int) -> np.ndarray:
    """Rows of positions 0..n-1 of one sequence from a paged cache [pages, page, ...]."""
    t = np.arange(n)
    return cache[block_row[t // page], t % page]


# ------------------------------------------------------------------ store

def store(k_u16: np.ndarray, m32: np.ndarray, fmt: str = "fp32") -> Tuple[np.ndarray, np.ndarray]:
    """Project and FP8-quantise keys.

    k_u16 [T, Hkv, d] bf16 bits; m32 [Hkv, r, d] float32 basis.
    Returns codes uint8 [T, Hkv, r] and stored scales [T, Hkv] (see quantise_rows)."""
    k = bf16_to_f64(k_u16)
    m = np.asarray(m32, dtype=np.float32).astype(np.float64)
    y = np.einsum("hrd,thd->thr", m, k)
    return quantise_rows(y, fmt)


SCALE_FORMATS = ("fp32", "e8m0", "none", "bf16")


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """OCP microscaling E8M0 scale byte -> 2^(E - 127) (E = 255, NaN, is never stored)."""
    return np.ldexp(1.0, np.asarray(b).astype(np.int64) - 127)


def quantise_rows(y: np.ndarray, fmt: str = "fp32") -> Tuple[np.ndarray, np.ndarray]:
    """Per-row (last axis) absmax scaling to the E4M3FN range.

    Returns (codes uint8 [..., S], stored scales): float32 for "fp32", uint8
    E8M0 bytes for "e8m0", None for "none".  "bf16" returns the bf16 values of
    y as bytes (uint8 [..., 2S], little-endian) and no scale."""
    if fmt == "none":
        return fp8.encode(y), None
    if fmt == "bf16":
        h = f64_to_bf16(y)
        return np.ascontiguousarray(h).view(np.uint8).reshape(h.shape[:-1] + (2 * h.shape[-1],)), None
    a = np.max(np.abs(y), axis=-1)
    scale = (a / fp8.MAX_FINITE).astype(np.float32)
    s64 = scale.astype(np.float64)
    if fmt == "e8m0":
        m, e = np.frexp(s64)                          # s = m 2^e, m in [0.5, 1): ceil(log2 s) = e, or e - 1 at m = 0.5
        e = np.clip(np.where(m == 0.5, e - 1, e), -127, 127)
        stored = np.where(s64 > 0, e + 127, 0).astype(np.uint8)
        s64 = np.where(s64 > 0, np.ldexp(1.0, e), 0.0)
    elif fmt != "fp32":
        raise ValueError(fmt)
    else:
        stored = scale
    safe = np.where(s64 > 0, s64, 1.0)
    codes = fp8.encode(y / safe[..., None])
    codes = np.where((s64 > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, stored


def scale_multiplier(stored, fmt: str = "fp32"):
    """Stored scales -> the factor the score is multiplied by (fp64)."""
    if fmt in ("none", "bf16"):
        return 1.0
    if fmt == "e8m0":
        return e8m0_decode(stored)
    return np.asarray(stored, dtype=np.float32).astype(np.float64)


# ------------------------------------------------------------------ project + score

def project_query(q_u16: np.ndarray, m32: np.ndarray, group: int) -> np.ndarray:
    """q_u16 [Hq, d] bf16 bits -> qhat [Hkv, r] = M_h qbar_h (fp64)."""
    qbar = group_mean(bf16_to_f64(q_u16), group)
    m = np.asarray(m32, dtype=np.float32).astype(np.float64)
    return np.einsum("hrd,hd->hr", m, qbar)


def decode_keys(codes: np.ndarray, fmt: str = "fp32") -> np.ndarray:
    """Stored projected-key elements -> fp64 values before the scale: FP8 codes
    [..., S], or for "bf16" the bytes [..., 2S] of S bf16 values."""
    if fmt == "bf16":
        c = np.ascontiguousarray(codes)
        return bf16_to_f64(c.view(np.uint16).reshape(c.shape[:-1] + (c.shape[-1] // 2,)))
    return fp8.decode(codes)


def scores(qhat: np.ndarray, codes: np.ndarray, scale, fmt: str = "fp32") -> np.ndarray:
    """Projected scores of one KV head: qhat [r], codes [N, r] (bf16: [N, 2r] bytes), stored scales [N]
    -> [N] fp64."""
    s = scale_multiplier(scale, fmt) * (decode_keys(codes, fmt) @ qhat)
    return np.where(s == 0.0, 0.0, s)


# ------------------------------------------------------------------ select

def select_topb(s: np.ndarray, budget: int) -> Tuple[np.ndarray, float]:
    """Top-B positions by (score desc, position asc); ascending, padded with -1.

    Returns (idx int32 [B], tau) where tau is the B-th score in that order
    (nan when nothing is selected)."""
    n = s.shape[0]
    k = min(budget, n)
    out = np.full(budget, -1, dtype=np.int32)
    if k == 0:
        return out, float("nan")
    order = np.lexsort((np.arange(n), -s))
    out[:k] = np.sort(order[:k])
    return out, float(s[order[k - 1]])


# ------------------------------------------------------------------ attend

def attend(q_u16: np.ndarray, k_u16: np.ndarray, v_u16: np.ndarray, sm: float) -> Tuple[np.ndarray, float]:
    """Softmax attention of one query [d] over rows k [n, d], v [n, dv] (bf16 bits) -> (o [dv], lse)."""
    k = bf16_to_f64(k_u16)
    v = bf16_to_f64(v_u16)
    if k.shape[0] == 0:
        return np.zeros(v.shape[1] if v.ndim == 2 else 0), float("-inf")
    q = bf16_to_f64(q_u16)
    x = sm * (k @ q)
    mx = x.max()
    e = np.exp(x - mx)
    l = e.sum()
    return (e @ v) / l, float(mx + np.log(l))


def attend_group(q_u16: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, idx: np.ndarray,
                 sm: float) -> Tuple[np.ndarray, np.ndarray]:
    """All G query heads of one KV head over one shared index set.

    q_u16 [G, d]; k_rows/v_rows [N, d] logical rows of the KV head; idx [B] (-1 padded).
    Returns o [G, d] and lse [G]."""
    sel = idx[idx >= 0]
    outs, lses = [], []
    for g in range(q_u16.shape[0]):
        o, l = attend(q_u16[g], k_rows[sel], v_rows[sel], sm)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.array(lses)


def window_indices(n: int, window: int) -> np.ndarray:
    """Dense positions [0, n) or, with window > 0, the last `window` of them."""
    lo = max(0, n - window) if window > 0 else 0
    return np.arange(lo, n, dtype=np.int32)


# ------------------------------------------------------------------ one full step

def decode_step(q_u16: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, m32: np.ndarray,
                budget: int, sm: float, codes: np.ndarray = None, scale: np.ndarray = None, fmt: str = "fp32"):
    """One sequence, all KV heads: store all keys (unless codes/scale given), select, attend.

    q_u16 [Hq, d]; k_rows, v_rows [N, Hkv, d]; m32 [Hkv, r, d].
    Returns dict(codes, scale, qhat, scores [Hkv, N], idx [Hkv, B], tau [Hkv], out [Hq, d], lse [Hq])."""
    hkv = k_rows.shape[1]
    group = q_u16.shape[0] // hkv
    if codes is None:
        codes, scale = store(k_rows, m32, fmt)
    qhat = project_query(q_u16, m32, group)
    n = k_rows.shape[0]
    sc = np.zeros((hkv, n))
    idx = np.zeros((hkv, budget), dtype=np.int32)
    tau = np.zeros(hkv)
    out = np.zeros((q_u16.shape[0], v_rows.shape[2]))
    lse = np.zeros(q_u16.shape[0])
    for h in range(hkv):
        sc[h] = scores(qhat[h], codes[:, h], None if scale is None else scale[:, h], fmt)
        idx[h], tau[h] = select_topb(sc[h], budget)
        o, l = attend_group(q_u16[h * group:(h + 1) * group], k_rows[:, h], v_rows[:, h], idx[h], sm)
        out[h * group:(h + 1) * group] = o
        lse[h * group:(h + 1) * group] = l
    return dict(codes=codes, scale=scale, qhat=qhat, scores=sc, idx=idx, tau=tau, out=out, lse=lse)
