"""Seeded synthetic decode workloads for the JSSA decode path.

This module only *generates inputs*: paged bf16 K/V caches, block tables,
decode-step queries and calibration sequences with the shapes and value
structure of the workloads the pages measure on (Llama-3.1-8B-dims layer at
32K/128K, a hybrid sliding-window/global stack, a DeepSeek-V3-shaped MLA
layer).  It holds none of the method's arithmetic: no basis, no projection,
no quantisation, no scoring, no selection and no attention.  Both the CPU
oracle (through the tests) and the HIP library (through the tests and the
benchmark) consume the tensors it returns.

Value recipe (builder's choice; the pages use model activations and a
"synthetic paged cache"):

* per (layer, KV head) a Haar-random orthogonal U (QR of a Gaussian, columns
  sign-fixed by the diagonal of R);
* keys   k = U diag(i^-0.8) z,  z ~ N(0, I_d);
* queries of each head of the group, independently,
         q = c_q U diag(i^-0.5) z',  c_q = sqrt(d / sum_i i^-2.6), which gives
  unit-std logits q.k/sqrt(d);
* values v ~ N(0, I_d);
* needles: floor(N/100) positions per (sequence, KV head), drawn without
  replacement from [0, N-1); each gets k += (8 sigma / |qbar|) qbar where qbar
  is the mean of the (bf16) queries of the group and sigma is the std of
  qbar.k over the base keys, so its exact score rises by 8 sigma;
* everything rounded to bf16 (round to nearest even) at the end;
* block table: a random permutation of all physical pages.

MLA rows are [c (512) ; k_pe (64)] with c = U_c diag(i^-0.8) z and k_pe drawn the
same way from its own U_pe; per-head queries use the same two bases with decay
i^-0.5.

Seeds: numpy SeedSequence(0, spawn_key=(model, layer, head, purpose)), one
32-bit torch generator seed per stream, so a workload is reproducible on a
given device type.  CPU and GPU generators give different (equally valid)
streams; a test always hands the *same* tensors to both sides.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

# purposes (part of the seed key)
P_BASIS, P_KEYS, P_QUERIES, P_VALUES, P_NEEDLES, P_CAL_K, P_CAL_Q, P_BLOCKS, P_PE_BASIS = range(9)

MODEL_IDS = {"tiny": 1, "llama8b": 2, "hybrid": 4, "mla": 5, "tiny_mla": 6, "test": 7}


@dataclass(frozen=True)
class Workload:
    name: str
    model: str                 # seed namespace: workloads of one model share bases
    kind: str                  # "gqa" | "mla"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int              # GQA d; MLA 576 = latent + rope
    seq_len: int               # N, including the token being decoded
    page_size: int
    rank: int                  # GQA r; MLA latent rank (scoring dims = rank + rope_dim)
    budget: int                # B
    calib_seqs: int
    calib_len: int
    num_layers: int = 1
    window: int = 0            # >0: even layers are dense sliding-window layers
    latent_dim: int = 0        # MLA only
    rope_dim: int = 0          # MLA only
    needle_frac: float = 0.01
    query_shift: int = 0       # >0: the query spectrum is rolled by this many of the basis' directions

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> float:
        if self.kind == "mla":
            return 1.0 / math.sqrt(128 + self.rope_dim)
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def pages_per_seq(self) -> int:
        return -(-self.seq_len // self.page_size)

    @property
    def num_pages(self) -> int:
        return self.batch * self.pages_per_seq

    @property
    def v_dim(self) -> int:
        return self.latent_dim if self.kind == "mla" else self.head_dim

    @property
    def score_dims(self) -> int:
        return self.rank + self.rope_dim if self.kind == "mla" else self.rank

    def global_layers(self) -> Tuple[int, ...]:
        """Layers that run the sparse path (all of them unless windowed)."""
        if self.window > 0:
            return tuple(l for l in range(self.num_layers) if l % 2 == 1)
        return tuple(range(self.num_layers))

    def window_layers(self) -> Tuple[int, ...]:
        if self.window > 0:
            return tuple(l for l in range(self.num_layers) if l % 2 == 0)
        return ()

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny GQA decode step
    "tiny": Workload("tiny", "tiny", "gqa", batch=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                     seq_len=4096, page_size=16, rank=32, budget=256, calib_seqs=2, calib_len=1024),
    # Llama-3-8B-shaped layer, 32K
    "llama8b_32k": Workload("llama8b_32k", "llama8b", "gqa", batch=16, num_q_heads=32, num_kv_heads=8,
                            head_dim=128, seq_len=32768, page_size=16, rank=32, budget=2048,
                            calib_seqs=4, calib_len=4096),
    # same layer (same bases, same calibration) at 128K
    "llama8b_128k": Workload("llama8b_128k", "llama8b", "gqa", batch=8, num_q_heads=32, num_kv_heads=8,
                             head_dim=128, seq_len=131072, page_size=16, rank=32, budget=2048,
                             calib_seqs=4, calib_len=4096),
    # hybrid sliding-window / global stack
    "hybrid_64k": Workload("hybrid_64k", "hybrid", "gqa", batch=8, num_q_heads=16, num_kv_heads=8,
                           head_dim=256, seq_len=65536, page_size=16, rank=48, budget=2048,
                           calib_seqs=4, calib_len=4096, num_layers=6, window=1024),
    # DeepSeek-V3-shaped MLA layer
    "mla_128k": Workload("mla_128k", "mla", "mla", batch=8, num_q_heads=128, num_kv_heads=1,
                         head_dim=576, seq_len=131072, page_size=64, rank=64, budget=2048,
                         calib_seqs=4, calib_len=4096, latent_dim=512, rope_dim=64),
    # small MLA case for CPU-sized parity
    "tiny_mla": Workload("tiny_mla", "tiny_mla", "mla", batch=2, num_q_heads=128, num_kv_heads=1,
                         head_dim=576, seq_len=3000, page_size=64, rank=64, budget=256,
                         calib_seqs=2, calib_len=512, latent_dim=512, rope_dim=64),
}


def seed_for(model: str, layer: int, head: int, purpose: int, extra: int = 0) -> int:
    ss = np.random.SeedSequence(0, spawn_key=(MODEL_IDS.get(model, 99), layer, head, purpose, extra))
    return int(ss.generate_state(1, dtype=np.uint32)[0])


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def haar_orthogonal(d: int, seed: int) -> np.ndarray:
    """Haar-distributed d x d orthogonal matrix (fp64)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((d, d))
    qm, rm = np.linalg.qr(a)
    return qm * np.sign(np.diag(rm))[None, :]


def key_spectrum(d: int) -> np.ndarray:
    return np.arange(1, d + 1, dtype=np.float64) ** -0.8


def query_spectrum(d: int) -> np.ndarray:
    return np.arange(1, d + 1, dtype=np.float64) ** -0.5


def query_amplitude(d: int, logit_dims: int) -> float:
    """c_q giving unit-std logits q.k / sqrt(logit_dims) (i^-0.5 * i^-0.8 = i^-1.3)."""
    return math.sqrt(logit_dims / float(np.sum(np.arange(1, d + 1, dtype=np.float64) ** -2.6)))


@functools.lru_cache(maxsize=256)
def _haar_cached(model: str, layer: int, head: int, d: int, purpose: int) -> np.ndarray:
    u = haar_orthogonal(d, seed_for(model, layer, head, purpose))
    u.setflags(write=False)
    return u


def _factor(w: Workload, layer: int, head: int, d: int, spectrum: np.ndarray, purpose=P_BASIS) -> np.ndarray:
    """U diag(spectrum) as fp64 (d x d)."""
    return _haar_cached(w.model, layer, head, d, purpose) * spectrum[None, :]


def _draw(shape, seed, device) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)


def _draw_rows(n: int, fac: np.ndarray, seed: int, device, scale: float = 1.0) -> torch.Tensor:
    """n rows of scale * fac @ z (fp32, [n, d])."""
    d = fac.shape[0]
    z = _draw((n, d), seed, device)
    f = torch.as_tensor(fac.T * scale, dtype=torch.float32, device=device)
    return z @ f


def _seq_lens(w: Workload, ragged: bool) -> np.ndarray:
    if ragged:
        return np.array([max(1, w.seq_len - 37 * b) for b in range(w.batch)], dtype=np.int32)
    return np.full(w.batch, w.seq_len, dtype=np.int32)


def make_block_table(w: Workload, pages_per_seq: Optional[int] = None) -> np.ndarray:
    pps = pages_per_seq or w.pages_per_seq
    rng = np.random.default_rng(seed_for(w.model, 0, 0, P_BLOCKS, w.batch * 1000003 + pps))
    perm = rng.permutation(w.batch * pps).astype(np.int32)
    return perm.reshape(w.batch, pps)


def _needles(n_valid: int, frac: float, seed: int) -> np.ndarray:
    cnt = int(math.floor(n_valid * frac))
    if cnt == 0 or n_valid < 2:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n_valid - 1, size=min(cnt, n_valid - 1), replace=False)).astype(np.int64)


def _plant(keys: torch.Tensor, qbar: torch.Tensor, pos: np.ndarray) -> None:
    """keys[pos] += (8 sigma/|qbar|) qbar, sigma = std_t(qbar . k_t) over the base keys."""
    if len(pos) == 0:
        return
    s = keys.double() @ qbar.double()
    sigma = float(s.std())
    direction = (8.0 * sigma / float(qbar.double().norm())) * qbar.double()
    idx = torch.as_tensor(pos, device=keys.device)
    keys[idx] = (keys[idx].double() + direction[None, :]).float()


@dataclass
class GQALayer:
    q: torch.Tensor            # bf16 [batch, Hq, d]
    k_cache: torch.Tensor      # bf16 [num_pages, page, Hkv, d]
    v_cache: torch.Tensor      # bf16 [num_pages, page, Hkv, d]
    needles: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)


@dataclass
class GQACase:
    w: Workload
    block_table: torch.Tensor  # int32 [batch, pages_per_seq]
    seq_lens: torch.Tensor     # int32 [batch]
    layers: Dict[int, GQALayer]


def make_gqa_layer(w: Workload, layer: int, block_table: np.ndarray, seq_lens: np.ndarray,
                   device="cpu", needles: bool = True) -> GQALayer:
    B, Hq, Hkv, d, P, G = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.group
    pps = block_table.shape[1]
    n_pages = int(block_table.max()) + 1
    kc = torch.zeros((n_pages, P, Hkv, d), dtype=torch.bfloat16, device=device)
    vc = torch.zeros((n_pages, P, Hkv, d), dtype=torch.bfloat16, device=device)
    q = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=device)
    cq = query_amplitude(d, d)
    kfacs = [_factor(w, layer, h, d, key_spectrum(d)) for h in range(Hkv)]
    qfacs = [_factor(w, layer, h, d, np.roll(query_spectrum(d), w.query_shift)) for h in range(Hkv)]
    bt = torch.as_tensor(block_table.astype(np.int64), device=device)
    planted = {}
    for b in range(B):
        n = int(seq_lens[b])
        npg = -(-n // P)
        for h in range(Hkv):
            for g in range(G):
                j = h * G + g
                q[b, j] = _draw_rows(1, qfacs[h], seed_for(w.model, layer, j, P_QUERIES, b), device, cq)[0].to(torch.bfloat16)
            keys = _draw_rows(npg * P, kfacs[h], seed_for(w.model, layer, h, P_KEYS, b), device)
            vals = _draw((npg * P, d), seed_for(w.model, layer, h, P_VALUES, b), device)
            if needles:
                qbar = q[b, h * G:(h + 1) * G].float().mean(0)
                pos = _needles(n, w.needle_frac, seed_for(w.model, layer, h, P_NEEDLES, b))
                _plant(keys[:n], qbar, pos)
                planted[(b, h)] = pos
            keys[n:] = 0
            vals[n:] = 0
            kc[bt[b, :npg], :, h, :] = keys.view(npg, P, d).to(torch.bfloat16)
            vc[bt[b, :npg], :, h, :] = vals.view(npg, P, d).to(torch.bfloat16)
    return GQALayer(q=q, k_cache=kc, v_cache=vc, needles=planted)


def make_gqa_case(w: Workload, device="cpu", ragged: bool = False, layers: Optional[Sequence[int]] = None,
                  needles: bool = True) -> GQACase:
    bt = make_block_table(w)
    sl = _seq_lens(w, ragged)
    todo = range(w.num_layers) if layers is None else layers
    out = {}
    for l in todo:
        out[l] = make_gqa_layer(w, l, bt, sl, device, needles=needles and l in w.global_layers())
    return GQACase(w=w, block_table=torch.as_tensor(bt, device=device),
                   seq_lens=torch.as_tensor(sl, device=device), layers=out)


def make_gqa_calibration(w: Workload, layer: int, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Calibration queries [T, Hq, d] and keys [T, Hkv, d] (bf16), no needles."""
    Hq, Hkv, d, G = w.num_q_heads, w.num_kv_heads, w.head_dim, w.group
    T = w.calib_seqs * w.calib_len
    cq = query_amplitude(d, d)
    qs = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=device)
    ks = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=device)
    for h in range(Hkv):
        kf = _factor(w, layer, h, d, key_spectrum(d))
        qf = _factor(w, layer, h, d, np.roll(query_spectrum(d), w.query_shift))
        ks[:, h] = _draw_rows(T, kf, seed_for(w.model, layer, h, P_CAL_K), device).to(torch.bfloat16)
        for g in range(G):
            j = h * G + g
            qs[:, j] = _draw_rows(T, qf, seed_for(w.model, layer, j, P_CAL_Q), device, cq).to(torch.bfloat16)
    return qs, ks


def population_basis(w: Workload, layer: int, head: int) -> np.ndarray:
    """The generator's own U_r^T (r x d): the leading directions of both spectra."""
    u = _haar_cached(w.model, layer, head, w.head_dim if w.kind == "gqa" else w.latent_dim, P_BASIS)
    return u[:, :w.rank].T.copy()


# ----------------------------------------------------------------------------- MLA

@dataclass
class MLACase:
    w: Workload
    q: torch.Tensor            # bf16 [batch, Hq, 576]
    latent: torch.Tensor       # bf16 [num_pages, page, 576]
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    needles: Dict[int, np.ndarray] = field(default_factory=dict)


def _mla_factors(w: Workload, spectrum_fn):
    dl, dr = w.latent_dim, w.rope_dim
    fc = _factor(w, 0, 0, dl, spectrum_fn(dl), P_BASIS)
    fr = _factor(w, 0, 0, dr, spectrum_fn(dr), P_PE_BASIS)
    return fc, fr


def _mla_rows(w: Workload, n: int, seed_c: int, seed_r: int, device, query: bool) -> torch.Tensor:
    dl, dr = w.latent_dim, w.rope_dim
    spec = query_spectrum if query else key_spectrum
    fc, fr = _mla_factors(w, spec)
    amp = 1.0
    if query:
        tot = float(np.sum(np.arange(1, dl + 1, dtype=np.float64) ** -2.6) +
                    np.sum(np.arange(1, dr + 1, dtype=np.float64) ** -2.6))
        amp = math.sqrt((128 + dr) / tot)
    c = _draw_rows(n, fc, seed_c, device, amp)
    r = _draw_rows(n, fr, seed_r, device, amp)
    return torch.cat([c, r], dim=1)


def make_mla_case(w: Workload, device="cpu", ragged: bool = False, needles: bool = True) -> MLACase:
    assert w.kind == "mla"
    B, Hq, P, D = w.batch, w.num_q_heads, w.page_size, w.head_dim
    bt = make_block_table(w)
    sl = _seq_lens(w, ragged)
    n_pages = int(bt.max()) + 1
    lat = torch.zeros((n_pages, P, D), dtype=torch.bfloat16, device=device)
    q = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=device)
    btt = torch.as_tensor(bt.astype(np.int64), device=device)
    planted = {}
    for b in range(B):
        n = int(sl[b])
        npg = -(-n // P)
        for j in range(Hq):
            q[b, j] = _mla_rows(w, 1, seed_for(w.model, 0, j, P_QUERIES, b),
                                seed_for(w.model, 1, j, P_QUERIES, b), device, True)[0].to(torch.bfloat16)
        rows = _mla_rows(w, npg * P, seed_for(w.model, 0, 0, P_KEYS, b), seed_for(w.model, 1, 0, P_KEYS, b),
                         device, False)
        if needles:
            qbar = q[b].float().mean(0)
            pos = _needles(n, w.needle_frac, seed_for(w.model, 0, 0, P_NEEDLES, b))
            _plant(rows[:n], qbar, pos)
            planted[b] = pos
        rows[n:] = 0
        lat[btt[b, :npg]] = rows.view(npg, P, D).to(torch.bfloat16)
    return MLACase(w=w, q=q, latent=lat, block_table=torch.as_tensor(bt, device=device),
                   seq_lens=torch.as_tensor(sl, device=device), needles=planted)


def make_mla_calibration(w: Workload, device="cpu", chunk: int = 512):
    """Yields (q [t, Hq, 576], latent [t, 576]) bf16 chunks of the calibration set."""
    T = w.calib_seqs * w.calib_len
    for c0 in range(0, T, chunk):
        t = min(chunk, T - c0)
        lat = _mla_rows(w, t, seed_for(w.model, 0, 0, P_CAL_K, c0), seed_for(w.model, 1, 0, P_CAL_K, c0),
                        device, False).to(torch.bfloat16)
        qs = torch.empty((t, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=device)
        for j in range(w.num_q_heads):
            qs[:, j] = _mla_rows(w, t, seed_for(w.model, 0, j, P_CAL_Q, c0), seed_for(w.model, 1, j, P_CAL_Q, c0),
                                 device, True).to(torch.bfloat16)
        yield qs, lat


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit pattern (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
