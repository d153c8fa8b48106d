"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, validates arguments before touching the device, and its host
eigensolver (jssa_basis) matches the oracle's calibration."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

L = pytest.importorskip("long_context_decode_amd")


def _declared():
    src = open(os.path.join(ROOT, "include", "jssa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(jssa_\w+)\s*\(", src)))


def test_header_symbols_exported():
    lib = ctypes.CDLL(L.LIB_PATH)
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


def test_status_strings():
    for s in range(-6, 1):
        assert L.status_string(s) and L.status_string(s) != "unknown status"
    assert L.status_string(7) == "unknown status"


def _shape(**kw):
    base = dict(kind=0, batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                max_pages_per_seq=8192, rank=32, budget=2048, select_mode=0)
    base.update(kw)
    return L.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=30), -2), (dict(budget=0), -2), (dict(budget=5000), -2), (dict(batch=0), -2),
    (dict(head_dim=64), -3), (dict(page_size=8), -3), (dict(rank=24), -3), (dict(rank=256, head_dim=256), -3),
    (dict(num_q_heads=48), -3), (dict(kind=7), -3), (dict(select_mode=4), -2), (dict(select_mode=-1), -2),
    (dict(select_mode=3), 0),
    (dict(kind=1, num_kv_heads=2, num_q_heads=128, head_dim=576, rank=64), -3),
    (dict(kind=1, num_kv_heads=1, num_q_heads=128, head_dim=576, rank=64, page_size=64), 0),
])
def test_shape_validation(kw, status):
    n = ctypes.c_size_t()
    st = L.raw_library().jssa_workspace_bytes(ctypes.byref(_shape(**kw)), ctypes.byref(n))
    assert st == status


@pytest.mark.parametrize("kw,mode,single", [
    # the tiny workload's shape: capacity 4096, G = 4, d = 128, r = 32
    (dict(batch=1, num_q_heads=8, num_kv_heads=2, max_pages_per_seq=256, budget=256), L.SELECT_AUTO, 1),
    (dict(batch=1, num_q_heads=8, num_kv_heads=2, max_pages_per_seq=256, budget=256), L.SELECT_FUSED, 1),
    (dict(batch=1, num_q_heads=8, num_kv_heads=2, max_pages_per_seq=256, budget=256), L.SELECT_SPLIT, 0),
    (dict(batch=1, num_q_heads=8, num_kv_heads=2, max_pages_per_seq=256, budget=256), L.SELECT_EXACT_STREAM, 0),
    (dict(max_pages_per_seq=768), L.SELECT_AUTO, 1),                      # capacity 12288: the limit
    (dict(max_pages_per_seq=769), L.SELECT_AUTO, 0),                      # one page more
    (dict(max_pages_per_seq=769), L.SELECT_FUSED, -3),
    (dict(max_pages_per_seq=192, page_size=64), L.SELECT_AUTO, 1),        # 12288 tokens in pages of 64
    (dict(max_pages_per_seq=256, num_q_heads=64), L.SELECT_AUTO, 0),      # G = 8: G * d = 1024
    (dict(max_pages_per_seq=256, head_dim=256, num_q_heads=16), L.SELECT_AUTO, 1),   # d = 256, G = 2
    (dict(max_pages_per_seq=256, head_dim=256), L.SELECT_AUTO, 0),        # d = 256, G = 4
    (dict(max_pages_per_seq=256, rank=64), L.SELECT_AUTO, 1),
    (dict(max_pages_per_seq=256, rank=80), L.SELECT_AUTO, 0),             # r > 64
    (dict(max_pages_per_seq=256, rank=80), L.SELECT_FUSED, -3),
    (dict(max_pages_per_seq=256, budget=4096), L.SELECT_AUTO, 1),
    (dict(), L.SELECT_AUTO, 0),                                           # the 128K layer: split path
    (dict(kind=1, num_kv_heads=1, num_q_heads=128, head_dim=576, rank=64, page_size=64, max_pages_per_seq=64),
     L.SELECT_AUTO, 0),                                                   # MLA: split path
])
def test_decode_path(kw, mode, single):
    """Which path jssa_decode takes (the single launch covers GQA with capacity <= 12288, r <= 64, G * d <= 512)."""
    v = ctypes.c_int32(-7)
    st = L.raw_library().jssa_decode_path(ctypes.byref(_shape(select_mode=mode, **kw)), ctypes.byref(v))
    if single < 0:
        assert st == single
    else:
        assert st == 0 and v.value == single


def test_workspace_and_page_sizes():
    s = _shape()
    ws = L.workspace_bytes(s)
    # candidate regions (one (key, position) slot per cached token and KV head) and the
    # gather-then-attend staging cache (B rows of K and V per sequence and KV head) dominate
    cand = 8 * 8 * 8192 * 16 * 8
    stage = 2 * 8 * 8 * 2048 * 128 * 2
    assert cand + stage < ws < cand + stage + 16 * 1024 * 1024
    assert L.kp_page_bytes(s) == (8 * 16 * 32, 8 * 16)
    m = _shape(kind=1, num_kv_heads=1, num_q_heads=128, head_dim=576, rank=64, page_size=64)
    assert L.kp_page_bytes(m) == (64 * 128, 64)
    # scale-free formats: no scale elements; BF16 keys take two bytes per element
    assert L.kp_page_bytes(_shape(scale_format=L.SCALE_NONE)) == (8 * 16 * 32, 0)
    assert L.kp_page_bytes(_shape(scale_format=L.KEYS_BF16)) == (2 * 8 * 16 * 32, 0)
    n = ctypes.c_size_t()
    assert L.raw_library().jssa_workspace_bytes(ctypes.byref(_shape(scale_format=4)), ctypes.byref(n)) == -3


def test_store_of_no_tokens_is_a_no_op_before_any_check():
    """T = 0 returns success before the pointers are looked at: nothing is launched (no device here)."""
    null = ctypes.c_void_p(0)
    assert L.raw_library().jssa_store(ctypes.byref(_shape()), null, null, 0, null, null, null, null) == 0
    assert L.raw_library().jssa_store(ctypes.byref(_shape()), null, null, -1, null, null, null, null) != 0


def test_entry_points_reject_before_launch():
    """Errors come back from host validation; nothing touches the device (there is none here)."""
    lib = L.raw_library()
    s = _shape()
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    ref = ctypes.byref(s)
    assert lib.jssa_select(ref, nul, fake, fake, fake, fake, fake, fake, nul, fake, 1 << 40, nul) == -1
    assert lib.jssa_select(ref, fake, fake, fake, fake, fake, fake, fake, nul, fake, 16, nul) == -4
    assert lib.jssa_attend(ref, fake, fake, fake, fake, fake, nul, 0.1, fake, nul, fake, 1 << 40, nul) == -1
    assert lib.jssa_attend(ref, fake, fake, fake, fake, fake, fake, 0.1, fake, nul, fake, 16, nul) == -4
    assert lib.jssa_full_decode(ref, fake, fake, fake, fake, fake, -1, 0.1, fake, nul, fake, 1 << 40, nul) == -2
    assert lib.jssa_gather_attend(ref, fake, fake, fake, fake, fake, nul, 0.1, fake, nul, fake, 1 << 40, nul) == -1
    assert lib.jssa_gather_attend(ref, fake, fake, fake, fake, fake, fake, 0.1, fake, nul, fake, 16, nul) == -4
    assert lib.jssa_decode(ref, fake, fake, nul, fake, fake, fake, fake, fake, fake, fake, fake, 0.1, fake, nul,
                           fake, 1 << 40, nul) == -1
    # the single-launch path refuses shapes it does not cover (capacity 131072 > 12288), before any launch
    fused = _shape(select_mode=L.SELECT_FUSED)
    assert lib.jssa_decode(ctypes.byref(fused), fake, nul, nul, fake, fake, fake, fake, fake, fake, fake, fake, 0.1,
                           fake, nul, fake, 1 << 40, nul) == -3
    assert lib.jssa_store(ref, nul, fake, 4, fake, fake, fake, nul) == -1
    assert lib.jssa_store(ref, fake, fake, -1, fake, fake, fake, nul) == -2
    assert lib.jssa_store(ref, nul, nul, 0, nul, nul, nul, nul) == 0          # T = 0: nothing to do
    bad = _shape(head_dim=64)
    assert lib.jssa_select(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, fake, nul, fake, 1 << 40, nul) == -3
    assert lib.jssa_calib_moments(ref, nul, fake, 4, fake, fake, fake, 1 << 30, nul) == -1
    assert lib.jssa_calib_moments(ref, fake, fake, 4, fake, fake, fake, 8, nul) == -4


def test_host_basis_matches_oracle_calibration():
    """jssa_basis (C++ Householder + QL) spans the oracle's subspace (numpy eigh)."""
    from oracle import calibrate as cal
    from synth import WORKLOADS, make_gqa_calibration, bf16_bits
    w = WORKLOADS["tiny"]
    q, k = make_gqa_calibration(w, 0)
    q64, k64 = cal.bf16_to_f64(bf16_bits(q)), cal.bf16_to_f64(bf16_bits(k))
    gq, gk = cal.moments_per_head(q64, k64, w.group)
    T = q64.shape[0]
    m = L.jssa_basis(L.shape_for(w), (gq * T).astype(np.float32), (gk * T).astype(np.float32))
    for h in range(w.num_kv_heads):
        mo = cal.basis(gq[h], gk[h], w.rank)
        mh = m[h].astype(np.float64)
        assert np.abs(mh @ mh.T - np.eye(w.rank)).max() < 1e-5
        # same projector (the eigengap keeps it well conditioned), same sign rule
        assert np.abs(mh.T @ mh - mo.T @ mo).max() < 1e-3
        assert abs(cal.l_marg(mh.T @ mh, gq[h], gk[h]) - cal.l_marg(mo.T @ mo, gq[h], gk[h])) < 1e-6
        for row in mh:
            assert row[np.argmax(np.abs(row))] > 0


def test_host_basis_exact_on_known_spectrum():
    """Diagonalisable input with a known eigenbasis: the rows come back exactly (up to fp32)."""
    from synth.workloads import haar_orthogonal
    d, r = 64, 16
    u = haar_orthogonal(d, 3)
    lam = np.linspace(2.0, 0.1, d)
    a = (u * lam) @ u.T
    s = L.make_shape(0, 1, 1, 1, 128, 16, 1, r, 16)
    # head_dim must be a supported d; embed the 64-dim problem in 128 dims
    big = np.zeros((128, 128))
    big[:64, :64] = a
    big[64:, 64:] = np.diag(np.linspace(0.05, 0.01, 64))
    m = L.jssa_basis(s, big[None].astype(np.float32), big[None].astype(np.float32))[0]
    for i in range(r):
        v = u[:, i]
        v = v * np.sign(v[np.argmax(np.abs(v))])
        assert np.abs(m[i, :64] - v).max() < 1e-4 and np.abs(m[i, 64:]).max() < 1e-6


def _split_shapes():
    """A seeded sample of GQA and MLA shapes, plus the ones where a window plan takes more splits than the
    full-capacity plan (129 pages of 16 at batch 8 and 8 KV heads; 257 pages at batch 4 and 8 KV heads)."""
    rng = np.random.default_rng(11)
    out = [_shape(batch=8, num_q_heads=32, num_kv_heads=8, max_pages_per_seq=129, budget=256),
           _shape(batch=4, num_q_heads=8, num_kv_heads=8, max_pages_per_seq=257, budget=1)]
    for _ in range(60):
        hkv = int(rng.choice([1, 2, 3, 8]))
        out.append(_shape(batch=int(rng.integers(1, 17)), num_kv_heads=hkv, num_q_heads=hkv * int(rng.choice([1, 2, 4, 8])),
                          page_size=int(rng.choice([16, 32, 64])), max_pages_per_seq=int(rng.integers(1, 3000)),
                          budget=int(rng.integers(1, 4097))))
    for _ in range(30):
        out.append(_shape(kind=1, num_kv_heads=1, num_q_heads=int(rng.choice([32, 64, 128])), head_dim=576, rank=64,
                          batch=int(rng.integers(1, 17)), page_size=int(rng.choice([16, 64])),
                          max_pages_per_seq=int(rng.integers(1, 3000)), budget=int(rng.integers(1, 4097))))
    return out


def test_attend_splits_fit_the_workspace():
    """Every attention call's split plan fits the partials the workspace holds: the sparse plan, the dense plan
    and the plan of every window from 1 to past the capacity (a window rounds its split length to fewer rows
    than the whole capacity does and can take more splits than the dense plan)."""
    for sh in _split_shapes():
        cap_tokens = sh.max_pages_per_seq * sh.page_size
        sp, cap = L.attend_splits(sh, True)
        assert 1 <= sp <= cap
        windows = sorted({1, 2, 255, 256, 257, 2047, 2048, 2049, cap_tokens - 1, cap_tokens, cap_tokens + 5}
                         | set(range(1, cap_tokens + 1, max(1, cap_tokens // 97))))
        for win in [0] + [x for x in windows if x > 0]:
            n, c = L.attend_splits(sh, False, win)
            assert c == cap and 1 <= n <= cap, (sh.batch, sh.num_kv_heads, sh.max_pages_per_seq, win, n, cap)


def test_attend_splits_known_shapes():
    """The two shapes where the window plan outgrows the full plan: 8 splits of 256 positions for a 2048-token
    window against 5 of 512 for the whole capacity, and 16 against 9."""
    sh = _split_shapes()[0]
    assert L.attend_splits(sh, False, 0)[0] == 5
    assert L.attend_splits(sh, False, 2048) == (8, 8)
    sh = _split_shapes()[1]
    assert L.attend_splits(sh, False, 0)[0] == 9
    assert L.attend_splits(sh, False, 4096) == (16, 16)
    with pytest.raises(L.JSSAError):
        L.attend_splits(sh, False, -1)


def test_noalloc_attend_refuses_oversized_and_null_before_any_launch():
    """jssa_attend_noalloc checks pointers, then the partials' size against its 64 MiB scratch array, before it
    touches a device (status codes only; the pointers are never dereferenced)."""
    lib = L.raw_library()
    fake = ctypes.c_void_p(16)
    # 256 sequences x 64 query heads x d 256: the partials exceed the scratch array
    big = _shape(batch=256, num_q_heads=64, num_kv_heads=8, head_dim=256, max_pages_per_seq=1024, budget=4096)
    splits, _ = L.attend_splits(big, True)
    assert 256 * 64 * splits * 4 * (256 + 2) * 4 > 64 << 20
    st = lib.jssa_attend_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake, ctypes.c_float(0.1), fake,
                                 None, None)
    assert st == -4                                           # JSSA_ERR_WORKSPACE
    small = _shape()
    st = lib.jssa_attend_noalloc(ctypes.byref(small), None, fake, fake, fake, fake, fake, ctypes.c_float(0.1), fake,
                                 None, None)
    assert st == -1                                           # JSSA_ERR_NULL
    st = lib.jssa_attend_noalloc(ctypes.byref(_shape(budget=0)), fake, fake, fake, fake, fake, fake,
                                 ctypes.c_float(0.1), fake, None, None)
    assert st == -2                                           # JSSA_ERR_SHAPE


# (entry point, argument kinds after the shape: "16" / "4" = a device pointer that must be 16- / 4-byte
# aligned, "i" = an int32 (4), "f" = the softmax scale, "z" = workspace bytes (0), "s" = the stream)
_ALIGN_CASES = [
    ("jssa_store", ["16", "4", "i", "16", "16", "4", "s"]),
    ("jssa_select", ["16", "16", "16", "4", "4", "4", "4", "4", "16", "z", "s"]),
    ("jssa_attend", ["16", "16", "16", "4", "4", "4", "f", "4", "4", "16", "z", "s"]),
    ("jssa_attend_noalloc", ["16", "16", "16", "4", "4", "4", "f", "4", "4", "s"]),
    ("jssa_decode", ["16", "16", "4", "16", "16", "4", "16", "16", "4", "4", "4", "f", "4", "4", "16", "z", "s"]),
    ("jssa_full_decode", ["16", "16", "16", "4", "4", "i", "f", "4", "4", "16", "z", "s"]),
    ("jssa_gather_attend", ["16", "16", "16", "4", "4", "4", "f", "4", "4", "16", "z", "s"]),
    ("jssa_calib_moments", ["16", "16", "i", "4", "4", "16", "z", "s"]),
]


@pytest.mark.parametrize("name,kinds", _ALIGN_CASES, ids=[c[0] for c in _ALIGN_CASES])
def test_misaligned_device_pointers_are_refused_before_any_launch(name, kinds):
    """Every device pointer that the kernels read with 16-byte vector loads must be 16-byte aligned, every
    other one 4-byte aligned; a pointer off by 8 (resp. 2) bytes returns JSSA_ERR_ALIGN, and the same call with
    every pointer aligned fails only on its zero workspace size.  The fake addresses are never dereferenced:
    validation ends before anything is launched."""
    lib = L.raw_library()
    fn = getattr(lib, name)
    sh = _shape()

    def args(bad=None):
        out = []
        for i, k in enumerate(kinds):
            if k in ("16", "4"):
                addr = 1 << 16
                if i == bad:
                    addr += 8 if k == "16" else 2
                out.append(ctypes.c_void_p(addr))
            elif k == "i":
                out.append(4)
            elif k == "f":
                out.append(ctypes.c_float(0.1))
            elif k == "z":
                out.append(0)
            else:
                out.append(None)
        return out

    for i, k in enumerate(kinds):
        if k in ("16", "4"):
            assert fn(ctypes.byref(sh), *args(i)) == L.ERR_ALIGN, (name, i)
    if "z" in kinds:
        assert fn(ctypes.byref(sh), *args()) == L.ERR_WORKSPACE
