"""CPU checks of the test helpers' layout conversion (the paged scoring-cache layout of include/jssa.h)."""
import numpy as np

from util import pack_kp, unpack_kp


def test_pack_unpack_roundtrip_and_layout():
    rng = np.random.default_rng(0)
    page, hkv, s = 16, 3, 48
    seq = [37, 50]
    bt = rng.permutation(8).astype(np.int32).reshape(2, 4)
    codes = [rng.integers(0, 256, (n, hkv, s), dtype=np.uint8) for n in seq]
    scales = [rng.random((n, hkv)).astype(np.float32) for n in seq]
    kp, ks = pack_kp(codes, scales, bt, page, 8, seq)
    # element i of (position t, head h) sits at kp[page][h][i // 16][slot][i % 16]
    t, h, i = 21, 2, 35
    assert kp[bt[1, t // page], h, i // 16, t % page, i % 16] == codes[1][t, h, i]
    assert ks[bt[1, t // page], h, t % page] == scales[1][t, h]
    for b, n in enumerate(seq):
        c, sc = unpack_kp(kp, ks, bt[b], n, page)
        assert np.array_equal(c, codes[b]) and np.array_equal(sc, scales[b])
