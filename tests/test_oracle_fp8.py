"""Pins for the oracle's OCP E4M3FN codec (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_spec_values.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        rows.append((int(c, 16), float(v)))
    return rows


def test_spec_values_decode_and_encode():
    for code, val in _golden():
        got = fp8.decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got)
            continue
        assert got == val and np.signbit(got) == np.signbit(val), hex(code)
        assert fp8.encode(np.array([val]))[0] == code, hex(code)


def test_exhaustive_roundtrip():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    back = fp8.encode(vals[finite])
    assert np.array_equal(back, codes[finite])


def test_positive_codes_strictly_increasing():
    vals = fp8.decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(vals) > 0)
    # neighbouring codes are one unit apart on the signed-magnitude line
    assert np.all(np.diff(fp8.signed_magnitude(np.arange(0, 0x7F, dtype=np.uint8))) == 1)


def test_midpoints_round_to_even():
    codes = np.arange(0, 0x7E, dtype=np.uint8)          # pairs (c, c+1) with c+1 <= 0x7E
    lo = fp8.decode(codes)
    hi = fp8.decode(codes + 1)
    mid = (lo + hi) / 2                                  # exact in fp64
    enc = fp8.encode(mid)
    even = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(enc, even.astype(np.uint8))
    assert np.array_equal(fp8.encode(-mid), (even | 0x80).astype(np.uint8))
    # just off the midpoint goes to the nearer neighbour
    assert np.array_equal(fp8.encode(np.nextafter(mid, 0)), codes)
    assert np.array_equal(fp8.encode(np.nextafter(mid, 1e9)), codes + 1)


def test_saturation_and_nan():
    x = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e6, -1e6, np.inf, -np.inf])
    assert list(fp8.encode(x)) == [0x7E] * 6 + [0xFE, 0x7E, 0xFE]
    assert fp8.encode(np.array([np.nan]))[0] in (0x7F, 0xFF)


def test_agrees_with_torch_float8_e4m3fn():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.uniform(-448, 448, 400_000),
        rng.standard_normal(300_000) * 4,
        rng.standard_normal(300_000) * 0.01,           # subnormal range
    ]).astype(np.float32).astype(np.float64)           # torch's cast goes through fp32 first
    ours = fp8.encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -12, 37.5])
def test_encode_error_within_half_ulp(scale):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(100_000) * scale
    x = x[np.abs(x) <= 448]
    err = np.abs(fp8.decode(fp8.encode(x)) - x)
    # half an ulp: 2^-4 relative in the normal range, 2^-10 absolute below 2^-6
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-15))
