"""Pins oracle/quant.py: error bound, brute-force nearest code, exact scale minimality, round trips."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import numerics, quant


def _weights(N, K, seed, dtype="bf16"):
    rng = np.random.Generator(np.random.PCG64(seed))
    W = rng.standard_normal((N, K)) * 0.02
    return numerics.store(W, dtype)


@pytest.mark.parametrize("K", [128, 256, 688, 300])
def test_w4_error_bound_and_nearest_code(K):
    W = _weights(24, K, K)
    codes, s, z = quant.quantize_w4(W)
    deq = quant.dequantize_w4(codes, s, z)
    for g, (a, b) in enumerate(quant.w4_groups(K)):
        blk = W[:, a:b]
        sg = s[:, g:g + 1]
        zg = z[:, g:g + 1].astype(np.float64)
        err = np.abs(blk - deq[:, a:b])
        assert np.all(err <= sg / 2 * (1 + 1e-12))
        # brute force: every code 0..15 -> the stored one is a nearest grid point
        grid = (np.arange(16)[None, None, :] - zg[:, :, None]) * sg[:, :, None]
        dist = np.abs(blk[:, :, None] - grid)
        best = dist.min(axis=2)
        assert np.allclose(err, best, rtol=0, atol=1e-15)
    assert codes.max() <= 15


def test_w4_scale_is_smallest_bf16_at_or_above_span():
    W = _weights(64, 256, 3)
    codes, s, z = quant.quantize_w4(W)
    for r in range(64):
        for g, (a, b) in enumerate(quant.w4_groups(256)):
            blk = W[r, a:b]
            lo = min(blk.min(), 0.0)
            hi = max(blk.max(), 0.0)
            exact = (Fraction(float(hi)) - Fraction(float(lo))) / 15
            sv = Fraction(float(s[r, g]))
            assert sv >= exact
            bits = int(numerics.f32_to_bf16_bits(np.array([s[r, g]], dtype=np.float32))[0])
            below = float(numerics.bf16_bits_to_f32(np.array([bits - 1], dtype=np.uint16))[0])
            assert Fraction(below) < exact
            # zero point: nearest integer to -lo/s, inside 0..15
            zz = int(z[r, g])
            assert 0 <= zz <= 15
            assert abs(Fraction(-float(lo)) / sv - zz) <= Fraction(1, 2)


def test_w4_on_grid_round_trip_and_zero_group():
    s = 2.0 ** -7
    z = 6
    codes = np.random.Generator(np.random.PCG64(0)).integers(0, 16, size=(4, 128))
    codes[:, 0] = 0
    codes[:, 1] = 15  # pin the span so the chosen scale is exactly s
    W = (codes - z) * s
    c2, s2, z2 = quant.quantize_w4(W)
    assert np.all(s2 == s) and np.all(z2 == z)
    assert np.array_equal(quant.dequantize_w4(c2, s2, z2), W)
    Z = np.zeros((3, 256))
    c3, s3, z3 = quant.quantize_w4(Z)
    assert np.all(s3 == 1.0) and np.all(z3 == 0) and np.all(c3 == 0)


def test_w4_pack_layout():
    codes = np.array([[1, 2, 3, 4, 5]], dtype=np.uint8)
    p = quant.pack_w4(codes)
    assert p.tolist() == [[0x21, 0x43, 0x05]]
    assert np.array_equal(quant.unpack_w4(p, 5), codes)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_w8_error_bound_and_nearest_code(dtype):
    W = _weights(40, 300, 11, dtype)
    q, s = quant.quantize_w8(W)
    deq = quant.dequantize_w8(q, s)
    err = np.abs(W - deq)
    assert np.all(err <= s[:, None] / 2 * (1 + 1e-12))
    codes = np.arange(-127, 128)
    grid = codes[None, None, :] * s[:, None, None]
    best = np.abs(W[:, :, None] - grid).min(axis=2)
    assert np.allclose(err, best, rtol=0, atol=1e-15)
    for r in range(40):
        exact = Fraction(float(np.max(np.abs(W[r])))) / 127
        assert Fraction(float(s[r])) >= exact
        below = float(np.nextafter(np.float32(s[r]), np.float32(0)))
        assert Fraction(below) < exact
    assert np.abs(q).max() <= 127


def test_w8_round_trip_and_zero_row():
    s = 2.0 ** -9
    q = np.random.Generator(np.random.PCG64(2)).integers(-127, 128, size=(3, 64))
    q[:, 0] = 127
    W = q * s
    q2, s2 = quant.quantize_w8(W)
    assert np.all(s2 == s) and np.array_equal(q2, q)
    q3, s3 = quant.quantize_w8(np.zeros((2, 16)))
    assert np.all(s3 == 1.0) and np.all(q3 == 0)
