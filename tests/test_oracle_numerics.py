"""Pins oracle/numerics.py: bf16 rounding against torch, round-up minimality exactly."""
from fractions import Fraction

import numpy as np
import torch

from oracle import numerics


def test_bf16_rne_matches_torch():
    rng = np.random.Generator(np.random.PCG64(5))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-40, -3.3e38], dtype=np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = numerics.f32_to_bf16_bits(x)
    assert np.array_equal(got, ref)
    back = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(numerics.round_bf16(x).astype(np.float32), back)


def _bf16_values_around(v):
    """All bf16 values in the binade of v and its neighbours, as Fractions (exact)."""
    t = np.float32(v)
    bits = int(numerics.f32_to_bf16_bits(np.array([t]))[0])
    cands = [int(b) for b in range(max(bits - 3, 1), bits + 4)]
    vals = numerics.bf16_bits_to_f32(np.array(cands, dtype=np.uint16)).astype(np.float64)
    return [Fraction(float(x)) for x in vals]


def test_bf16_round_up_is_minimal_exactly():
    rng = np.random.Generator(np.random.PCG64(9))
    for _ in range(2000):
        hi = float(numerics.round_bf16(abs(rng.standard_normal()) * 0.05)[0])
        lo = -float(numerics.round_bf16(abs(rng.standard_normal()) * 0.05)[0])
        exact = (Fraction(hi) - Fraction(lo)) / 15
        s = float(numerics.bf16_round_up(np.array([(hi - lo) / 15.0]))[0])
        assert Fraction(s) >= exact
        smaller = [c for c in _bf16_values_around(s) if c < Fraction(s)]
        assert all(c < exact for c in smaller)


def test_f32_round_up_is_minimal_exactly():
    rng = np.random.Generator(np.random.PCG64(10))
    for _ in range(2000):
        amax = float(np.float32(abs(rng.standard_normal()) * 0.1))
        exact = Fraction(amax) / 127
        s = float(numerics.f32_round_up(np.array([amax / 127.0]))[0])
        assert Fraction(s) >= exact
        below = float(np.nextafter(np.float32(s), np.float32(0)))
        assert Fraction(below) < exact
