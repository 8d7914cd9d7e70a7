"""Storage-type helpers for the oracle (bf16 / fp32 rounding).

The pages fix only that the target runs in bf16 (p1, "关键模块" item 1: the
drafter is a W4/W8 quantization of the target's own weights; the target keeps
its native precision).  Where a value is *stored* in bf16 or fp32, the oracle
rounds it exactly as that storage would: round-to-nearest-even for data, and
round-toward-+inf where a quantizer scale must not shrink (so that every weight
of the row or group stays inside the representable range).

Pinned by tests/test_oracle_numerics.py against torch's own bf16 conversion
and against exact rational arithmetic (fractions.Fraction).
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r = np.where(nan, np.uint16(0x7FC0), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_bf16(x) -> np.ndarray:
    """Value of x (float32 or float64) after storage in bf16, returned as float64.

    float64 inputs are first rounded to float32 (the GPU holds them as float32
    registers before the bf16 store), then to bf16.
    """
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def store(x, dtype: str) -> np.ndarray:
    """Round to the model's storage type ('bf16' or 'f32'), result as float64."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def f32_round_up(v: np.ndarray) -> np.ndarray:
    """Smallest float32 >= v (v float64, v > 0)."""
    v = np.asarray(v, dtype=np.float64)
    t = v.astype(np.float32)
    low = t.astype(np.float64) < v
    t = np.where(low, np.nextafter(t, np.float32(np.inf)), t)
    return t.astype(np.float32)


def bf16_round_up(v: np.ndarray) -> np.ndarray:
    """Smallest bf16 >= v for v > 0 (v float64); returned as float64 values."""
    t = f32_round_up(v)
    u = t.view(np.uint32).astype(np.uint64)
    hi = u >> 16
    hi = np.where((u & 0xFFFF) != 0, hi + 1, hi).astype(np.uint16)
    return bf16_bits_to_f32(hi).astype(np.float64)


def rint(x) -> np.ndarray:
    """Round half to even (numpy's rint)."""
    return np.rint(x)
