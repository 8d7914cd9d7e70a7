"""Weight quantizers that build the self-drafter from the target's own weights.

Source: p1 (EfficientRollout), section "关键模块" (key modules), item 1: the
drafter is obtained by quantizing the target model's weights, e.g. W4 or W8,
with no separate training; section "与现有工作流的接口" (workflow interface)
names the W4A16 format.  The pages do not print the quantizer, so the plain
reading is used:

* W8, symmetric, one scale per output row (output channel):
  s_r = max_k |W[r,k]| / 127, rounded *up* to fp32 (the scale's storage type);
  q = clamp(rint(w / s_r), -127, 127); deq = q * s_r.  An all-zero row uses s = 1.
* W4, asymmetric, one (scale, zero) per output row and per group of 128 inputs:
  lo = min(min w, 0), hi = max(max w, 0) (so 0 is always representable);
  s = (hi - lo) / 15, rounded *up* to bf16; z = clamp(rint(-lo / s), 0, 15);
  q = clamp(rint(w / s) + z, 0, 15); deq = (q - z) * s.  An all-zero group uses
  s = 1, z = 0.  A last group shorter than 128 (K not a multiple of 128) is
  quantized the same way over its own elements.

rint is round-half-to-even.  Scales and quotients are computed in float64; the
rounding-up makes every |w / s| fit the code range, so |w - deq| <= s/2.

Pinned by tests/test_oracle_quant.py: the s/2 error bound, brute-force nearest
grid point over all 16 (or 255) codes, exact minimality of the rounded-up
scale (fractions.Fraction), exact round-trip of on-grid values, all-zero groups.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round_up, f32_round_up


def quantize_w8(W: np.ndarray):
    """W [N, K] (float values exactly as stored) -> (q int8 [N,K], scale float64 [N] (fp32 values))."""
    W = np.asarray(W, dtype=np.float64)
    amax = np.max(np.abs(W), axis=1)
    s = np.where(amax > 0, f32_round_up(amax / 127.0).astype(np.float64), 1.0)
    q = np.clip(np.rint(W / s[:, None]), -127, 127).astype(np.int8)
    return q, s


def dequantize_w8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return q.astype(np.float64) * s[:, None]


def w4_groups(K: int, group: int = 128):
    """Start/end of each input group along K (last one may be ragged)."""
    starts = list(range(0, K, group))
    return [(a, min(a + group, K)) for a in starts]


def quantize_w4(W: np.ndarray, group: int = 128):
    """W [N, K] -> (codes uint8 [N,K] in 0..15, scale float64 [N,G] (bf16 values), zero uint8 [N,G])."""
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    groups = w4_groups(K, group)
    G = len(groups)
    codes = np.zeros((N, K), dtype=np.uint8)
    scale = np.zeros((N, G), dtype=np.float64)
    zero = np.zeros((N, G), dtype=np.uint8)
    for g, (a, b) in enumerate(groups):
        blk = W[:, a:b]
        lo = np.minimum(blk.min(axis=1), 0.0)
        hi = np.maximum(blk.max(axis=1), 0.0)
        span = hi - lo
        nz = span > 0
        s = np.ones(N, dtype=np.float64)
        if np.any(nz):
            s[nz] = bf16_round_up(span[nz] / 15.0)
        z = np.where(nz, np.clip(np.rint(-lo / s), 0, 15), 0.0)
        q = np.clip(np.rint(blk / s[:, None]) + z[:, None], 0, 15)
        codes[:, a:b] = q.astype(np.uint8)
        scale[:, g] = s
        zero[:, g] = z.astype(np.uint8)
    return codes, scale, zero


def dequantize_w4(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int = 128) -> np.ndarray:
    N, K = codes.shape
    out = np.empty((N, K), dtype=np.float64)
    for g, (a, b) in enumerate(w4_groups(K, group)):
        out[:, a:b] = (codes[:, a:b].astype(np.float64) - zero[:, g:g + 1].astype(np.float64)) * scale[:, g:g + 1]
    return out


def pack_w4(codes: np.ndarray) -> np.ndarray:
    """Canonical W4 byte layout: uint8 [N, ceil(K/2)], low nibble = even k, high nibble = odd k."""
    N, K = codes.shape
    Kp = (K + 1) // 2
    c = np.zeros((N, 2 * Kp), dtype=np.uint8)
    c[:, :K] = codes
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_w4(packed: np.ndarray, K: int) -> np.ndarray:
    lo = packed & 0x0F
    hi = packed >> 4
    N = packed.shape[0]
    out = np.empty((N, 2 * packed.shape[1]), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out[:, :K]
