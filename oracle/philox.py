"""Philox4x32-10 counter-based generator and the uniforms the sampler draws.

Philox is the generator of Salmon, Moraes, Dror and Shaw, "Parallel random
numbers: as easy as 1, 2, 3" (SC'11): a 10-round network on a 128-bit counter
and a 64-bit key.  Each round multiplies counter words 0 and 2 by the constants
0xD2511F53 and 0xCD9E8D57 (keeping the high and low 32-bit halves), mixes the
high halves with counter words 1 and 3 and with the round key, and permutes;
between rounds the key is bumped by the Weyl constants 0x9E3779B9 and
0xBB67AE85.  The first round uses the key as given.

The speculative sampler's draws are keyed as the method requires (a
counter-based Philox keyed by seed, sequence, position and draft index):

* key     = (seed mod 2^32, seed >> 32)
* counter = (seq_id, pos, draft_idx, purpose), where seq_id is the *global*
  rollout index, pos is the 0-based absolute position of the token being
  decided, draft_idx is j for draft position j, gamma+1 for the bonus and 0 for
  an autoregressive step, and purpose is 0 draft sample, 1 accept test,
  2 residual/bonus sample, 3 autoregressive sample.  (The purpose word is this
  build's reading: the pages name only seed, sequence, position and draft
  index, and separate words keep the three draws of one position independent.)
* u = ((out0 >> 8) + 1) * 2^-24, which lies in (0, 1] and is exact in fp32.

Pinned by tests/test_oracle_philox.py against PyTorch's independent C++
Philox4x32-10 engine (ATen's PhiloxRNGEngine.h, compiled with g++ in the test)
on arbitrary counters and keys, plus uniformity and avalanche checks.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK = 0xFFFFFFFF

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_RESIDUAL = 2
PURPOSE_AR = 3


def _mulhilo(a: np.ndarray, b: int):
    p = a.astype(np.uint64) * np.uint64(b)
    return (p >> np.uint64(32)) & np.uint64(MASK), p & np.uint64(MASK)


def philox4x32_10(ctr, key):
    """ctr: 4 arrays (or ints) of uint32 words, key: 2 words. Returns 4 uint64 arrays of 32-bit outputs."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & np.uint64(MASK) for c in ctr)
    k0, k1 = (np.asarray(k, dtype=np.uint64) & np.uint64(MASK) for k in key)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(W0)) & np.uint64(MASK)
            k1 = (k1 + np.uint64(W1)) & np.uint64(MASK)
        hi0, lo0 = _mulhilo(c0, M0)
        hi1, lo1 = _mulhilo(c2, M1)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform(seed: int, seq_id, pos, draft_idx, purpose) -> np.ndarray:
    """u in (0, 1] for the given counter fields (broadcasting numpy arrays); float64 values exact in fp32."""
    key = (seed & MASK, (seed >> 32) & MASK)
    out0, _, _, _ = philox4x32_10((seq_id, pos, draft_idx, purpose), key)
    return ((out0 >> np.uint64(8)).astype(np.float64) + 1.0) * (2.0 ** -24)


def u1(seed: int, seq_id: int, pos: int, draft_idx: int, purpose: int) -> float:
    return float(uniform(seed, seq_id, pos, draft_idx, purpose))
