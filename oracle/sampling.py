"""Token distributions and draws used by the speculative sampler.

* pi(z; T, top_p): the sampling distribution a logits row defines.  T = 0 is
  greedy (one-hot at the argmax, lowest index on ties).  Otherwise softmax(z/T)
  in float64, and for top_p < 1 the nucleus: sort by probability descending
  (equal probabilities by index ascending), keep the shortest prefix whose
  cumulative mass reaches top_p (the crossing token included), zero the rest
  and renormalize.  top_p >= 1 leaves the softmax untouched.  The pages leave
  these details open (config 4 only states top-p 0.95); the same pi is applied
  to the target's p and the drafter's q, so the lossless guarantee holds for
  the filtered target distribution.
* sample(w, u): the smallest index i, in vocabulary order, whose running sum
  sum_{k<=i} w_k reaches u * sum(w) (inverse CDF, u in (0, 1]).
* accept(p, q, d, u): accept draft token d iff u * q[d] <= p[d], i.e. with
  probability min(1, p[d]/q[d]) for u uniform on (0, 1].
* residual(p, q): normalize(max(0, p - q)), falling back to p when the
  positive part has no mass.

Accept rule, residual and bonus are standard speculative sampling (Leviathan,
Kalman and Matias, ICML 2023; Chen et al. 2023), which is the lossless
acceptance the pages require: p2 (abstract) calls speculative decoding a
lossless primitive that preserves the target's output distribution, and p3
(section 1, "target 为什么能一次检查多个位置") says every draft after the first
rejected one is discarded.

Pinned by tests/test_oracle_sampling.py: hand-computed 4-token examples
(top-p crossing, ties), exact inverse-CDF frequencies over a fine u grid, the
T -> 0 limit, and (with oracle/spec.py) the brute-force lossless enumeration.
"""
from __future__ import annotations

import numpy as np


def softmax64(z: np.ndarray, T: float) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z)
    w = np.exp((z - m) / T)
    return w / np.sum(w)


def pi(z: np.ndarray, T: float, top_p: float) -> np.ndarray:
    """Sampling distribution of one logits row (float64 probabilities summing to 1)."""
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    if T == 0.0:
        out = np.zeros(V, dtype=np.float64)
        out[int(np.argmax(z))] = 1.0  # np.argmax returns the first maximum
        return out
    p = softmax64(z, T)
    if top_p >= 1.0:
        return p
    order = np.lexsort((np.arange(V), -p))  # primary: p descending; secondary: index ascending
    cum = np.cumsum(p[order])
    n_keep = int(np.searchsorted(cum, top_p, side="left")) + 1
    n_keep = min(n_keep, V)
    keep = np.zeros(V, dtype=bool)
    keep[order[:n_keep]] = True
    out = np.where(keep, p, 0.0)
    return out / np.sum(out)


def sample(w: np.ndarray, u: float) -> int:
    """Smallest index i with sum_{k<=i} w_k >= u * sum(w), scanning in vocabulary order."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    target = u * c[-1]
    i = int(np.searchsorted(c, target, side="left"))
    return min(i, w.shape[0] - 1)


def accept(p: np.ndarray, q: np.ndarray, d: int, u: float) -> bool:
    return bool(u * q[d] <= p[d])


def accept_prob(p: np.ndarray, q: np.ndarray, d: int) -> float:
    if q[d] <= 0.0:
        return 1.0
    return float(min(1.0, p[d] / q[d]))


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    r = np.maximum(0.0, np.asarray(p, np.float64) - np.asarray(q, np.float64))
    s = np.sum(r)
    if s <= 0.0:
        return np.asarray(p, np.float64) / np.sum(p)
    return r / s


def cdf_margin(w: np.ndarray, u: float, i: int) -> float:
    """Distance (relative to sum(w)) between u*sum(w) and the CDF edges of the chosen bucket i.

    A small value means the draw sits on a bucket edge, where a different
    (but equally valid) summation order can pick the neighbouring token.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    tot = c[-1]
    t = u * tot
    lo = c[i - 1] if i > 0 else 0.0
    hi = c[i]
    return float(min(abs(t - lo), abs(hi - t)) / tot)
