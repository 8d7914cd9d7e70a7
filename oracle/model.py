"""Plain pre-norm decoder transformer (target and self-drafter) with a KV cache.

The model family is the one the workloads name (Qwen2.5 / Llama-3 shaped
decoders: RMSNorm, rotary position embedding, grouped-query attention, SwiGLU
feed-forward).  The pages give only shapes, so each layer is the standard
published one:

* layer:  h <- h + Attn(RMSNorm(h));  m = RMSNorm(h);
          h <- h + W_down (silu(W_gate m) * (W_up m))
* logits = W_lm RMSNorm_f(h); untied embedding and lm_head; no biases.
* RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g.
* RoPE, rotate-half: pairs (i, i + hd/2), theta_i = base^(-2i/hd), 0-based
  absolute positions.
* GQA: query head h reads KV head floor(h / (hq/hkv)); scores scaled by
  1/sqrt(hd); causal mask (a query at position t sees keys 0..t);
  max-subtracted softmax.

The drafter is the same network with every linear replaced by its dequantized
W8/W4 copy (lm_head included) and it reads and writes the *same* KV store:
p1 ("关键模块", item 1) says the quantized drafter shares the target's KV cache
and needs no extra storage.  Its K/V for draft positions are provisional and
the target's verify pass overwrites them.

Storage precision (bf16 build): weights, the inputs of every linear layer,
the KV entries and the attention query are stored in bf16 (round to nearest
even); the residual stream, accumulations and everything else run in float64
here.  fp32 build: the same points are rounded to fp32.

Pinned by tests/test_oracle_model.py: KV-cached incremental decode equals a
full causal forward; a (gamma+1)-token verify block equals gamma+1 single-token
decodes; RoPE is the identity at position 0 and q(m).k(n) depends only on m-n;
hq = hkv reduces to multi-head attention; one layer re-expressed with PyTorch's
library routines (scaled_dot_product_attention, rms_norm, silu).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .numerics import store


@dataclass
class Config:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str = "bf16"  # storage type of weights / KV / linear inputs: 'bf16' or 'f32'
    rms_eps: float = 1e-6
    rope_theta: float = 1e4


@dataclass
class Weights:
    """float64 arrays holding exactly the stored values (bf16 or fp32)."""
    embed: np.ndarray        # [V, d]
    final_norm: np.ndarray   # [d]
    lm_head: np.ndarray      # [V, d]
    attn_norm: list          # L x [d]
    wqkv: list               # L x [(hq + 2 hkv) * hd, d]  (q rows, then k rows, then v rows)
    wo: list                 # L x [d, hq * hd]
    mlp_norm: list           # L x [d]
    wgate_up: list           # L x [2F, d]  (gate rows, then up rows)
    wdown: list              # L x [d, F]


class KVStore:
    """Per-sequence, per-layer K and V rows indexed by absolute position."""

    def __init__(self, cfg: Config, capacity: int):
        L, hkv, hd = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
        self.k = np.zeros((L, capacity, hkv, hd), dtype=np.float64)
        self.v = np.zeros((L, capacity, hkv, hd), dtype=np.float64)
        self.capacity = capacity

    def copy(self) -> "KVStore":
        c = KVStore.__new__(KVStore)
        c.k = self.k.copy()
        c.v = self.v.copy()
        c.capacity = self.capacity
        return c


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope_cos_sin(positions: np.ndarray, hd: int, theta: float):
    half = hd // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """x [T, heads, hd] rotated by position (rotate-half pairing)."""
    hd = x.shape[-1]
    half = hd // 2
    cos, sin = rope_cos_sin(positions, hd, theta)
    cos = cos[:, None, :]
    sin = sin[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attention(q: np.ndarray, kv: KVStore, layer: int, positions: np.ndarray, cfg: Config) -> np.ndarray:
    """q [T, hq, hd] (stored values) for query positions -> out [T, hq*hd]; query t sees keys 0..positions[t]."""
    T = q.shape[0]
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    grp = hq // hkv
    out = np.zeros((T, hq, hd), dtype=np.float64)
    scale = 1.0 / np.sqrt(hd)
    for t in range(T):
        n = int(positions[t]) + 1
        for h in range(hq):
            g = h // grp
            K = kv.k[layer, :n, g, :]
            V = kv.v[layer, :n, g, :]
            s = (K @ q[t, h]) * scale
            s = s - np.max(s)
            w = np.exp(s)
            w = w / np.sum(w)
            out[t, h] = w @ V
    return out.reshape(T, hq * hd)


def forward(cfg: Config, W: Weights, tokens, positions, kv: KVStore, lin=None) -> np.ndarray:
    """Run tokens (one sequence) at the given absolute positions; write K/V; return logits [T, V].

    `lin` optionally replaces the linear weights (the drafter's dequantized
    copies); it is a Weights-like object whose wqkv/wo/wgate_up/wdown/lm_head
    are used instead of W's.  Embedding and norm gains always come from W.
    """
    st = cfg.dtype
    M = lin if lin is not None else W
    tokens = np.asarray(tokens, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    T = tokens.shape[0]
    hq, hkv, hd, F = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    h = W.embed[tokens].astype(np.float64)
    for l in range(cfg.n_layers):
        x = store(rmsnorm(h, W.attn_norm[l], cfg.rms_eps), st)
        qkv = x @ M.wqkv[l].T
        q = qkv[:, : hq * hd].reshape(T, hq, hd)
        k = qkv[:, hq * hd: (hq + hkv) * hd].reshape(T, hkv, hd)
        v = qkv[:, (hq + hkv) * hd:].reshape(T, hkv, hd)
        q = store(rope(q, positions, cfg.rope_theta), st)
        k = store(rope(k, positions, cfg.rope_theta), st)
        v = store(v, st)
        kv.k[l, positions] = k
        kv.v[l, positions] = v
        a = store(attention(q, kv, l, positions, cfg), st)
        h = h + a @ M.wo[l].T
        x = store(rmsnorm(h, W.mlp_norm[l], cfg.rms_eps), st)
        gu = x @ M.wgate_up[l].T
        act = store(silu(gu[:, :F]) * gu[:, F:], st)
        h = h + act @ M.wdown[l].T
    x = store(rmsnorm(h, W.final_norm, cfg.rms_eps), st)
    return x @ M.lm_head.T


@dataclass
class DraftLinears:
    """Dequantized linear weights of the self-drafter (float64)."""
    wqkv: list = field(default_factory=list)
    wo: list = field(default_factory=list)
    wgate_up: list = field(default_factory=list)
    wdown: list = field(default_factory=list)
    lm_head: np.ndarray = None


def config_from(shape) -> Config:
    """Config from a workload shape (an object with the same field names)."""
    return Config(n_layers=shape.n_layers, d_model=shape.d_model, n_q_heads=shape.n_q_heads,
                  n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim, ffn=shape.ffn,
                  vocab=shape.vocab, dtype=shape.dtype, rms_eps=shape.rms_eps,
                  rope_theta=shape.rope_theta)


def weights_from(cfg: Config, arrays: dict) -> Weights:
    """Weights from name -> array (any float dtype holding the stored values)."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    L = cfg.n_layers
    return Weights(
        embed=f(arrays["embed"]), final_norm=f(arrays["final_norm"]), lm_head=f(arrays["lm_head"]),
        attn_norm=[f(arrays[f"attn_norm.{l}"]) for l in range(L)],
        wqkv=[f(arrays[f"wqkv.{l}"]) for l in range(L)],
        wo=[f(arrays[f"wo.{l}"]) for l in range(L)],
        mlp_norm=[f(arrays[f"mlp_norm.{l}"]) for l in range(L)],
        wgate_up=[f(arrays[f"wgate_up.{l}"]) for l in range(L)],
        wdown=[f(arrays[f"wdown.{l}"]) for l in range(L)],
    )
