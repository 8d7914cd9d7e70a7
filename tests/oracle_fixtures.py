"""Small random models for the oracle's own pin tests (numpy, float64 values)."""
import numpy as np

from oracle.model import Config, KVStore, Weights
from oracle.numerics import store


def tiny_config(V=16, d=32, hq=4, hkv=2, hd=8, F=48, L=2, dtype="f32", theta=1e4):
    return Config(n_layers=L, d_model=d, n_q_heads=hq, n_kv_heads=hkv, head_dim=hd, ffn=F, vocab=V,
                  dtype=dtype, rms_eps=1e-6, rope_theta=theta)


def tiny_weights(cfg: Config, seed=0, std=0.3, gains=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    d, V, hq, hkv, hd, F, L = cfg.d_model, cfg.vocab, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.n_layers
    n = lambda *s: store(rng.standard_normal(s) * std, cfg.dtype)
    g = (lambda: store(1.0 + 0.1 * rng.standard_normal(d), cfg.dtype)) if gains else (lambda: np.ones(d))
    return Weights(
        embed=n(V, d), final_norm=g(), lm_head=n(V, d),
        attn_norm=[g() for _ in range(L)], wqkv=[n((hq + 2 * hkv) * hd, d) for _ in range(L)],
        wo=[n(d, hq * hd) for _ in range(L)], mlp_norm=[g() for _ in range(L)],
        wgate_up=[n(2 * F, d) for _ in range(L)], wdown=[n(d, F) for _ in range(L)])
