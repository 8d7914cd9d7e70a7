"""Pins oracle/model.py against library routines and invariants."""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import model
from oracle.model import KVStore, forward

from oracle_fixtures import tiny_config, tiny_weights


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_incremental_equals_full_causal(dtype):
    cfg = tiny_config(dtype=dtype)
    W = tiny_weights(cfg, gains=True)
    toks = np.random.Generator(np.random.PCG64(1)).integers(0, cfg.vocab, 12)
    kv1 = KVStore(cfg, 16)
    full = forward(cfg, W, toks, np.arange(12), kv1)
    kv2 = KVStore(cfg, 16)
    rows = [forward(cfg, W, toks[t:t + 1], [t], kv2)[0] for t in range(12)]
    assert np.allclose(np.array(rows), full, rtol=0, atol=1e-11)
    assert np.allclose(kv1.k, kv2.k, atol=1e-12) and np.allclose(kv1.v, kv2.v, atol=1e-12)


def test_verify_block_equals_sequential_decodes():
    cfg = tiny_config()
    W = tiny_weights(cfg, seed=3)
    toks = np.random.Generator(np.random.PCG64(2)).integers(0, cfg.vocab, 10)
    kv = KVStore(cfg, 20)
    forward(cfg, W, toks[:5], np.arange(5), kv)
    kv_a, kv_b = kv.copy(), kv.copy()
    blk = forward(cfg, W, toks[5:10], np.arange(5, 10), kv_a)
    seq = [forward(cfg, W, toks[t:t + 1], [t], kv_b)[0] for t in range(5, 10)]
    assert np.allclose(blk, np.array(seq), rtol=0, atol=1e-11)


def test_rope_identity_at_zero_and_relative():
    rng = np.random.Generator(np.random.PCG64(4))
    x = rng.standard_normal((1, 3, 16))
    assert np.allclose(model.rope(x, np.array([0]), 1e4), x, atol=0)
    q = rng.standard_normal(16)
    k = rng.standard_normal(16)
    dots = []
    for m, n in [(5, 2), (13, 10), (103, 100), (7003, 7000)]:
        qm = model.rope(q[None, None, :], np.array([m]), 1e4)[0, 0]
        kn = model.rope(k[None, None, :], np.array([n]), 1e4)[0, 0]
        dots.append(qm @ kn)
    assert np.allclose(dots, dots[0], rtol=0, atol=1e-9)
    # rotation preserves norms
    y = model.rope(x, np.array([37]), 1e4)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))


def test_gqa_with_equal_heads_is_mha():
    # hq == hkv: each query head reads its own KV head
    cfg = tiny_config(hq=2, hkv=2)
    W = tiny_weights(cfg, seed=5)
    toks = np.arange(6) % cfg.vocab
    kv = KVStore(cfg, 8)
    out = forward(cfg, W, toks, np.arange(6), kv)
    assert np.all(np.isfinite(out))
    # duplicating KV heads (hkv=1 -> both q heads share head 0) changes the result only through wqkv
    q = np.random.Generator(np.random.PCG64(0)).standard_normal((1, 2, cfg.head_dim))
    a = model.attention(q, kv, 0, np.array([5]), cfg)
    for h in range(2):
        K = kv.k[0, :6, h]
        V = kv.v[0, :6, h]
        s = K @ q[0, h] / np.sqrt(cfg.head_dim)
        w = np.exp(s - s.max())
        w /= w.sum()
        assert np.allclose(a[0, h * cfg.head_dim:(h + 1) * cfg.head_dim], w @ V)


def test_one_layer_against_torch_library_routines():
    cfg = tiny_config(L=1, hq=4, hkv=2, hd=8, d=32, F=48, V=16)
    W = tiny_weights(cfg, seed=6, gains=True)
    T = 7
    toks = np.random.Generator(np.random.PCG64(7)).integers(0, cfg.vocab, T)
    kv = KVStore(cfg, T)
    got = forward(cfg, W, toks, np.arange(T), kv)

    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    hq, hkv, hd, F, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.d_model
    h = t(W.embed)[torch.tensor(toks)]
    x = Fn.rms_norm(h, (d,), weight=t(W.attn_norm[0]), eps=cfg.rms_eps)
    qkv = x @ t(W.wqkv[0]).T
    q = qkv[:, :hq * hd].view(T, hq, hd)
    k = qkv[:, hq * hd:(hq + hkv) * hd].view(T, hkv, hd)
    v = qkv[:, (hq + hkv) * hd:].view(T, hkv, hd)
    # rotary embedding (rotate-half) written with torch ops on complex numbers
    half = hd // 2
    inv = 1e4 ** (-torch.arange(half, dtype=torch.float64) * 2 / hd)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    def rope_c(a):
        c = torch.complex(a[..., :half], a[..., half:]) * rot
        return torch.cat([c.real, c.imag], dim=-1)
    q, k = rope_c(q), rope_c(k)
    grp = hq // hkv
    k = k.repeat_interleave(grp, dim=1)
    v = v.repeat_interleave(grp, dim=1)
    o = Fn.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True)
    o = o.transpose(0, 1).reshape(T, hq * hd)
    h = h + o @ t(W.wo[0]).T
    m = Fn.rms_norm(h, (d,), weight=t(W.mlp_norm[0]), eps=cfg.rms_eps)
    gu = m @ t(W.wgate_up[0]).T
    h = h + (Fn.silu(gu[:, :F]) * gu[:, F:]) @ t(W.wdown[0]).T
    logits = Fn.rms_norm(h, (d,), weight=t(W.final_norm), eps=cfg.rms_eps) @ t(W.lm_head).T
    # the oracle stores linear inputs / KV in fp32 for an 'f32' model; torch keeps fp64 -> ~1e-7
    assert np.allclose(got, logits.numpy(), rtol=0, atol=2e-6)
