"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic.  Everything here is random init (there are no trained
weights or datasets): the pages' workloads (RL on math-reasoning prompts,
p1 "局限"; GRPO on a math dataset, p5 section 5) are stood in for by uniform
random prompts and lognormal per-sequence stop lengths.

Recipe:
* every weight matrix (embedding, q/k/v/o, gate/up/down, untied lm_head) is
  i.i.d. N(0, 0.02); RMSNorm gains are 1; no biases.  bf16 models round the
  draws to bf16 (round to nearest even).
* prompts are i.i.d. uniform over the vocabulary.
* stop lengths: L = min(cap, max(1, rint(exp(ln(median) + 0.75 * Z)))), Z ~ N(0,1).

CPU tensors come from torch's CPU generator; large models are generated on
the GPU with torch's device generator (same recipe, different stream of
numbers).  Each tensor has its own seed so a reduced-depth model holds exactly
the first layers of the full one.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Shape:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str          # 'bf16' or 'f32'
    rms_eps: float
    rope_theta: float
    quant: str          # drafter format: 'w8' or 'w4'


SHAPES = {
    "tiny": Shape("tiny", 2, 256, 4, 2, 64, 688, 1024, "f32", 1e-6, 1e4, "w8"),
    # small bf16 decoder with the 7B family's head layout (hd 128, GQA) and a
    # vocabulary that is not a multiple of the sampler's 2048-token chunks
    "mini-bf16": Shape("mini-bf16", 2, 512, 4, 2, 128, 1536, 8000, "bf16", 1e-6, 1e6, "w4"),
    "qwen2.5-7b": Shape("qwen2.5-7b", 28, 3584, 28, 4, 128, 18944, 152064, "bf16", 1e-6, 1e6, "w4"),
    "qwen2.5-14b": Shape("qwen2.5-14b", 48, 5120, 40, 8, 128, 13824, 152064, "bf16", 1e-6, 1e6, "w4"),
    "qwen2.5-32b": Shape("qwen2.5-32b", 64, 5120, 40, 8, 128, 27648, 152064, "bf16", 1e-6, 1e6, "w4"),
    "llama-3-8b": Shape("llama-3-8b", 32, 4096, 32, 8, 128, 14336, 128256, "bf16", 1e-5, 5e5, "w8"),
}


def shape(name: str, **over) -> Shape:
    s = SHAPES[name]
    if over:
        d = dict(s.__dict__)
        d.update(over)
        s = Shape(**d)
    return s


def tensor_shapes(s: Shape):
    """(name, shape) of every weight tensor, in a fixed order."""
    hq, hkv, hd, d, F, V = s.n_q_heads, s.n_kv_heads, s.head_dim, s.d_model, s.ffn, s.vocab
    out = [("embed", (V, d)), ("final_norm", (d,)), ("lm_head", (V, d))]
    for l in range(s.n_layers):
        out += [
            (f"attn_norm.{l}", (d,)),
            (f"wqkv.{l}", ((hq + 2 * hkv) * hd, d)),
            (f"wo.{l}", (d, hq * hd)),
            (f"mlp_norm.{l}", (d,)),
            (f"wgate_up.{l}", (2 * F, d)),
            (f"wdown.{l}", (d, F)),
        ]
    return out


def _tensor_seed(seed: int, name: str) -> int:
    base = {"embed": 1, "final_norm": 2, "lm_head": 3}
    if name in base:
        idx = base[name]
    else:
        kind, l = name.split(".")
        kinds = ["attn_norm", "wqkv", "wo", "mlp_norm", "wgate_up", "wdown"]
        idx = 16 + 8 * int(l) + kinds.index(kind)
    return (seed * 1_000_003 + idx) & 0x7FFFFFFFFFFFFFFF


def weights(s: Shape, seed: int = 0, device: str = "cpu", std: float = 0.02):
    """dict name -> torch tensor (float32 for 'f32' models, bfloat16 for 'bf16') on `device`."""
    import torch

    dt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    out = {}
    for name, shp in tensor_shapes(s):
        if name.endswith("norm") or "norm." in name:
            out[name] = torch.ones(shp, dtype=dt, device=device)
            continue
        g = torch.Generator(device=device)
        g.manual_seed(_tensor_seed(seed, name))
        t = torch.randn(shp, generator=g, dtype=torch.float32, device=device)
        t.mul_(std)
        out[name] = t.to(dt)
    return out


def prompts(n: int, length: int, vocab: int, seed: int = 0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed + 17))
    return rng.integers(0, vocab, size=(n, length), dtype=np.int64).astype(np.int32)


def stop_lengths(n: int, median: float, cap: int, seed: int = 0, sigma: float = 0.75) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed + 29))
    z = rng.standard_normal(n)
    L = np.rint(np.exp(np.log(median) + sigma * z))
    return np.minimum(cap, np.maximum(1, L)).astype(np.int32)


def kv_fill(shape_, seed: int = 0, device: str = "cpu"):
    """Synthetic bf16 KV contents (N(0,1)) for fixed-context sweeps."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed + 41)
    return torch.randn(shape_, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
