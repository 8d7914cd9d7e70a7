"""Self-speculative decoding step, autoregressive step and rollout loops.

One speculative step for a sequence whose pending token sits at position n
(KV valid for 0..n-1), with draft length gamma:

1. Draft (p1 "关键模块" item 1): for j = 1..gamma the drafter (quantized
   self-model, shared KV) runs the pending token (j = 1) or d_{j-1} at
   position n+j-1, writing provisional K/V there; q_j = pi(drafter logits);
   d_j = sample(q_j, u(s, n+j, j, draft)).
2. Verify (p3 section 1, "target 为什么能一次检查多个位置"): one target forward
   over [pending, d_1..d_gamma] at positions n..n+gamma scores every position
   at once and overwrites the provisional K/V; p_j = pi(target logits row j).
3. Accept (p2 abstract: lossless, the target distribution is preserved; p3:
   everything after the first failed draft is discarded): for j = 1..gamma,
   accept d_j iff u(s, n+j, j, accept) * q_j(d_j) <= p_j(d_j).  At the first
   rejection emit d_1..d_{j-1} and a sample of normalize(max(0, p_j - q_j))
   (u(s, n+j, j, residual)) and stop.  If all pass, emit d_1..d_gamma and a
   bonus sample of p_{gamma+1} (u(s, n+gamma+1, gamma+1, residual)).
4. Roll back: KV stays valid for 0..n+a (a = accepted drafts); the last
   emitted token becomes the new pending token at n+a+1.
5. A sequence stops at its preset length; tokens past it are dropped
   (p1 "问题背景": long-tail responses dominate a batch, which shrinks as
   samples finish).

At temperature 0 this reduces to: accept iff d_j = argmax p_j, and on a
rejection emit argmax p_j, so greedy speculation reproduces greedy
autoregressive decoding token for token.

The autoregressive step (the baseline of p1 "实验设计") samples
pi(p_1) with u(s, n+1, 0, ar).  Prefill runs the target over the prompt and
draws the first generated token as an autoregressive sample.

Pinned by tests/test_oracle_spec.py: greedy SD == greedy AR; brute-force
enumeration of the exact output distribution on a tiny vocabulary (gamma <= 2)
equals the target's (lossless); q == p always emits gamma+1 tokens; disjoint
supports emit one token distributed as p_1; the mean emitted length matches
(1 - alpha^(gamma+1)) / (1 - alpha) for context-free p, q; gamma = 0 == AR.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import philox
from .model import Config, DraftLinears, KVStore, Weights, forward
from .quant import dequantize_w4, dequantize_w8, quantize_w4, quantize_w8
from .sampling import accept, pi, residual, sample


# ---------------------------------------------------------------------------
# Drafter construction (p1 "关键模块" item 1; re-derived after every policy update)
# ---------------------------------------------------------------------------

def build_drafter(W: Weights, quant: str, group: int = 128, quant_lm_head: bool = True) -> DraftLinears:
    def dq(M):
        if quant == "w8":
            q, s = quantize_w8(M)
            return dequantize_w8(q, s)
        if quant == "w4":
            c, s, z = quantize_w4(M, group)
            return dequantize_w4(c, s, z, group)
        raise ValueError(quant)

    D = DraftLinears()
    D.wqkv = [dq(m) for m in W.wqkv]
    D.wo = [dq(m) for m in W.wo]
    D.wgate_up = [dq(m) for m in W.wgate_up]
    D.wdown = [dq(m) for m in W.wdown]
    D.lm_head = dq(W.lm_head) if quant_lm_head else W.lm_head
    return D


@dataclass
class SamplingParams:
    """Sampler settings.  The library receives the temperature and top_p as 32-bit floats (its
    rollout descriptor), so they are held here as those float32 values: where a decision sits within
    float32 rounding of the threshold (a nucleus whose cumulative mass lies between float32(0.95) and
    0.95), both sides then decide on the same number."""
    seed: int = 0
    temperature: float = 1.0
    top_p: float = 1.0

    def __post_init__(self):
        self.temperature = float(np.float32(self.temperature))
        self.top_p = float(np.float32(self.top_p))


@dataclass
class SeqState:
    seq_id: int
    pending: int            # token at position n (its KV not yet written by the target)
    n: int                  # position of the pending token
    kv: KVStore
    stop_len: int           # total generated tokens allowed (including the first, from prefill)
    generated: list = field(default_factory=list)

    @property
    def done(self) -> bool:
        return len(self.generated) >= self.stop_len


@dataclass
class StepRecord:
    """What one speculative step did for one sequence (for lockstep comparison)."""
    drafts: list
    q_logits: np.ndarray    # [gamma, V]
    p_logits: np.ndarray    # [gamma+1, V]
    n_accepted: int
    emitted: list


def spec_decide(p_logits: np.ndarray, q_logits: np.ndarray, drafts, seq_id: int, n: int,
                sp: SamplingParams):
    """Accept/resample/bonus decision from logits rows (no model involved).

    p_logits [gamma+1, V], q_logits [gamma, V], drafts [gamma] -> (n_accepted, emitted tokens).
    """
    gamma = len(drafts)
    for j in range(1, gamma + 1):
        p = pi(p_logits[j - 1], sp.temperature, sp.top_p)
        q = pi(q_logits[j - 1], sp.temperature, sp.top_p)
        d = int(drafts[j - 1])
        u = philox.u1(sp.seed, seq_id, n + j, j, philox.PURPOSE_ACCEPT)
        if not accept(p, q, d, u):
            r = residual(p, q)
            t = sample(r, philox.u1(sp.seed, seq_id, n + j, j, philox.PURPOSE_RESIDUAL))
            return j - 1, [int(x) for x in drafts[: j - 1]] + [t]
    p = pi(p_logits[gamma], sp.temperature, sp.top_p)
    t = sample(p, philox.u1(sp.seed, seq_id, n + gamma + 1, gamma + 1, philox.PURPOSE_RESIDUAL))
    return gamma, [int(x) for x in drafts] + [t]


def draft_sample(q_logits_row: np.ndarray, seq_id: int, pos: int, j: int, sp: SamplingParams) -> int:
    q = pi(q_logits_row, sp.temperature, sp.top_p)
    return sample(q, philox.u1(sp.seed, seq_id, pos, j, philox.PURPOSE_DRAFT))


def ar_sample(logits_row: np.ndarray, seq_id: int, pos: int, sp: SamplingParams) -> int:
    p = pi(logits_row, sp.temperature, sp.top_p)
    return sample(p, philox.u1(sp.seed, seq_id, pos, 0, philox.PURPOSE_AR))


def spec_step(cfg: Config, W: Weights, D: DraftLinears, st: SeqState, gamma: int,
              sp: SamplingParams) -> StepRecord:
    n = st.n
    drafts = []
    q_rows = []
    tok = st.pending
    for j in range(1, gamma + 1):
        zq = forward(cfg, W, [tok], [n + j - 1], st.kv, lin=D)[0]
        q_rows.append(zq)
        tok = draft_sample(zq, st.seq_id, n + j, j, sp)
        drafts.append(tok)
    vt = [st.pending] + drafts
    zp = forward(cfg, W, vt, list(range(n, n + gamma + 1)), st.kv)
    q_logits = np.array(q_rows).reshape(gamma, cfg.vocab)
    a, emitted = spec_decide(zp, q_logits, drafts, st.seq_id, n, sp)
    commit(st, emitted, a)
    return StepRecord(drafts=drafts, q_logits=q_logits, p_logits=zp, n_accepted=a, emitted=emitted)


def commit(st: SeqState, emitted, n_accepted: int) -> list:
    """Apply an emitted run: truncate at the stop length, advance the pending token."""
    room = st.stop_len - len(st.generated)
    kept = list(emitted[:room])
    st.generated.extend(kept)
    # KV valid for 0..n+a; the last emitted token is pending at n+a+1.
    st.n = st.n + n_accepted + 1
    st.pending = int(emitted[-1])
    return kept


def ar_step(cfg: Config, W: Weights, st: SeqState, sp: SamplingParams) -> np.ndarray:
    z = forward(cfg, W, [st.pending], [st.n], st.kv)[0]
    t = ar_sample(z, st.seq_id, st.n + 1, sp)
    commit(st, [t], 0)
    return z


def prefill(cfg: Config, W: Weights, seq_id: int, prompt, stop_len: int, capacity: int,
            sp: SamplingParams) -> SeqState:
    """Target forward over prompt positions 0..P-1; the first token is an AR draw at position P."""
    P = len(prompt)
    kv = KVStore(cfg, capacity)
    z = forward(cfg, W, list(prompt), list(range(P)), kv)
    t = ar_sample(z[-1], seq_id, P, sp)
    st = SeqState(seq_id=seq_id, pending=t, n=P, kv=kv, stop_len=stop_len, generated=[t])
    return st


def rollout_ar(cfg, W, prompts, stop_lens, sp: SamplingParams, seq_ids=None):
    seq_ids = list(range(len(prompts))) if seq_ids is None else list(seq_ids)
    out = []
    for sid, pr, L in zip(seq_ids, prompts, stop_lens):
        st = prefill(cfg, W, sid, pr, L, len(pr) + L + 2, sp)
        while not st.done:
            ar_step(cfg, W, st, sp)
        out.append(st.generated)
    return out


def rollout_spec(cfg, W, D, prompts, stop_lens, gamma: int, sp: SamplingParams, seq_ids=None):
    seq_ids = list(range(len(prompts))) if seq_ids is None else list(seq_ids)
    out = []
    for sid, pr, L in zip(seq_ids, prompts, stop_lens):
        st = prefill(cfg, W, sid, pr, L, len(pr) + L + gamma + 2, sp)
        while not st.done:
            spec_step(cfg, W, D, st, gamma, sp)
        out.append(st.generated)
    return out
