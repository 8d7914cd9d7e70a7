"""Pins oracle/spec.py: greedy equivalence, brute-force losslessness, closed forms."""
import itertools

import numpy as np
import pytest

from oracle import philox, spec
from oracle.model import KVStore, forward
from oracle.sampling import accept_prob, pi, residual
from oracle.spec import SamplingParams

from oracle_fixtures import tiny_config, tiny_weights


def _setup(V=16, quant="w8", seed=0, std=0.3, L=1):
    cfg = tiny_config(V=V, L=L)
    W = tiny_weights(cfg, seed=seed, std=std)
    D = spec.build_drafter(W, quant, group=128)
    return cfg, W, D


@pytest.mark.parametrize("quant", ["w8", "w4"])
def test_greedy_spec_equals_greedy_ar(quant):
    cfg, W, D = _setup(V=64, quant=quant, L=2)
    rng = np.random.Generator(np.random.PCG64(3))
    prompts = [list(rng.integers(0, 64, 6)) for _ in range(3)]
    sp = SamplingParams(seed=0, temperature=0.0, top_p=1.0)
    ar = spec.rollout_ar(cfg, W, prompts, [20, 20, 20], sp)
    for gamma in (1, 3, 5):
        sd = spec.rollout_spec(cfg, W, D, prompts, [20, 20, 20], gamma, sp)
        assert sd == ar


def _exact_joint_sd(cfg, W, D, prompt, gamma, T, top_p):
    """Exact distribution of the first gamma+1 tokens: one SD step, then target AR (enumerated)."""
    V = cfg.vocab
    P = len(prompt)
    cache = {}

    def target_dist(tokens):
        key = tuple(tokens)
        if key not in cache:
            kv = KVStore(cfg, len(tokens) + 1)
            z = forward(cfg, W, list(tokens), list(range(len(tokens))), kv)[-1]
            cache[key] = pi(z, T, top_p)
        return cache[key]

    # prefix state: KV of the prompt written by the target; the pending token is the last prompt token
    base = KVStore(cfg, P + gamma + 2)
    forward(cfg, W, prompt[:-1], list(range(P - 1)), base)
    n = P - 1
    joint = {}

    def extend(emitted, prob):
        # AR extension from the target up to gamma+1 tokens
        if prob == 0.0:
            return
        if len(emitted) == gamma + 1:
            joint[tuple(emitted)] = joint.get(tuple(emitted), 0.0) + prob
            return
        p = target_dist(list(prompt) + list(emitted))
        for t in range(V):
            if p[t] > 0:
                extend(emitted + [t], prob * p[t])

    for drafts in itertools.product(range(V), repeat=gamma):
        kv = base.copy()
        tok = prompt[-1]
        qs = []
        pd = 1.0
        for j in range(gamma):
            zq = forward(cfg, W, [tok], [n + j], kv, lin=D)[0]
            q = pi(zq, T, top_p)
            qs.append(q)
            pd *= q[drafts[j]]
            tok = drafts[j]
        if pd == 0.0:
            continue
        zp = forward(cfg, W, [prompt[-1]] + list(drafts), list(range(n, n + gamma + 1)), kv)
        ps = [pi(zp[j], T, top_p) for j in range(gamma + 1)]
        reach = pd
        for j in range(gamma):
            a = accept_prob(ps[j], qs[j], drafts[j])
            r = residual(ps[j], qs[j])
            for t in range(V):
                if r[t] > 0:
                    extend(list(drafts[:j]) + [t], reach * (1 - a) * r[t])
            reach *= a
        for t in range(V):
            if ps[gamma][t] > 0:
                extend(list(drafts) + [t], reach * ps[gamma][t])

    target = {}
    def tgt(prefix, prob):
        if len(prefix) == gamma + 1:
            target[tuple(prefix)] = prob
            return
        p = target_dist(list(prompt) + prefix)
        for t in range(V):
            if p[t] > 0:
                tgt(prefix + [t], prob * p[t])
    tgt([], 1.0)
    return joint, target


@pytest.mark.parametrize("V,gamma,quant,T,top_p", [
    (8, 1, "w8", 1.0, 1.0),
    (8, 2, "w4", 1.0, 1.0),
    (16, 2, "w8", 1.0, 1.0),
    (8, 2, "w8", 0.7, 0.8),
])
def test_brute_force_lossless(V, gamma, quant, T, top_p):
    cfg, W, D = _setup(V=V, quant=quant, std=0.5)
    joint, target = _exact_joint_sd(cfg, W, D, [1, 5, 3], gamma, T, top_p)
    keys = set(joint) | set(target)
    diff = max(abs(joint.get(k, 0.0) - target.get(k, 0.0)) for k in keys)
    assert abs(sum(joint.values()) - 1.0) < 1e-12
    assert diff < 1e-12


def test_monte_carlo_step_code_matches_target():
    """The Philox-driven step code (not just the enumerated rule) reproduces the target joint."""
    V, gamma = 6, 1
    cfg, W, D = _setup(V=V, quant="w4", std=0.6)
    prompt = [2, 4]
    _, target = _exact_joint_sd(cfg, W, D, prompt, gamma, 1.0, 1.0)
    N = 6000
    counts = {}
    sp = SamplingParams(seed=11, temperature=1.0, top_p=1.0)
    for sid in range(N):
        kv = KVStore(cfg, 8)
        forward(cfg, W, prompt[:-1], [0], kv)
        st = spec.SeqState(seq_id=sid, pending=prompt[-1], n=1, kv=kv, stop_len=10, generated=[])
        spec.spec_step(cfg, W, D, st, gamma, sp)
        while len(st.generated) < gamma + 1:
            spec.ar_step(cfg, W, st, sp)
        k = tuple(st.generated[:gamma + 1])
        counts[k] = counts.get(k, 0) + 1
    chi2 = 0.0
    for k, pr in target.items():
        e = N * pr
        chi2 += (counts.get(k, 0) - e) ** 2 / e
    dof = len(target) - 1
    assert chi2 < dof + 5 * np.sqrt(2 * dof)


def test_q_equals_p_emits_gamma_plus_one():
    cfg, W, _ = _setup(V=32)
    D = spec.DraftLinears(wqkv=W.wqkv, wo=W.wo, wgate_up=W.wgate_up, wdown=W.wdown, lm_head=W.lm_head)
    sp = SamplingParams(seed=5)
    for sid in range(20):
        kv = KVStore(cfg, 40)
        forward(cfg, W, [3, 1, 4], [0, 1, 2], kv)
        st = spec.SeqState(seq_id=sid, pending=1, n=3, kv=kv, stop_len=100, generated=[])
        for _ in range(3):
            rec = spec.spec_step(cfg, W, D, st, 4, sp)
            assert rec.n_accepted == 4 and len(rec.emitted) == 5


def test_disjoint_support_emits_one_token_from_p():
    V = 10
    p_log = np.full(V, -np.inf)
    p_log[:4] = np.log([0.1, 0.2, 0.3, 0.4])
    q_log = np.full(V, -np.inf)
    q_log[6:] = 0.0
    sp = SamplingParams(seed=2)
    counts = np.zeros(V)
    N = 8000
    for sid in range(N):
        drafts = []
        for j in range(1, 4):
            drafts.append(spec.draft_sample(q_log, sid, 10 + j, j, sp))
        a, em = spec.spec_decide(np.stack([p_log] * 4), np.stack([q_log] * 3), drafts, sid, 10, sp)
        assert a == 0 and len(em) == 1
        counts[em[0]] += 1
    exp = N * np.array([0.1, 0.2, 0.3, 0.4])
    chi2 = float(np.sum((counts[:4] - exp) ** 2 / exp))
    assert counts[4:].sum() == 0 and chi2 < 3 + 5 * np.sqrt(6)


@pytest.mark.parametrize("gamma", [1, 3, 6])
def test_mean_emitted_closed_form(gamma):
    V = 12
    rng = np.random.Generator(np.random.PCG64(gamma))
    p_log = rng.standard_normal(V)
    q_log = p_log + 0.7 * rng.standard_normal(V)
    p, q = pi(p_log, 1.0, 1.0), pi(q_log, 1.0, 1.0)
    alpha = float(np.sum(np.minimum(p, q)))
    sp = SamplingParams(seed=9)
    N = 8000
    lens = np.zeros(N)
    for sid in range(N):
        drafts = [spec.draft_sample(q_log, sid, 100 + j, j, sp) for j in range(1, gamma + 1)]
        _, em = spec.spec_decide(np.stack([p_log] * (gamma + 1)), np.stack([q_log] * gamma), drafts, sid, 100, sp)
        lens[sid] = len(em)
    en = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(lens.mean() - en) < 4 * lens.std() / np.sqrt(N)


def test_gamma_zero_is_a_target_sample():
    V = 8
    p_log = np.log(np.arange(1, V + 1, dtype=float))
    p = pi(p_log, 1.0, 1.0)
    sp = SamplingParams(seed=4)
    N = 8000
    counts = np.zeros(V)
    for sid in range(N):
        a, em = spec.spec_decide(p_log[None, :], np.zeros((0, V)), [], sid, 3, sp)
        assert a == 0 and len(em) == 1
        counts[em[0]] += 1
    chi2 = float(np.sum((counts - N * p) ** 2 / (N * p)))
    assert chi2 < 7 + 5 * np.sqrt(14)


@pytest.mark.parametrize("quant", ["w8", "w4"])
def test_kv_after_rejection_equals_target_prefill(quant):
    """KV rollback (speculative sampling over a shared paged KV): after every step, rows
    0..n-1 must be the target's own K/V for the committed tokens, as a fresh target
    prefill of prompt + emitted tokens writes them, whatever the drafter or the rejected
    drafts wrote into those rows; the pending position n = P + len(generated) - 1 until
    the stop length cuts the last emitted run (then only the kept tokens are compared)."""
    cfg, W, D = _setup(V=64, quant=quant, L=2, std=0.6)
    prompt = [5, 17, 42, 3, 9]
    sp = SamplingParams(seed=11, temperature=1.0, top_p=1.0)
    gamma, stop = 4, 24
    st = spec.prefill(cfg, W, 0, prompt, stop, len(prompt) + stop + gamma + 2, sp)
    rejected = 0
    while not st.done:
        rec = spec.spec_step(cfg, W, D, st, gamma, sp)
        rejected += rec.n_accepted < gamma
        toks = list(prompt) + st.generated[:-1]
        m = len(toks)
        if not st.done:
            assert st.n == m and st.pending == st.generated[-1]
        ref = KVStore(cfg, st.kv.capacity)
        forward(cfg, W, toks, list(range(m)), ref)
        np.testing.assert_allclose(st.kv.k[:, :m], ref.k[:, :m], rtol=0, atol=1e-12)
        np.testing.assert_allclose(st.kv.v[:, :m], ref.v[:, :m], rtol=0, atol=1e-12)
    assert rejected > 0
