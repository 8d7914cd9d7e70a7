"""Forked sequences (er_kv_fork): children share the parent's committed KV blocks and copy its partial
last block, then continue on their own Philox streams.  Checked against the oracle, whose child state is
the parent's state (KV rows, pending token, position, generated tokens) under the child's sequence id.

Tiny fp32 decoder (W8 drafter): logits within 1e-4 relative, tokens exact on the GPU's logits.
"""
import copy

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from oracle import spec as OSP  # noqa: E402
from oracle.model import config_from, forward, weights_from  # noqa: E402


def _engine(shape, wts, **kw):
    from speculative_decoding_rl_amd import Engine, _lib
    kw.setdefault("max_seqs", 16)
    kw.setdefault("max_batch", 16)
    kw.setdefault("max_ctx", 256)
    kw.setdefault("prefill_chunk", 256)
    kw.setdefault("kv_blocks", 128)
    kw.setdefault("policy", _lib.ER_POLICY_FORCE_AR)
    kw.setdefault("hbm_bytes_per_s", 8e12)
    kw.setdefault("flops_per_s", 2.5e15)
    kw.setdefault("t_fwd_s", 0.0)
    return Engine(shape, {k: v.cuda() for k, v in wts.items()}, "w8", **kw)


@pytest.fixture(scope="module")
def tiny():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = synth.shape("tiny")
    wts = synth.weights(shape, seed=0)
    cfg = config_from(shape)
    W = weights_from(cfg, {k: v.float().numpy() for k, v in wts.items()})
    return shape, wts, cfg, W


def _child_state(st, seq_id, stop_len):
    c = copy.copy(st)
    c.kv = st.kv.copy()
    c.generated = list(st.generated)
    c.seq_id = seq_id
    c.stop_len = stop_len
    return c


def _ar_lockstep(eng, cfg, W, ids, states, sp, steps):
    for _ in range(steps):
        tok, _ = eng.ar_step(ids)
        for i, st in enumerate(states):
            gz = eng.debug_logits(1, i)[0]
            z = forward(cfg, W, [st.pending], [st.n], st.kv)[0]
            assert np.max(np.abs(gz - z)) / np.max(np.abs(z)) < 1e-4
            assert OSP.ar_sample(gz.astype(np.float64), st.seq_id, st.n + 1, sp) == tok[i]
            OSP.commit(st, [int(tok[i])], 0)


@pytest.mark.parametrize("steps_before", [5, 12])   # 20 + 5 = 25 keys (partial block), 20 + 12 = 32 (none)
def test_forked_children_continue_like_the_oracle(tiny, steps_before):
    shape, wts, cfg, W = tiny
    sp = OSP.SamplingParams(seed=7, temperature=1.0)
    eng = _engine(shape, wts, seed=7)
    free0, _ = eng.free_blocks()
    prompt = list(synth.prompts(1, 20, shape.vocab, seed=7)[0])
    pid = int(eng.kv_alloc([20], [60])[0])
    first = eng.prefill([pid], [prompt])
    par = OSP.prefill(cfg, W, pid, prompt, 60, 128, sp)
    assert par.pending == first[0]
    _ar_lockstep(eng, cfg, W, [pid], [par], sp, steps_before)
    n = par.n
    before = eng.free_blocks()[0]
    kids = [int(k) for k in eng.kv_fork(pid, [50, 55, 60])]
    # a partial last block is copied once per child; full blocks are shared
    assert before - eng.free_blocks()[0] == (3 if n % 16 else 0)
    for k in kids:
        g, ctx, fin = eng.seq_info(k)
        assert (g, ctx, fin) == eng.seq_info(pid)
    states = [par] + [_child_state(par, k, m) for k, m in zip(kids, [50, 55, 60])]
    _ar_lockstep(eng, cfg, W, [pid] + kids, states, sp, 8)
    gens = [tuple(s.generated[-8:]) for s in states[1:]]
    assert len(set(gens)) > 1            # the children draw from their own streams
    eng.kv_free(kids)
    eng.kv_free([pid])
    assert eng.free_blocks()[0] == free0


def test_greedy_speculation_over_forks_equals_greedy_ar(tiny):
    """At T = 0 every branch of a fork continues the same way; drafts written into the children's and the
    parent's private blocks must not touch the shared ones, so all of them equal the oracle's greedy AR."""
    shape, wts, cfg, W = tiny
    from speculative_decoding_rl_amd import _lib
    eng = _engine(shape, wts, seed=3, temperature=0.0, policy=_lib.ER_POLICY_FORCE_SD)
    eng.set_gamma(3)
    prompt = list(synth.prompts(1, 27, shape.vocab, seed=3)[0])
    pid = int(eng.kv_alloc([27], [70])[0])
    first = eng.prefill([pid], [prompt])
    gen = {pid: [int(first[0])]}
    for _ in range(3):
        tok, ne, _ = eng.step([pid])
        gen[pid] += [int(t) for t in tok[0, :ne[0]]]
    kids = [int(k) for k in eng.kv_fork(pid, [70, 70])]
    for k in kids:
        gen[k] = list(gen[pid])
    act = [pid] + kids
    while act:
        tok, ne, _ = eng.step(act)
        for i, a in enumerate(act):
            gen[a] += [int(t) for t in tok[i, :ne[i]]]
        act = [a for a in act if not eng.seq_info(a)[2]]
    ref = OSP.rollout_ar(cfg, W, [prompt], [70], OSP.SamplingParams(seed=3, temperature=0.0))[0]
    for a in [pid] + kids:
        assert gen[a] == ref, a
    eng.close()


def test_fork_refuses_bad_requests(tiny):
    shape, wts, cfg, W = tiny
    from speculative_decoding_rl_amd import _lib
    eng = _engine(shape, wts, seed=1, max_seqs=3, max_batch=3)
    prompt = list(synth.prompts(1, 10, shape.vocab, seed=1)[0])
    pid = int(eng.kv_alloc([10], [20])[0])
    with pytest.raises(_lib.ErError) as e:
        eng.kv_fork(pid, [20])                      # not prefilled
    assert e.value.code == _lib.ER_ESTATE
    eng.prefill([pid], [prompt])
    with pytest.raises(_lib.ErError) as e:
        eng.kv_fork(pid, [1])                       # cap not above the generated count
    assert e.value.code == _lib.ER_EINVAL
    with pytest.raises(_lib.ErError) as e:
        eng.kv_fork(pid, [20, 20, 20])              # max_seqs
    assert e.value.code == _lib.ER_ENOMEM
    free = eng.free_blocks()[0]
    assert eng.seq_info(pid) == (1, 10, 0) and eng.free_blocks()[0] == free
    eng.close()
