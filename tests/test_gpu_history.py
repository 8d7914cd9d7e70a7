"""History steps (drafts copied from earlier rollouts, er_history_step / ER_POLICY_HISTORY) against the
oracle: the library's drafts equal oracle.history's on the oracle's token history, the verify logits
equal the oracle's target forward (tiny fp32 decoder, 1e-4 relative), the proposal rows are point
masses, and the emitted tokens equal the oracle's lossless decision with point-mass proposals on the
GPU's logits, exactly.  Greedy: a rollout drafted from an earlier greedy rollout of the same prompt
accepts every draft and equals greedy AR in fewer steps."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from oracle import spec as OSP  # noqa: E402
from oracle.history import HistoryCache, point_mass_logits  # noqa: E402
from oracle.model import config_from, forward, weights_from  # noqa: E402


def _engine(shape, wts, **kw):
    from speculative_decoding_rl_amd import Engine, _lib
    kw.setdefault("max_seqs", 8)
    kw.setdefault("max_batch", 8)
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


def test_history_steps_match_the_oracle(tiny):
    from speculative_decoding_rl_amd import History
    shape, wts, cfg, W = tiny
    V, g, L = shape.vocab, 3, 1
    sp = OSP.SamplingParams(seed=4, temperature=1.0)
    prompts = [list(p) for p in synth.prompts(3, 12, V, seed=4)]
    # earlier rollouts: the oracle's own samples of the same prompts under another seed, plus a short
    # sequence of tokens the prompts end with, so that some keys hit and some miss
    earlier = OSP.rollout_ar(cfg, W, prompts, [40] * 3, OSP.SamplingParams(seed=99, temperature=1.0))
    ora, lib = HistoryCache(L), History(L)
    for i, (p, r) in enumerate(zip(prompts, earlier)):
        ora.add(p, r, float(i))
        lib.add(p, r, float(i))
    eng = _engine(shape, wts, seed=4)
    eng.set_history(lib, gamma=g, max_batch=8)
    ids = [int(i) for i in eng.kv_alloc([12] * 3, [30] * 3)]
    first = eng.prefill(ids, prompts)
    states = [OSP.prefill(cfg, W, ids[i], prompts[i], 30, 128, sp) for i in range(3)]
    assert [s.pending for s in states] == list(first)
    accepted = 0
    act = list(range(3))
    while act:
        tok, ne, info = eng.history_step([ids[i] for i in act])
        assert info.mode == 3
        drafts = eng.debug_drafts(len(act), g)
        for slot, i in enumerate(act):
            st = states[i]
            d = ora.propose(prompts[i], prompts[i] + st.generated, g)
            d = d + [st.pending] * (g - len(d))
            assert list(drafts[slot]) == d, (i, st.n)
            gp = eng.debug_logits(1, slot).astype(np.float64)
            gq = eng.debug_logits(0, slot)
            for j in range(g):
                assert gq[j][d[j]] == 0.0 and np.all(np.delete(gq[j], d[j]) <= -1e29)
            kv = st.kv.copy()
            op = forward(cfg, W, [st.pending] + d, list(range(st.n, st.n + g + 1)), kv)
            assert np.max(np.abs(gp - op)) / np.max(np.abs(op)) < 1e-4
            q = np.stack([point_mass_logits(x, V) for x in d])
            a, em = OSP.spec_decide(gp, q, d, st.seq_id, st.n, sp)
            kept = int(ne[slot])
            assert em[:kept] == list(tok[slot, :kept]), (i, st.n)
            accepted += a
            forward(cfg, W, [st.pending] + d[:a], list(range(st.n, st.n + a + 1)), st.kv)
            OSP.commit(st, em, a)
        act = [i for i in act if not eng.seq_info(ids[i])[2]]
    st = eng.stats()
    assert st["history_steps"] > 0 and st["history_accepted"] == accepted
    eng.close()
    lib.close()


def test_greedy_history_rollout_equals_greedy_ar_in_fewer_steps(tiny):
    """At T = 0 an earlier greedy rollout of the same prompt is what the target will say again: drafted
    from it, the rollout equals greedy AR token for token, in the steps the cache's drafts predict."""
    from speculative_decoding_rl_amd import History, _lib
    shape, wts, cfg, W = tiny
    g = 4
    prompt = list(synth.prompts(1, 16, shape.vocab, seed=8)[0])
    greedy = OSP.SamplingParams(seed=8, temperature=0.0)
    # the earlier rollout runs past this one's stop, so that its drafts cover the last step too
    ref_long = OSP.rollout_ar(cfg, W, [prompt], [71], greedy)[0]
    ref = ref_long[:61]
    hist = History(4)
    hist.add(prompt, ref_long, 1.0)
    eng = _engine(shape, wts, seed=8, temperature=0.0, policy=_lib.ER_POLICY_HISTORY)
    eng.set_history(hist, gamma=g, max_batch=8)
    sid = int(eng.kv_alloc([16], [61])[0])
    out = [int(eng.prefill([sid], [prompt])[0])]
    steps = 0
    while not eng.seq_info(sid)[2]:
        tok, ne, info = eng.step([sid])
        assert info.mode == _lib.ER_MODE_HISTORY
        out += [int(t) for t in tok[0, :ne[0]]]
        steps += 1
    assert out == ref
    # the same steps on the oracle's cache: at T = 0 a draft is accepted exactly when it is the greedy
    # token, so the accepted count and the number of steps follow from the drafts alone (a key that
    # recurs in the record offers its last continuation, which a greedy loop need not repeat)
    ora = HistoryCache(4)
    ora.add(prompt, ref_long, 1.0)
    gen, acc, n_steps = [ref[0]], 0, 0
    while len(gen) < len(ref):
        d = ora.propose(prompt, prompt + gen, g)
        d = d + [gen[-1]] * (g - len(d))
        a = 0
        while a < g and d[a] == ref_long[len(gen) + a]:
            a += 1
        acc += a
        gen = gen + ref_long[len(gen):len(gen) + a + 1]
        n_steps += 1
    st = eng.stats()
    assert steps == n_steps and st["history_accepted"] == acc, (steps, n_steps, st["history_accepted"], acc)
    assert steps < 60 // 2                      # far fewer than AR's 60 steps
    eng.close()


def test_history_policy_falls_back_to_ar(tiny):
    """ER_POLICY_HISTORY takes AR steps without a record in the cache and above its batch limit."""
    from speculative_decoding_rl_amd import History, _lib
    shape, wts, cfg, W = tiny
    eng = _engine(shape, wts, seed=2, policy=_lib.ER_POLICY_HISTORY)
    hist = History(2)
    eng.set_history(hist, gamma=2, max_batch=2)
    ids = [int(i) for i in eng.kv_alloc([8] * 3, [20] * 3)]
    eng.prefill(ids, [list(p) for p in synth.prompts(3, 8, shape.vocab, seed=2)])
    _, _, info = eng.step(ids[:1])
    assert info.mode == _lib.ER_MODE_AR          # empty cache
    hist.add([1, 2, 3], [4, 5, 6], 0.0)
    _, _, info = eng.step(ids[:2])
    assert info.mode == _lib.ER_MODE_HISTORY
    _, _, info = eng.step(ids)
    assert info.mode == _lib.ER_MODE_AR          # 3 > max_batch
    eng.close()
