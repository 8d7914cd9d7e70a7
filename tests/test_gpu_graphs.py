"""Bucketed graph capture (er_set_graphs) against the oracle.

With graphs on, steps run as their batch bucket (1 .. 16 as they are, larger
batches padded to a power of two) and replay graphs recorded per (kind,
bucket, gamma, context capacity).  Every replay is
checked: the speculative lockstep (tests/lockstep.py) compares each step's
drafter and target logits with the oracle's (tiny fp32 decoder within 1e-4
relative; the bf16 decoder within 3e-2 absolute) and the tokens exactly on the
GPU's own logits, while the batch shrinks through the buckets 32, 16, ..., 1 and
the host's own work and synchronizations run between replays.  AR steps with
a padded bucket are checked the same way, a history step reuses the verify
graph recorded by a self-drafted step of the same key, and the settings that
must not replay (kernel profile on) or must drop graphs (new weights) do so.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from oracle import spec as OSP  # noqa: E402
from oracle.model import config_from, forward, weights_from  # noqa: E402

from lockstep import run_lockstep  # noqa: E402


def _engine(shape, wts, quant, **kw):
    from speculative_decoding_rl_amd import Engine, _lib
    kw.setdefault("max_seqs", 16)
    kw.setdefault("max_batch", 8)
    kw.setdefault("max_ctx", 512)
    kw.setdefault("prefill_chunk", 512)
    kw.setdefault("kv_blocks", 256)
    kw.setdefault("policy", _lib.ER_POLICY_FORCE_SD)
    kw.setdefault("hbm_bytes_per_s", 8e12)
    kw.setdefault("flops_per_s", 2.5e15)
    kw.setdefault("t_fwd_s", 0.0)
    return Engine(shape, {k: v.cuda() for k, v in wts.items()}, quant, **kw)


def _setup(name, quant):
    shape = synth.shape(name)
    wts = synth.weights(shape, seed=0)
    cfg = config_from(shape)
    W = weights_from(cfg, {k: v.float().numpy() for k, v in wts.items()})
    D = OSP.build_drafter(W, quant)
    return shape, wts, cfg, W, D


@pytest.fixture(scope="module")
def tiny():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _setup("tiny", "w8")


@pytest.fixture(scope="module")
def mini():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = synth.shape("mini-bf16")
    return _setup("mini-bf16", shape.quant)


@pytest.mark.parametrize("n,T,top_p", [(5, 1.0, 1.0), (5, 0.8, 0.9), (18, 1.0, 1.0)])
def test_tiny_fp32_graph_lockstep(tiny, n, T, top_p):
    """5 sequences (buckets of their own) and 18 (bucket 32, fourteen padding rows, then their own
    buckets from 16 down) with ragged prompts, shrinking to one."""
    shape, wts, cfg, W, D = tiny
    prompts = [list(p) for p in synth.prompts(n, 40, shape.vocab, seed=7)]
    prompts = [p[:20 + (4 * i) % 20] for i, p in enumerate(prompts)]
    eng = _engine(shape, wts, "w8", seed=7, temperature=T, top_p=top_p, gamma_max=8, max_seqs=40, max_batch=32,
                  kv_blocks=512)
    eng.set_graphs(32)
    sp = OSP.SamplingParams(seed=7, temperature=T, top_p=top_p)
    gen, tally = run_lockstep(eng, cfg, W, D, prompts, 60, 4, sp)
    gs = eng.graph_stats()
    eng.close()
    print(f"steps={tally.steps} flagged={tally.flagged} rel_q={tally.max_rel_q:.2e} rel_p={tally.max_rel_p:.2e} "
          f"graphs={gs}")
    assert tally.max_rel_q < 1e-4 and tally.max_rel_p < 1e-4
    assert tally.unflagged_mismatch == 0
    assert all(len(g) == 60 for g in gen)
    # every speculative step replayed a drafter and a verify graph; most replays reuse a recorded graph
    assert gs["replays"] == 2 * tally.steps
    assert 2 <= gs["captures"] < gs["replays"]


@pytest.mark.parametrize("n_seq,gamma", [(3, 4), (6, 2)])
def test_mini_bf16_graph_lockstep(mini, n_seq, gamma):
    """bf16 fused forward through graphs: MFMA attention with a fixed number of units per item."""
    shape, wts, cfg, W, D = mini
    prompts = [list(p) for p in synth.prompts(n_seq, 37, shape.vocab, seed=5)]
    eng = _engine(shape, wts, shape.quant, seed=5, temperature=1.0, top_p=1.0)
    eng.set_graphs(8)
    sp = OSP.SamplingParams(seed=5, temperature=1.0, top_p=1.0)
    gen, tally = run_lockstep(eng, cfg, W, D, prompts, 40, gamma, sp)
    gs = eng.graph_stats()
    eng.close()
    print(f"steps={tally.steps} flagged={tally.flagged} abs_q={tally.max_abs_q:.2e} abs_p={tally.max_abs_p:.2e} "
          f"graphs={gs}")
    assert tally.max_abs_q < 3e-2 and tally.max_abs_p < 3e-2
    assert tally.unflagged_mismatch == 0
    assert gs["replays"] == 2 * tally.steps and gs["captures"] < gs["replays"]


@pytest.mark.parametrize("n", [3, 17])
def test_graph_ar_steps_match_the_oracle(tiny, n):
    """AR steps of 3 sequences (bucket 3) and of 17 (bucket 32, fifteen padding rows); logits and tokens
    of every step against the oracle."""
    shape, wts, cfg, W, D = tiny
    from speculative_decoding_rl_amd import _lib
    prompts = synth.prompts(n, 20, shape.vocab, seed=2)
    eng = _engine(shape, wts, "w8", seed=2, policy=_lib.ER_POLICY_FORCE_AR, max_seqs=40, max_batch=32,
                  kv_blocks=512)
    eng.set_graphs(32)
    ids = eng.kv_alloc([20] * n, [12] * n)
    first = eng.prefill(ids, list(prompts))
    sp = OSP.SamplingParams(seed=2)
    states = [OSP.prefill(cfg, W, int(ids[i]), list(prompts[i]), 12, 40, sp) for i in range(n)]
    assert [s.pending for s in states] == list(first)
    for _ in range(8):
        tok, info = eng.ar_step(ids)
        for i in range(n):
            gz = eng.debug_logits(1, i)[0]
            z = forward(cfg, W, [states[i].pending], [states[i].n], states[i].kv)[0]
            assert np.max(np.abs(gz - z)) / np.max(np.abs(z)) < 1e-4
            assert OSP.ar_sample(gz.astype(np.float64), int(ids[i]), states[i].n + 1, sp) == tok[i]
            OSP.commit(states[i], [int(tok[i])], 0)
    gs = eng.graph_stats()
    eng.close()
    assert gs["replays"] == 8 and gs["captures"] == 1


def test_greedy_graph_rollout_equals_eager_and_oracle(tiny):
    """Greedy speculative rollouts with and without graphs equal the oracle's greedy AR rollout."""
    shape, wts, cfg, W, D = tiny
    prompts = synth.prompts(5, 24, shape.vocab, seed=9)
    outs = {}
    for graphs in (0, 8):
        eng = _engine(shape, wts, "w8", seed=9, temperature=0.0)
        eng.set_graphs(graphs)
        eng.set_gamma(3)
        ids = eng.kv_alloc([24] * 5, [40] * 5)
        first = eng.prefill(ids, list(prompts))
        out, lens, st = eng.rollout(ids, 48)
        outs[graphs] = [[int(first[i])] + list(out[i, :lens[i]]) for i in range(5)]
        gs = eng.graph_stats()
        eng.close()
        assert (gs["replays"] > 0) == (graphs > 0)
    ref = OSP.rollout_ar(cfg, W, [list(p) for p in prompts], [40] * 5, OSP.SamplingParams(seed=9, temperature=0.0))
    assert outs[8] == outs[0] == ref


def test_history_step_reuses_the_verify_graph(tiny):
    """A history step of the same (bucket, gamma, capacity) replays the verify graph a self-drafted step
    recorded: no new recording, one more replay; its tokens follow the lossless decision on its logits."""
    from speculative_decoding_rl_amd import History
    shape, wts, cfg, W, D = tiny
    prompts = [list(p) for p in synth.prompts(2, 16, shape.vocab, seed=3)]
    hist = History(1)
    for p in prompts:
        hist.add(p, list(p[:8]), 1.0)
    eng = _engine(shape, wts, "w8", seed=3)
    eng.set_graphs(8)
    eng.set_gamma(4)
    eng.set_history(hist, gamma=4, max_batch=8)
    ids = [int(i) for i in eng.kv_alloc([16] * 2, [30] * 2)]
    eng.prefill(ids, prompts)
    eng.spec_step(ids)
    g1 = eng.graph_stats()
    assert g1["captures"] == 2 and g1["replays"] == 2
    tok, ne, info = eng.history_step(ids)
    assert info.mode == 3
    g2 = eng.graph_stats()
    assert g2["captures"] == 2 and g2["replays"] == 3
    sp = OSP.SamplingParams(seed=3)
    drafts = eng.debug_drafts(2, 4)
    for slot in range(2):
        gp = eng.debug_logits(1, slot).astype(np.float64)
        gq = eng.debug_logits(0, slot).astype(np.float64)
        _, n_ctx, _ = eng.seq_info(ids[slot])
        n0 = n_ctx - int(ne[slot])
        a, em = OSP.spec_decide(gp, gq, list(drafts[slot]), ids[slot], n0, sp)
        assert em[:int(ne[slot])] == list(tok[slot, :int(ne[slot])])
    eng.close()


def test_graphs_off_under_profile_and_dropped_on_new_weights(tiny):
    shape, wts, cfg, W, D = tiny
    from speculative_decoding_rl_amd import _lib
    eng = _engine(shape, wts, "w8", seed=1)
    eng.set_graphs(8)
    eng.set_gamma(2)
    ids = [int(i) for i in eng.kv_alloc([16] * 2, [40] * 2)]
    eng.prefill(ids, [list(p) for p in synth.prompts(2, 16, shape.vocab, seed=1)])
    eng.spec_step(ids)
    assert eng.graph_stats()["cached"] == 2
    eng.set_kernel_profile(_lib.ER_KPROF_ALL)
    eng.spec_step(ids)
    eng.set_kernel_profile(_lib.ER_KPROF_OFF)
    assert eng.graph_stats()["replays"] == 2          # the profiled step ran eagerly
    eng.update_weights({k: v.cuda() for k, v in wts.items()})
    assert eng.graph_stats()["cached"] == 0
    eng.spec_step(ids)
    gs = eng.graph_stats()
    assert gs["cached"] == 2 and gs["captures"] == 4
    free0, total = eng.free_blocks()
    eng.set_graphs(0)
    free1, _ = eng.free_blocks()
    assert free1 == free0 + 1                           # the padding block went back to the pool
    eng.close()
