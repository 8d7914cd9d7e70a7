"""The roofline policy as it runs inside the library (ER_POLICY_AUTO), the
drafter rebuild after a policy update, and shared-prefix groups, through the
C ABI against the oracle.

* AUTO: at every er_step the draft length the library runs equals
  oracle.controller.plan on the same state, batch, mean context and
  acceptance estimate; after a speculative step the trials-based acceptance
  and its EMA (beta = 0.3 on the new sample) equal oracle.controller.alpha_step
  and ema on the per-sequence accepted counts; the policy state equals the
  oracle's.  The cost constants are chosen so that speculation pays at the
  prior and not at the measured acceptance, which makes the policy switch to
  AR and probe (EfficientRollout "关键模块" items 2-3).
* er_update_weights: after a re-point at new weights the drafter is the new
  weights' quantized copy (EfficientRollout "关键模块" item 1: the drafter
  tracks the policy).
* Shared prefixes: a GRPO-style group sharing its prompt's KV blocks rolls
  out exactly as the same sequences with private blocks, and lockstep with
  the oracle over speculative steps (W8 drafter on a bf16 model).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from oracle import controller as OC  # noqa: E402
from oracle import spec as OSP  # noqa: E402
from oracle.model import KVStore, config_from, forward, weights_from  # noqa: E402

from lockstep import abs_err, greedy_paths_agree, rel_err, run_lockstep, teacher_forced  # noqa: E402

ABS_TOL = 3e-2


def _engine(shape, wts, quant, **kw):
    from speculative_decoding_rl_amd import Engine, _lib
    kw.setdefault("max_seqs", 16)
    kw.setdefault("max_batch", 16)
    kw.setdefault("max_ctx", 512)
    kw.setdefault("prefill_chunk", 512)
    kw.setdefault("kv_blocks", 256)
    kw.setdefault("policy", _lib.ER_POLICY_FORCE_SD)
    kw.setdefault("hbm_bytes_per_s", 8e12)
    kw.setdefault("flops_per_s", 2.5e15)
    kw.setdefault("t_fwd_s", 0.0)
    return Engine(shape, {k: v.cuda() for k, v in wts.items()}, quant, **kw)


def _setup(shape, quant, seed=0):
    wts = synth.weights(shape, seed=seed)
    cfg = config_from(shape)
    W = weights_from(cfg, {k: v.float().numpy() for k, v in wts.items()})
    D = OSP.build_drafter(W, quant)
    return shape, wts, cfg, W, D


@pytest.fixture(scope="module")
def mini():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _setup(synth.shape("mini-bf16"), "w4")


def _cost(shape, q_bytes):
    return OC.ModelCost(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                        shape.vocab, 2.0, q_bytes, 2.0)


def _switching_t_fwd(m, bw, fl, B, C):
    """A per-forward time at which speculation pays at alpha 0.9 but not at 0.6."""
    for t in np.geomspace(1e-8, 1e-2, 400):
        r = OC.Roofline(bw, fl, float(t))
        if OC.choose(m, r, B, C, 0.9, 1, 8) > 0 and OC.choose(m, r, B, C, 0.6, 1, 8) == 0:
            return float(t)
    raise AssertionError("no switching regime")


def test_auto_policy_live_loop_matches_oracle(mini):
    from speculative_decoding_rl_amd import _lib
    shape, wts, cfg, W, D = mini
    B, plen = 3, 40
    m = _cost(shape, 0.5 + 3.0 / 128)
    bw, fl = 8e12, 2.5e15
    t_fwd = _switching_t_fwd(m, bw, fl, B, 100.0)
    r = OC.Roofline(bw, fl, t_fwd)
    # T = 0.02: near-greedy sampling on this model accepts about 0.6 of the W4 drafts
    eng = _engine(shape, wts, "w4", seed=3, temperature=0.02, policy=_lib.ER_POLICY_AUTO, alpha_init=0.9,
                  hbm_bytes_per_s=bw, flops_per_s=fl, t_fwd_s=t_fwd)
    ids = [int(i) for i in eng.kv_alloc([plen] * B, [450] * B)]
    eng.prefill(ids, [list(p) for p in synth.prompts(B, plen, shape.vocab, seed=3)])
    cm = eng.cost_model()
    assert cm["t_fwd_s"] == t_fwd and cm["hbm_bytes_per_s"] == bw and cm["flops_per_s"] == fl
    # the descriptor holds alpha_init, beta and the margin as fp32: the library computes with those values
    f32 = lambda x: float(np.float32(x))
    a_init, beta, margin = f32(0.9), f32(0.3), f32(1.02)
    st = OC.PlanState()
    alpha = a_init
    n_sd = n_ar = n_probe = 0
    for step in range(200):
        ctx = [eng.seq_info(i)[1] for i in ids]
        if max(ctx) > 440:
            break
        want = OC.plan(m, r, st, OC.POLICY_AUTO, B, float(np.mean(ctx)), alpha, a_init, 1, 8, margin)
        tok, ne, info = eng.step(ids)
        got = int(info.gamma) if info.mode == _lib.ER_MODE_SD else 0
        assert got == want, step
        ps = eng.plan_state()
        assert (ps["choice"], ps["ar_streak"], ps["probe_every"]) == (st.choice, st.ar_streak, st.probe_every), step
        if got:
            acc = [int(n) - 1 for n in ne]          # no stop truncation here: emitted = accepted + 1
            assert info.accepted == sum(acc) and info.emitted == sum(acc) + B
            a_step = OC.alpha_step(acc, [got] * B)
            assert abs(info.alpha_step - a_step) < 1e-6, step
            alpha = OC.ema(alpha, a_step, beta)
            n_sd += 1
            n_probe += st.choice == 0
        else:
            assert list(ne) == [1] * B
            n_ar += 1
        assert abs(eng.stats()["alpha_ema"] - alpha) < 1e-12, step
    eng.close()
    print(f"sd={n_sd} ar={n_ar} probes={n_probe} alpha_end={alpha:.3f}")
    assert n_sd > 0 and n_ar > 0 and n_probe > 0


def test_auto_policy_greedy_tokens_equal_ar(mini):
    """Under the roofline policy at T = 0 the tokens are the target's greedy tokens, whatever mix of
    speculative and AR steps the policy chose."""
    from speculative_decoding_rl_amd import _lib
    shape, wts, cfg, W, D = mini
    B, plen = 3, 33
    m = _cost(shape, 0.5 + 3.0 / 128)
    t_fwd = _switching_t_fwd(m, 8e12, 2.5e15, B, 80.0)
    prompts = [list(p) for p in synth.prompts(B, plen, shape.vocab, seed=4)]
    outs = {}
    for pol in (_lib.ER_POLICY_AUTO, _lib.ER_POLICY_FORCE_AR):
        eng = _engine(shape, wts, "w4", seed=4, temperature=0.0, policy=pol, alpha_init=0.9, t_fwd_s=t_fwd)
        ids = eng.kv_alloc([plen] * B, [90] * B)
        first = eng.prefill(ids, prompts)
        out, lens, stt = eng.rollout(ids, 128)
        outs[pol] = [[int(first[i])] + list(out[i, :lens[i]]) for i in range(B)]
        if pol == _lib.ER_POLICY_AUTO:
            assert stt["sd_steps"] > 0
        eng.close()
    # The verify pass scores B*(gamma+1) rows and the AR pass B rows through GEMMs that may sum in other
    # orders (from some row count the library GEMM), so on bf16 the paths agree up to the first near-tie.
    checked = greedy_paths_agree(cfg, W, prompts, outs[_lib.ER_POLICY_FORCE_AR], outs[_lib.ER_POLICY_AUTO],
                                 2.0 * ABS_TOL)
    assert checked >= 30, checked


@pytest.mark.parametrize("name,quant,tol_kind", [("tiny", "w8", "rel"), ("mini-bf16", "w4", "abs")])
def test_update_weights_rebuilds_the_drafter(name, quant, tol_kind):
    """A context built on weights A and re-pointed at weights B drafts and verifies as B's oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = synth.shape(name)
    _, wts_a, cfg, _, _ = _setup(shape, quant, seed=0)
    _, wts_b, _, W_b, D_b = _setup(shape, quant, seed=1)
    eng = _engine(shape, wts_a, quant, seed=2, temperature=1.0, max_ctx=256, prefill_chunk=256, kv_blocks=128)
    eng.update_weights({k: v.cuda() for k, v in wts_b.items()})
    gamma, plen = 3, 21
    eng.set_gamma(gamma)
    prompts = [list(p) for p in synth.prompts(2, plen, shape.vocab, seed=2)]
    ids = eng.kv_alloc([plen] * 2, [20] * 2)
    first = eng.prefill(ids, prompts)
    sp = OSP.SamplingParams(seed=2)
    err = rel_err if tol_kind == "rel" else abs_err
    tol = 1e-4 if tol_kind == "rel" else ABS_TOL
    states = []
    for i in range(2):
        kv = KVStore(cfg, plen + 40)
        z = forward(cfg, W_b, prompts[i], list(range(plen)), kv)
        assert err(eng.debug_logits(1, i)[0], z[-1]) < tol
        states.append(OSP.SeqState(seq_id=int(ids[i]), pending=int(first[i]), n=plen, kv=kv, stop_len=20,
                                   generated=[int(first[i])]))
    tok, ne, info = eng.spec_step([int(i) for i in ids])
    drafts = eng.debug_drafts(2, gamma)
    for i in range(2):
        oq, op = teacher_forced(cfg, W_b, D_b, states[i], drafts[i])
        assert err(eng.debug_logits(0, i), oq) < tol, "drafter logits after the update"
        assert err(eng.debug_logits(1, i), op) < tol, "target logits after the update"
    eng.close()


@pytest.fixture(scope="module")
def mini_w8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _setup(synth.shape("mini-bf16"), "w8")


@pytest.mark.parametrize("plen", [45, 48])
def test_shared_prefix_group_equals_private_blocks(mini_w8, plen):
    """A group of four sharing one prompt's KV blocks (45 tokens: two shared blocks plus a copied
    partial block; 48: three shared blocks) rolls out bit for bit as the same four sequences with
    private blocks (same seed, same sequence ids, so the same Philox streams)."""
    from speculative_decoding_rl_amd import _lib
    shape, wts, cfg, W, D = mini_w8
    prompt = list(synth.prompts(1, plen, shape.vocab, seed=9)[0])
    outs = []
    for share in ([0, 0, 0, 0], None):
        eng = _engine(shape, wts, "w8", seed=9, temperature=1.0, policy=_lib.ER_POLICY_FORCE_SD)
        # bit for bit needs the same kernels on both sides: the library GEMM's row threshold would put
        # the private prefill (4 x plen rows) and the group's (plen rows) on different GEMMs, whose fp32
        # sums run in another order
        eng.set_library_gemm(0)
        eng.set_gamma(3)
        free0, _ = eng.free_blocks()
        ids = eng.kv_alloc([plen] * 4, [40] * 4, share_group=share)
        assert list(ids) == [0, 1, 2, 3]
        first = eng.prefill(ids, [prompt] * 4)
        out, lens, st = eng.rollout(ids, 64)
        outs.append([[int(first[i])] + list(out[i, :lens[i]]) for i in range(4)])
        assert st["sd_steps"] > 0
        assert eng.free_blocks()[0] == free0
        eng.close()
    assert outs[0] == outs[1]
    # the members drew different continuations (different sequence ids)
    assert len({tuple(o) for o in outs[0]}) == 4


def test_shared_prefix_group_lockstep_w8_bf16(mini_w8):
    """The group, lockstep against the oracle over speculative steps (drafter and target logits
    within the bf16 bound, decisions exact on the GPU's logits)."""
    shape, wts, cfg, W, D = mini_w8
    prompt = list(synth.prompts(1, 45, shape.vocab, seed=10)[0])
    eng = _engine(shape, wts, "w8", seed=10, temperature=1.0)
    sp = OSP.SamplingParams(seed=10)
    gen, tally = run_lockstep(eng, cfg, W, D, [prompt] * 4, 24, 4, sp, share_group=[0, 0, 0, 0])
    eng.close()
    print(f"steps={tally.steps} flagged={tally.flagged} abs_q={tally.max_abs_q:.2e} abs_p={tally.max_abs_p:.2e}")
    assert tally.steps >= 4
    assert tally.max_abs_q < ABS_TOL and tally.max_abs_p < ABS_TOL
    assert tally.unflagged_mismatch == 0
    assert all(len(g) == 24 for g in gen)
