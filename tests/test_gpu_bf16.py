"""bf16 parity of the speculative rollout (fused bf16 forward) against the oracle.

bf16 models run the fused forward: RMSNorm formed on the linear's input
load, RoPE and the paged-KV append in the QKV projection's epilogue, SwiGLU in
the gate/up projection's epilogue and the residual add (with the next norm's
sums of squares) in the output projections.  Logits must agree with the oracle
within 3e-2 absolute; tokens exactly on the GPU's own logits, and with the
oracle's logits except on flagged steps (tests/lockstep.py).

Workloads: a 2-layer bf16 decoder with head_dim 128 and a ragged vocabulary
(W4 drafter), batches that put the verify pass on both the skinny path
(M <= 32) and the tiled GEMM (M > 32); and the Qwen2.5-7B widths at reduced
depth (2 layers, full vocabulary), where the projections run at their real
shapes.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from oracle import spec as OSP  # noqa: E402
from oracle.model import KVStore, config_from, forward, weights_from  # noqa: E402

from lockstep import greedy_paths_agree, run_lockstep  # noqa: E402

ABS_TOL = 3e-2
# Two GPU runs that each agree with the oracle within the bf16 bound agree with
# each other within twice it (triangle inequality).
ABS_TOL_GPU_VS_GPU = 2 * ABS_TOL
# Relative perturbation of every pre-rounding value for the oracle's own
# envelope at full width: 2^-20, i.e. 16 fp32 ulps.  An fp32 sum of K terms
# taken in another order typically moves by about sqrt(K) * 2^-24 relative
# (3.6e-6 at K = 3584, 8.2e-6 at K = 18944), so this understates what a
# different accumulation order does; a bf16 store can then round the other way
# and random-init layers amplify each flip.
ENVELOPE_REL = 2.0 ** -20


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


def _setup(shape):
    wts = synth.weights(shape, seed=0)
    cfg = config_from(shape)
    W = weights_from(cfg, {k: v.float().numpy() for k, v in wts.items()})
    D = OSP.build_drafter(W, shape.quant)
    return shape, wts, cfg, W, D


@pytest.fixture(scope="module")
def mini():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _setup(synth.shape("mini-bf16"))


@pytest.mark.parametrize("n_seq,gamma,T,top_p,fused", [
    (4, 4, 1.0, 1.0, True),     # verify M = 20: skinny MFMA path
    (9, 4, 1.0, 0.95, True),    # verify M = 45: tiled GEMM, ragged m-tile
    (3, 8, 0.7, 1.0, True),     # long drafts
    (4, 4, 1.0, 1.0, False),    # the unfused kernel sequence
])
def test_mini_bf16_lockstep(mini, n_seq, gamma, T, top_p, fused):
    shape, wts, cfg, W, D = mini
    prompts = [list(p) for p in synth.prompts(n_seq, 37, shape.vocab, seed=5)]
    eng = _engine(shape, wts, shape.quant, seed=5, temperature=T, top_p=top_p)
    eng.set_fused(fused)
    sp = OSP.SamplingParams(seed=5, temperature=T, top_p=top_p)
    gen, tally = run_lockstep(eng, cfg, W, D, prompts, 40, gamma, sp)
    eng.close()
    print(f"steps={tally.steps} flagged={tally.flagged} abs_q={tally.max_abs_q:.2e} abs_p={tally.max_abs_p:.2e}")
    assert tally.max_abs_q < ABS_TOL and tally.max_abs_p < ABS_TOL
    assert tally.unflagged_mismatch == 0
    assert all(len(g) == 40 for g in gen)


def test_mini_bf16_greedy_spec_equals_ar(mini):
    shape, wts, cfg, W, D = mini
    from speculative_decoding_rl_amd import _lib
    prompts = [list(p) for p in synth.prompts(5, 29, shape.vocab, seed=6)]
    outs = {}
    for mode in ("sd", "ar"):
        eng = _engine(shape, wts, shape.quant, seed=6, temperature=0.0,
                      policy=_lib.ER_POLICY_FORCE_SD if mode == "sd" else _lib.ER_POLICY_FORCE_AR)
        eng.set_gamma(5)
        ids = eng.kv_alloc([29] * 5, [33] * 5)
        first = eng.prefill(ids, prompts)
        out, lens, st = eng.rollout(ids, 64)
        outs[mode] = [[int(first[i])] + list(out[i, :lens[i]]) for i in range(5)]
        eng.close()
    # bf16 rounding can differ between a 1-row and a (gamma+1)-row forward only
    # through accumulation order: the two GPU paths agree token for token up to
    # each sequence's first greedy near-tie (oracle margin under twice the bound)
    checked = greedy_paths_agree(cfg, W, prompts, outs["ar"], outs["sd"], 2.0 * ABS_TOL)
    assert checked >= 50, checked


def test_mini_bf16_shared_prefix_group(mini):
    """Sequences of one group share the prompt's KV blocks (prefilled once)."""
    shape, wts, cfg, W, D = mini
    from speculative_decoding_rl_amd import _lib
    prompt = list(synth.prompts(1, 45, shape.vocab, seed=7)[0])
    eng = _engine(shape, wts, shape.quant, seed=7, temperature=1.0, policy=_lib.ER_POLICY_FORCE_SD)
    eng.set_gamma(3)
    free0, _ = eng.free_blocks()
    ids = eng.kv_alloc([45] * 4, [12] * 4, share_group=[0, 0, 0, 0])
    first = eng.prefill(ids, [prompt] * 4)
    sp = OSP.SamplingParams(seed=7)
    kv = KVStore(cfg, 80)
    z = forward(cfg, W, prompt, list(range(45)), kv)[-1]
    for i in range(4):
        gz = eng.debug_logits(1, i)[0]
        assert np.max(np.abs(gz - z)) < ABS_TOL
        assert OSP.ar_sample(gz.astype(np.float64), int(ids[i]), 45, sp) == first[i]
    out, lens, st = eng.rollout(ids, 32)
    assert list(lens) == [11] * 4
    assert eng.free_blocks()[0] == free0
    eng.kv_free(ids)


@pytest.fixture(scope="module")
def qwen7_2l():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _setup(synth.shape("qwen2.5-7b", n_layers=2))


def test_qwen7b_width_lockstep(qwen7_2l):
    """Real 7B projection shapes (2 layers, vocab 152064): prefill through the
    tiled GEMM, drafter through the W4 streaming path, verify at M = 15.
    Logits must agree within the bf16 bound, or within the oracle's own spread
    when its stores are perturbed by a few fp32 ulps (two shadow oracles on
    the same committed tokens) where that spread is larger."""
    shape, wts, cfg, W, D = qwen7_2l
    prompts = [list(p) for p in synth.prompts(3, 24, shape.vocab, seed=8)]
    eng = _engine(shape, wts, shape.quant, seed=8, max_seqs=4, max_batch=4, max_ctx=128, prefill_chunk=128,
                  kv_blocks=64)
    sp = OSP.SamplingParams(seed=8)
    gen, tally = run_lockstep(eng, cfg, W, D, prompts, 40, 4, sp, max_steps=6, envelope_rel=ENVELOPE_REL,
                              envelope_seeds=2)
    eng.close()
    bound = max(ABS_TOL, tally.envelope)
    print(f"steps={tally.steps} flagged={tally.flagged} abs_q={tally.max_abs_q:.2e} abs_p={tally.max_abs_p:.2e} "
          f"oracle envelope={tally.envelope:.2e} bound={bound:.2e}")
    assert tally.steps == 6
    assert tally.max_abs_q < bound and tally.max_abs_p < bound
    assert tally.unflagged_mismatch == 0


def test_many_chunk_prefill_matches_one_chunk(qwen7_2l):
    """A prefill cut into nine chunks gives the same logits as one chunk, at
    the prompt's end and one decode step later (which reads every chunk's KV).
    Each chunk's metadata goes up from one pinned host region by a queued
    copy; the chunks must not overwrite a copy's source before it has run."""
    from speculative_decoding_rl_amd import _lib
    shape, wts, cfg, W, D = qwen7_2l
    prompts = [list(p) for p in synth.prompts(3, 700, shape.vocab, seed=12)]
    got = []
    for chunk in (256, 4096):
        eng = _engine(shape, wts, shape.quant, seed=12, max_seqs=4, max_batch=4, max_ctx=1024,
                      prefill_chunk=chunk, kv_blocks=256, policy=_lib.ER_POLICY_FORCE_AR)
        ids = eng.kv_alloc([700] * 3, [8] * 3)
        first = eng.prefill(ids, prompts)
        at_prompt = [eng.debug_logits(1, s)[0].copy() for s in range(3)]
        eng.ar_step([int(i) for i in ids])
        after = [eng.debug_logits(1, s)[0].copy() for s in range(3)]
        eng.close()
        got.append((first, at_prompt, after))
    for s in range(3):
        # the decode step's input is the token drawn at the prompt's end: a
        # near-tie may draw differently under the two chunkings
        for k in ((1, 2) if got[0][0][s] == got[1][0][s] else (1,)):
            d = float(np.abs(got[0][k][s] - got[1][k][s]).max())
            assert d < ABS_TOL_GPU_VS_GPU, (s, k, d)
