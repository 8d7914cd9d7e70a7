"""Lockstep comparison of the GPU rollout against the oracle (test helper).

The GPU runs a step; the oracle recomputes, on the GPU's committed prefix and
with the GPU's drafts, the drafter and target logits (compared within the
logits tolerance), re-runs the sampler on the GPU's own logits (must give the
GPU's tokens exactly), runs the sampler on its own logits (must agree unless
the step is flagged), and then commits the GPU's tokens so that one boundary
case does not cascade.

Flags (decisions that rounding may legitimately flip): an acceptance test
whose ratio p/q lies within 1e-3 of the uniform draw, a greedy decision whose
top-2 logit margin is under 1e-2, and -- for categorical draws, which those two
rules do not cover -- a draw whose outcome flips when the oracle's logits
replace the GPU's.
"""
from __future__ import annotations

import numpy as np

from oracle import philox as OP
from oracle import sampling as OS
from oracle import spec as OSP
from oracle.model import KVStore, forward


def rel_err(got, ref):
    """max |got - ref| / max |ref| (per call)."""
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def abs_err(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)))


def teacher_forced(cfg, W, D, st: OSP.SeqState, drafts):
    """Oracle drafter and target logits of one step on the given drafts (writes st.kv)."""
    n = st.n
    g = len(drafts)
    q_rows = []
    tok = st.pending
    for j in range(g):
        q_rows.append(forward(cfg, W, [tok], [n + j], st.kv, lin=D)[0])
        tok = int(drafts[j])
    p_rows = forward(cfg, W, [st.pending] + [int(d) for d in drafts], list(range(n, n + g + 1)), st.kv)
    return np.array(q_rows).reshape(g, cfg.vocab), p_rows


def greedy_margin(z):
    s = np.sort(np.asarray(z, np.float64))
    return float(s[-1] - s[-2])


def decision_flags(p_rows, q_rows, drafts, seq_id, n, sp: OSP.SamplingParams, n_acc):
    """Is any acceptance test of this step within 1e-3 of its draw (or greedy margin < 1e-2)?"""
    g = len(drafts)
    flagged = False
    for j in range(1, min(n_acc + 1, g) + 1):
        if sp.temperature == 0.0:
            flagged |= greedy_margin(p_rows[j - 1]) < 1e-2 or greedy_margin(q_rows[j - 1]) < 1e-2
            continue
        p = OS.pi(p_rows[j - 1], sp.temperature, sp.top_p)
        q = OS.pi(q_rows[j - 1], sp.temperature, sp.top_p)
        d = int(drafts[j - 1])
        u = OP.u1(sp.seed, seq_id, n + j, j, OP.PURPOSE_ACCEPT)
        if q[d] > 0:
            flagged |= abs(p[d] / q[d] - u) < 1e-3
    if sp.temperature == 0.0 and n_acc == g:
        flagged |= greedy_margin(p_rows[g]) < 1e-2
    return flagged


class Tally:
    def __init__(self):
        self.steps = 0
        self.flagged = 0
        self.unflagged_mismatch = 0
        self.max_rel_q = 0.0
        self.max_rel_p = 0.0
        self.max_abs_q = 0.0
        self.max_abs_p = 0.0
        self.first_flag_step = None

    def logits(self, gq, oq, gp, op):
        if gq is not None and len(gq):
            self.max_rel_q = max(self.max_rel_q, rel_err(gq, oq))
            self.max_abs_q = max(self.max_abs_q, abs_err(gq, oq))
        self.max_rel_p = max(self.max_rel_p, rel_err(gp, op))
        self.max_abs_p = max(self.max_abs_p, abs_err(gp, op))


def run_lockstep(eng, cfg, W, D, prompts, new, gamma, sp: OSP.SamplingParams, max_steps=None):
    """Prefill `prompts` on the engine and run spec steps at fixed gamma until
    every sequence has `new` tokens (or `max_steps`), checking each step
    against the oracle.  Returns (generated tokens per sequence, Tally)."""
    n_seq = len(prompts)
    eng.set_gamma(gamma)
    ids = eng.kv_alloc([len(p) for p in prompts], [new] * n_seq)
    first = eng.prefill(ids, [list(p) for p in prompts])
    tally = Tally()
    states = []
    for i in range(n_seq):
        kv = KVStore(cfg, len(prompts[i]) + new + gamma + 4)
        z = forward(cfg, W, list(prompts[i]), list(range(len(prompts[i]))), kv)
        gz = eng.debug_logits(1, i)
        tally.logits(None, None, gz[0], z[-1])
        # sampler on the GPU's logits reproduces the GPU's token exactly
        assert OSP.ar_sample(gz[0].astype(np.float64), int(ids[i]), len(prompts[i]), sp) == first[i]
        st = OSP.SeqState(seq_id=int(ids[i]), pending=int(first[i]), n=len(prompts[i]), kv=kv, stop_len=new,
                          generated=[int(first[i])])
        states.append(st)
    gen = [[int(first[i])] for i in range(n_seq)]
    active = list(range(n_seq))
    while active and (max_steps is None or tally.steps < max_steps):
        b_ids = [int(ids[i]) for i in active]
        tok, ne, info = eng.spec_step(b_ids)
        drafts = eng.debug_drafts(len(active), gamma)
        tally.steps += 1
        nxt = []
        for slot, i in enumerate(active):
            st = states[i]
            gq = eng.debug_logits(0, slot)
            gp = eng.debug_logits(1, slot)
            oq, op = teacher_forced(cfg, W, D, st, drafts[slot])
            tally.logits(gq, oq, gp, op)
            # drafts: the oracle sampler on the GPU's drafter logits gives the GPU's drafts
            for j in range(gamma):
                assert OSP.draft_sample(gq[j].astype(np.float64), st.seq_id, st.n + j + 1, j + 1, sp) == drafts[slot][j]
            # decision on the GPU's logits: exact
            a_g, em_g = OSP.spec_decide(gp.astype(np.float64), gq.astype(np.float64), drafts[slot], st.seq_id, st.n, sp)
            kept = int(ne[slot])
            assert em_g[:kept] == list(tok[slot, :kept]), (tally.steps, slot)
            # decision on the oracle's logits: equal unless flagged
            a_o, em_o = OSP.spec_decide(op, oq, drafts[slot], st.seq_id, st.n, sp)
            if (a_o, em_o) != (a_g, em_g):
                if decision_flags(op, oq, drafts[slot], st.seq_id, st.n, sp, min(a_o, a_g)) or \
                        decision_flags(gp.astype(np.float64), gq.astype(np.float64), drafts[slot], st.seq_id, st.n,
                                       sp, min(a_o, a_g)) or a_o == a_g:
                    tally.flagged += 1
                    if tally.first_flag_step is None:
                        tally.first_flag_step = tally.steps
                else:
                    tally.unflagged_mismatch += 1
            OSP.commit(st, em_g, a_g)
            gen[i].extend(int(t) for t in tok[slot, :kept])
            if len(st.generated) < new:
                nxt.append(i)
        active = nxt
    eng.kv_free(ids)
    return gen, tally
