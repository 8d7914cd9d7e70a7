"""Lockstep comparison of the GPU rollout against the oracle (test helper).

The GPU runs a step; the oracle recomputes, on the GPU's committed prefix and
with the GPU's drafts, the drafter and target logits (compared within the
logits tolerance), re-runs the sampler on the GPU's own logits (must give the
GPU's tokens exactly), runs the sampler on its own logits (must agree unless
the step is flagged), and then commits the GPU's tokens so that one boundary
case does not cascade.

Flags (the benchmark spec tolerance clause): an acceptance test whose ratio p/q lies
within 1e-3 of the uniform draw, a greedy decision whose top-2 logit margin is
under 1e-2, and -- for categorical draws, which that clause does not cover -- a
draw whose outcome flips when the oracle's logits replace the GPU's.
"""
from __future__ import annotations

import numpy as np

from oracle import philox as OP
from oracle import sampling as OS
from oracle import spec as OSP
from oracle.model import forward


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
