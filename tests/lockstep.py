"""Lockstep comparison of the GPU rollout against the oracle (test helper).

The GPU runs a step; the oracle recomputes, on the GPU's committed prefix and
with the GPU's drafts, the drafter and target logits (compared within the
logits tolerance), re-runs the sampler on the GPU's own logits (must give the
GPU's tokens exactly), runs the sampler on its own logits (must agree unless
the step is flagged), and then commits the GPU's tokens so that one boundary
case does not cascade.

Flags (decisions that rounding may legitimately flip).  A step whose
decision differs between the GPU's and the oracle's logits is flagged only if
the difference is explained by the logit error measured on that step; any
other difference is an unflagged mismatch.

* Greedy (T = 0): the top-2 logit margin at a tested position is under
  max(1e-2, 2 eps), eps the larger max |logit difference| of the two rows.
* Acceptance tests: |p/q - u| < 1e-3 (the rule of the parity contract), or
  within the ratio's own error bound: p/q moves by at most a factor
  exp(2 (eps_p + eps_q) / T) when every logit moves by at most eps (softmax
  ratios move by exp(eps/T) per logit and by the same bound through the
  normalizer).
* Categorical draws (residual or bonus), same accept count: u lies within
  delta of an edge of the drawn token's CDF interval, with delta bounding how
  far the normalized CDF can move: kappa = exp(2 eps / T) - 1 per
  distribution; delta = kappa_p for the bonus draw from p;
  delta = 2 (kappa_p + kappa_q) / S for the residual max(0, p - q) of mass S.
* Nucleus (top_p < 1): the kept sets of the two rows differ and the mass
  before or after the last kept token lies within kappa of top_p.
"""
from __future__ import annotations

from contextlib import contextmanager

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


@contextmanager
def perturbed_stores(rel, rng):
    """Run the oracle with every stored (rounded) value perturbed before its rounding by a relative
    N(0, rel) amount: the spread this gives is how far a different fp32 accumulation order (which
    moves pre-rounding values by a few ulps) can move the oracle's own logits."""
    import oracle.model as OM
    base = OM.store

    def store(x, dt):
        x = np.asarray(x, np.float64)
        return base(x * (1.0 + rel * rng.standard_normal(x.shape)), dt)

    OM.store = store
    try:
        yield
    finally:
        OM.store = base


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


def greedy_paths_agree(cfg, W, prompts, ref, other, bound):
    """Two greedy rollouts of the same prompts by two GPU paths that may sum in
    different orders (a 1-row and a (gamma+1)-row target forward).  With the
    oracle teacher-forced on `ref`: wherever the greedy top-2 margin is at least
    `bound` (twice the per-path logit bound), `ref` holds the oracle's argmax;
    the two rollouts agree token for token up to their first difference, which
    must sit at a position whose margin is under `bound` (either argmax is then
    the target's) and ends the comparison of that sequence.  Returns the tokens
    compared."""
    checked = 0
    for i, pr in enumerate(prompts):
        a, b = list(ref[i]), list(other[i])
        assert len(a) == len(b), i
        toks = list(pr) + a[:-1]
        z = forward(cfg, W, toks, list(range(len(toks))), KVStore(cfg, len(toks)))[len(pr) - 1:]
        for k in range(len(a)):
            near_tie = greedy_margin(z[k]) < bound
            if not near_tie:
                assert a[k] == int(np.argmax(z[k])), (i, k)
            if a[k] != b[k]:
                assert near_tie, (i, k, greedy_margin(z[k]))
                break
            checked += 1
    return checked


def _kappa(eps, T):
    return float(np.expm1(2.0 * eps / T))


def _nucleus_flips(zg, zo, T, top_p, eps):
    """Do the nucleus sets of the two rows differ (and is that explained by eps)?  -> (differ, explained)"""
    if top_p >= 1.0 or T == 0.0:
        return False, True
    pg = OS.pi(zg, T, top_p) > 0
    po = OS.pi(zo, T, top_p) > 0
    if np.array_equal(pg, po):
        return False, True
    p = OS.softmax64(zg, T)
    order = np.lexsort((np.arange(p.shape[0]), -p))
    cum = np.cumsum(p[order])
    k = int(np.count_nonzero(pg))
    before = cum[k - 2] if k >= 2 else 0.0
    k_eps = _kappa(eps, T)
    return True, abs(before - top_p) <= k_eps + 1e-12 or abs(cum[k - 1] - top_p) <= k_eps + 1e-12


def mismatch_explained(gp, gq, op, oq, drafts, seq_id, n, sp: OSP.SamplingParams):
    """The GPU's and the oracle's decisions on this step differ: is the difference within what the
    measured logit error can flip (see the module docstring)?"""
    g = len(drafts)
    T = sp.temperature
    gp = np.asarray(gp, np.float64)
    gq = np.asarray(gq, np.float64)
    eps_p = [abs_err(gp[j], op[j]) for j in range(g + 1)]
    eps_q = [abs_err(gq[j], oq[j]) for j in range(g)]
    if T == 0.0:
        rows = [(gp[j], max(eps_p[j], eps_q[j] if j < g else 0.0)) for j in range(g + 1)]
        rows += [(gq[j], max(eps_p[j], eps_q[j])) for j in range(g)]
        return any(greedy_margin(z) < max(1e-2, 2.0 * e) for z, e in rows)
    for j in range(1, g + 1):
        for z_g, z_o, e in ((gp[j - 1], op[j - 1], eps_p[j - 1]), (gq[j - 1], oq[j - 1], eps_q[j - 1])):
            differ, ok = _nucleus_flips(z_g, z_o, T, sp.top_p, e)
            if differ:
                return ok
        pg_, qg_ = OS.pi(gp[j - 1], T, sp.top_p), OS.pi(gq[j - 1], T, sp.top_p)
        po_, qo_ = OS.pi(op[j - 1], T, sp.top_p), OS.pi(oq[j - 1], T, sp.top_p)
        d = int(drafts[j - 1])
        u = OP.u1(sp.seed, seq_id, n + j, j, OP.PURPOSE_ACCEPT)
        acc_g, acc_o = OS.accept(pg_, qg_, d, u), OS.accept(po_, qo_, d, u)
        if acc_g != acc_o:
            bound = np.expm1(2.0 * (eps_p[j - 1] + eps_q[j - 1]) / T)
            for p_, q_ in ((pg_, qg_), (po_, qo_)):
                if q_[d] > 0:
                    ratio = p_[d] / q_[d]
                    if abs(ratio - u) < max(1e-3, ratio * bound + 1e-12):
                        return True
            return False
        if not acc_g:
            # same rejection at j: the residual draws differ
            r = np.maximum(0.0, pg_ - qg_)
            S = float(np.sum(r))
            if S <= 0.0:
                r, S = pg_, 1.0
            k = OS.sample(r, OP.u1(sp.seed, seq_id, n + j, j, OP.PURPOSE_RESIDUAL))
            delta = 2.0 * (_kappa(eps_p[j - 1], T) + _kappa(eps_q[j - 1], T)) / S
            return OS.cdf_margin(r, OP.u1(sp.seed, seq_id, n + j, j, OP.PURPOSE_RESIDUAL), k) <= delta + 1e-12
    # every draft accepted on both sides: the bonus draws differ
    differ, ok = _nucleus_flips(gp[g], op[g], T, sp.top_p, eps_p[g])
    if differ:
        return ok
    pb = OS.pi(gp[g], T, sp.top_p)
    u = OP.u1(sp.seed, seq_id, n + g + 1, g + 1, OP.PURPOSE_RESIDUAL)
    k = OS.sample(pb, u)
    return OS.cdf_margin(pb, u, k) <= _kappa(eps_p[g], T) + 1e-12


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
        self.first_flag_len = {}   # sequence -> tokens generated before its first flagged step
        self.envelope = 0.0        # max |perturbed oracle - oracle| over the compared rows

    def logits(self, gq, oq, gp, op):
        if gq is not None and len(gq):
            self.max_rel_q = max(self.max_rel_q, rel_err(gq, oq))
            self.max_abs_q = max(self.max_abs_q, abs_err(gq, oq))
        self.max_rel_p = max(self.max_rel_p, rel_err(gp, op))
        self.max_abs_p = max(self.max_abs_p, abs_err(gp, op))


def run_lockstep(eng, cfg, W, D, prompts, new, gamma, sp: OSP.SamplingParams, max_steps=None,
                 envelope_rel=0.0, envelope_seeds=0, share_group=None):
    """Prefill `prompts` on the engine and run spec steps at fixed gamma until
    every sequence has `new` tokens (or `max_steps`), checking each step
    against the oracle.  Returns (generated tokens per sequence, Tally).

    envelope_seeds > 0 also runs that many shadow oracles with perturbed
    stores (perturbed_stores) on the same committed tokens and records in
    tally.envelope how far their logits move from the oracle's.  share_group is
    passed to er_kv_alloc (sequences of one group share their prompt's KV
    blocks; their prompts must be equal)."""
    n_seq = len(prompts)
    eng.set_gamma(gamma)
    ids = eng.kv_alloc([len(p) for p in prompts], [new] * n_seq, share_group=share_group)
    first = eng.prefill(ids, [list(p) for p in prompts])
    tally = Tally()
    states = []
    z_pref = []
    for i in range(n_seq):
        kv = KVStore(cfg, len(prompts[i]) + new + gamma + 4)
        z = forward(cfg, W, list(prompts[i]), list(range(len(prompts[i]))), kv)
        gz = eng.debug_logits(1, i)
        z_pref.append(z[-1])
        tally.logits(None, None, gz[0], z[-1])
        # sampler on the GPU's logits reproduces the GPU's token exactly
        assert OSP.ar_sample(gz[0].astype(np.float64), int(ids[i]), len(prompts[i]), sp) == first[i]
        st = OSP.SeqState(seq_id=int(ids[i]), pending=int(first[i]), n=len(prompts[i]), kv=kv, stop_len=new,
                          generated=[int(first[i])])
        states.append(st)
    shadows = []
    for e in range(envelope_seeds):
        rng = np.random.Generator(np.random.PCG64(1000 + e))
        row = []
        for i in range(n_seq):
            kv = KVStore(cfg, len(prompts[i]) + new + gamma + 4)
            with perturbed_stores(envelope_rel, rng):
                zp = forward(cfg, W, list(prompts[i]), list(range(len(prompts[i]))), kv)
            tally.envelope = max(tally.envelope, abs_err(zp[-1], z_pref[i]))
            row.append((OSP.SeqState(seq_id=int(ids[i]), pending=int(first[i]), n=len(prompts[i]), kv=kv,
                                     stop_len=new, generated=[int(first[i])]), rng))
        shadows.append(row)
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
                if mismatch_explained(gp, gq, op, oq, drafts[slot], st.seq_id, st.n, sp):
                    tally.flagged += 1
                    if tally.first_flag_step is None:
                        tally.first_flag_step = tally.steps
                    tally.first_flag_len.setdefault(i, len(gen[i]))
                else:
                    tally.unflagged_mismatch += 1
            for row in shadows:
                sh, rng = row[i]
                with perturbed_stores(envelope_rel, rng):
                    sq, spp = teacher_forced(cfg, W, D, sh, drafts[slot])
                tally.envelope = max(tally.envelope, abs_err(sq, oq), abs_err(spp, op))
                OSP.commit(sh, em_g, a_g)
            OSP.commit(st, em_g, a_g)
            gen[i].extend(int(t) for t in tok[slot, :kept])
            if len(st.generated) < new:
                nxt.append(i)
        active = nxt
    eng.kv_free(ids)
    return gen, tally
