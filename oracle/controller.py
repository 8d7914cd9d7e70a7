"""Roofline SD on/off toggle and acceptance-aware draft length (pure functions).

Sources:
* p1 "关键模块" item 2 (system-aware SD toggle): model decode latency with a
  roofline; speculation pays only when a small active batch leaves decode
  memory-bound, and costs more than it saves when the batch is large and
  decode is compute-bound.  p1 "局限": the compute/memory boundary is
  calibrated per GPU.  p3 section 2 ("Elastic enable", "动态选参"): enable SD
  only below an active-request threshold, and pick draft depth and verify
  width per batch size.
* p1 "关键模块" item 3 (acceptance-aware draft length): raise gamma when recent
  acceptance is high, lower it when low.
* p5 section 2.2: an EMA coefficient of 0.3 for the online score and a 1.02
  margin before switching branches.

Plain reading used here (the pages print no formula):

  alpha_ema <- (1 - beta) * alpha_ema + beta * alpha_step,  beta = 0.3 weighting
  the new sample, alpha_step = sum(accepted) / sum(trials) over the step's
  sequences, trials = accepted + 1 after a rejection and gamma after a full
  acceptance (the maximum-likelihood acceptance of the geometric model).

  E[n](alpha, gamma) = (1 - alpha^(gamma+1)) / (1 - alpha)  (tokens per SD step;
  gamma + 1 when alpha = 1).

  Forward time T(bytes, flops) = t_fwd + (rows - 1) * t_row + max(bytes / BW, flops / FLOPS),
  rows = the forward's rows (B for AR and a draft forward, B*(g+1) for the
  verify), t_row = t_row_draft for drafter forwards and t_row_target for the
  target's.  t_fwd and the per-row terms are what the GPU's forwards take
  beyond the roofline at 1 row and per further row (p1 "局限": calibrated per
  GPU; measured at init from forwards of 1 and 16 rows); zero unless measured.
  AR step:    bytes = wb*P + B*C*kvb + B*kvb + B*V*4,  flops = 2*P*B + 4*B*C*hq*hd*L
  draft fwd:  bytes = bq*P + B*C*kvb + B*kvb + B*V*4,  flops = 2*P*B + 4*B*C*hq*hd*L
  verify fwd: bytes = wb*P + B*C*kvb + B*(g+1)*kvb + B*(g+1)*V*4,
              flops = 2*P*B*(g+1) + 4*B*(g+1)*C*hq*hd*L
  SD step:    g * T(draft) + T(verify)
  (P = streamed linear parameters incl. lm_head, wb = target bytes/param,
  bq = drafter bytes/param, kvb = KV bytes per token, C = mean committed context.)

  score(0) = B / T(AR);  score(g) = B * E[n](alpha, g) / T_SD(g);
  g* = argmax over {0} U [g_min, g_max] (ties to the smaller g); keep the
  current choice unless g*'s score exceeds it by the switch margin.
  g = 0 means autoregressive, so one rule covers both the toggle and gamma.

Pinned by tests/test_oracle_controller.py: E[n] against direct summation of
the geometric series and Monte Carlo; the toggle is off above the roofline
crossover and on below it; g* is non-decreasing in alpha; the margin's
hysteresis.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass
class ModelCost:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    w_bytes: float        # target bytes per linear parameter (2 bf16, 4 fp32)
    q_bytes: float        # drafter bytes per linear parameter (0.5 + 3/128 for W4-g128, ~1 for W8)
    kv_bytes_el: float    # bytes per KV element (2 bf16, 4 fp32)

    @property
    def p_lin(self) -> float:
        L, d, hq, hkv, hd, F, V = (self.n_layers, self.d_model, self.n_q_heads, self.n_kv_heads,
                                   self.head_dim, self.ffn, self.vocab)
        per_layer = d * (hq + 2 * hkv) * hd + hq * hd * d + 2 * F * d + F * d
        return float(L * per_layer + V * d)

    @property
    def kvb(self) -> float:
        return float(self.n_layers * 2 * self.n_kv_heads * self.head_dim * self.kv_bytes_el)


@dataclass
class Roofline:
    bw: float = 8.0e12        # bytes/s
    flops: float = 2.5e15     # flop/s
    t_fwd: float = 0.0        # fixed seconds per forward (launch overhead)
    t_row_draft: float = 0.0  # seconds per drafter-forward row beyond the first, beyond the roofline
    t_row_target: float = 0.0 # seconds per target-forward row beyond the first, beyond the roofline


def expected_tokens(alpha: float, gamma: int) -> float:
    if gamma <= 0:
        return 1.0
    if alpha >= 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def fwd_time(r: Roofline, nbytes: float, nflops: float, extra: float = 0.0) -> float:
    return r.t_fwd + extra + max(nbytes / r.bw, nflops / r.flops)


def ar_time(m: ModelCost, r: Roofline, B: int, C: float) -> float:
    P, kvb = m.p_lin, m.kvb
    by = m.w_bytes * P + B * C * kvb + B * kvb + B * m.vocab * 4.0
    fl = 2.0 * P * B + 4.0 * B * C * m.n_q_heads * m.head_dim * m.n_layers
    return fwd_time(r, by, fl, r.t_row_target * (B - 1))


def sd_time(m: ModelCost, r: Roofline, B: int, C: float, g: int) -> float:
    P, kvb = m.p_lin, m.kvb
    att = 4.0 * C * m.n_q_heads * m.head_dim * m.n_layers
    d_by = m.q_bytes * P + B * C * kvb + B * kvb + B * m.vocab * 4.0
    d_fl = 2.0 * P * B + B * att
    v_by = m.w_bytes * P + B * C * kvb + B * (g + 1) * kvb + B * (g + 1) * m.vocab * 4.0
    v_fl = 2.0 * P * B * (g + 1) + B * (g + 1) * att
    return (g * fwd_time(r, d_by, d_fl, r.t_row_draft * (B - 1)) +
            fwd_time(r, v_by, v_fl, r.t_row_target * (B * (g + 1) - 1)))


def score(m: ModelCost, r: Roofline, B: int, C: float, alpha: float, g: int) -> float:
    if g == 0:
        return B / ar_time(m, r, B, C)
    return B * expected_tokens(alpha, g) / sd_time(m, r, B, C, g)


def choose(m: ModelCost, r: Roofline, B: int, C: float, alpha: float, g_min: int, g_max: int,
           current: int = -1, margin: float = 1.02, allow_ar: bool = True) -> int:
    """allow_ar=False restricts the argmax to speculation (the forced-SD policy and probes)."""
    cands = ([0] if allow_ar else []) + list(range(g_min, g_max + 1))
    best, best_s = 0, -1.0
    for g in cands:
        s = score(m, r, B, C, alpha, g)
        if s > best_s:
            best, best_s = g, s
    if current in cands and current != best:
        if best_s <= margin * score(m, r, B, C, alpha, current):
            return current
    return best


# ---------------------------------------------------------------------------
# The step-by-step policy around choose().  The acceptance estimate moves only
# on speculative steps, and the pages do not say how it is refreshed while the
# toggle holds AR.  Reading used here: while the choice stays AR in a regime
# where the initial estimate alpha_init would make speculation pay, every
# probe_every-th consecutive AR choice runs one speculative step instead (the
# recorded choice stays AR); the gap starts at 32 and doubles after each probe
# up to 1024, and a speculative choice resets it to 32.
# ---------------------------------------------------------------------------
POLICY_AUTO, POLICY_FORCE_SD, POLICY_FORCE_AR = 0, 1, 2
PROBE_FIRST, PROBE_MAX = 32, 1024


@dataclass
class PlanState:
    choice: int = -1       # last recorded choice, 0 = AR, -1 = none yet
    ar_streak: int = 0     # consecutive AR choices since the last probe / speculative choice
    probe_every: int = 0   # current probe gap, 0 = not started


def plan(m: ModelCost, r: Roofline, st: PlanState, policy: int, B: int, C: float, alpha_ema: float,
         alpha_init: float, g_lo: int, g_hi: int, margin: float = 1.02) -> int:
    """Draft length to run this step (0 = AR); updates st."""
    if policy == POLICY_FORCE_AR:
        return 0
    allow_ar = policy == POLICY_AUTO
    g = choose(m, r, B, C, alpha_ema, g_lo, g_hi, current=st.choice, margin=margin, allow_ar=allow_ar)
    st.choice = g
    if g > 0 or not allow_ar:
        st.ar_streak = 0
        if g > 0:
            st.probe_every = PROBE_FIRST
        return g
    if st.probe_every <= 0:
        st.probe_every = PROBE_FIRST
    st.ar_streak += 1
    if st.ar_streak < st.probe_every:
        return 0
    st.ar_streak = 0
    if choose(m, r, B, C, alpha_init, g_lo, g_hi, current=-1, margin=1.0) == 0:
        return 0          # speculation would not pay even at the prior: no probe
    st.probe_every = min(2 * st.probe_every, PROBE_MAX)
    return choose(m, r, B, C, alpha_ema, g_lo, g_hi, current=-1, margin=1.0, allow_ar=False)


def ema(alpha_ema: float, alpha_step: float, beta: float = 0.3) -> float:
    return (1.0 - beta) * alpha_ema + beta * alpha_step


def alpha_step(accepted, gammas) -> float:
    """accepted[i] drafts accepted of gammas[i] drafted -> trials-based acceptance rate."""
    num = 0
    den = 0
    for a, g in zip(accepted, gammas):
        num += a
        den += (a + 1) if a < g else g
    return num / den if den > 0 else 0.0


# ---------------------------------------------------------------------------
# Measured-timing guard (the timing_guard policy of the History Tree Dynamic
# RL page: section 2.2 gives the parameters, section 3.3 the logic).  Plain
# reading used here, with autoregressive decoding as the default branch (the
# page's history branch) and speculation as the alternative (its EAGLE3
# branch); the history-cache warm-up rules have no counterpart:
#
# * large batches (above max_sd_batch) always take the default branch;
# * per batch bucket (ceil(log2(batch))) a tokens/ms EMA is kept for each
#   branch, weight ema_alpha on the new sample, the first sample setting it;
# * the alternative is compared only after compare_after default steps in the
#   bucket, and taken only while its score beats the default's by `margin`;
# * without a score for it, the alternative is probed for probe_steps steps
#   when the batch is at most probe_max_batch;
# * a speculative step whose tokens/ms falls below bad_ratio x the default
#   score is bad: back to the default branch, the speculative score is
#   dropped, and the bucket cools down for `cooldown` steps, a length that
#   grows by cooldown_growth up to cooldown_max with each consecutive bad
#   probe and returns to `cooldown` once a probe completes.
# ---------------------------------------------------------------------------
@dataclass
class GuardParams:
    max_sd_batch: int = 8
    probe_max_batch: int = 2
    compare_after: int = 64
    probe_steps: int = 8
    ema_alpha: float = 0.3
    margin: float = 1.02
    cooldown: int = 8192
    cooldown_max: int = 65536
    cooldown_growth: float = 4.0
    bad_ratio: float = 0.98


def guard_bucket(batch: int) -> int:
    """Smallest b with 2**b >= batch."""
    b = 0
    while (1 << b) < batch:
        b += 1
    return b


class TimingGuard:
    AR, SD = 0, 1

    def __init__(self, p: GuardParams | None = None):
        self.p = p or GuardParams()
        self.step = 0
        self.ema = {}          # (bucket, branch) -> tokens/ms
        self.n_ar = {}         # bucket -> default-branch steps observed
        self.probe_left = {}   # bucket -> speculative probe steps still to run
        self.cool_until = {}   # bucket -> first step after the cooldown
        self.cool_len = {}     # bucket -> length of the next cooldown

    def choose(self, batch: int) -> int:
        p = self.p
        now = self.step
        self.step += 1
        if batch > p.max_sd_batch:
            return self.AR
        b = guard_bucket(batch)
        if self.probe_left.get(b, 0) > 0:
            return self.SD
        if self.n_ar.get(b, 0) < p.compare_after:
            return self.AR
        if now < self.cool_until.get(b, 0):
            return self.AR
        sd = self.ema.get((b, self.SD))
        if sd is not None:
            ar = self.ema.get((b, self.AR))
            return self.SD if sd > p.margin * ar else self.AR
        if batch <= p.probe_max_batch:
            self.probe_left[b] = p.probe_steps
            return self.SD
        return self.AR

    def _bad_probe(self, b: int) -> None:
        p = self.p
        n = self.cool_len.get(b, p.cooldown)
        self.cool_until[b] = self.step + n
        self.cool_len[b] = min(int(n * p.cooldown_growth), p.cooldown_max)
        self.probe_left[b] = 0
        self.ema.pop((b, self.SD), None)

    def observe(self, batch: int, branch: int, tokens: float, ms: float) -> None:
        p = self.p
        if batch > p.max_sd_batch:
            return
        b = guard_bucket(batch)
        rate = tokens / ms
        if branch == self.AR:
            self.n_ar[b] = self.n_ar.get(b, 0) + 1
        else:
            ar = self.ema.get((b, self.AR))
            if ar is not None and rate < p.bad_ratio * ar:
                self._bad_probe(b)
                return
            if self.probe_left.get(b, 0) > 0:
                self.probe_left[b] -= 1
                if self.probe_left[b] == 0:
                    self.cool_len[b] = p.cooldown
        old = self.ema.get((b, branch))
        self.ema[(b, branch)] = rate if old is None else (1.0 - p.ema_alpha) * old + p.ema_alpha * rate
