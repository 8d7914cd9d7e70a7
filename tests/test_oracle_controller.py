"""Pins oracle/controller.py: closed forms, monotonicity, toggle regime, hysteresis."""
import numpy as np
import pytest

from oracle import controller as C


def qwen7b_cost():
    return C.ModelCost(n_layers=28, d_model=3584, n_q_heads=28, n_kv_heads=4, head_dim=128, ffn=18944,
                       vocab=152064, w_bytes=2.0, q_bytes=0.5 + 3.0 / 128, kv_bytes_el=2.0)


def test_parameter_and_kv_counts_match_the_published_shape():
    m = qwen7b_cost()
    # Qwen2.5-7B linear parameters without embedding: 28 layers + untied lm_head
    assert m.p_lin == 7_070_285_824
    assert m.kvb == 57_344


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.77, 0.99, 1.0])
def test_expected_tokens_is_the_geometric_sum(alpha):
    for g in range(0, 9):
        direct = sum(alpha ** k for k in range(g + 1)) if g > 0 else 1.0
        assert abs(C.expected_tokens(alpha, g) - direct) < 1e-12


def test_expected_tokens_monte_carlo():
    rng = np.random.Generator(np.random.PCG64(0))
    alpha, g = 0.73, 5
    acc = rng.random((200000, g)) < alpha
    first_rej = np.where(acc.all(axis=1), g, np.argmin(acc, axis=1))
    emitted = first_rej + 1
    assert abs(emitted.mean() - C.expected_tokens(alpha, g)) < 4 * emitted.std() / np.sqrt(len(emitted))


def test_toggle_off_at_large_batch_on_in_the_tail():
    m = qwen7b_cost()
    r = C.Roofline(bw=8e12, flops=2.5e15, t_fwd=0.0)
    # short context, moderate acceptance: the verify forward turns compute-bound at large B
    big = C.choose(m, r, 256, 128, 0.6, 1, 8)
    small = C.choose(m, r, 1, 128, 0.6, 1, 8)
    assert big == 0 and small > 0
    # monotone: once off at B, stays off at every larger B
    seen_off = False
    for B in range(1, 257):
        g = C.choose(m, r, B, 128, 0.6, 1, 8)
        if g == 0:
            seen_off = True
        else:
            assert not seen_off, B


def test_gamma_non_decreasing_in_alpha():
    m = qwen7b_cost()
    r = C.Roofline()
    for B in (1, 4, 16):
        prev = -1
        for a in np.linspace(0.0, 0.99, 60):
            g = C.choose(m, r, B, 1024, float(a), 1, 8)
            assert g >= prev
            prev = g


def test_margin_hysteresis():
    m = qwen7b_cost()
    r = C.Roofline()
    # find alpha where the best gamma changes between 2 and 3 at B=1
    alphas = np.linspace(0.3, 0.95, 400)
    gs = [C.choose(m, r, 1, 512, float(a), 1, 8) for a in alphas]
    i = next(k for k in range(1, len(gs)) if gs[k] != gs[k - 1])
    a_sw = float(alphas[i])
    new, old = gs[i], gs[i - 1]
    s_new = C.score(m, r, 1, 512, a_sw, new)
    s_old = C.score(m, r, 1, 512, a_sw, old)
    assert s_new > s_old
    if s_new <= 1.02 * s_old:
        assert C.choose(m, r, 1, 512, a_sw, 1, 8, current=old) == old
    assert C.choose(m, r, 1, 512, a_sw, 1, 8, current=old, margin=1.0) == new


def test_alpha_step_and_ema():
    assert C.alpha_step([4, 1, 0], [4, 4, 4]) == 5 / (4 + 2 + 1)
    assert C.ema(0.5, 1.0, 0.3) == pytest.approx(0.65)


# ---- hand-computed points of the step-time model -----------------------------
# A toy shape small enough to evaluate every term by hand:
#   L=1, d=2, hq=hkv=1, hd=2, F=1, V=3, wb=2, bq=1, KV element 2 bytes
#   P   = d(hq+2hkv)hd + hq hd d + 2Fd + Fd + Vd = 12 + 4 + 4 + 2 + 6 = 28
#   kvb = L * 2 * hkv * hd * 2 = 8 bytes per token
# At B=2, C=5, gamma=2:
#   AR bytes     = wb P + B C kvb + B kvb + 4 B V          = 56 + 80 + 16 + 24      = 176
#   AR flops     = 2 P B + 4 B C hq hd L                    = 112 + 80              = 192
#   draft bytes  = bq P + B C kvb + B kvb + 4 B V          = 28 + 80 + 16 + 24      = 148
#   draft flops  = 2 P B + 4 B C hq hd L                    = 112 + 80              = 192
#   verify bytes = wb P + B C kvb + B(g+1)kvb + 4B(g+1)V   = 56 + 80 + 48 + 72      = 256
#   verify flops = 2 P B (g+1) + 4 B (g+1) C hq hd L       = 336 + 240             = 576
# Each term changes the total if dropped, so a missing or mistyped term fails.
def toy_cost():
    return C.ModelCost(n_layers=1, d_model=2, n_q_heads=1, n_kv_heads=1, head_dim=2, ffn=1, vocab=3,
                       w_bytes=2.0, q_bytes=1.0, kv_bytes_el=2.0)


# (bw, flops, t_fwd, t_row_draft, t_row_target) -> (AR step, SD step at gamma 2), worked by hand from the
# table above (B = 2: the AR and draft forwards have 2 rows, 1 beyond the first; the verify has 6, 5 beyond)
TOY_TIMES = [
    ((1.0, 1e30, 0.0, 0.0, 0.0), (176.0, 2 * 148.0 + 256.0)),               # bytes-bound: 176, 552
    ((1e30, 1.0, 0.0, 0.0, 0.0), (192.0, 2 * 192.0 + 576.0)),               # flop-bound: 192, 960
    ((1.0, 1e30, 0.5, 0.0, 0.0), (176.5, 2 * 148.5 + 256.5)),               # fixed time per forward: 176.5, 553.5
    ((1.0, 1.5, 0.0, 0.0, 0.0), (176.0, 2 * max(148.0, 128.0) + 384.0)),    # the max is per forward: 176, 680
    # per-row terms: AR 176 + 1 * 0.125; SD 2 * (148 + 1 * 0.25) + 256 + 5 * 0.125 = 553.125
    ((1.0, 1e30, 0.0, 0.25, 0.125), (176.125, 553.125)),
]


def test_toy_shape_counts():
    m = toy_cost()
    assert m.p_lin == 28.0 and m.kvb == 8.0


@pytest.mark.parametrize("rates,want", TOY_TIMES)
def test_step_times_at_hand_computed_points(rates, want):
    m = toy_cost()
    r = C.Roofline(*rates)
    assert C.ar_time(m, r, 2, 5.0) == pytest.approx(want[0], rel=1e-12)
    assert C.sd_time(m, r, 2, 5.0, 2) == pytest.approx(want[1], rel=1e-12)


def test_choice_at_a_hand_computed_point():
    # bytes-bound toy at B=2, C=5: score(AR) = 2/176 = 0.011364; score(2) = 2 E[n] / 552.
    # E[n](0.9, 2) = 1 + 0.9 + 0.81 = 2.71 -> 0.009819 < AR;  at alpha = 1, E = 3 -> 0.010870 < AR.
    m = toy_cost()
    r = C.Roofline(1.0, 1e30, 0.0)
    assert C.choose(m, r, 2, 5.0, 0.9, 2, 2) == 0
    assert C.choose(m, r, 2, 5.0, 1.0, 2, 2) == 0
    # gamma = 1: draft 148 + verify (56 + 80 + 32 + 48 = 216) = 364; at alpha = 1, 2*2/364 = 0.010989 < AR
    assert C.sd_time(m, r, 2, 5.0, 1) == pytest.approx(364.0)
    # with a cheaper drafter (bq = 0.1 -> draft bytes 122.8): gamma 1 at alpha 1 = 4 / 338.8 = 0.011806 > AR
    m2 = C.ModelCost(1, 2, 1, 1, 2, 1, 3, 2.0, 0.1, 2.0)
    assert C.sd_time(m2, r, 2, 5.0, 1) == pytest.approx(122.8 + 216.0)
    assert C.choose(m2, r, 2, 5.0, 1.0, 1, 1) == 1


# ---- the step-by-step policy (acceptance probes) ------------------------------
def _probe_regime():
    """Qwen2.5-7B shape at B=1, C=2048: speculation pays at alpha 0.9, not at 0.05."""
    m = qwen7b_cost()
    r = C.Roofline(8e12, 2.5e15, 0.0)
    assert C.choose(m, r, 1, 2048.0, 0.9, 1, 8) > 0
    assert C.choose(m, r, 1, 2048.0, 0.05, 1, 8) == 0
    return m, r


def test_probe_schedule_doubles_to_its_cap():
    m, r = _probe_regime()
    st = C.PlanState()
    probes = []
    for call in range(1, 4100):
        g = C.plan(m, r, st, C.POLICY_AUTO, 1, 2048.0, 0.05, 0.9, 1, 8)
        if g:
            probes.append(call)
            # a probe speculates with the argmax over gamma >= 1 at the current estimate
            assert g == C.choose(m, r, 1, 2048.0, 0.05, 1, 8, allow_ar=False)
        assert st.choice == 0
    # gaps 32, 64, 128, 256, 512, 1024, 1024, ... consecutive AR choices
    assert probes == [32, 96, 224, 480, 992, 2016, 3040, 4064]


def test_no_probe_when_the_prior_says_ar():
    m, r = _probe_regime()
    st = C.PlanState()
    assert all(C.plan(m, r, st, C.POLICY_AUTO, 1, 2048.0, 0.05, 0.05, 1, 8) == 0 for _ in range(3000))


def test_speculative_choice_resets_the_probe_gap():
    m, r = _probe_regime()
    st = C.PlanState()
    for _ in range(96):                      # probes at calls 32 and 96: the gap is now 128
        C.plan(m, r, st, C.POLICY_AUTO, 1, 2048.0, 0.05, 0.9, 1, 8)
    assert st.probe_every == 128
    assert C.plan(m, r, st, C.POLICY_AUTO, 1, 2048.0, 0.9, 0.9, 1, 8) > 0
    assert st.probe_every == 32 and st.ar_streak == 0
    calls = 0
    while True:
        calls += 1
        if C.plan(m, r, st, C.POLICY_AUTO, 1, 2048.0, 0.05, 0.9, 1, 8):
            break
    assert calls == 32


def test_forced_policies():
    m, r = _probe_regime()
    st = C.PlanState()
    assert all(C.plan(m, r, st, C.POLICY_FORCE_AR, 1, 2048.0, 0.9, 0.9, 1, 8) == 0 for _ in range(10))
    assert all(C.plan(m, r, st, C.POLICY_FORCE_SD, 64, 2048.0, 0.01, 0.9, 1, 8) >= 1 for _ in range(10))
