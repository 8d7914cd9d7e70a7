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
