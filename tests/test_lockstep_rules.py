"""CPU checks of the lockstep flag rules (tests/lockstep.py): a decision that the
measured logit error can flip is explained; one it cannot flip is not."""
import numpy as np

from lockstep import mismatch_explained
from oracle import philox as OP
from oracle import sampling as OS
from oracle import spec as OSP

SP = OSP.SamplingParams(seed=3, temperature=1.0, top_p=1.0)


def _bonus_case(V=16, seq=5, n=40, g=1):
    """Target/drafter rows where the one draft is always accepted (q == p at the draft), so the
    step ends in a bonus draw from p_{g+1}; returns rows and the bonus uniform."""
    rng = np.random.Generator(np.random.PCG64(1))
    z = rng.normal(size=(g + 1, V))
    q = z[:g].copy()
    drafts = [int(np.argmax(z[0]))]
    u = OP.u1(SP.seed, seq, n + g + 1, g + 1, OP.PURPOSE_RESIDUAL)
    return z, q, drafts, u, seq, n


def test_bonus_draw_flip_near_an_edge_is_explained():
    z, q, drafts, u, seq, n = _bonus_case()
    k = OS.sample(OS.pi(z[1], 1.0, 1.0), u)
    # smallest shift of logit k that makes the oracle's bonus draw differ (bisection)
    lo, hi = 0.0, 8.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        zo = z.copy()
        zo[1, k] -= mid
        if OS.sample(OS.pi(zo[1], 1.0, 1.0), u) != k:
            hi = mid
        else:
            lo = mid
    zo = z.copy()
    zo[1, k] -= hi
    assert OS.sample(OS.pi(zo[1], 1.0, 1.0), u) != k
    assert mismatch_explained(z, q, zo, q, drafts, seq, n, SP)


def test_bonus_draw_flip_far_from_an_edge_is_not_explained():
    z, q, drafts, u, seq, n = _bonus_case()
    p = OS.pi(z[1], 1.0, 1.0)
    k = OS.sample(p, u)
    assert OS.cdf_margin(p, u, k) > 1e-4
    # rows 1e-7 apart cannot move the CDF by the draw's margin: a differing draw there is a real error
    assert not mismatch_explained(z, q, z + 1e-7, q + 1e-7, drafts, seq, n, SP)
    # rows far apart can
    assert mismatch_explained(z, q, z + np.roll(z, 3, axis=1), q, drafts, seq, n, SP)


def test_acceptance_ratio_rule():
    rng = np.random.Generator(np.random.PCG64(2))
    V, seq, n = 12, 2, 10
    z = rng.normal(size=(2, V))
    q = rng.normal(size=(1, V))
    d = int(np.argmax(OS.pi(q[0], 1.0, 1.0)))
    u = OP.u1(SP.seed, seq, n + 1, 1, OP.PURPOSE_ACCEPT)
    p_, q_ = OS.pi(z[0], 1.0, 1.0), OS.pi(q[0], 1.0, 1.0)
    ratio = p_[d] / q_[d]
    # shift the target logit of d so that the oracle's ratio lands on the other side of u
    target = u * 1.02 if ratio < u else u * 0.98
    zo = z.copy()
    zo[0, d] += np.log(target / ratio)  # approximately (the normalizer moves too)
    acc_g = OS.accept(p_, q_, d, u)
    acc_o = OS.accept(OS.pi(zo[0], 1.0, 1.0), q_, d, u)
    if acc_g != acc_o:
        # eps is |log(target/ratio)|: the bound exp(2 eps) covers the move
        assert mismatch_explained(z, q, zo, q, [d], seq, n, SP)


def test_greedy_margin_rule():
    sp0 = OSP.SamplingParams(seed=0, temperature=0.0)
    z = np.array([[0.0, 1.0, 1.004, -2.0], [0.5, 0.1, 0.2, 0.3]])
    q = np.array([[0.0, 1.0, 1.004, -2.0]])
    zo = z.copy()
    zo[0, 1] += 0.01
    assert mismatch_explained(z, q, zo, q, [2], 0, 5, sp0)      # margin 0.004 < 1e-2
    z2 = np.array([[0.0, 1.0, 1.5, -2.0], [0.5, 0.1, 0.2, 0.3]])
    assert not mismatch_explained(z2, z2[:1], z2 + 1e-6, z2[:1] + 1e-6, [2], 0, 5, sp0)
