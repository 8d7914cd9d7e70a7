"""Pins oracle/sampling.py: hand-computed examples, inverse-CDF frequencies, greedy limit."""
import json
import os

import numpy as np

from oracle import sampling

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sampling_examples.json")


def test_hand_computed_examples():
    cases = json.load(open(GOLD))["cases"]
    for c in cases:
        z = np.log(np.array(c["weights"], dtype=np.float64))
        got = sampling.pi(z, c["T"], c["top_p"])
        assert np.allclose(got, np.array(c["expect"], dtype=np.float64), rtol=0, atol=1e-15), c["name"]


def test_greedy_and_low_temperature_limit():
    z = np.array([0.5, 2.0, -1.0, 2.0, 1.9])
    assert sampling.pi(z, 0.0, 1.0).tolist() == [0, 1, 0, 0, 0]  # lowest index among ties
    p = sampling.pi(z, 1e-3, 1.0)
    assert abs(p[1] - 0.5) < 1e-12 and abs(p[3] - 0.5) < 1e-12


def test_sample_inverse_cdf_exact_frequencies():
    w = np.array([0.0, 1.0, 0.0, 3.0, 4.0, 0.0])  # total 8
    N = 4096
    counts = np.zeros(6, dtype=int)
    for k in range(1, N + 1):
        counts[sampling.sample(w, k / N)] += 1
    assert counts.tolist() == [0, N // 8, 0, 3 * N // 8, 4 * N // 8, 0]
    assert sampling.sample(w, 1.0) == 4  # never a trailing zero-weight token
    assert sampling.sample(w, 2.0 ** -24) == 1


def test_accept_rule_measure():
    p = np.array([0.2, 0.5, 0.3])
    q = np.array([0.4, 0.4, 0.2])
    # fraction of u on a fine grid that accepts token 0 is p/q = 0.5
    N = 10000
    acc = sum(sampling.accept(p, q, 0, k / N) for k in range(1, N + 1))
    assert acc == N // 2
    assert all(sampling.accept(p, q, 1, k / N) for k in range(1, N + 1))  # p >= q always accepts
    assert sampling.accept_prob(p, q, 0) == 0.5


def test_residual():
    p = np.array([0.2, 0.5, 0.3])
    q = np.array([0.4, 0.4, 0.2])
    r = sampling.residual(p, q)
    assert np.allclose(r, [0.0, 0.5, 0.5])
    assert np.allclose(sampling.residual(p, p), p)  # zero mass falls back to p


def test_top_p_nucleus_is_the_smallest_set_reaching_p():
    """Nucleus sampling keeps the smallest set of tokens whose probability mass
    reaches top_p (renormalized).  With distinct probabilities that set is unique:
    found here by enumerating every subset of a 6-token vocabulary."""
    import itertools
    rng = np.random.Generator(np.random.PCG64(21))
    for trial in range(60):
        V = 6
        z = rng.normal(0.0, 2.0, V)
        T = float(rng.choice([0.5, 1.0, 1.7]))
        top_p = float(rng.uniform(0.05, 0.995))
        w = np.exp((z - z.max()) / T)
        p = w / w.sum()
        best = None
        for k in range(1, V + 1):
            sets = [s for s in itertools.combinations(range(V), k) if p[list(s)].sum() >= top_p]
            if sets:
                best = max(sets, key=lambda s: p[list(s)].sum())
                break
        want = np.zeros(V)
        want[list(best)] = p[list(best)] / p[list(best)].sum()
        np.testing.assert_allclose(sampling.pi(z, T, top_p), want, rtol=1e-12, atol=0)
