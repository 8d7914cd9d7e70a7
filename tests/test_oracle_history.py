"""Pins of oracle.history (the model-free history drafter's cache).

Hand-worked cases of every rule of the reading (key = the last L tokens, the
continuation in the recorded response, reward first then the latest record, the
prompt's own map before the global one), and a brute-force search over every
recorded occurrence that must agree with the maps on random streams.
"""
import numpy as np

from oracle.history import HistoryCache


def test_hand_worked_lookups():
    h = HistoryCache(2)
    h.add([1, 2, 3], [4, 5, 6, 7], reward=1.0)
    assert h.propose([1, 2, 3], [9, 2, 3], 3) == [4, 5, 6]      # key (2, 3): the response from its start
    assert h.propose([1, 2, 3], [1, 2, 3, 4, 5], 4) == [6, 7]   # the record ends after two tokens
    assert h.propose([1, 2, 3], [1, 2, 3, 5, 4], 4) == []       # no occurrence of (5, 4)
    assert h.propose([1, 2, 3], [3], 4) == []                   # shorter than the prefix
    assert h.propose([1, 2, 3], [2, 3], 0) == []


def test_reward_first_then_latest():
    h = HistoryCache(2)
    h.add([1, 2, 3], [4, 5, 6], reward=1.0)
    h.add([1, 2, 3], [4, 8, 9], reward=0.5)                      # lower: (2, 3) keeps the first
    assert h.propose([1, 2, 3], [2, 3], 3) == [4, 5, 6]
    assert h.propose([1, 2, 3], [3, 4], 3) == [5, 6]
    h.add([1, 2, 3], [4, 7, 7], reward=1.0)                      # equal reward: the later record wins
    assert h.propose([1, 2, 3], [2, 3], 3) == [4, 7, 7]
    h.add([1, 2, 3], [4, 1, 1], reward=2.0)                      # higher
    assert h.propose([1, 2, 3], [3, 4], 2) == [1, 1]


def test_prompt_map_before_global_fallback():
    h = HistoryCache(1)
    h.add([10], [11, 12], reward=0.0)
    h.add([20], [11, 13], reward=5.0)                            # higher reward, other prompt
    assert h.propose([10], [10, 11], 2) == [12]                  # its own map, despite the lower reward
    assert h.propose([30], [11], 2) == [13]                      # unknown prompt: global, highest reward
    assert h.propose([20], [11], 1) == [13]


def _brute(records, L, prompt, context, gamma):
    """Every occurrence of the context's last L tokens in a recorded response: the prompt's own records
    first; among them the highest reward, ties to the last recorded (record order, then position)."""
    if gamma < 1 or len(context) < L:
        return []
    key = list(context[-L:])
    for own in (True, False):
        best = None
        for rid, (p, toks, rw) in enumerate(records):
            if own and list(p) != list(prompt):
                continue
            for i in range(len(p), len(toks)):
                if i >= L and toks[i - L:i] == key and (best is None or rw >= best[0]):
                    best = (rw, rid, i)
        if best is not None:
            return records[best[1]][1][best[2]:best[2] + gamma]
    return []


def test_maps_equal_brute_force_search():
    rng = np.random.default_rng(5)
    for trial in range(40):
        L = int(rng.integers(1, 4))
        h = HistoryCache(L)
        records = []
        prompts = [list(rng.integers(0, 6, size=int(rng.integers(1, 5)))) for _ in range(3)]
        for _ in range(int(rng.integers(1, 8))):
            p = prompts[int(rng.integers(0, 3))]
            resp = list(rng.integers(0, 6, size=int(rng.integers(1, 12))))
            rw = float(rng.integers(0, 3))
            h.add(p, resp, rw)
            records.append((p, [int(t) for t in p] + [int(t) for t in resp], rw))
        for _ in range(30):
            p = prompts[int(rng.integers(0, 3))] if rng.random() < 0.8 else [9]
            ctx = list(p) + list(rng.integers(0, 6, size=int(rng.integers(0, 6))))
            g = int(rng.integers(0, 6))
            assert h.propose(p, ctx, g) == _brute(records, L, p, ctx, g), (trial, p, ctx, g)


def test_point_mass_proposal_accepts_with_the_target_probability():
    """With q the point mass on d, min(1, p(d)/q(d)) = p(d), and the residual max(0, p - q) is p with d
    removed: the enumeration over (accept, redraw) outcomes gives back p exactly (lossless)."""
    from oracle import sampling as OS
    from oracle.history import point_mass_logits
    rng = np.random.default_rng(1)
    for _ in range(20):
        V = 6
        z = rng.normal(size=V)
        p = OS.pi(z, 1.0, 1.0)
        d = int(rng.integers(0, V))
        q = OS.pi(point_mass_logits(d, V), 1.0, 1.0)
        assert q[d] == 1.0 and q.sum() == 1.0
        assert abs(OS.accept_prob(p, q, d) - p[d]) < 1e-15
        r = OS.residual(p, q)
        out = np.zeros(V)
        out[d] += OS.accept_prob(p, q, d)
        out += (1.0 - OS.accept_prob(p, q, d)) * r / r.sum()
        assert np.allclose(out, p, atol=1e-14)
