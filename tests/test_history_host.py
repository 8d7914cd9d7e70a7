"""The library's history cache (er_history_*, host code) against oracle.history on the same streams:
identical drafts for every query, through the C ABI (no GPU needed)."""
import numpy as np
import pytest

from oracle.history import HistoryCache


@pytest.fixture(scope="module")
def History():
    from speculative_decoding_rl_amd import History as H
    return H


def test_library_cache_equals_the_oracle(History):
    rng = np.random.default_rng(11)
    for trial in range(60):
        L = int(rng.integers(1, 5))
        lib, ora = History(L), HistoryCache(L)
        prompts = [list(map(int, rng.integers(0, 7, size=int(rng.integers(1, 6))))) for _ in range(3)]
        for _ in range(int(rng.integers(1, 10))):
            p = prompts[int(rng.integers(0, 3))]
            resp = list(map(int, rng.integers(0, 7, size=int(rng.integers(0, 15)))))
            rw = float(rng.integers(0, 3)) + (0.5 if rng.random() < 0.2 else 0.0)
            lib.add(p, resp, rw)
            ora.add(p, resp, rw)
        for _ in range(40):
            p = prompts[int(rng.integers(0, 3))] if rng.random() < 0.85 else [6, 6]
            ctx = list(p) + list(map(int, rng.integers(0, 7, size=int(rng.integers(0, 8)))))
            g = int(rng.integers(0, 7))
            assert lib.propose(p, ctx, g) == ora.propose(p, ctx, g), (trial, L, p, ctx, g)
        assert lib.records() == len(ora.records)
        lib.close()


def test_bad_arguments_are_refused(History):
    from speculative_decoding_rl_amd import _lib
    with pytest.raises(_lib.ErError):
        History(0)
    h = History(2)
    with pytest.raises(_lib.ErError):
        h.add([1, 2], [3], float("nan"))
    assert h.records() == 0
    h.close()
