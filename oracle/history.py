"""Model-free history drafter: drafts copied from earlier rollouts of the same prompt.

Test infrastructure: only tests/, the smoke entry point and the benchmark's CPU
baseline use this package.

Source: p5 ("History Tree Dynamic RL 投机解码"), section 1 (history_tree: drafts
taken from responses of earlier rollouts, high-reward pieces first, for later
rollouts of the same prompt or similar contexts) and section 3.3 (a fixed-prefix
history cache per prompt plus a global fallback cache; candidates extracted at a
fixed prefix length; updates by reward first); section 2.2 (4 draft tokens by
default, at most 64 requests speculate).

Plain reading used here (the page names the pieces, not the rule):

* A record is one earlier rollout: its prompt, its response and one reward.
* The key of a position i of a record (i inside the response) is the L tokens
  just before it in prompt + response; its candidate draft is the record's
  tokens from i on.
* Each prompt has its own map key -> candidate, and one global map holds every
  prompt's keys.  A key keeps the candidate of the highest reward; among equal
  rewards the one recorded last (later record, then later position).
* To draft for a sequence, take the last L tokens of its prompt + generated
  tokens (the last generated token being the one not yet verified); look the
  key up in the sequence's prompt map, else in the global map; the draft is the
  first gamma tokens of the candidate (fewer when the record ends), or none.

Pinned by tests/test_oracle_history.py: hand-worked cases of each rule, and a
brute-force search over every recorded occurrence on random streams.
"""
from __future__ import annotations


class HistoryCache:
    def __init__(self, prefix_len: int):
        if prefix_len < 1:
            raise ValueError("prefix_len must be >= 1")
        self.L = int(prefix_len)
        self.records: list[list[int]] = []
        self.per_prompt: dict[tuple, dict[tuple, tuple]] = {}
        self.glob: dict[tuple, tuple] = {}

    def add(self, prompt, response, reward: float) -> None:
        toks = [int(t) for t in prompt] + [int(t) for t in response]
        P = len(prompt)
        rid = len(self.records)
        self.records.append(toks)
        mine = self.per_prompt.setdefault(tuple(int(t) for t in prompt), {})
        for i in range(P, len(toks)):
            if i < self.L:
                continue
            key = tuple(toks[i - self.L:i])
            for m in (mine, self.glob):
                old = m.get(key)
                if old is None or reward >= old[2]:
                    m[key] = (rid, i, float(reward))

    def propose(self, prompt, context, gamma: int) -> list[int]:
        if gamma < 1 or len(context) < self.L:
            return []
        key = tuple(int(t) for t in context[-self.L:])
        e = self.per_prompt.get(tuple(int(t) for t in prompt), {}).get(key)
        if e is None:
            e = self.glob.get(key)
        if e is None:
            return []
        rid, i, _ = e
        return self.records[rid][i:i + gamma]


def point_mass_logits(draft: int, vocab: int):
    """Logits whose distribution is the point mass on `draft` (a deterministic proposal): the lossless
    rule then accepts with probability p(draft) and resamples a rejection from p without the draft."""
    import numpy as np
    z = np.full(vocab, -np.inf)
    z[int(draft)] = 0.0
    return z
