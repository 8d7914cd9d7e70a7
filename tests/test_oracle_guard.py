"""Pins of the timing-guard oracle (oracle/controller.py TimingGuard) to the
rules and constants the History Tree Dynamic RL page states: section 2.2
(EMA weight 0.3, switch margin 1.02, probe 8 steps, compare after 64 steps,
cooldown 8192 growing x4 to at most 65536, bad-step ratio 0.98, probing only
at batch <= 2, speculation only at batch <= 8) and section 3.3 (large batches
take the default branch; switch only past the margin; a bad probe falls back
and cools down)."""
import pytest

from oracle.controller import GuardParams, TimingGuard, guard_bucket

AR, SD = TimingGuard.AR, TimingGuard.SD


def _warm(g, batch, rate=1.0, n=64):
    for _ in range(n):
        assert g.choose(batch) == AR
        g.observe(batch, AR, rate * batch, 1.0)


def test_page_defaults():
    p = GuardParams()
    assert (p.max_sd_batch, p.probe_max_batch, p.compare_after, p.probe_steps) == (8, 2, 64, 8)
    assert (p.ema_alpha, p.margin, p.cooldown, p.cooldown_max, p.cooldown_growth, p.bad_ratio) == \
        (0.3, 1.02, 8192, 65536, 4.0, 0.98)


def test_buckets_are_powers_of_two():
    assert [guard_bucket(b) for b in (1, 2, 3, 4, 5, 8, 9, 16, 17)] == [0, 1, 2, 2, 3, 3, 4, 4, 5]


def test_large_batch_always_default():
    g = TimingGuard()
    for _ in range(500):
        assert g.choose(9) == AR
        g.observe(9, AR, 9.0, 1.0)
    assert guard_bucket(9) not in g.n_ar


def test_no_comparison_before_compare_after_then_probe_of_eight():
    g = TimingGuard()
    _warm(g, 1, n=63)
    g.choose(1)  # 64th decision: still AR (63 observed)
    g.observe(1, AR, 1.0, 1.0)
    picks = []
    for _ in range(8):
        picks.append(g.choose(1))
        g.observe(1, SD, 1.0, 1.0)   # as fast as AR: not bad, not better
    assert picks == [SD] * 8
    assert g.choose(1) == AR          # score known, not past the margin


def test_ema_weight_on_new_sample():
    g = TimingGuard()
    g.choose(2)
    g.observe(2, AR, 10.0, 1.0)      # first sample sets the score
    for n in range(1, 12):
        g.choose(2)
        g.observe(2, AR, 4.0, 1.0)
        assert g.ema[(1, AR)] == pytest.approx(4.0 + 6.0 * 0.7 ** n, rel=1e-12)


@pytest.mark.parametrize("ratio,want", [(1.01, AR), (1.03, SD)])
def test_switch_only_past_margin(ratio, want):
    g = TimingGuard()
    _warm(g, 1)
    for _ in range(8):
        assert g.choose(1) == SD
        g.observe(1, SD, ratio, 1.0)
    assert g.choose(1) == want


def test_cooldown_sequence_exact():
    g = TimingGuard()
    _warm(g, 1)
    seen = []
    for _ in range(4):
        while g.choose(1) == AR:
            g.observe(1, AR, 1.0, 1.0)
        # a probe step was chosen
        g.observe(1, SD, 0.5, 1.0)              # bad
        seen.append(g.cool_until[0] - g.step)
    assert seen == [8192, 32768, 65536, 65536]


def test_completed_probe_resets_cooldown_length():
    g = TimingGuard()
    _warm(g, 1)
    assert g.choose(1) == SD
    g.observe(1, SD, 0.5, 1.0)                   # bad -> cooldown 8192, next 32768
    while g.choose(1) == AR:
        g.observe(1, AR, 1.0, 1.0)
    for _ in range(8):                          # this probe completes (rate equal to AR)
        g.observe(1, SD, 1.0, 1.0)
        if g.probe_left[0] == 0:
            break
        assert g.choose(1) == SD
    assert g.cool_len[0] == 8192


def test_probe_only_at_small_batch():
    g = TimingGuard()
    _warm(g, 4)
    for _ in range(1000):
        assert g.choose(4) == AR                # bucket 3-4: no score, no probing above batch 2
        g.observe(4, AR, 4.0, 1.0)


def test_buckets_independent():
    g = TimingGuard()
    _warm(g, 1)
    _warm(g, 2)
    assert g.choose(1) == SD
    g.observe(1, SD, 0.1, 1.0)                   # bucket 0 cools down
    assert g.choose(2) == SD                     # bucket 1 probes regardless
