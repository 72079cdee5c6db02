"""Pins of the next-token sampling oracle (CPU).

The oracle restates the linkmax.top walkthrough's generate step (section 3.3):
softmax at a temperature, nucleus (top-p) cut, draw from the renormalised kept
probabilities.  These tests pin it to facts fixed independently of its code:
hand-computed cases, the distribution its draw induces, limits in the
temperature, invariances, and tie handling.  A planted mistake in each rule
is shown to fail a pin.
"""
import numpy as np
import pytest

from oracle import sample as osm


def _logits_for(probs):
    return np.log(np.asarray(probs, dtype=np.float64))


def test_hand_computed_cut_and_draw():
    # probabilities 0.5, 0.3, 0.15, 0.05: mass before each = 0, 0.5, 0.8, 0.95
    lg = _logits_for([0.15, 0.5, 0.05, 0.3])          # ids 1, 3, 0, 2 in sorted order
    p = osm.softmax_temperature(lg, 1.0)
    np.testing.assert_allclose(p, [0.15, 0.5, 0.05, 0.3], rtol=1e-12)
    assert list(osm.top_p_keep(p, 0.79)) == [1, 3]      # 0.8 > 0.79 drops id 0
    assert list(osm.top_p_keep(p, 0.81)) == [1, 3, 0]   # 0.8 <= 0.81 keeps it; 0.95 drops id 2
    assert list(osm.top_p_keep(p, 0.0)) == [1]          # the first token is always kept
    assert list(osm.top_p_keep(p, 1.0)) == [1, 3, 0, 2]
    # kept {1, 3} renormalised: 0.625, 0.375
    assert osm.sample_row(lg, 1.0, 0.79, 0.0) == 1
    assert osm.sample_row(lg, 1.0, 0.79, 0.62) == 1
    assert osm.sample_row(lg, 1.0, 0.79, 0.63) == 3
    assert osm.sample_row(lg, 1.0, 0.79, 0.999) == 3
    # kept {1, 3, 0}: cdf 0.5/0.95, 0.8/0.95, 1
    assert osm.sample_row(lg, 1.0, 0.81, 0.52) == 1
    assert osm.sample_row(lg, 1.0, 0.81, 0.53) == 3
    assert osm.sample_row(lg, 1.0, 0.81, 0.842) == 3    # 0.8/0.95 = 0.84211
    assert osm.sample_row(lg, 1.0, 0.81, 0.8422) == 0
    assert osm.sample_row(lg, 1.0, 0.81, 0.99) == 0


def test_hand_computed_decision_margins():
    # The GPU sampling tests compare a draw exactly only where this helper says
    # the float32 arithmetic cannot flip it.  Same four tokens: mass before each
    # in sorted order 0, 0.5, 0.8, 0.95.
    lg = _logits_for([0.15, 0.5, 0.05, 0.3])
    mp, mu = osm.decision_margins(lg, 1.0, 0.75, 0.6)
    assert mp == pytest.approx(0.05, abs=1e-12)         # |0.8 - 0.75|
    assert mu == pytest.approx(0.025, abs=1e-12)        # kept {1, 3}: cdf 0.625, 1; |0.625 - 0.6|
    mp, mu = osm.decision_margins(lg, 1.0, 0.81, 0.9)
    assert mp == pytest.approx(0.01, abs=1e-12)         # |0.8 - 0.81|
    assert mu == pytest.approx(0.9 - 0.8 / 0.95, abs=1e-12)  # kept {1, 3, 0}: cdf .5/.95, .8/.95, 1
    mp, mu = osm.decision_margins(lg, 1.0, 0.5, 0.5)    # exactly on the cut and on a boundary
    assert mp == 0.0
    assert mu == pytest.approx(0.125, abs=1e-12)        # the cut keeps {1, 3}: |0.625 - 0.5|


def test_draw_induces_the_renormalised_kept_distribution():
    rng = np.random.default_rng(7)
    lg = rng.normal(0.0, 2.0, 50)
    T, top_p = 0.7, 0.9
    p = osm.softmax_temperature(lg, T)
    kept = osm.top_p_keep(p, top_p)
    want = np.zeros(50)
    want[kept] = p[kept] / p[kept].sum()
    n = 200_000
    u = (np.arange(n) + 0.5) / n                       # an evenly spaced grid over [0, 1)
    counts = np.bincount([osm.sample_row(lg, T, top_p, x) for x in u], minlength=50)
    # each token owns an interval of the cdf: its share of a uniform grid is exact to 1/n
    np.testing.assert_allclose(counts / n, want, atol=1.0 / n + 1e-12)
    assert set(np.flatnonzero(counts)) == set(kept)


def test_temperature_limits_and_zero():
    rng = np.random.default_rng(3)
    lg = rng.normal(0.0, 1.0, 1000)
    am = int(np.argmax(lg))
    for u in (0.0, 0.3, 0.99):
        assert osm.sample_row(lg, 1e-4, 0.95, u) == am     # cold: all mass on the argmax
        assert osm.sample_row(lg, 0.0, 0.95, u) == am      # greedy
    p = osm.softmax_temperature(lg, 1e6)                   # hot: uniform
    np.testing.assert_allclose(p, 1.0 / 1000, rtol=1e-4)
    # softmax at temperature T equals the closed form exp(l/T) / sum exp(l/T)
    e = np.exp(lg / 0.8)
    np.testing.assert_allclose(osm.softmax_temperature(lg, 0.8), e / e.sum(), rtol=1e-12)


def test_shift_invariance_and_full_nucleus():
    rng = np.random.default_rng(11)
    lg = rng.normal(0.0, 1.5, 300)
    us = rng.random(40)
    a = [osm.sample_row(lg, 0.9, 0.8, u) for u in us]
    b = [osm.sample_row(lg + 123.25, 0.9, 0.8, u) for u in us]
    assert a == b
    p = osm.softmax_temperature(lg, 0.9)
    assert len(osm.top_p_keep(p, 1.0)) == 300


def test_ties_are_ordered_by_token_id():
    lg = np.zeros(10)
    lg[[3, 7]] = 5.0                                      # an exact tie at the top
    p = osm.softmax_temperature(lg, 1.0)
    assert list(osm.sorted_order(p)[:2]) == [3, 7]
    assert osm.sample_row(lg, 1.0, 1e-9, 0.99) == 3        # only the first of the tie is kept
    half = p[3] / (p[3] + p[7])                            # = 0.5: kept {3, 7} with a tiny nucleus above p[3]
    assert osm.sample_row(lg, 1.0, p[3] * 1.0001, half - 0.01) == 3
    assert osm.sample_row(lg, 1.0, p[3] * 1.0001, half + 0.01) == 7
    assert osm.sample_row(lg, 0.0, 0.9, 0.5) == 3          # greedy: the first maximum


def test_planted_mistakes_fail_the_pins(monkeypatch):
    # (1) an inclusive cut (cumsum > p instead of cumsum - prob > p) drops the token that crosses p
    inclusive = lambda probs, top_p: osm.sorted_order(probs)[np.cumsum(np.sort(probs)[::-1]) <= top_p]
    monkeypatch.setattr(osm, "top_p_keep", inclusive)
    with pytest.raises(AssertionError):
        test_hand_computed_cut_and_draw()
    monkeypatch.undo()
    # (2) ties ordered by descending id
    monkeypatch.setattr(osm, "sorted_order", lambda probs: np.lexsort((-np.arange(probs.shape[-1]), -probs)))
    with pytest.raises(AssertionError):
        test_ties_are_ordered_by_token_id()
    monkeypatch.undo()
    # (3) a draw that ignores the renormalisation (u compared with unnormalised kept mass)
    def unnormalised(logits, temperature, top_p, u):
        probs = osm.softmax_temperature(logits, temperature)
        kept = osm.top_p_keep(probs, top_p)
        j = int(np.searchsorted(np.cumsum(probs[kept]), u, side="right"))
        return int(kept[min(j, len(kept) - 1)])
    monkeypatch.setattr(osm, "sample_row", unnormalised)
    with pytest.raises(AssertionError):
        test_draw_induces_the_renormalised_kept_distribution()
