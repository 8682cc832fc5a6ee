"""Pins of the bias controller oracle (oracle/balance.py)."""

import numpy as np

from oracle import balance as ob


def test_sign_rule_by_hand():
    # loads 6, 2, 4, 4 over E = 4 experts: mean 4 -> down, up, unchanged, unchanged
    offsets = [0, 6, 8, 12, 16, 16 + 5]          # last group: the shared expert, ignored
    b = np.array([0.5, -0.25, 0.0, 1.0], np.float32)
    got = ob.bias_update(b, offsets, 4, 0.125)
    assert np.array_equal(got, np.array([0.375, -0.125, 0.0, 1.0], np.float32))


def test_fractional_mean_and_fp32_rounding():
    # 3 assignments over 2 experts: mean 1.5, loads 2 and 1 -> down, up
    offsets = [0, 2, 3]
    b = np.array([1.0, 1.0], np.float32)
    g = np.float32(1e-8)                          # below half an ulp of 1.0: no change
    assert np.array_equal(ob.bias_update(b, offsets, 2, g), b)
    g = np.float32(0.001)
    got = ob.bias_update(b, offsets, 2, g)
    assert got[0] == np.float32(np.float32(1.0) - g) and got[1] == np.float32(np.float32(1.0) + g)
    assert got.dtype == np.float32


def test_balanced_loads_leave_bias():
    offsets = np.arange(0, 5 * 8, 8)              # every expert at the mean (E = 4)
    b = np.random.default_rng(0).standard_normal(4).astype(np.float32)
    assert np.array_equal(ob.bias_update(b, offsets, 4, 0.3), b)


def _zipf_scores(seed, n=512, E=8):
    """A toy whose preferred routing is skewed: expert e is the best for a
    Zipf-like share of the tokens, with small random margins."""
    rng = np.random.default_rng(seed)
    pref = rng.choice(E, size=n, p=(1.0 / np.arange(1, E + 1)) / np.sum(1.0 / np.arange(1, E + 1)))
    s = rng.uniform(0.0, 3.0, (n, E))
    s[np.arange(n), pref] += 3.0
    return s


def test_controller_settles_with_small_gain_and_oscillates_with_large():
    # The walk-through's toy behaviour: a small step brings max/min occupancy
    # down and keeps it there; a step much larger than the score spread makes
    # the loads swing instead of settling.
    s = _zipf_scores(1)
    loads, _ = ob.toy_balance(s, 0.05, 300)
    ratio = loads.max(1) / np.maximum(loads.min(1), 1)
    assert ratio[0] > 5 and ratio[-50:].max() < 2.5
    loads8, _ = ob.toy_balance(s, 8.0, 300)
    ratio8 = loads8.max(1) / np.maximum(loads8.min(1), 1)
    assert ratio8[-50:].min() > 5


def test_bias_never_enters_the_gate():
    # selection changes with the bias, the scores used for weighting do not:
    # with top-1 on a fixed score matrix, the chosen expert's score is read
    # from the unbiased matrix whatever the bias
    s = _zipf_scores(2, n=64)
    _, b = ob.toy_balance(s, 0.5, 40)
    sel = np.argmax(s + b, axis=1)
    gate = s[np.arange(64), sel]
    assert np.array_equal(gate, np.take_along_axis(s, sel[:, None], 1)[:, 0])
    assert not np.array_equal(sel, np.argmax(s, axis=1))
