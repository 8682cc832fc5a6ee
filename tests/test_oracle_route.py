"""Pins of the oracle's router (CPU only)."""

import itertools
import math

import numpy as np
import pytest

from oracle import route as R


def logit(p):
    return math.log(p / (1.0 - p))


def one_hot_inputs(affinities):
    """x = e_0 and wg[e, 0] = logit(s_e): the router then sees affinity s_e."""
    E = len(affinities)
    x = np.zeros((1, 4))
    x[0, 0] = 1.0
    wg = np.zeros((E, 4))
    wg[:, 0] = [logit(p) for p in affinities]
    return x, wg


def test_toy_mixture(golden):
    g = golden["toy_mixture"]
    x, wg = one_hot_inputs(g["affinities"])
    r = R.route(x, wg, None, n_groups=1, topk_groups=1, k=g["k"], route_scale=1.0)
    assert list(r["idx"][0]) == g["selected"]
    assert [round(float(v), 3) for v in r["w"][0]] == g["weights_3dp"]
    contrib = float(np.dot(r["w"][0], g["expert_outputs"]))
    assert round(contrib, 1) == g["routed_contribution_1dp"]


def test_bias_changes_selection_not_weights(golden):
    g = golden["bias_example"]
    x, wg = one_hot_inputs(g["affinities"])
    r0 = R.route(x, wg, None, 1, 1, g["k"], 1.0)
    assert list(r0["idx"][0]) == g["selected_without_bias"]
    r = R.route(x, wg, np.array(g["bias"], np.float32), 1, 1, g["k"], 1.0)
    assert np.allclose(r["z"][0], g["selection_scores"], atol=1e-7)
    assert list(r["idx"][0]) == g["selected"]
    assert [round(float(v), 3) for v in r["w"][0]] == g["weights_3dp"]
    # with the routed scaling factor the weights scale, the selection does not
    r25 = R.route(x, wg, np.array(g["bias"], np.float32), 1, 1, g["k"], 2.5)
    assert np.array_equal(r25["idx"], r["idx"])
    assert np.allclose(r25["w"] / 2.5, r["w"], rtol=1e-6)


def sigmoid_py(v):
    return 1.0 / (1.0 + math.exp(-v))


def brute_force(z_row, s_row, E, G, M, k):
    """Independent formulation: the group score is the largest sum of K_r/M
    members; the kept groups are the M-subset with the largest total score;
    the experts are the k-subset of allowed experts with the largest total z."""
    per = E // G
    n_top = k // M
    gscore = []
    for g in range(G):
        members = z_row[g * per:(g + 1) * per]
        gscore.append(max(sum(c) for c in itertools.combinations(members, n_top)))
    best_groups = max(itertools.combinations(range(G), M), key=lambda c: sum(gscore[i] for i in c))
    allowed = [e for g in best_groups for e in range(g * per, (g + 1) * per)]
    best = max(itertools.combinations(allowed, k), key=lambda c: sum(z_row[e] for e in c))
    return sorted(best), best_groups


@pytest.mark.parametrize("E,G,M,k", [(8, 4, 2, 4), (12, 3, 2, 2), (16, 4, 2, 4), (16, 8, 4, 4), (12, 6, 3, 3)])
def test_brute_force_tiny(E, G, M, k):
    rng = np.random.default_rng(E * 100 + G * 10 + M + k)
    T, d = 40, 16
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (rng.standard_normal((E, d)) / 3).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    r = R.route(x, wg, b, G, M, k, 2.5)
    checked = 0
    for t in range(T):
        if r["near_tie"][t]:
            continue
        s_row = [sigmoid_py(sum(float(x[t, i]) * float(wg[e, i]) for i in range(d))) for e in range(E)]
        z_row = [s_row[e] + float(b[e]) for e in range(E)]
        sel, groups = brute_force(z_row, s_row, E, G, M, k)
        assert list(r["idx"][t]) == sel
        tot = sum(s_row[e] for e in sel)
        assert np.allclose(r["w"][t], [2.5 * s_row[e] / tot for e in sel], rtol=1e-6)
        checked += 1
    assert checked >= T - 2


def test_invariants_v3_shape():
    """k distinct ids, from at most M groups, weights sum to route_scale,
    gates use the unbiased affinity."""
    rng = np.random.default_rng(5)
    T, d, E, G, M, k = 300, 64, 256, 8, 4, 8
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (rng.standard_normal((E, d)) / 8).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    r = R.route(x, wg, b, G, M, k, 2.5)
    idx = r["idx"]
    assert idx.shape == (T, k)
    for t in range(T):
        assert len(set(idx[t])) == k and list(idx[t]) == sorted(idx[t])
        assert len(set(idx[t] // (E // G))) <= M
    ws = r["w"].astype(np.float64).sum(axis=1) / 2.5
    assert np.all(np.abs(ws - 1.0) < 8 * 2.0 ** -24 * 2)
    s_sel = np.take_along_axis(r["s"], idx.astype(np.int64), axis=1)
    assert np.all(s_sel > 0) and np.all(s_sel < 1)


def test_uniform_bias_shift_and_masking_bias_leave_weights():
    """Adding the same constant to every bias keeps every selection and every
    weight; pushing unselected experts down keeps the weights too."""
    rng = np.random.default_rng(9)
    T, d, E, G, M, k = 200, 32, 64, 8, 4, 8
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (rng.standard_normal((E, d)) / 6).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    r = R.route(x, wg, b, G, M, k, 2.5)
    r2 = R.route(x, wg, (b + np.float32(0.25)).astype(np.float32), G, M, k, 2.5)
    ok = ~(r["near_tie"] | r2["near_tie"])
    assert np.array_equal(r["idx"][ok], r2["idx"][ok])
    assert np.array_equal(r["w"][ok], r2["w"][ok])
    # per token: remove all non-selected experts by a large negative bias
    for t in np.nonzero(ok)[0][:20]:
        bb = np.full(E, -5.0, np.float32)
        bb[r["idx"][t]] = 0.0
        rt = R.route(x[t:t + 1], wg, bb, G, M, k, 2.5)
        assert np.array_equal(rt["idx"][0], r["idx"][t])
        assert np.array_equal(rt["w"][0], r["w"][t])


def test_negative_scores_respect_group_limit():
    """Biased scores can be negative; masked experts must still never be picked."""
    E, G, M, k = 16, 4, 2, 4
    x = np.zeros((1, 2))
    x[0, 0] = 1.0
    wg = np.zeros((E, 2))
    wg[:, 0] = -30.0                       # s ~ 1e-13 for all experts
    b = np.full(E, -0.04, np.float32)
    b[[0, 1, 4, 5]] = -0.01                # groups 0 and 1 are best
    r = R.route(x, wg, b, G, M, k, 2.5)
    assert set(r["idx"][0] // 4) <= {0, 1}
    assert list(r["idx"][0]) == [0, 1, 4, 5]


def test_tie_breaks_to_lower_index():
    E, G, M, k = 8, 2, 1, 2
    x = np.zeros((1, 1))
    wg = np.zeros((E, 1))                  # all affinities 0.5 exactly
    r = R.route(x, wg, None, G, M, k, 2.5)
    assert list(r["idx"][0]) == [0, 1]
    assert r["near_tie"][0]
    assert np.allclose(r["w"][0], [1.25, 1.25])
