"""Property tier of the oracle's router and dispatch (CPU): invariants that
hold for any routing configuration, checked on randomly drawn ones
(hypothesis, seeded and bounded).  They complement the pins in the other
test_oracle_*.py files: a pin fixes values on chosen cases, a property fixes
structure on many.

Router ("DeepSeek-V3" summary page, section 1 DeepSeekMoE paragraph and
"Node-limited routing", section 2 "Auxiliary-loss-free load balancing"; the
book's chapter 7 "Selecting and combining experts", chapter 8 "V3's
routing-only bias" and "Restricting target nodes"):
  * the selection depends on the tokens one by one: permuting tokens permutes
    the result;
  * the group rule is the same for every group: permuting whole groups (their
    centroid rows and biases) relabels the selected ids;
  * with one group, or with every group kept, the selection is the plain
    top-k of the biased scores;
  * raising the bias of a selected expert keeps the selection and leaves the
    gates bit for bit (the bias enters the selection only);
  * gates are proportional to the unbiased affinities of the selected
    experts and sum to the routed scaling factor;
  * the selection is k distinct experts from at most M groups.
Dispatch (chapter 15 "What dispatch must do"): every assignment gets exactly
one row; the rows of an expert are contiguous, in token order; the counts
are the per-expert assignment counts.
"""

import numpy as np
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import route as oroute, permute as operm

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def routing_case(draw):
    G = draw(st.sampled_from([1, 2, 3, 4, 8]))
    per = draw(st.integers(1, 12))
    E = G * per
    M = draw(st.integers(1, G))
    n_top = draw(st.integers(1, per))
    k = M * n_top
    T = draw(st.integers(1, 24))
    d = draw(st.sampled_from([4, 8, 16]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rho = draw(st.sampled_from([1.0, 2.5]))
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    return dict(x=x, wg=wg, bias=bias, G=G, M=M, k=k, rho=rho, rng=rng)


def run(c, x=None, wg=None, bias="same"):
    return oroute.route(c["x"] if x is None else x, c["wg"] if wg is None else wg,
                        c["bias"] if isinstance(bias, str) else bias, c["G"], c["M"], c["k"], c["rho"])


@SETTINGS
@given(routing_case())
def test_selection_shape_and_gates(c):
    r = run(c)
    E, k, G, M = c["wg"].shape[0], c["k"], c["G"], c["M"]
    per = E // G
    for t in range(c["x"].shape[0]):
        ids = r["idx"][t]
        assert len(set(ids.tolist())) == k and np.all(np.diff(ids) > 0)
        assert len(set((ids // per).tolist())) <= M
        s = r["s"][t, ids]
        w = r["w"][t].astype(np.float64)
        assert np.all(w > 0)
        assert abs(w.sum() - c["rho"]) <= 1e-6 * c["rho"]
        np.testing.assert_allclose(w / w.sum(), s / s.sum(), rtol=1e-6)


@SETTINGS
@given(routing_case())
def test_token_permutation(c):
    T = c["x"].shape[0]
    p = c["rng"].permutation(T)
    a, b = run(c), run(c, x=c["x"][p])
    assert np.array_equal(a["idx"][p], b["idx"])
    assert np.array_equal(a["w"][p], b["w"])


@SETTINGS
@given(routing_case())
def test_group_relabelling(c):
    E, G = c["wg"].shape[0], c["G"]
    per = E // G
    gp = c["rng"].permutation(G)                       # new group j holds old group gp[j]
    ep = (gp[:, None] * per + np.arange(per)[None, :]).reshape(-1)
    a = run(c)
    b = run(c, wg=c["wg"][ep], bias=c["bias"][ep])
    ok = ~(a["near_tie"] | b["near_tie"])
    inv = np.argsort(ep)                               # old id -> new id
    mapped = np.sort(inv[a["idx"]], axis=1)
    assert np.array_equal(mapped[ok], b["idx"][ok])


@SETTINGS
@given(routing_case())
def test_no_group_limit_is_plain_topk(c):
    E, k, G0 = c["wg"].shape[0], c["k"], c["G"]
    cases = [(1, 1)]
    if k % G0 == 0 and k // G0 <= E // G0:     # every group kept (the rule needs k/M per group)
        cases.append((G0, G0))
    for G, M in cases:
        r = oroute.route(c["x"], c["wg"], c["bias"], G, M, k, c["rho"])
        z = r["s"] + c["bias"].astype(np.float64)[None, :]
        for t in range(c["x"].shape[0]):
            if r["near_tie"][t]:
                continue
            top = np.sort(np.argsort(-z[t], kind="stable")[:c["k"]])
            assert np.array_equal(r["idx"][t], top)


@SETTINGS
@given(routing_case())
def test_bias_raise_on_selected_keeps_everything(c):
    a = run(c)
    T = c["x"].shape[0]
    t = int(c["rng"].integers(0, T))
    e = int(a["idx"][t, int(c["rng"].integers(0, c["k"]))])
    b2 = c["bias"].copy()
    b2[e] += np.float32(0.25)
    b = oroute.route(c["x"][t:t + 1], c["wg"], b2, c["G"], c["M"], c["k"], c["rho"])
    if a["near_tie"][t]:
        return
    assert np.array_equal(b["idx"][0], a["idx"][t])
    assert np.array_equal(b["w"][0], a["w"][t])


@SETTINGS
@given(st.integers(1, 40), st.integers(1, 8), st.integers(1, 70), st.integers(0, 2 ** 31 - 1))
def test_dispatch_structure(T, k, E, seed):
    if k > E:
        k = E
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)
    offsets, pos, row_token = operm.permute(idx, E)
    assert offsets[0] == 0 and offsets[E] == T * k and offsets[E + 1] == T * k + T
    assert np.array_equal(np.diff(offsets[:E + 1]), np.bincount(idx.ravel(), minlength=E))
    assert np.array_equal(np.sort(pos.ravel()), np.arange(T * k))      # one row per assignment
    for t in range(T):
        for j in range(k):
            r = pos[t, j]
            assert row_token[r] == t
            assert offsets[idx[t, j]] <= r < offsets[idx[t, j] + 1]
    for e in range(E):
        toks = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(toks) > 0)                                # token order within an expert
