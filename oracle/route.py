"""Router: sigmoid affinity, selection-only bias, group-limited top-k (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix:
  * affinity s_{i,t} = Sigmoid(u_t . e_i) with e_i the expert centroid; the
    outputs do not sum to one ("DeepSeek-V3" summary page, section 1
    "Architecture recap", DeepSeekMoE paragraph; the book's chapter 7 "The
    router's affinity scores");
  * a per-expert bias b_i enters the selection score s + b only; the gate uses
    the unbiased s (summary page section 2 "Auxiliary-loss-free load
    balancing"; chapter 8 "V3's routing-only bias" and its worked example);
  * a token may use experts in at most M groups, ranked by the sum of the
    highest K_r/M affinities in each group (summary page, "Node-limited
    routing"; chapter 8 "Restricting target nodes", where the inference example
    sums each group's top-2 *biased* scores);
  * the gates are the selected affinities normalised to sum to one
    (summary page, DeepSeekMoE paragraph, Eq. 13 of the report; chapter 7
    "Selecting and combining experts"), then multiplied by the routed scaling
    factor (2.5 for V3, chapter 7: applied after normalisation);
  * no token is dropped (summary page, "No token dropping").

Readings where the pages are silent:
  * group g holds the contiguous experts [g*E/G, (g+1)*E/G);
  * ties in group rank go to the lower group index, ties in expert rank to the
    lower expert index;
  * experts outside the kept groups are masked with -inf (biased scores can be
    negative, so a 0 mask would not enforce the group limit);
  * the selected ids are reported in ascending expert order;
  * the router is evaluated in float64 from the BF16 inputs (the report keeps
    gating in higher precision; chapter 17 "High-precision exceptions").
A token is flagged "near tie" when, among allowed experts, the k-th and
(k+1)-th biased scores differ by less than 1e-6, or when the M-th and (M+1)-th
group scores do; such tokens have two correct selections.
"""

import numpy as np

NEAR_TIE = 1e-6


def affinity(x, wg):
    """s[t, e] = sigmoid(x_t . wg_e) in float64 (BF16 products are exact)."""
    logits = np.asarray(x, np.float64) @ np.asarray(wg, np.float64).T
    return 1.0 / (1.0 + np.exp(-logits))


def route(x, wg, bias, n_groups, topk_groups, k, route_scale):
    """Route T tokens.

    x [T, d], wg [E, d] (BF16 values as float32), bias [E] float32 or None.
    Returns dict with
      idx      int32 [T, k]  selected experts, ascending
      w        float32 [T, k] route_scale * s / sum(s over the selected set)
      s        float64 [T, E] affinities
      near_tie bool [T]      k-th/(k+1)-th expert or M-th/(M+1)-th group gap < 1e-6
      tie_kind int8 [T]      bit 0: expert boundary, bit 1: group boundary
    """
    x = np.asarray(x, np.float64)
    wg = np.asarray(wg, np.float64)
    T = x.shape[0]
    E = wg.shape[0]
    assert E % n_groups == 0 and 1 <= topk_groups <= n_groups
    per_group = E // n_groups
    assert k % topk_groups == 0
    n_top = k // topk_groups                 # K_r / M highest scores per group
    assert 1 <= n_top <= per_group and k <= topk_groups * per_group

    s = affinity(x, wg)
    b = np.zeros(E) if bias is None else np.asarray(bias, np.float32).astype(np.float64)
    z = s + b[None, :]

    zg = z.reshape(T, n_groups, per_group)
    top_in_group = -np.sort(-zg, axis=2)[:, :, :n_top]
    gscore = top_in_group.sum(axis=2)                        # [T, G]
    gorder = np.argsort(-gscore, axis=1, kind="stable")      # ties -> lower group
    kept = gorder[:, :topk_groups]
    allowed_g = np.zeros((T, n_groups), bool)
    np.put_along_axis(allowed_g, kept, True, axis=1)
    allowed = np.repeat(allowed_g, per_group, axis=1)        # [T, E]
    zm = np.where(allowed, z, -np.inf)

    eorder = np.argsort(-zm, axis=1, kind="stable")          # ties -> lower expert
    sel = np.sort(eorder[:, :k], axis=1)
    s_sel = np.take_along_axis(s, sel, axis=1)
    w = route_scale * s_sel / s_sel.sum(axis=1, keepdims=True)

    tie_kind = np.zeros(T, np.int8)
    n_allowed = topk_groups * per_group
    if k < n_allowed:
        zs = np.take_along_axis(zm, eorder[:, k - 1:k + 1], axis=1)
        tie_kind |= (np.abs(zs[:, 0] - zs[:, 1]) < NEAR_TIE).astype(np.int8)
    if topk_groups < n_groups:
        gs = np.take_along_axis(gscore, gorder[:, topk_groups - 1:topk_groups + 1], axis=1)
        tie_kind |= ((np.abs(gs[:, 0] - gs[:, 1]) < NEAR_TIE).astype(np.int8) << 1)

    return {
        "idx": sel.astype(np.int32),
        "w": w.astype(np.float32),
        "s": s,
        "z": z,
        "near_tie": tie_kind != 0,
        "tie_kind": tie_kind,
    }
