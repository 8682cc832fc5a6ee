"""Auxiliary-loss-free load balancing: the per-expert bias controller (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix ("DeepSeek-V3: the recipe, and the interconnect that shaped
it", section "Auxiliary-loss-free balancing"; the "DeepSeek-V3" summary page,
section 2; the book's chapter 8 "V3's routing-only bias"):
  * after each step, every expert's load over the batch is compared with the
    mean load; an overloaded expert's bias goes down by gamma, an underloaded
    expert's bias goes up by gamma (a fixed step, sign only);
  * the bias enters the selection score only, never the gate.

Readings where the pages are silent:
  * load = number of (token, routed expert) assignments of the expert in the
    batch (the shared expert has no bias and is not counted);
  * an expert exactly at the mean keeps its bias (sign 0);
  * the comparison is made on integers (load * E against the total
    assignments), the bias update in FP32 with one rounding (the bias is an
    FP32 vector).
"""

import numpy as np


def expert_loads(offsets, E):
    """Per routed expert: rows in its group of the grouped buffer."""
    off = np.asarray(offsets, np.int64)
    return off[1:E + 1] - off[:E]


def bias_update(bias, offsets, E, gamma):
    """One controller step: b - gamma * sign(load - mean load), FP32."""
    load = expert_loads(offsets, E)
    total = int(np.asarray(offsets, np.int64)[E])
    s = np.sign(load * E - total).astype(np.float32)          # exact: integers
    return (np.asarray(bias, np.float32) - np.float32(gamma) * s).astype(np.float32)


def toy_balance(scores, gamma, steps, k=1):
    """The thermostat on a fixed score matrix (tokens x experts): route top-k
    by score + bias, update the bias from the loads, repeat.  Returns the
    per-step loads [steps, E] and the final bias.  Used to check the
    controller's qualitative behaviour (it settles with a small gain and
    oscillates with a large one)."""
    scores = np.asarray(scores, np.float64)
    n, E = scores.shape
    bias = np.zeros(E, np.float32)
    loads = []
    for _ in range(steps):
        sel = np.argsort(-(scores + bias.astype(np.float64)), axis=1, kind="stable")[:, :k]
        load = np.bincount(sel.reshape(-1), minlength=E)
        offsets = np.concatenate([[0], np.cumsum(load)])
        loads.append(load)
        bias = bias_update(bias, offsets, E, gamma)
    return np.asarray(loads), bias
