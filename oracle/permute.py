"""Permutation of token rows into per-expert groups, and the matching gather (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Experts are applied by grouping the token assignments by expert so that each
expert runs one batched matrix product (the book's chapter 7 "Batches change
what is active"); the grouping keeps metadata that identifies the original
token and its mixture weight so the outputs can be restored (chapter 15 "What
dispatch must do"); FP8 codes are what is moved (summary page section 6,
"Storage and communication": quantise before dispatch).

Readings: within one expert the rows keep token order (a stable sort), so the
permutation is unique; the shared expert (index E, always on) owns the last T
rows in token order.
"""

import numpy as np


def permute(idx, n_experts):
    """idx int [T, k] (distinct experts per token).
    Returns offsets int32 [E+2], pos int32 [T, k], row_token int32 [T*k].

    offsets[e]..offsets[e+1] are expert e's rows; offsets[E] = T*k and
    offsets[E+1] = T*k + T bound the shared expert's rows.  pos[t, j] is the row
    holding (t, idx[t, j]); row_token[r] is the token of routed row r.
    """
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    flat_e = idx.reshape(-1)
    flat_t = np.repeat(np.arange(T), k)
    counts = np.bincount(flat_e, minlength=n_experts)
    offsets = np.zeros(n_experts + 2, np.int64)
    offsets[1:n_experts + 1] = np.cumsum(counts)
    offsets[n_experts + 1] = T * k + T
    order = np.lexsort((flat_t, flat_e))        # primary key expert, then token
    row_token = flat_t[order]
    pos = np.empty(T * k, np.int64)
    pos[order] = np.arange(T * k)
    return offsets.astype(np.int32), pos.reshape(T, k).astype(np.int32), row_token.astype(np.int32)


def gather_rows(a, row_token, T):
    """Permuted copy of per-token rows: routed rows then the T shared rows."""
    a = np.asarray(a)
    return np.concatenate([a[np.asarray(row_token, np.int64)], a[:T]], axis=0)
