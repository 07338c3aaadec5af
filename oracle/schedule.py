"""The schedule: per-expert counts, exclusive scan, and the token-slot permutation
(oracle).

[AREX] first design decision: one schedule table drives dispatch, combine,
reverse-combine and reverse-dispatch; [ALPHA] section 一: the receiver places
tokens in the order each expert needs.  [AREX] second design decision: tokens
stream through a fixed-size ring buffer (macrobatch) that is filled and
drained at minibatch granularity; [AREX] third decision: the minibatch size is
a tunable number of tokens.

Notation: token t has slots s = t*k + j, j in [0, k).  Macrobatch m covers
tokens [m*M, (m+1)*M) and so slots [m*M*k, (m+1)*M*k); its rows are the same
range of global row numbers.  Within a macrobatch the rows are grouped by
expert (expert 0 first) and, within an expert, ordered by ascending slot id
(a stable counting sort).  Because a minibatch is a contiguous token range,
each minibatch occupies a contiguous sub-range of every expert's group.
"""
from __future__ import annotations

import numpy as np


def schedule(idx, E: int, macrobatch: int = 0, minibatch: int = 0):
    """Build the schedule for routing indices idx int [T,k].

    Returns a dict of int64 arrays:
      counts      [n_macro, E]        rows of expert e in macrobatch m
      offsets     [n_macro, E+1]      exclusive scan of counts (macrobatch-local)
      mini_counts [n_macro, E, n_mini] rows of expert e from minibatch i of m
      row_of_slot [S]                 global row of slot s
      slot_of_row [S]                 inverse permutation
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    M = macrobatch or T
    mb = minibatch or M
    if T % M or M % mb:
        raise ValueError("macrobatch must divide T and minibatch must divide macrobatch")
    n_macro, n_mini = T // M, M // mb
    S = T * k
    Sm = M * k
    flat = idx.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert index out of range")

    counts = np.zeros((n_macro, E), dtype=np.int64)
    offsets = np.zeros((n_macro, E + 1), dtype=np.int64)
    mini_counts = np.zeros((n_macro, E, n_mini), dtype=np.int64)
    row_of_slot = np.empty(S, dtype=np.int64)
    for m in range(n_macro):
        local = flat[m * Sm:(m + 1) * Sm]
        counts[m] = np.bincount(local, minlength=E)
        offsets[m, 1:] = np.cumsum(counts[m])
        for i in range(n_mini):
            part = local[i * mb * k:(i + 1) * mb * k]
            mini_counts[m, :, i] = np.bincount(part, minlength=E)
        # stable counting sort: slot order within each expert is preserved
        order = np.argsort(local, kind="stable")           # local slot of each local row
        rows = np.empty(Sm, dtype=np.int64)
        rows[order] = np.arange(Sm)
        row_of_slot[m * Sm:(m + 1) * Sm] = m * Sm + rows
    slot_of_row = np.empty(S, dtype=np.int64)
    slot_of_row[row_of_slot] = np.arange(S)
    return {
        "counts": counts,
        "offsets": offsets,
        "mini_counts": mini_counts,
        "row_of_slot": row_of_slot,
        "slot_of_row": slot_of_row,
        "n_macro": n_macro,
        "n_mini": n_mini,
        "macro_rows": Sm,
    }
