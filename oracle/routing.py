"""Top-k routing (oracle).

[ALPHA] section 一: a router chooses a few experts per token; section 四: the
public micro-benchmark routes synthetic Gaussian logits with a plain top-k.
[ALPHA] section 二: the router projection sits outside the layer, so the
logits are an input here.

Reading taken where the pages are silent:
  * the k selected experts are the k largest logits; among equal logits the
    lower expert index wins (IEEE comparison, so -0.0 and +0.0 tie);
  * slot j of a token is the j-th selected expert in that order (descending
    logit, ties by ascending index);
  * the combine weights are the softmax over the k selected logits only.
"""
from __future__ import annotations

import numpy as np


def route(logits, k: int):
    """Return (idx int32 [T,k], w float64 [T,k]) for fp32 logits [T,E].

    idx[t] lists the k experts with the largest logits of token t, ordered by
    (logit descending, expert index ascending); w[t] is the softmax of those k
    logits, evaluated in float64 with the largest logit subtracted first.
    """
    L = np.asarray(logits)
    if L.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(L)):
        raise ValueError("logits must be finite")
    Ld = L.astype(np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    experts = np.arange(E)
    for t in range(T):
        # lexsort sorts by the last key first: primary -logit, secondary index
        order = np.lexsort((experts, -Ld[t]))
        sel = order[:k]
        idx[t] = sel
        z = Ld[t, sel] - Ld[t, sel[0]]
        ez = np.exp(z)
        w[t] = ez / ez.sum()
    return idx, w
