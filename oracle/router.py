"""The router projection and its backward (oracle).

[ALPHA] section 二: the router projection that turns token activations into
expert logits sits outside the MoE layer proper (the layer starts from the
logits), and section 三: the layer benchmark excludes it.  It is built here as
the step upstream of the routing, so that the logit gradient the layer
returns reaches the router weights and the tokens.

Definitions (x [T, H], W_r [E, H], rows of W_r are experts):
  logits = x W_r^T                               [T, E]
  given dL/dlogits = d_logits [T, E]:
    dx_router  = d_logits W_r                    [T, H]  (added to the layer's dx)
    dW_router  = d_logits^T x                    [E, H]
Plain float64 products; no blocking or reordering.
"""
from __future__ import annotations

import numpy as np


def router_logits(x, w_router):
    """logits [T, E] = x [T, H] @ W_r[E, H]^T, float64."""
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def router_backward(x, w_router, d_logits):
    """(dx_router [T, H], dW_router [E, H]) of logits = x W_r^T given d_logits [T, E]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w_router, np.float64)
    dl = np.asarray(d_logits, np.float64)
    return dl @ w, dl.T @ x
