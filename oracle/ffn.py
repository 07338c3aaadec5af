"""Dispatch, expert SwiGLU FFN, weighted combine, and the backward (oracle).

[ALPHA] section 一: dispatch sends each token to its chosen experts, the
experts run a SwiGLU FFN (routed experts, and a shared expert in the forward
kernel), and combine brings the results back to the token; section 二: the
router-weighted sum over a token's expert outputs is the last step of the
layer, and the layer's output is bitwise reproducible because the order of
floating-point accumulation is fixed.  [AREX] closing design paragraph and
[AIGWX] "详细发生了什么": the backward computes the router-weight gradient
alongside the SwiGLU backward, and offers BF16 and MXFP8 modes.

Definitions used (token t, its slots j = 0..k-1, expert e = idx[t, j]):
  g = W_gate[e] x_t,  u = W_up[e] x_t,  h = SiLU(g) * u,  o = W_down[e] h
  y_t = FFN_shared(x_t) + sum_j w[t, j] * o_(t, j)     (shared term only if present)
Backward, with dy_t the upstream gradient:
  dw[t, j] = <dy_t, o_(t, j)>
  dh = w[t, j] * (W_down[e]^T dy_t)
  dg = dh * u * sigma(g) * (1 + g * (1 - sigma(g))),  du = dh * SiLU(g)
  dx_t = (W_sh_gate^T dg_sh + W_sh_up^T du_sh) + sum_j (W_gate[e]^T dg + W_up[e]^T du)
  dW_down[e] = sum over e's slots of (w dy_t) h^T, dW_gate[e] = sum dg x_t^T,
  dW_up[e] = sum du x_t^T
  d_logit[t, idx[t, j]] = w_j (dw_j - sum_i w_i dw_i); zero for unselected experts.

MXFP4-weight mode (mx="w4", forward only): the weights of every forward GEMM
in MXFP4 (E2M1 elements, E8M0 scales per 32 along K), the activations (x, h)
in MXFP8, both along K.

MXFP8 mode quantises each GEMM operand along that GEMM's reduction axis
(oracle.mx) before float64 arithmetic.  Every product of the layer goes
through mm(A, B, mx) = Q(A along its last axis) @ Q(B along its first axis),
so the axis of each operand is the contraction axis by construction:
  forward:   x along H, W_gate / W_up rows along H; h along I, W_down rows along I.
  backward:  dy along H and W_down along H (for W_down^T dy); dg, du along I and
             W_gate, W_up along I (for the input gradient); for the weight
             gradients, whose reduction runs over an expert's rows, the row
             operands in blocks of 32 consecutive rows of the expert's group
             (ascending slot order, one group per macrobatch, last block
             zero-padded); the shared expert's group in a macrobatch is that
             macrobatch's tokens.
Pins of the MXFP8 mode (tests/test_oracle_mx.py): mm's two axes (operands
exact along the contraction axis only); each forward operand's axis (x, h,
W_gate / W_up, W_down: the MXFP8 layer equals the exact layer on operands
exact along the intended axis and lossy along the other); the backward's
dy, dg / du and W_down^T axes (dx and dw); the 32-row blocks per macrobatch
group (a two-macrobatch stream whose blocks would straddle the boundary).
"""
from __future__ import annotations

import numpy as np

from .mx import mx_roundtrip, mxfp4_roundtrip


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def mm(A, B, mx=False):
    """A [.., K] @ B [K, ..]; in MXFP8 mode both operands are first quantised
    along K, the contraction axis (A along its last axis, B along its first).
    mx == "w4" (the MXFP4-weight forward): A, the activations, in MXFP8 and B,
    the weights, in MXFP4, both along K."""
    A, B = _f64(A), _f64(B)
    if mx == "w4":
        return mx_roundtrip(A, -1) @ mxfp4_roundtrip(B, 0)
    if mx:
        A = mx_roundtrip(A, -1)
        B = mx_roundtrip(B, 0)
    return A @ B


def sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def swiglu(g, u):
    """SiLU(g) * u."""
    return g * sigmoid(g) * u


def swiglu_grad(g, u, dh):
    """(dg, du) of h = SiLU(g) * u given dh."""
    s = sigmoid(g)
    dg = dh * u * s * (1.0 + g * (1.0 - s))
    du = dh * g * s
    return dg, du


def expert_forward(X, wg, wu, wd, mx=False):
    """One expert's FFN on rows X [n, H]: returns g, u, h [n, I] and o [n, H]."""
    X, wg, wu, wd = _f64(X), _f64(wg), _f64(wu), _f64(wd)
    g = mm(X, wg.T, mx)
    u = mm(X, wu.T, mx)
    h = swiglu(g, u)
    o = mm(h, wd.T, mx)
    return g, u, h, o


def forward(x, wg, wu, wd, idx, w, shared=None, tokens=None, mx=False):
    """Layer forward.

    x [T, H]; wg[e], wu[e] -> [I, H]; wd[e] -> [H, I] (arrays or lazy indexables);
    idx [T, k], w [T, k] from route(); shared = (sg, su, sd) or None;
    tokens: token ids to evaluate (default all).  Returns a dict with
    y [n, H] and the per-slot g, u, h [n, k, I] and o [n, k, H].
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    n = tokens.size
    sel = idx[tokens]
    X_all = _f64(np.asarray(x)[tokens])
    H = X_all.shape[1]
    first = wg[int(sel.flat[0])] if sel.size else None
    I = np.asarray(first).shape[0] if first is not None else 0
    g = np.zeros((n, k, I)); u = np.zeros((n, k, I)); h = np.zeros((n, k, I))
    o = np.zeros((n, k, H))
    for e in np.unique(sel):
        ti, jj = np.nonzero(sel == e)
        ge, ue, he, oe = expert_forward(X_all[ti], wg[e], wu[e], wd[e], mx)
        g[ti, jj], u[ti, jj], h[ti, jj], o[ti, jj] = ge, ue, he, oe
    wsel = _f64(w)[tokens]
    y = np.zeros((n, H))
    if shared is not None:
        y = y + expert_forward(X_all, *shared, mx=mx)[3]
    for j in range(k):
        y = y + wsel[:, j:j + 1] * o[:, j]
    return {"y": y, "g": g, "u": u, "h": h, "o": o, "tokens": tokens}


def _wgrad(A, B, mx, groups=None):
    """sum over rows r of A[r] (outer) B[r]: A [n, P], B [n, Q] -> [P, Q];
    the reduction runs over the rows.  groups: row-index arrays (one per
    macrobatch) summed separately, so that MXFP8 blocks of 32 rows never span
    two macrobatches; the partial sums are added in the given order."""
    A, B = _f64(A), _f64(B)
    if groups is None:
        groups = [np.arange(A.shape[0])]
    acc = np.zeros((A.shape[1], B.shape[1]))
    for rows in groups:
        if len(rows):
            acc = acc + mm(A[rows].T, B[rows], mx)
    return acc


def backward(x, wg, wu, wd, idx, w, dy, shared=None, mx=False, sched=None,
             tokens=None, experts=None):
    """Layer backward.

    tokens:  token ids whose dx, dw and d_logits are wanted (default all).
    experts: expert ids whose weight gradients are wanted (default: all
             experts when tokens is None, else none).  Weight gradients use
             every slot routed to the expert.
    sched:   the schedule (oracle.schedule); needed in MXFP8 mode, where the
             weight gradients quantise rows in blocks of the expert's group of
             each macrobatch.
    Returns a dict with dx [n, H]; dw [n, k], the router-weight gradient
    (<dy, o> in exact arithmetic; in MXFP8 mode the fused <Q(dy) Q(W_down), h>);
    dw_direct [n, k] (= <dy, o>); dw_fused [n, k] (= <W_down^T dy, h>, with the
    MXFP8 operands in MXFP8 mode); dl_sel [n, k] (the
    logit gradient at the selected experts; zero elsewhere); dWg, dWu, dWd
    (dicts by expert) and, when shared is given and tokens is None, the shared
    expert's dW_sg, dW_su, dW_sd.
    """
    if mx == "w4":
        raise ValueError("the MXFP4-weight variant is forward-only")
    idx = np.asarray(idx)
    T, k = idx.shape
    all_tokens = tokens is None
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    if experts is None:
        experts = [] if not all_tokens else sorted(set(int(e) for e in np.unique(idx)))
    wf = _f64(w)
    out = {}

    # ---- per-token quantities: dw, d_logits, dx -------------------------
    fw = forward(x, wg, wu, wd, idx, w, shared=shared, tokens=tokens, mx=mx)
    X = _f64(np.asarray(x)[tokens])
    DY = _f64(np.asarray(dy)[tokens])
    n = tokens.size
    H = X.shape[1]
    sel = idx[tokens]
    dw = np.einsum("tjh,th->tj", fw["o"], DY)       # <dy_t, o_(t,j)>
    dw_fused = np.zeros_like(dw)                    # <W_down^T dy_t, h_(t,j)>
    dXd_slot = np.zeros((n, k, H))                  # input gradient of each slot
    for e in np.unique(sel):
        ti, jj = np.nonzero(sel == e)
        wge, wue, wde = _f64(wg[e]), _f64(wu[e]), _f64(wd[e])
        a = mm(DY[ti], wde, mx)                         # W_down^T dy, per row
        dw_fused[ti, jj] = np.sum(a * fw["h"][ti, jj], axis=1)
        dh = wf[tokens[ti], jj][:, None] * a
        dg, du = swiglu_grad(fw["g"][ti, jj], fw["u"][ti, jj], dh)
        dXd_slot[ti, jj] = mm(dg, wge, mx) + mm(du, wue, mx)
    # reverse-dispatch: shared term first, then slots j = 0..k-1
    dx = np.zeros((n, H))
    if shared is not None:
        sg, su, sd = (_f64(a) for a in shared)
        g, u, h, _ = expert_forward(X, sg, su, sd, mx)
        a = mm(DY, sd, mx)
        dgs, dus = swiglu_grad(g, u, a)
        dx = dx + mm(dgs, sg, mx) + mm(dus, su, mx)
        if all_tokens:
            # the shared expert's group in macrobatch m is that macrobatch's
            # tokens; the partial sums are added in the backward's order
            # (macrobatches in reverse)
            groups = None
            if mx:
                if sched is None:
                    raise ValueError("MXFP8 weight gradients need the schedule")
                M = sched["macro_rows"] // k
                groups = [np.arange(m * M, (m + 1) * M) for m in range(sched["n_macro"])][::-1]
            out["dW_sd"] = _wgrad(DY, h, mx, groups)
            out["dW_sg"] = _wgrad(dgs, X, mx, groups)
            out["dW_su"] = _wgrad(dus, X, mx, groups)
    for j in range(k):
        dx = dx + dXd_slot[:, j]
    # The router-weight gradient is computed inside the SwiGLU backward, from
    # W_down^T dy ([AREX] closing paragraph).  In exact arithmetic that equals
    # <dy, o>; in MXFP8 mode W_down^T dy is itself an MXFP8 GEMM, so the
    # method's gradient is the fused form.
    dw_direct = dw
    if mx:
        dw = dw_fused
    wsel = wf[tokens]
    centre = np.sum(wsel * dw, axis=1, keepdims=True)
    dl_sel = wsel * (dw - centre)
    out.update({"dx": dx, "dw": dw, "dw_direct": dw_direct, "dw_fused": dw_fused,
                "dl_sel": dl_sel, "tokens": tokens, "fwd": fw})

    # ---- weight gradients of the requested experts ----------------------
    dWg, dWu, dWd = {}, {}, {}
    flat = idx.reshape(-1)
    for e in experts:
        slots = np.nonzero(flat == e)[0]          # ascending slot id
        groups = [slots]
        if mx:
            if sched is None:
                raise ValueError("MXFP8 weight gradients need the schedule")
            Sm = sched["macro_rows"]
            groups = [slots[(slots // Sm) == m] for m in range(sched["n_macro"])][::-1]
        wge, wue, wde = _f64(wg[e]), _f64(wu[e]), _f64(wd[e])
        accg = np.zeros(wge.shape); accu = np.zeros(wue.shape); accd = np.zeros(wde.shape)
        for sl in groups:
            if sl.size == 0:
                continue
            t, j = sl // k, sl % k
            Xe = _f64(np.asarray(x)[t])
            DYe = _f64(np.asarray(dy)[t])
            ge, ue, he, _ = expert_forward(Xe, wge, wue, wde, mx)
            a = mm(DYe, wde, mx)
            ws = wf[t, j][:, None]
            dge, due = swiglu_grad(ge, ue, ws * a)
            accd = accd + _wgrad(ws * DYe, he, mx)
            accg = accg + _wgrad(dge, Xe, mx)
            accu = accu + _wgrad(due, Xe, mx)
        dWg[e], dWu[e], dWd[e] = accg, accu, accd
    out.update({"dWg": dWg, "dWu": dWu, "dWd": dWd})
    return out


def d_logits_dense(idx, dl_sel, E, tokens=None):
    """Scatter the selected-logit gradients into a dense [n, E] array."""
    idx = np.asarray(idx)
    tokens = np.arange(idx.shape[0]) if tokens is None else np.asarray(tokens)
    out = np.zeros((tokens.size, E))
    rows = np.arange(tokens.size)[:, None]
    out[rows, idx[tokens]] = dl_sel
    return out
