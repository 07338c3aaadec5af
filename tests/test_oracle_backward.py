"""Pins for the backward oracle: central finite differences in float64 of the
scalar loss sum_t <dy_t, y_t>, plus identities that hold exactly."""
import math

import numpy as np
import pytest

import oracle

EPS = 1e-6


def _layer(seed, T=4, H=8, I=4, E=4, k=2, shared=False):
    rng = np.random.default_rng(seed)
    while True:
        L = rng.standard_normal((T, E)).astype(np.float32)
        srt = -np.sort(-L.astype(np.float64), axis=1)
        # top-k is piecewise constant: keep draws whose k-th / (k+1)-th gap is wide
        if k == E or np.all(srt[:, k - 1] - srt[:, k] > 100 * EPS):
            break
    p = {
        "x": rng.standard_normal((T, H)),
        "wg": rng.standard_normal((E, I, H)) / math.sqrt(H),
        "wu": rng.standard_normal((E, I, H)) / math.sqrt(H),
        "wd": rng.standard_normal((E, H, I)) / math.sqrt(I),
        "L": L.astype(np.float64),
        "dy": rng.standard_normal((T, H)),
    }
    if shared:
        p["sg"] = rng.standard_normal((I, H)) / math.sqrt(H)
        p["su"] = rng.standard_normal((I, H)) / math.sqrt(H)
        p["sd"] = rng.standard_normal((H, I)) / math.sqrt(I)
    return p, k


def _loss(p, k, w_override=None):
    idx, w = oracle.route(p["L"], k)          # float64 logits keep the FD exact
    if w_override is not None:
        w = w_override
    sh = (p["sg"], p["su"], p["sd"]) if "sg" in p else None
    y = oracle.forward(p["x"], p["wg"], p["wu"], p["wd"], idx, w, shared=sh)["y"]
    return float(np.sum(y * p["dy"]))


def _fd(p, k, name):
    arr = p[name]
    g = np.zeros_like(arr)
    for i in np.ndindex(arr.shape):
        old = arr[i]
        arr[i] = old + EPS
        lp = _loss(p, k)
        arr[i] = old - EPS
        lm = _loss(p, k)
        arr[i] = old
        g[i] = (lp - lm) / (2 * EPS)
    return g


def _analytic(p, k):
    idx, w = oracle.route(p["L"], k)
    sh = (p["sg"], p["su"], p["sd"]) if "sg" in p else None
    b = oracle.backward(p["x"], p["wg"], p["wu"], p["wd"], idx, w, p["dy"], shared=sh)
    return idx, w, b


def _close(a, b):
    scale = max(1.0, float(np.max(np.abs(b))))
    assert float(np.max(np.abs(a - b))) <= 1e-6 * scale, float(np.max(np.abs(a - b)))


@pytest.mark.parametrize("seed,shared", [(0, False), (1, False), (2, True)])
def test_finite_differences(seed, shared):
    p, k = _layer(seed, shared=shared)
    idx, w, b = _analytic(p, k)
    E = p["wg"].shape[0]
    _close(b["dx"], _fd(p, k, "x"))
    fd_wg, fd_wu, fd_wd = _fd(p, k, "wg"), _fd(p, k, "wu"), _fd(p, k, "wd")
    for e in range(E):
        zero = np.zeros_like(p["wg"][e])
        _close(b["dWg"].get(e, zero), fd_wg[e])
        _close(b["dWu"].get(e, zero), fd_wu[e])
        _close(b["dWd"].get(e, np.zeros_like(p["wd"][e])), fd_wd[e])
    dl = oracle.ffn.d_logits_dense(idx, b["dl_sel"], E)
    _close(dl, _fd(p, k, "L"))
    if shared:
        _close(b["dW_sg"], _fd(p, k, "sg"))
        _close(b["dW_su"], _fd(p, k, "su"))
        _close(b["dW_sd"], _fd(p, k, "sd"))
    # the router-weight gradient, by perturbing the weights themselves
    fd_w = np.zeros_like(w)
    for i in np.ndindex(w.shape):
        wp, wm = w.copy(), w.copy()
        wp[i] += EPS
        wm[i] -= EPS
        fd_w[i] = (_loss(p, k, wp) - _loss(p, k, wm)) / (2 * EPS)
    _close(b["dw"], fd_w)


def test_exact_identities():
    p, k = _layer(5, T=16, H=12, I=6, E=6, k=3)
    idx, w, b = _analytic(p, k)
    # <dy, W_down h> == <W_down^T dy, h>
    np.testing.assert_allclose(b["dw_fused"], b["dw"], rtol=1e-12, atol=1e-12)
    # the softmax gradient sums to zero over a token's selected logits
    np.testing.assert_allclose(b["dl_sel"].sum(1), 0.0, atol=1e-12)
    # identical experts: every slot returns the same output, so the logits get no gradient
    for nm in ("wg", "wu", "wd"):
        p[nm][:] = p[nm][0]
    idx, w, b = _analytic(p, k)
    np.testing.assert_allclose(b["dl_sel"], 0.0, atol=1e-12)


def test_subsets_match_full():
    p, k = _layer(6, T=12, H=8, I=4, E=5, k=2)
    idx, w, full = _analytic(p, k)
    tok = np.array([5, 0, 11])
    sub = oracle.backward(p["x"], p["wg"], p["wu"], p["wd"], idx, w, p["dy"], tokens=tok,
                          experts=[1, 3])
    np.testing.assert_allclose(sub["dx"], full["dx"][tok], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sub["dw"], full["dw"][tok], rtol=1e-13, atol=1e-13)
    for e in (1, 3):
        np.testing.assert_allclose(sub["dWd"][e], full["dWd"][e], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(sub["dWg"][e], full["dWg"][e], rtol=1e-13, atol=1e-13)
