"""Pins for the router projection oracle (oracle.router): central finite
differences in float64 of the whole chain x, W_r -> logits -> top-k routing
-> MoE layer -> sum_t <dy_t, y_t>, whose gradients with respect to W_r and x
must equal router_backward applied to the layer's logit gradient (plus, for
x, the layer's own input gradient); and a hand-worked example."""
import math

import numpy as np

import oracle

EPS = 1e-6


def _chain(seed, T=4, H=8, I=4, E=4, k=2):
    rng = np.random.default_rng(seed)
    while True:
        p = {"x": rng.standard_normal((T, H)), "wr": rng.standard_normal((E, H)),
             "wg": rng.standard_normal((E, I, H)) / math.sqrt(H),
             "wu": rng.standard_normal((E, I, H)) / math.sqrt(H),
             "wd": rng.standard_normal((E, H, I)) / math.sqrt(I),
             "dy": rng.standard_normal((T, H))}
        L = oracle.router_logits(p["x"], p["wr"])
        srt = -np.sort(-L, axis=1)
        # top-k is piecewise constant: keep draws whose k-th / (k+1)-th gap is wide
        if np.all(srt[:, k - 1] - srt[:, k] > 1e4 * EPS):
            return p, k


def _loss(p, k):
    L = oracle.router_logits(p["x"], p["wr"])
    idx, w = oracle.route(L, k)
    y = oracle.forward(p["x"], p["wg"], p["wu"], p["wd"], idx, w)["y"]
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


def test_router_gradients_match_finite_differences_of_the_chain():
    for seed in range(3):
        p, k = _chain(seed)
        L = oracle.router_logits(p["x"], p["wr"])
        idx, w = oracle.route(L, k)
        b = oracle.backward(p["x"], p["wg"], p["wu"], p["wd"], idx, w, p["dy"])
        dl = oracle.ffn.d_logits_dense(idx, b["dl_sel"], p["wr"].shape[0])
        dx_r, dw_r = oracle.router_backward(p["x"], p["wr"], dl)
        fd_w = _fd(p, k, "wr")
        fd_x = _fd(p, k, "x")
        scale = max(1.0, np.max(np.abs(fd_w)))
        assert np.max(np.abs(dw_r - fd_w)) <= 1e-6 * scale
        scale = max(1.0, np.max(np.abs(fd_x)))
        assert np.max(np.abs(b["dx"] + dx_r - fd_x)) <= 1e-6 * scale


def test_router_hand_worked():
    # x = [[1, 2], [0, -1]], W_r = [[1, 0], [1, 1], [0, 3]] (E = 3, H = 2)
    x = np.array([[1.0, 2.0], [0.0, -1.0]])
    wr = np.array([[1.0, 0.0], [1.0, 1.0], [0.0, 3.0]])
    np.testing.assert_array_equal(oracle.router_logits(x, wr), [[1.0, 3.0, 6.0], [0.0, -1.0, -3.0]])
    dl = np.array([[1.0, 0.0, -1.0], [0.5, 2.0, 0.0]])
    dx, dw = oracle.router_backward(x, wr, dl)
    # dx = dl W_r: row 0 = [1,0] - [0,3] = [1, -3]; row 1 = 0.5 [1,0] + 2 [1,1] = [2.5, 2]
    np.testing.assert_array_equal(dx, [[1.0, -3.0], [2.5, 2.0]])
    # dW_r = dl^T x: expert 0 = 1 [1,2] + 0.5 [0,-1] = [1, 1.5]; expert 1 = 2 [0,-1];
    # expert 2 = -1 [1, 2]
    np.testing.assert_array_equal(dw, [[1.0, 1.5], [0.0, -2.0], [-1.0, -2.0]])
