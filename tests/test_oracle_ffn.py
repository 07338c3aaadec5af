"""Pins for the forward oracle: a hand-worked layer, dense brute force, and
special cases that reduce to textbook results."""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            key, *nums = line.split()
            vals[key] = [float(v) for v in nums]
    return vals


def _two_expert_case():
    x = np.array([[1.0, 2.0]])
    wg = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    wu = np.array([[[0.0, 1.0]], [[1.0, 0.0]]])
    wd = np.array([[[1.0], [-1.0]], [[2.0], [0.0]]])
    logits = np.zeros((1, 2), np.float32)
    return x, wg, wu, wd, logits


def test_hand_worked_two_expert_layer():
    ref = _golden("swiglu_two_experts.txt")
    x, wg, wu, wd, logits = _two_expert_case()
    idx, w = oracle.route(logits, 2)
    f = oracle.forward(x, wg, wu, wd, idx, w)
    np.testing.assert_allclose(f["h"][0, :, 0], [ref["h0"][0], ref["h1"][0]], rtol=1e-15)
    np.testing.assert_allclose(f["y"][0], ref["y"], rtol=1e-15)
    b = oracle.backward(x, wg, wu, wd, idx, w, np.array([[1.0, 0.0]]))
    np.testing.assert_allclose(b["dw"][0], ref["dw"], rtol=1e-15)
    np.testing.assert_allclose(b["dl_sel"][0], ref["dlogits"], rtol=1e-14)


def _ffn_by_loops(xt, wg, wu, wd):
    """One expert on one token with explicit loops."""
    I, H = wg.shape
    h = []
    for i in range(I):
        g = sum(wg[i, c] * xt[c] for c in range(H))
        u = sum(wu[i, c] * xt[c] for c in range(H))
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [sum(wd[r, i] * h[i] for i in range(I)) for r in range(H)]


def _rand_layer(seed, T, H, I, E, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((E, I, H)) * scale / math.sqrt(H)
    wu = rng.standard_normal((E, I, H)) * scale / math.sqrt(H)
    wd = rng.standard_normal((E, H, I)) / math.sqrt(I)
    L = rng.standard_normal((T, E)).astype(np.float32)
    return x, wg, wu, wd, L


@pytest.mark.parametrize("seed,T,H,I,E,k", [(0, 7, 5, 3, 4, 2), (1, 5, 6, 4, 6, 3), (2, 4, 3, 2, 3, 1)])
def test_dense_brute_force(seed, T, H, I, E, k):
    x, wg, wu, wd, L = _rand_layer(seed, T, H, I, E)
    idx, w = oracle.route(L, k)
    y = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    for t in range(T):
        acc = [0.0] * H
        for e in range(E):               # every expert on every token, masked
            gate = 0.0
            for j in range(k):
                if idx[t, j] == e:
                    gate = w[t, j]
            o = _ffn_by_loops(x[t], wg[e], wu[e], wd[e])
            acc = [a + gate * v for a, v in zip(acc, o)]
        np.testing.assert_allclose(y[t], acc, rtol=1e-12, atol=1e-12)


def test_single_expert_is_swiglu_mlp():
    x, wg, wu, wd, _ = _rand_layer(4, 9, 6, 5, 1)
    idx, w = oracle.route(np.zeros((9, 1), np.float32), 1)
    y = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    g = x @ wg[0].T
    u = x @ wu[0].T
    ref = (g / (1 + np.exp(-g)) * u) @ wd[0].T
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_all_experts_is_softmax_mixture():
    from scipy.special import softmax

    x, wg, wu, wd, L = _rand_layer(5, 6, 4, 3, 5)
    idx, w = oracle.route(L, 5)
    y = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    p = softmax(L.astype(np.float64), axis=1)
    ref = np.zeros_like(y)
    for e in range(5):
        g = x @ wg[e].T
        u = x @ wu[e].T
        ref += p[:, e:e + 1] * ((g / (1 + np.exp(-g)) * u) @ wd[e].T)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_give_one_ffn():
    x, wg, wu, wd, L = _rand_layer(6, 12, 8, 4, 6)
    wg[:] = wg[0]; wu[:] = wu[0]; wd[:] = wd[0]
    idx, w = oracle.route(L, 3)
    y = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    g = x @ wg[0].T
    u = x @ wu[0].T
    np.testing.assert_allclose(y, (g / (1 + np.exp(-g)) * u) @ wd[0].T, rtol=1e-12, atol=1e-12)


def test_down_projection_linearity():
    x, wg, wu, wd, L = _rand_layer(7, 10, 8, 4, 5)
    idx, w = oracle.route(L, 2)
    y = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    assert np.all(oracle.forward(x, wg, wu, 0 * wd, idx, w)["y"] == 0)
    y3 = oracle.forward(x, wg, wu, -3.0 * wd, idx, w)["y"]
    np.testing.assert_allclose(y3, -3.0 * y, rtol=1e-13, atol=1e-13)


def test_shared_expert_adds_one_dense_ffn():
    x, wg, wu, wd, L = _rand_layer(8, 10, 8, 4, 5)
    rng = np.random.default_rng(80)
    sh = (rng.standard_normal((4, 8)), rng.standard_normal((4, 8)), rng.standard_normal((8, 4)))
    idx, w = oracle.route(L, 2)
    y0 = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    y1 = oracle.forward(x, wg, wu, wd, idx, w, shared=sh)["y"]
    for t in range(10):
        np.testing.assert_allclose(y1[t] - y0[t], _ffn_by_loops(x[t], *sh), rtol=1e-11, atol=1e-11)


def test_token_subset_matches_full():
    x, wg, wu, wd, L = _rand_layer(9, 20, 8, 4, 6)
    idx, w = oracle.route(L, 2)
    full = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    sub = oracle.forward(x, wg, wu, wd, idx, w, tokens=np.array([3, 17, 0]))["y"]
    np.testing.assert_allclose(sub, full[[3, 17, 0]], rtol=1e-13, atol=1e-14)
