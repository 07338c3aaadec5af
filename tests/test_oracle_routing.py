"""Pins for the routing oracle: hand-worked cases, brute force, invariants."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(row, k):
    """k rounds of 'take the best remaining expert' by an explicit scan."""
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:      # strict: ties keep the lower index
                best = e
        chosen.append(best)
    return chosen


def _load_routing_examples():
    cases = []
    for line in open(os.path.join(GOLDEN, "routing_examples.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        lg, k, idx, w = (p.strip() for p in line.split("|"))
        cases.append((np.array([float(v) for v in lg.split()], dtype=np.float32), int(k),
                      [int(v) for v in idx.split()], [float(v) for v in w.split()]))
    return cases


@pytest.mark.parametrize("case", _load_routing_examples())
def test_hand_worked_examples(case):
    logits, k, idx_ref, w_ref = case
    idx, w = oracle.route(logits[None, :], k)
    assert idx[0].tolist() == idx_ref
    np.testing.assert_allclose(w[0], w_ref, rtol=1e-15, atol=0)


@pytest.mark.parametrize("seed,T,E,k,kind", [
    (0, 50, 8, 2, "normal"), (1, 40, 16, 5, "ties"), (2, 30, 7, 7, "ties"),
    (3, 40, 33, 1, "zeros"), (4, 20, 64, 10, "ties"),
])
def test_against_brute_force(seed, T, E, k, kind):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        L = rng.standard_normal((T, E)).astype(np.float32)
    elif kind == "ties":
        L = rng.integers(-1, 2, size=(T, E)).astype(np.float32)
    else:
        L = np.where(rng.random((T, E)) < 0.5, np.float32(-0.0), np.float32(0.0))
        L[:, ::3] = -1.0
    idx, w = oracle.route(L, k)
    for t in range(T):
        ref = _brute_topk(L[t].tolist(), k)
        assert idx[t].tolist() == ref, (t, L[t], idx[t], ref)
        z = np.exp(L[t, ref].astype(np.float64) - L[t, ref[0]])
        # softmax restricted to the selected logits, written out per element
        for j in range(k):
            assert abs(w[t, j] - z[j] / z.sum()) <= 1e-15


def test_invariants():
    rng = np.random.default_rng(7)
    L = rng.standard_normal((200, 64)).astype(np.float32)
    k = 6
    idx, w = oracle.route(L, k)
    assert idx.dtype == np.int32
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)                  # weights follow logit order
    for t in range(L.shape[0]):
        assert len(set(idx[t].tolist())) == k
        mask = np.ones(64, bool)
        mask[idx[t]] = False
        assert L[t, idx[t]].min() >= L[t, mask].max()


def test_k_equals_E_is_full_softmax():
    from scipy.special import softmax

    rng = np.random.default_rng(3)
    L = rng.standard_normal((10, 5)).astype(np.float32)
    idx, w = oracle.route(L, 5)
    full = softmax(L.astype(np.float64), axis=1)
    for t in range(10):
        np.testing.assert_allclose(w[t], full[t, idx[t]], rtol=1e-14)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.route(np.zeros((2, 3), np.float32), 4)
    with pytest.raises(ValueError):
        oracle.route(np.array([[np.nan, 0.0]], np.float32), 1)
