"""Pins for the schedule oracle: O(S^2) counting brute force and invariants."""
import numpy as np
import pytest

import oracle


def _brute_rows(idx, E, M):
    """row of every slot by explicit counting, macrobatch by macrobatch."""
    T, k = idx.shape
    flat = idx.reshape(-1)
    Sm = M * k
    rows = []
    for s in range(flat.size):
        m = s // Sm
        lo = m * Sm
        e = flat[s]
        before_experts = sum(1 for q in range(lo, lo + Sm) if flat[q] < e)
        before_slots = sum(1 for q in range(lo, s) if flat[q] == e)
        rows.append(lo + before_experts + before_slots)
    return rows


@pytest.mark.parametrize("seed,T,E,k,M,mb", [
    (0, 24, 5, 2, 0, 0), (1, 40, 8, 3, 20, 5), (2, 16, 3, 3, 8, 2), (3, 12, 16, 4, 0, 0),
])
def test_against_brute_force(seed, T, E, k, M, mb):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = oracle.route(L, k)
    s = oracle.schedule(idx, E, M, mb)
    assert s["row_of_slot"].tolist() == _brute_rows(idx, E, M or T)
    Mm = M or T
    for m in range(T // Mm):
        local = idx.reshape(-1)[m * Mm * k:(m + 1) * Mm * k]
        for e in range(E):
            assert s["counts"][m, e] == sum(1 for v in local if v == e)
            assert s["offsets"][m, e] == sum(1 for v in local if v < e)


def test_invariants_zipf_like():
    rng = np.random.default_rng(11)
    T, E, k, M, mb = 256, 32, 4, 64, 16
    L = rng.standard_normal((T, E)).astype(np.float32) + np.linspace(3, -3, E).astype(np.float32)
    idx, _ = oracle.route(L, k)
    s = oracle.schedule(idx, E, M, mb)
    S = T * k
    r, q = s["row_of_slot"], s["slot_of_row"]
    assert sorted(r.tolist()) == list(range(S))                     # bijection
    assert np.array_equal(q[r], np.arange(S))                       # inverse
    assert np.all(s["counts"].sum(1) == M * k)
    assert np.array_equal(s["offsets"][:, 1:], np.cumsum(s["counts"], 1))
    assert np.array_equal(s["mini_counts"].sum(2), s["counts"])
    flat = idx.reshape(-1)
    for m in range(T // M):
        base = m * M * k
        for e in range(E):
            lo, hi = base + s["offsets"][m, e], base + s["offsets"][m, e + 1]
            slots = q[lo:hi]
            assert np.all(flat[slots] == e)
            assert np.all(np.diff(slots) > 0)                       # stable: ascending slot
            # each minibatch is a contiguous piece of the expert's group
            mini_of = (slots - base) // (mb * k)
            assert np.all(np.diff(mini_of) >= 0)
            assert np.array_equal(np.bincount(mini_of, minlength=M // mb), s["mini_counts"][m, e])


def test_empty_experts_and_single_expert():
    idx = np.zeros((10, 1), dtype=np.int32)
    s = oracle.schedule(idx, 4)
    assert s["counts"].tolist() == [[10, 0, 0, 0]]
    assert s["offsets"].tolist() == [[0, 10, 10, 10, 10]]
    assert s["row_of_slot"].tolist() == list(range(10))


def test_rejects_bad_shapes():
    idx = np.zeros((10, 2), dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.schedule(idx, 4, macrobatch=3)
    with pytest.raises(ValueError):
        oracle.schedule(idx, 4, macrobatch=10, minibatch=4)
    with pytest.raises(ValueError):
        oracle.schedule(idx + 4, 4)
