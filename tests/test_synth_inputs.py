"""The seeded input generator: slices regenerate exactly, streams differ,
and the distribution has the stated mean and spread."""
import numpy as np
import torch

import synth_inputs as si


def test_slices_regenerate_exactly():
    shape = si.custom_shape("t", T=16, H=64, I=32, E=4, k=2, seed=9)
    wg, wu, wd = si.all_expert_weights(shape)
    for e in range(4):
        a, b, c = si.expert_weights(shape, e)
        assert torch.equal(a, wg[e]) and torch.equal(b, wu[e]) and torch.equal(c, wd[e])
    x = si.tokens(shape)
    assert torch.equal(si.tokens(shape, rows=[3, 0, 15]), x[[3, 0, 15]])
    dy = si.grad_out(shape)
    assert torch.equal(si.grad_out(shape, rows=[7]), dy[[7]])


def test_chunking_does_not_change_values():
    a = si.normal((1000,), 5, 2, 0.5, torch.bfloat16)
    b = si.normal((1000,), 5, 2, 0.5, torch.bfloat16, chunk=37)
    assert torch.equal(a, b)


def test_streams_and_seeds_differ():
    a = si.normal((4096,), 1, si.S_X)
    assert not torch.equal(a, si.normal((4096,), 1, si.S_DY))
    assert not torch.equal(a, si.normal((4096,), 2, si.S_X))


def test_distribution():
    v = si.normal((1 << 20,), 3, si.S_X, 0.25).double()
    assert abs(v.mean().item()) < 3e-3
    assert abs(v.std().item() - 0.25) < 2e-3
    assert v.dtype == torch.float64


def test_zipf_bias_and_permutation():
    b = si.zipf_bias(512).numpy().astype(np.float64)
    assert np.all(np.diff(b) < 0)                      # expert 0 hottest
    p = np.exp(b / 2)
    assert abs(p.sum() - 1.0) < 1e-5
    assert abs(p[0] / p[1] - 2 ** 1.1) < 1e-4
    perm = si.permutation(1000, 2, si.S_PERM)
    assert sorted(perm.tolist()) == list(range(1000))


def test_balanced_ep_share_logits():
    """One GPU's expert-parallel share: every expert gets exactly T/E rows, each
    row routed top-1 to its assigned expert with weight 1."""
    import oracle
    sh = si.SHAPES["e8_ep_share"]
    L = si.logits(sh, "cpu").numpy()
    assert set(np.unique(L)) == {0.0, 1.0} and np.all(L.sum(1) == 1.0)
    idx, w = oracle.route(L.astype(np.float64), sh.k)
    assert np.array_equal(idx[:, 0], si.balanced_assignment(sh).numpy())
    assert np.array_equal(np.bincount(idx[:, 0], minlength=sh.E), np.full(sh.E, sh.T // sh.E))
    assert np.all(w == 1.0)
