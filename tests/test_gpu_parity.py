"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Exact for routing indices and the schedule; within 1e-2 * max|ref| for every
bf16 output and gradient (the tolerance the layer is specified to); the
combine weights within fp32 rounding.  Small shapes are compared element by
element; the 512-expert shapes on sampled tokens and experts.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_cases import Case, assert_close, assert_rerun_bitwise, f32, ring_samples

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": si.SHAPES["tiny"],
    "ragged": si.custom_shape("ragged", T=100, H=256, I=256, E=7, k=3, seed=11),
    "sparse_experts": si.custom_shape("sparse_experts", T=40, H=128, I=128, E=16, k=1, seed=12),
    "single_expert": si.custom_shape("single_expert", T=70, H=128, I=256, E=1, k=1, seed=13),
    "ring_shared": si.custom_shape("ring_shared", T=512, H=256, I=128, E=16, k=4, seed=14,
                                   n_shared=1, macrobatch=128, minibatch=64),
    "zipf_ring": si.custom_shape("zipf_ring", T=1024, H=128, I=128, E=32, k=4, seed=15,
                                 macrobatch=256, minibatch=128, zipf=True),
    # wider outputs: weight-gradient slabs of 8 and 16 column tiles (the
    # latter dealt over two blocks); the ring variant accumulates them across
    # two macrobatches in fp32
    "stripes": si.custom_shape("stripes", T=256, H=512, I=512, E=16, k=4, seed=17),
    "stripes_ring": si.custom_shape("stripes_ring", T=512, H=512, I=1024, E=32, k=2, seed=18,
                                    n_shared=1, macrobatch=256, minibatch=128),
    # groups of ~256 rows: the 128-row tiles of the row-grouped GEMMs
    "dense_experts": si.custom_shape("dense_experts", T=512, H=256, I=256, E=8, k=4, seed=19),
    # 128-row tiles with an odd number of 128-column tiles (the last block of
    # the two-tile K loops holds one tile), for the routed experts and a dense
    # shared expert; their weight gradients take the deep kernels
    "odd_tiles": si.custom_shape("odd_tiles", T=512, H=1152, I=384, E=4, k=2, seed=20, n_shared=1),
    # k = E: every token goes to every expert (the dense softmax mixture)
    "all_experts": si.custom_shape("all_experts", T=96, H=128, I=128, E=4, k=4, seed=28),
    # the largest k the library takes (32): 32 slots per token in the combine
    # and the reverse-dispatch, 32 selection rounds in the routing
    "max_k": si.custom_shape("max_k", T=64, H=128, I=128, E=64, k=32, seed=29),
    # the largest E (1024): ten ballot rounds over the expert-id bits, most
    # experts empty
    "max_e": si.custom_shape("max_e", T=256, H=128, I=128, E=1024, k=8, seed=32),
    # top-1 routing without a shared expert over several macrobatches: the
    # down projection and the gate/up input gradient write y and dx rows
    # directly (no combine or reverse-dispatch pass)
    "top1_ring": si.custom_shape("top1_ring", T=512, H=256, I=256, E=8, k=1, seed=34,
                                 macrobatch=128, minibatch=64),
    # groups of several hundred rows over two macrobatches, with a dense
    # shared expert of 512 rows per macrobatch: the down projection's
    # 256 x 256 tiles (groups of at least 256 rows, ragged tails) beside the
    # 128-row tiles of the smaller groups
    "big_tiles": si.custom_shape("big_tiles", T=1024, H=512, I=256, E=4, k=2, seed=36,
                                 n_shared=1, macrobatch=512, minibatch=256),
    # Zipf-skewed groups: a few hot experts in 256-row tiles, the rest in
    # 128-row tiles, top-1 (rows written straight to y)
    "big_zipf_top1": si.custom_shape("big_zipf_top1", T=4096, H=256, I=128, E=16, k=1, seed=37,
                                     zipf=True),
    # groups of ~500 rows over two macrobatches: an expert's weight gradient
    # moves between the 256 x 256 kernels (>= 512 rows) and the 128 x 128
    # deep kernels from one macrobatch to the next, through its fp32 sums
    "big_wgrad": si.custom_shape("big_wgrad", T=2048, H=256, I=256, E=4, k=2, seed=38,
                                 macrobatch=1024, minibatch=512),
    # Zipf-skewed groups with a dense shared expert of 768 rows: every weight
    # gradient form in one macrobatch (256 x 256, deep 128 x 128, slabs)
    "big_wgrad_zipf": si.custom_shape("big_wgrad_zipf", T=1536, H=256, I=256, E=6, k=3, seed=39,
                                      n_shared=1, macrobatch=768, minibatch=256, zipf=True),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.device_supported(), "the library requires gfx950"


def test_generator_is_bit_exact_on_gpu():
    sh = SMALL["ragged"]
    assert torch.equal(si.tokens(sh, "cuda").cpu(), si.tokens(sh, "cpu"))
    assert torch.equal(si.logits(SMALL["zipf_ring"], "cuda").cpu(), si.logits(SMALL["zipf_ring"], "cpu"))
    big = si.SHAPES["e512_t2048"]
    wg, wu, wd = si.all_expert_weights(sh, "cuda")
    for e in range(sh.E):
        a, b, c = si.expert_weights(sh, e, "cpu")
        assert torch.equal(wg[e].cpu(), a) and torch.equal(wu[e].cpu(), b) and torch.equal(wd[e].cpu(), c)
    for e in (0, 300, 511):
        a, b, c = si.expert_weights(big, e, "cuda")
        a2, b2, c2 = si.expert_weights(big, e, "cpu")
        assert torch.equal(a.cpu(), a2) and torch.equal(b.cpu(), b2) and torch.equal(c.cpu(), c2)


def _check_schedule(case: Case):
    idx, w, sch = case.oracle_schedule()
    s = case.sched
    np.testing.assert_array_equal(s["topk_idx"].cpu().numpy(), idx)
    np.testing.assert_array_equal(s["counts"].cpu().numpy(), sch["counts"])
    np.testing.assert_array_equal(s["offsets"].cpu().numpy(), sch["offsets"])
    np.testing.assert_array_equal(s["mini_counts"].cpu().numpy(), sch["mini_counts"])
    np.testing.assert_array_equal(s["row_of_slot"].cpu().numpy(), sch["row_of_slot"])
    np.testing.assert_array_equal(s["slot_of_row"].cpu().numpy(), sch["slot_of_row"])
    gw = s["topk_w"].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gw - w)) <= 2e-6, np.max(np.abs(gw - w))
    return idx, w, sch


@pytest.mark.parametrize("name", list(SMALL))
def test_schedule_small(name):
    case = Case(SMALL[name], with_backward=False)
    case.schedule()
    _check_schedule(case)


def test_schedule_with_ties_and_signed_zeros():
    shape = si.custom_shape("ties", T=512, H=128, I=128, E=64, k=6, seed=16, macrobatch=256,
                            minibatch=64)
    g = torch.Generator().manual_seed(0)
    L = torch.randint(-1, 2, (512, 64), generator=g).float()
    L[::3] = torch.where(torch.rand(L[::3].shape, generator=g) < 0.5, -0.0, 0.0)
    case = Case(shape, logits_override=L, with_backward=False)
    case.schedule()
    _check_schedule(case)


@pytest.mark.parametrize("name", ["e512_t2048", "e512_t65536_zipf", "e8_ep_share"])
def test_schedule_full_size(name):
    from gpu_cases import cfg_of
    from mixture_experts_layer_dispatch_amd import binding as B

    case = Case.__new__(Case)          # schedule only: no weights needed
    case.shape = si.SHAPES[name]
    case.cfg = cfg_of(case.shape)
    case.logits = si.logits(case.shape, "cuda")
    case.ws = B.alloc_workspace(case.cfg)
    case.sched = B.alloc_schedule(case.cfg)
    case.schedule()
    _check_schedule(case)
    assert B.moe_check_device_error(case.ws) == 0


def _oracle_forward(case: Case, idx, w, tokens=None):
    x = f32(case.x)
    return oracle.forward(x, case.expert_view(case.wg), case.expert_view(case.wu),
                          case.expert_view(case.wd), idx, w, shared=case.shared_np(), tokens=tokens)


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    case = Case(SMALL[name], with_backward=False)
    case.schedule()
    idx, w, sch = _check_schedule(case)
    case.forward()
    torch.cuda.synchronize()
    ref = _oracle_forward(case, idx, w)
    assert_close("y", f32(case.y), ref["y"])
    # saved g, u are stored by schedule row
    rows = sch["row_of_slot"].reshape(case.shape.T, case.shape.k)
    g = f32(case.saved["g"])[rows]
    u = f32(case.saved["u"])[rows]
    assert_close("g", g, ref["g"])
    assert_close("u", u, ref["u"])
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(case.ws) == 0


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_small(name):
    case = Case(SMALL[name])
    case.schedule()
    idx, w, sch = case.oracle_schedule()
    case.forward()
    case.backward()
    torch.cuda.synchronize()
    x, dy = f32(case.x), f32(case.dy)
    ref = oracle.backward(x, case.expert_view(case.wg), case.expert_view(case.wu),
                          case.expert_view(case.wd), idx, w, dy, shared=case.shared_np(),
                          experts=list(range(case.shape.E)))
    assert_close("dx", f32(case.dx), ref["dx"])
    assert_close("dw", case.dw.cpu().numpy(), ref["dw"])
    dl = oracle.ffn.d_logits_dense(idx, ref["dl_sel"], case.shape.E)
    assert_close("d_logits", case.dlogits.cpu().numpy(), dl)
    E = case.shape.E
    zero_g = np.zeros((case.shape.I, case.shape.H))
    zero_d = np.zeros((case.shape.H, case.shape.I))
    dWg = np.stack([ref["dWg"].get(e, zero_g) for e in range(E)])
    dWu = np.stack([ref["dWu"].get(e, zero_g) for e in range(E)])
    dWd = np.stack([ref["dWd"].get(e, zero_d) for e in range(E)])
    assert_close("dW_gate", f32(case.grads["d_w_gate"]), dWg)
    assert_close("dW_up", f32(case.grads["d_w_up"]), dWu)
    assert_close("dW_down", f32(case.grads["d_w_down"]), dWd)
    if case.sw is not None:
        assert_close("dW_shared_gate", f32(case.grads["d_s_gate"]), ref["dW_sg"])
        assert_close("dW_shared_up", f32(case.grads["d_s_up"]), ref["dW_su"])
        assert_close("dW_shared_down", f32(case.grads["d_s_down"]), ref["dW_sd"])
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(case.ws) == 0


def test_bitwise_determinism_and_grouping_independence():
    base = SMALL["ring_shared"]
    case = Case(base)
    case.schedule()
    case.forward()
    case.backward()
    y1, dx1 = case.y.clone(), case.dx.clone()
    g1 = {k: v.clone() for k, v in case.grads.items()}
    dw1 = case.dw.clone()
    for _ in range(2):
        case.poison_outputs()
        case.schedule()
        case.forward()
        case.backward()
        assert torch.equal(case.y, y1) and torch.equal(case.dx, dx1) and torch.equal(case.dw, dw1)
        for k in g1:
            assert torch.equal(case.grads[k], g1[k]), k
    # the routed rows' math does not depend on how tokens are grouped into
    # macrobatches and minibatches (the shared expert's neither)
    other = si.custom_shape("ring_shared_b", T=base.T, H=base.H, I=base.I, E=base.E, k=base.k,
                            seed=base.seed, n_shared=1, macrobatch=256, minibatch=32)
    c2 = Case(other)
    c2.schedule()
    c2.forward()
    assert torch.equal(c2.y, y1)


# ------------------------------------------------------------------ full size
def _full_case():
    return Case(si.SHAPES["e512_t2048"])


def test_forward_backward_full_size_sampled():
    case = _full_case()
    case.schedule()
    idx, w, sch = _check_schedule(case)
    case.forward()
    case.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(case.ws) == 0
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(case.shape.T, size=24, replace=False))
    tokens[0] = 0
    tokens[-1] = case.shape.T - 1
    x, dy = f32(case.x), f32(case.dy)
    wgv, wuv, wdv = case.expert_view(case.wg), case.expert_view(case.wu), case.expert_view(case.wd)
    ref = oracle.forward(x, wgv, wuv, wdv, idx, w, tokens=tokens)
    assert_close("y[sampled]", f32(case.y)[tokens], ref["y"])
    experts = [int(idx[0, 0]), int(idx[-1, -1]), 257]
    rb = oracle.backward(x, wgv, wuv, wdv, idx, w, dy, tokens=tokens, experts=experts)
    assert_close("dx[sampled]", f32(case.dx)[tokens], rb["dx"])
    assert_close("dw[sampled]", case.dw.cpu().numpy()[tokens], rb["dw"])
    dl = oracle.ffn.d_logits_dense(idx, rb["dl_sel"], case.shape.E, tokens=tokens)
    assert_close("d_logits[sampled]", case.dlogits.cpu().numpy()[tokens], dl)
    for e in experts:
        assert_close(f"dW_gate[{e}]", f32(case.grads["d_w_gate"][e]), rb["dWg"][e])
        assert_close(f"dW_up[{e}]", f32(case.grads["d_w_up"][e]), rb["dWu"][e])
        assert_close(f"dW_down[{e}]", f32(case.grads["d_w_down"][e]), rb["dWd"][e])
    # every expert's weight gradient is written (no stale memory): norms are finite and
    # zero exactly where the expert received no rows
    counts = sch["counts"][0]
    n = case.grads["d_w_down"].float().flatten(1).abs().amax(1).cpu().numpy()
    assert np.all(np.isfinite(n)) and np.all((n == 0) == (counts == 0))
    assert_rerun_bitwise(case)


def test_forward_backward_ring_full_size_sampled():
    """The 65 536-token Zipf workload at full size: four macrobatches through
    the ring (two halves, minibatch dispatch), a shared expert, and the weight
    gradients summed over the reverse macrobatch walk in fp32."""
    case = Case(si.SHAPES["e512_t65536_zipf"])
    case.schedule()
    idx, w, sch = _check_schedule(case)
    case.forward()
    case.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(case.ws) == 0
    tokens, experts = ring_samples(case, sch)
    x, dy = f32(case.x), f32(case.dy)
    wgv, wuv, wdv = case.expert_view(case.wg), case.expert_view(case.wu), case.expert_view(case.wd)
    ref = oracle.forward(x, wgv, wuv, wdv, idx, w, shared=case.shared_np(), tokens=tokens)
    assert_close("y[sampled]", f32(case.y)[tokens], ref["y"])
    rb = oracle.backward(x, wgv, wuv, wdv, idx, w, dy, shared=case.shared_np(), tokens=tokens,
                         experts=experts)
    assert_close("dx[sampled]", f32(case.dx)[tokens], rb["dx"])
    assert_close("dw[sampled]", case.dw.cpu().numpy()[tokens], rb["dw"])
    dl = oracle.ffn.d_logits_dense(idx, rb["dl_sel"], case.shape.E, tokens=tokens)
    assert_close("d_logits[sampled]", case.dlogits.cpu().numpy()[tokens], dl)
    for e in experts:
        assert_close(f"dW_gate[{e}]", f32(case.grads["d_w_gate"][e]), rb["dWg"][e])
        assert_close(f"dW_up[{e}]", f32(case.grads["d_w_up"][e]), rb["dWu"][e])
        assert_close(f"dW_down[{e}]", f32(case.grads["d_w_down"][e]), rb["dWd"][e])
    assert_rerun_bitwise(case)


def test_forward_backward_ep_share_full_size_sampled():
    """One GPU's expert-parallel share: 8 experts with 2560 rows each, top-1."""
    case = Case(si.SHAPES["e8_ep_share"])
    case.schedule()
    idx, w, sch = _check_schedule(case)
    case.forward()
    case.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(case.ws) == 0
    rng = np.random.default_rng(7)
    tokens = np.sort(rng.choice(case.shape.T, size=24, replace=False))
    x, dy = f32(case.x), f32(case.dy)
    wgv, wuv, wdv = case.expert_view(case.wg), case.expert_view(case.wu), case.expert_view(case.wd)
    ref = oracle.forward(x, wgv, wuv, wdv, idx, w, tokens=tokens)
    assert_close("y[sampled]", f32(case.y)[tokens], ref["y"])
    rb = oracle.backward(x, wgv, wuv, wdv, idx, w, dy, tokens=tokens, experts=[0, 7])
    assert_close("dx[sampled]", f32(case.dx)[tokens], rb["dx"])
    assert_close("dw[sampled]", case.dw.cpu().numpy()[tokens], rb["dw"])
    for e in (0, 7):
        assert_close(f"dW_gate[{e}]", f32(case.grads["d_w_gate"][e]), rb["dWg"][e])
        assert_close(f"dW_up[{e}]", f32(case.grads["d_w_up"][e]), rb["dWu"][e])
        assert_close(f"dW_down[{e}]", f32(case.grads["d_w_down"][e]), rb["dWd"][e])


def test_forward_backward_many_big_tiles_sampled():
    """A macrobatch of 131 072 routed rows over eight experts (I = 512): enough
    256 x 256 tiles of the down dgrad (512 row tiles x 2 column tiles) for its
    256 x 256 form, with router weights, gathered dy and the dw partials of its
    two 128-column halves per tile, checked on sampled tokens and experts."""
    shape = si.custom_shape("many_big_tiles", T=32768, H=256, I=512, E=8, k=4, seed=40)
    case = Case(shape)
    case.schedule()
    idx, w, sch = _check_schedule(case)
    case.forward()
    case.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(case.ws) == 0
    rng = np.random.default_rng(9)
    tokens = np.sort(rng.choice(shape.T, size=24, replace=False))
    tokens[0], tokens[-1] = 0, shape.T - 1
    x, dy = f32(case.x), f32(case.dy)
    wgv, wuv, wdv = case.expert_view(case.wg), case.expert_view(case.wu), case.expert_view(case.wd)
    ref = oracle.forward(x, wgv, wuv, wdv, idx, w, tokens=tokens)
    assert_close("y[sampled]", f32(case.y)[tokens], ref["y"])
    rb = oracle.backward(x, wgv, wuv, wdv, idx, w, dy, tokens=tokens, experts=[1, 3])
    assert_close("dx[sampled]", f32(case.dx)[tokens], rb["dx"])
    assert_close("dw[sampled]", case.dw.cpu().numpy()[tokens], rb["dw"])
    dl = oracle.ffn.d_logits_dense(idx, rb["dl_sel"], shape.E, tokens=tokens)
    assert_close("d_logits[sampled]", case.dlogits.cpu().numpy()[tokens], dl)
    for e in (1, 3):
        assert_close(f"dW_gate[{e}]", f32(case.grads["d_w_gate"][e]), rb["dWg"][e])
        assert_close(f"dW_up[{e}]", f32(case.grads["d_w_up"][e]), rb["dWu"][e])
        assert_close(f"dW_down[{e}]", f32(case.grads["d_w_down"][e]), rb["dWd"][e])
    assert_rerun_bitwise(case)


def test_dense_shared_expert_big_weight_gradient_tiles():
    """A shared expert whose weight gradients have enough 256 x 256 tiles to
    fill their persistent grid (H = I = 4096: 256 tiles of dW_down, 512 of
    dW_gate | dW_up) takes that form; smaller dense groups take the 128 x 128
    tiles.  Checked in full against the oracle (about 20 s of float64 on the
    host)."""
    shape = si.custom_shape("dense_big_wgrad", T=512, H=4096, I=4096, E=2, k=1, seed=41, n_shared=1)
    case = Case(shape)
    case.schedule()
    idx, w, sch = _check_schedule(case)
    case.forward()
    case.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(case.ws) == 0
    x, dy = f32(case.x), f32(case.dy)
    wgv, wuv, wdv = case.expert_view(case.wg), case.expert_view(case.wu), case.expert_view(case.wd)
    rb = oracle.backward(x, wgv, wuv, wdv, idx, w, dy, shared=case.shared_np())
    assert_close("dx", f32(case.dx), rb["dx"])
    assert_close("dW_shared_gate", f32(case.grads["d_s_gate"]), rb["dW_sg"])
    assert_close("dW_shared_up", f32(case.grads["d_s_up"]), rb["dW_su"])
    assert_close("dW_shared_down", f32(case.grads["d_s_down"]), rb["dW_sd"])
    for e in (0, 1):
        assert_close(f"dW_down[{e}]", f32(case.grads["d_w_down"][e]), rb["dWd"][e])


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_256_row_tiles_give_the_bits_of_the_smaller_tiles(precision):
    """The same tokens as one macrobatch (groups of ~512 rows, a 1024-row shared
    expert: the 256 x 256 tile forms) and as eight macrobatches (groups of ~64
    rows: 64-row tiles).  Every output whose rows do not mix across
    macrobatches (y, dx, the router-weight and logit gradients) is bit for bit
    the same: each row's products are summed in the same order in every tile
    form."""
    from mixture_experts_layer_dispatch_amd import binding as B
    prec = B.PREC_BF16 if precision == "bf16" else B.PREC_MXFP8
    kw = dict(T=1024, H=512, I=256, E=4, k=2, seed=42, n_shared=1)
    one = Case(si.custom_shape("tiles_one_macrobatch", **kw), precision=prec)
    many = Case(si.custom_shape("tiles_eight_macrobatches", macrobatch=128, minibatch=64, **kw),
                precision=prec)
    for c in (one, many):
        c.schedule()
        c.forward()
        c.backward()
    torch.cuda.synchronize()
    assert B.moe_check_device_error(one.ws) == 0 and B.moe_check_device_error(many.ws) == 0
    _, _, sch = one.oracle_schedule()
    assert (sch["counts"] >= 256).any()                      # the large form runs in `one`
    for name in ("y", "dx", "dw", "dlogits"):
        assert torch.equal(getattr(one, name), getattr(many, name)), name
