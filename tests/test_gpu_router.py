"""GPU parity of the router projection (moe_router_forward / moe_router_backward)
against the oracle (oracle.router): logits within fp32 accumulation error of the
exact product of the bf16 inputs, the router's share of dx and dW_router within
the bf16 bar; the router backward composed after the layer's backward."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_cases import Case, assert_close, f32

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny": si.SHAPES["tiny"],
    "ragged": si.custom_shape("ragged_router", T=100, H=256, I=128, E=7, k=3, seed=80),
    "wide_e": si.custom_shape("wide_e_router", T=192, H=384, I=128, E=200, k=4, seed=81),
    "e512_t2048": si.SHAPES["e512_t2048"],
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", list(SHAPES))
def test_router_forward_backward(name):
    from mixture_experts_layer_dispatch_amd import binding as B
    from gpu_cases import cfg_of
    shape = SHAPES[name]
    cfg = cfg_of(shape)
    x = si.tokens(shape, "cuda")
    wr = si.router_weights(shape, "cuda")
    logits = torch.full((shape.T, shape.E), float("nan"), device="cuda")
    B.moe_router_forward(cfg, x, wr, logits)
    dl = si.normal((shape.T, shape.E), shape.seed + 1000, si.S_LOGITS, 1.0, torch.float32, "cuda")
    dx0 = si.grad_out(shape, "cuda")                   # stands for the layer's dx
    dx = dx0.clone()
    dwr = torch.full((shape.E, shape.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = B.alloc_workspace(cfg)
    B.moe_router_backward(cfg, x, wr, dl, dx, dwr, ws)
    torch.cuda.synchronize()
    xs, ws_ = f32(x).astype(np.float64), f32(wr).astype(np.float64)
    ref = oracle.router_logits(xs, ws_)
    assert_close("logits", logits.cpu().numpy(), ref, 1e-4)
    # the oracle's d_logits operand: the GPU rounds d_logits to bf16 once
    dl16 = f32(dl.to(torch.bfloat16)).astype(np.float64)
    rdx, rdw = oracle.router_backward(xs, ws_, dl16)
    assert_close("dx (layer + router)", f32(dx), f32(dx0) + rdx)
    assert_close("dW_router", f32(dwr), rdw)


def test_router_after_the_layer_backward():
    """logits from the router feed the schedule; the layer's d_logits feed the
    router backward, whose dx completes the layer's."""
    from mixture_experts_layer_dispatch_amd import binding as B
    shape = si.custom_shape("router_chain", T=256, H=256, I=128, E=16, k=4, seed=83)
    wr = si.router_weights(shape, "cuda")
    x = si.tokens(shape, "cuda")
    logits = torch.empty(shape.T, shape.E, device="cuda")
    c = Case(shape, logits_override=torch.zeros(shape.T, shape.E))
    B.moe_router_forward(c.cfg, x, wr, logits)
    c.logits = logits
    c.schedule()
    c.forward()
    c.backward()
    dwr = torch.empty(shape.E, shape.H, dtype=torch.bfloat16, device="cuda")
    dx_layer = c.dx.clone()
    B.moe_router_backward(c.cfg, x, wr, c.dlogits, c.dx, dwr, c.ws)
    torch.cuda.synchronize()
    assert B.moe_check_device_error(c.ws) == 0
    # the oracle routes its own logits; the seeded input keeps every token's
    # k-th / (k+1)-th logit gap far above fp32 accumulation error, so both
    # sides must pick the same experts
    L = oracle.router_logits(f32(x).astype(np.float64), f32(wr).astype(np.float64))
    srt = -np.sort(-L, axis=1)
    assert np.min(srt[:, shape.k - 1] - srt[:, shape.k]) > 1e-3
    idx, w = oracle.route(L, shape.k)
    np.testing.assert_array_equal(c.sched["topk_idx"].cpu().numpy(), idx)
    ref = oracle.backward(f32(x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd), idx, w,
                          f32(c.dy))
    dl = oracle.ffn.d_logits_dense(idx, ref["dl_sel"], shape.E)
    rdx, rdw = oracle.router_backward(f32(x), f32(wr), dl)
    assert_close("dx (layer + router)", f32(c.dx), ref["dx"] + rdx)
    assert_close("dW_router", f32(dwr), rdw)
    assert not torch.equal(c.dx, dx_layer)
