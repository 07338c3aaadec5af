"""GPU parity of the recompute mode (MOE_FLAG_RECOMPUTE): nothing but the
schedule is saved for the backward, which walks the macrobatches in reverse,
takes the last macrobatch's gate/up projections from the workspace and
recomputes every earlier one's (arex-research.com "Cursor 放出 MoK", design
section, second decision).

The recomputation runs the forward's own gate/up GEMM on the same inputs, so
every output of the backward must be bit-identical to the saving mode's; one
shape per precision is also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_cases import Case, assert_close, f32

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny": si.SHAPES["tiny"],
    # four macrobatches, a shared expert: three of them recomputed
    "ring_shared": si.custom_shape("ring_shared_rc", T=512, H=256, I=128, E=16, k=4, seed=40,
                                   n_shared=1, macrobatch=128, minibatch=64),
    # hot experts past one K step of the weight gradients, 128-row tiles
    "zipf_ring": si.custom_shape("zipf_ring_rc", T=1024, H=256, I=256, E=32, k=4, seed=41,
                                 macrobatch=256, minibatch=128, zipf=True),
    "odd_tiles": si.custom_shape("odd_tiles_rc", T=512, H=1152, I=384, E=4, k=2, seed=42,
                                 n_shared=1, macrobatch=256),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(shape, precision, recompute):
    c = Case(shape, precision=precision, recompute=recompute)
    c.schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(c.ws) == 0
    return c


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
@pytest.mark.parametrize("name", list(SHAPES))
def test_recompute_matches_saving_mode_bitwise(name, prec):
    from mixture_experts_layer_dispatch_amd import binding as B
    p = B.PREC_MXFP8 if prec == "mxfp8" else B.PREC_BF16
    ref = _run(SHAPES[name], p, False)
    rc = _run(SHAPES[name], p, True)
    assert rc.saved == {}
    assert torch.equal(rc.y, ref.y)
    assert torch.equal(rc.dx, ref.dx)
    assert torch.equal(rc.dw, ref.dw)
    assert torch.equal(rc.dlogits, ref.dlogits)
    for k in ref.grads:
        assert torch.equal(rc.grads[k], ref.grads[k]), k


@pytest.mark.parametrize("prec,tol", [("bf16", 1e-2), ("mxfp8", 3e-2)])
def test_recompute_against_oracle(prec, tol):
    from mixture_experts_layer_dispatch_amd import binding as B
    shape = SHAPES["ring_shared"]
    mx = prec == "mxfp8"
    c = _run(shape, B.PREC_MXFP8 if mx else B.PREC_BF16, True)
    idx, w, sch = c.oracle_schedule()
    ref = oracle.backward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd),
                          idx, w, f32(c.dy), shared=c.shared_np(), mx=mx, sched=sch,
                          experts=list(range(shape.E)))
    assert_close("y", f32(c.y), ref["fwd"]["y"], tol)
    assert_close("dx", f32(c.dx), ref["dx"], tol)
    assert_close("dw", c.dw.cpu().numpy(), ref["dw"], tol)
    E = shape.E
    zg = np.zeros((shape.I, shape.H))
    zd = np.zeros((shape.H, shape.I))
    assert_close("dW_gate", f32(c.grads["d_w_gate"]), np.stack([ref["dWg"].get(e, zg) for e in range(E)]), tol)
    assert_close("dW_down", f32(c.grads["d_w_down"]), np.stack([ref["dWd"].get(e, zd) for e in range(E)]), tol)
    assert_close("dW_shared_up", f32(c.grads["d_s_up"]), ref["dW_su"], tol)
