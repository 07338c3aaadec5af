"""GPU parity of the MXFP4-weight forward (MOE_PREC_MXFP4: E2M1 weights with
E8M0 scales per 32 along K, MXFP8 activations) against the oracle's "w4"
mode: the quantised weights bit for bit, the layer's output within
3e-2 * max|ref| (the oracle applies the same quantisation; what is left is
fp32 summation order and the bf16 storage of o), bit-identical reruns; the
backward is refused."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_cases import Case, assert_close, f32

pytestmark = pytest.mark.gpu

MX_TOL = 3e-2

SHAPES = {
    "tiny": si.SHAPES["tiny"],
    "ragged": si.custom_shape("ragged_mx4", T=100, H=256, I=256, E=7, k=3, seed=90),
    "ring_shared": si.custom_shape("ring_shared_mx4", T=512, H=256, I=128, E=16, k=4, seed=91,
                                   n_shared=1, macrobatch=128, minibatch=64),
    # groups of ~256 rows: the 128-row tiles
    "dense_experts": si.custom_shape("dense_experts_mx4", T=512, H=256, I=256, E=8, k=4, seed=92),
    "odd_tiles": si.custom_shape("odd_tiles_mx4", T=512, H=1152, I=384, E=4, k=2, seed=93, n_shared=1),
    "max_k": si.custom_shape("max_k_mx4", T=64, H=128, I=128, E=64, k=32, seed=94),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(shape, **kw):
    from mixture_experts_layer_dispatch_amd import binding as B
    return Case(shape, precision=B.PREC_MXFP4, **kw)


def _unpack(codes):
    """[.., K/2] bytes -> [.., K] nibbles (element 2q in the low nibble of byte q)."""
    c = codes.cpu().numpy()
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def _check_quantised(w_bf16, codes, scales):
    ref_c, ref_s = oracle.mxfp4_quantize(f32(w_bf16).astype(np.float64), axis=1)
    ks = scales.cpu().numpy()
    got_s = ks.transpose(1, 0, 2).reshape(ks.shape[1], ks.shape[0] * 4)
    np.testing.assert_array_equal(got_s, ref_s)
    np.testing.assert_array_equal(_unpack(codes), ref_c)


@pytest.mark.parametrize("name", ["tiny", "ring_shared", "odd_tiles"])
def test_mxfp4_weight_quantiser_bit_exact(name):
    c = _case(SHAPES[name], with_backward=False)
    torch.cuda.synchronize()
    for e in range(c.shape.E):
        _check_quantised(c.wg[e], c.wq4["w_gate_q"][e], c.wq4["w_gate_s"][e])
        _check_quantised(c.wu[e], c.wq4["w_up_q"][e], c.wq4["w_up_s"][e])
        _check_quantised(c.wd[e], c.wq4["w_down_q"][e], c.wq4["w_down_s"][e])
    if c.sw is not None:
        _check_quantised(c.sw[0], c.wq4["s_gate_q"], c.wq4["s_gate_s"])
        _check_quantised(c.sw[2], c.wq4["s_down_q"], c.wq4["s_down_s"])


def test_mxfp4_quantiser_edge_values():
    """Ties, saturation, signed zeros, zero blocks, element by element."""
    from mixture_experts_layer_dispatch_amd import binding as B
    shape = si.custom_shape("edge4", T=8, H=128, I=128, E=1, k=1, seed=0)
    c = _case(shape, with_backward=False)
    vals = torch.tensor([0.0, -0.0, 0.5, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 100.0, -9.0, 0.25, 0.75,
                         2.9, 0.3], dtype=torch.float32)
    w = torch.zeros(128, 128, dtype=torch.float32)
    w[:, :16] = vals                       # block 0 of every row mixes everything
    w[5] = 0.0                             # an all-zero row
    w[7] *= -1
    wb = w.to(torch.bfloat16).cuda()
    weights = {"w_gate": wb[None].contiguous(), "w_up": wb[None].contiguous(),
               "w_down": wb[None].contiguous()}
    q = B.alloc_weights_mx4(c.cfg)
    B.moe_quantize_weights_mxfp4(c.cfg, weights, q)
    torch.cuda.synchronize()
    _check_quantised(wb, q["w_gate_q"][0], q["w_gate_s"][0])
    _check_quantised(wb, q["w_down_q"][0], q["w_down_s"][0])


@pytest.mark.parametrize("name", list(SHAPES))
def test_mxfp4_forward_small(name):
    c = _case(SHAPES[name], with_backward=False)
    c.schedule()
    idx, w, sch = c.oracle_schedule()
    c.forward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(c.ws) == 0
    ref = oracle.forward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd),
                         idx, w, shared=c.shared_np(), mx="w4")
    assert_close("y (mxfp4 weights)", f32(c.y), ref["y"], MX_TOL)
    rows = sch["row_of_slot"].reshape(c.shape.T, c.shape.k)
    assert_close("g (mxfp4 weights)", f32(c.saved["g"])[rows], ref["g"], MX_TOL)
    assert_close("u (mxfp4 weights)", f32(c.saved["u"])[rows], ref["u"], MX_TOL)
    # the 4-bit weights really are 4-bit: the MXFP8 layer is measurably different
    mx8 = oracle.forward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd),
                         idx, w, shared=c.shared_np(), mx=True)["y"]
    assert np.max(np.abs(mx8 - ref["y"])) > 3 * np.max(np.abs(f32(c.y) - ref["y"]))


def test_mxfp4_forward_full_size_sampled_and_reruns():
    c = _case(si.SHAPES["e512_t2048"], with_backward=False)
    c.schedule()
    c.forward()
    torch.cuda.synchronize()
    idx, w = oracle.route(f32(c.logits), c.shape.k)
    np.testing.assert_array_equal(c.sched["topk_idx"].cpu().numpy(), idx)
    rng = np.random.default_rng(3)
    tokens = np.sort(rng.choice(c.shape.T, size=16, replace=False))
    ref = oracle.forward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd),
                         idx, w, tokens=tokens, mx="w4")
    assert_close("y[sampled] (mxfp4 weights)", f32(c.y)[tokens], ref["y"], MX_TOL)
    for e in (0, 511):
        _check_quantised(c.wg[e], c.wq4["w_gate_q"][e], c.wq4["w_gate_s"][e])
        _check_quantised(c.wd[e], c.wq4["w_down_q"][e], c.wq4["w_down_s"][e])
    y1 = c.y.clone()
    c.poison_outputs()
    c.schedule()
    c.forward()
    assert torch.equal(c.y, y1)


def test_mxfp4_backward_is_refused():
    from mixture_experts_layer_dispatch_amd import binding as B
    c = _case(SHAPES["tiny"])
    c.schedule()
    c.forward()
    with pytest.raises(B.MoEError) as ei:
        c.backward()
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED
