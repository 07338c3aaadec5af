"""GPU parity of the MXFP8 path against the oracle's MXFP8 mode.

Quantised weights (codes and E8M0 scales, both orientations) must equal the
oracle's quantiser bit for bit; the layer's outputs must be within
3e-2 * max|ref| of the oracle run in MXFP8 mode (same quantisation rule, so
the tolerance covers only fp32 summation order, bf16 storage of o, dX and the
outputs, and the rare quantisation code that flips because a GPU operand
differs from the oracle's in the last fp32 bits).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_cases import Case, assert_close, assert_rerun_bitwise, f32, ring_samples

pytestmark = pytest.mark.gpu

MX_TOL = 3e-2

SHAPES = {
    "tiny": si.SHAPES["tiny"],
    "ragged": si.custom_shape("ragged_mx", T=100, H=256, I=256, E=7, k=3, seed=21),
    "ring_shared": si.custom_shape("ring_shared_mx", T=512, H=256, I=128, E=16, k=4, seed=22,
                                   n_shared=1, macrobatch=128, minibatch=64),
    # hot experts past one K step of the weight gradients (zipf), and experts
    # with many rows each (the 128-row weight-gradient slabs)
    "zipf_ring": si.custom_shape("zipf_ring_mx", T=1024, H=256, I=128, E=32, k=4, seed=23,
                                 macrobatch=256, minibatch=128, zipf=True),
    "dense_experts": si.custom_shape("dense_experts_mx", T=512, H=256, I=256, E=8, k=4, seed=24),
    # wider outputs: weight-gradient slabs of 8 and 16 column tiles (the
    # latter dealt over two blocks), and their fp32 accumulation across
    # macrobatches
    "stripes": si.custom_shape("stripes_mx", T=256, H=512, I=512, E=16, k=4, seed=25),
    "stripes_ring": si.custom_shape("stripes_ring_mx", T=512, H=512, I=1024, E=32, k=2, seed=26,
                                    n_shared=1, macrobatch=256, minibatch=128),
    # 128-row tiles with an odd number of 128-column tiles (the two-tile K
    # loops end on a single tile), for the routed experts and a dense shared
    # expert; their weight gradients take the deep kernels
    "odd_tiles": si.custom_shape("odd_tiles_mx", T=512, H=1152, I=384, E=4, k=2, seed=27,
                                 n_shared=1),
    # k = E (every token to every expert) and the largest k (32)
    "all_experts": si.custom_shape("all_experts_mx", T=96, H=128, I=128, E=4, k=4, seed=30),
    "max_k": si.custom_shape("max_k_mx", T=64, H=128, I=128, E=64, k=32, seed=31),
    "max_e": si.custom_shape("max_e_mx", T=256, H=128, I=128, E=1024, k=8, seed=33),
    "top1_ring": si.custom_shape("top1_ring_mx", T=512, H=256, I=256, E=8, k=1, seed=35,
                                 macrobatch=128, minibatch=64),
    # groups of ~256 rows over two macrobatches with a dense shared expert of
    # 512 rows: the gate/up GEMM's 256 x 256 tiles beside its 128-row tiles
    "big_tiles": si.custom_shape("big_tiles_mx", T=1024, H=512, I=256, E=4, k=2, seed=41,
                                 n_shared=1, macrobatch=512, minibatch=256),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class MXCase(Case):
    def __init__(self, shape, **kw):
        from mixture_experts_layer_dispatch_amd import binding as B
        super().__init__(shape, precision=B.PREC_MXFP8, **kw)


def _check_quantised(w_bf16, codes, scales, axis):
    """codes/scales from the GPU vs the oracle's quantiser of w along `axis`.
    The GPU's scales are K-step-major, [K/128, rows, 4]: scale (row r, block b)
    sits at [b // 4, r, b % 4]."""
    ref_c, ref_s = oracle.mx_quantize(f32(w_bf16).astype(np.float64), axis=axis)
    got_c, ks = codes.cpu().numpy(), scales.cpu().numpy()
    assert ks.ndim == 3 and ks.shape[1:] == (got_c.shape[0], 4) and ks.shape[0] * 128 == got_c.shape[1]
    got_s = ks.transpose(1, 0, 2).reshape(got_c.shape[0], got_c.shape[1] // 32)
    if axis == 0:                       # the GPU stores the transposed copy
        got_c, got_s = got_c.T, got_s.T
    np.testing.assert_array_equal(got_s, ref_s)
    np.testing.assert_array_equal(got_c, ref_c)


@pytest.mark.parametrize("name", list(SHAPES))
def test_weight_quantiser_bit_exact(name):
    c = MXCase(SHAPES[name], with_backward=False)
    torch.cuda.synchronize()
    for e in range(c.shape.E):
        _check_quantised(c.wg[e], c.wq["w_gate_q"][e], c.wq["w_gate_s"][e], 1)
        _check_quantised(c.wu[e], c.wq["w_up_q"][e], c.wq["w_up_s"][e], 1)
        _check_quantised(c.wd[e], c.wq["w_down_q"][e], c.wq["w_down_s"][e], 1)
        _check_quantised(c.wg[e], c.wq["w_gate_tq"][e], c.wq["w_gate_ts"][e], 0)
        _check_quantised(c.wu[e], c.wq["w_up_tq"][e], c.wq["w_up_ts"][e], 0)
        _check_quantised(c.wd[e], c.wq["w_down_tq"][e], c.wq["w_down_ts"][e], 0)
    if c.sw is not None:
        _check_quantised(c.sw[0], c.wq["s_gate_q"], c.wq["s_gate_s"], 1)
        _check_quantised(c.sw[2], c.wq["s_down_q"], c.wq["s_down_s"], 1)
        _check_quantised(c.sw[1], c.wq["s_up_tq"], c.wq["s_up_ts"], 0)


def test_quantiser_edge_values():
    """Saturation, ties, subnormals, zero blocks and huge blocks, element by element."""
    from mixture_experts_layer_dispatch_amd import binding as B
    shape = si.custom_shape("edge", T=8, H=128, I=128, E=1, k=1, seed=0)
    c = MXCase(shape, with_backward=False)
    vals = torch.tensor([0.0, -0.0, 1.0, 1.0625, 1.1875, 448.0, 464.0, 500.0, 2.0 ** -9,
                         2.0 ** -10, 3 * 2.0 ** -10, -1000.0, 2.0 ** 100, 2.0 ** -100, 7.0, 0.1],
                        dtype=torch.float32)
    w = torch.zeros(128, 128, dtype=torch.float32)
    w[:, :16] = vals                       # block 0 of every row mixes everything
    w[5] = 0.0                             # an all-zero row
    w[6, 32:64] = 2.0 ** -130              # a block far below 2^-127 (bf16 keeps it)
    w[7] *= -1
    wb = w.to(torch.bfloat16).cuda()
    weights = {"w_gate": wb[None].contiguous(), "w_up": wb[None].contiguous(),
               "w_down": wb[None].contiguous()}
    q = B.alloc_weights_mx(c.cfg)
    B.moe_quantize_weights_mxfp8(c.cfg, weights, q)
    torch.cuda.synchronize()
    _check_quantised(wb, q["w_gate_q"][0], q["w_gate_s"][0], 1)
    _check_quantised(wb, q["w_down_tq"][0], q["w_down_ts"][0], 0)


@pytest.mark.parametrize("name", list(SHAPES))
def test_forward_mx_small(name):
    c = MXCase(SHAPES[name], with_backward=False)
    c.schedule()
    idx, w, sch = c.oracle_schedule()
    c.forward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(c.ws) == 0
    ref = oracle.forward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd),
                         idx, w, shared=c.shared_np(), mx=True)
    assert_close("y (mxfp8)", f32(c.y), ref["y"], MX_TOL)
    rows = sch["row_of_slot"].reshape(c.shape.T, c.shape.k)
    assert_close("g (mxfp8)", f32(c.saved["g"])[rows], ref["g"], MX_TOL)
    assert_close("u (mxfp8)", f32(c.saved["u"])[rows], ref["u"], MX_TOL)
    # the quantisation is really applied: the bf16 oracle is measurably different
    exact = oracle.forward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu),
                           c.expert_view(c.wd), idx, w, shared=c.shared_np())["y"]
    assert np.max(np.abs(exact - ref["y"])) > 3 * np.max(np.abs(f32(c.y) - ref["y"]))


def test_forward_mx_full_size_sampled():
    c = MXCase(si.SHAPES["e512_t2048"], with_backward=False)
    c.schedule()
    c.forward()
    torch.cuda.synchronize()
    idx, w = oracle.route(f32(c.logits), c.shape.k)       # the oracle's own routing
    rng = np.random.default_rng(1)
    tokens = np.sort(rng.choice(c.shape.T, size=16, replace=False))
    ref = oracle.forward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd),
                         idx, w, tokens=tokens, mx=True)
    assert_close("y[sampled] (mxfp8)", f32(c.y)[tokens], ref["y"], MX_TOL)
    for e in (0, 511):
        _check_quantised(c.wg[e], c.wq["w_gate_q"][e], c.wq["w_gate_s"][e], 1)
        _check_quantised(c.wd[e], c.wq["w_down_tq"][e], c.wq["w_down_ts"][e], 0)


@pytest.mark.parametrize("name", list(SHAPES))
def test_backward_mx_small(name):
    c = MXCase(SHAPES[name])
    c.schedule()
    idx, w, sch = c.oracle_schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(c.ws) == 0
    E = c.shape.E
    ref = oracle.backward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd),
                          idx, w, f32(c.dy), shared=c.shared_np(), mx=True, sched=sch,
                          experts=list(range(E)))
    assert_close("dx (mxfp8)", f32(c.dx), ref["dx"], MX_TOL)
    assert_close("dw (mxfp8)", c.dw.cpu().numpy(), ref["dw"], MX_TOL)
    dl = oracle.ffn.d_logits_dense(idx, ref["dl_sel"], E)
    assert_close("d_logits (mxfp8)", c.dlogits.cpu().numpy(), dl, MX_TOL)
    zg = np.zeros((c.shape.I, c.shape.H))
    zd = np.zeros((c.shape.H, c.shape.I))
    assert_close("dW_gate (mxfp8)", f32(c.grads["d_w_gate"]),
                 np.stack([ref["dWg"].get(e, zg) for e in range(E)]), MX_TOL)
    assert_close("dW_up (mxfp8)", f32(c.grads["d_w_up"]),
                 np.stack([ref["dWu"].get(e, zg) for e in range(E)]), MX_TOL)
    assert_close("dW_down (mxfp8)", f32(c.grads["d_w_down"]),
                 np.stack([ref["dWd"].get(e, zd) for e in range(E)]), MX_TOL)
    if c.sw is not None:
        assert_close("dW_shared_gate (mxfp8)", f32(c.grads["d_s_gate"]), ref["dW_sg"], MX_TOL)
        assert_close("dW_shared_up (mxfp8)", f32(c.grads["d_s_up"]), ref["dW_su"], MX_TOL)
        assert_close("dW_shared_down (mxfp8)", f32(c.grads["d_s_down"]), ref["dW_sd"], MX_TOL)


def test_backward_mx_full_size_sampled():
    c = MXCase(si.SHAPES["e512_t2048"])
    c.schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(c.ws) == 0
    idx, w, sch = c.oracle_schedule()
    rng = np.random.default_rng(2)
    tokens = np.sort(rng.choice(c.shape.T, size=12, replace=False))
    experts = [int(idx[0, 0]), 300]
    rb = oracle.backward(f32(c.x), c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd),
                         idx, w, f32(c.dy), mx=True, sched=sch, tokens=tokens, experts=experts)
    assert_close("dx[sampled] (mxfp8)", f32(c.dx)[tokens], rb["dx"], MX_TOL)
    assert_close("dw[sampled] (mxfp8)", c.dw.cpu().numpy()[tokens], rb["dw"], MX_TOL)
    for e in experts:
        assert_close(f"dW_gate[{e}] (mxfp8)", f32(c.grads["d_w_gate"][e]), rb["dWg"][e], MX_TOL)
        assert_close(f"dW_up[{e}] (mxfp8)", f32(c.grads["d_w_up"][e]), rb["dWu"][e], MX_TOL)
        assert_close(f"dW_down[{e}] (mxfp8)", f32(c.grads["d_w_down"][e]), rb["dWd"][e], MX_TOL)
    assert_rerun_bitwise(c)


def test_forward_backward_mx_ring_full_size_sampled():
    """MXFP8 on the 65 536-token Zipf workload: four macrobatches, the shared
    expert, per-macrobatch 32-row blocks of the weight-gradient operands."""
    c = MXCase(si.SHAPES["e512_t65536_zipf"])
    c.schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(c.ws) == 0
    idx, w, sch = c.oracle_schedule()
    assert np.array_equal(c.sched["topk_idx"].cpu().numpy(), idx)
    tokens, experts = ring_samples(c, sch)
    x, dy = f32(c.x), f32(c.dy)
    wgv, wuv, wdv = c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd)
    ref = oracle.forward(x, wgv, wuv, wdv, idx, w, shared=c.shared_np(), tokens=tokens, mx=True)
    assert_close("y[sampled] (mxfp8)", f32(c.y)[tokens], ref["y"], MX_TOL)
    rb = oracle.backward(x, wgv, wuv, wdv, idx, w, dy, shared=c.shared_np(), mx=True, sched=sch,
                         tokens=tokens, experts=experts)
    assert_close("dx[sampled] (mxfp8)", f32(c.dx)[tokens], rb["dx"], MX_TOL)
    assert_close("dw[sampled] (mxfp8)", c.dw.cpu().numpy()[tokens], rb["dw"], MX_TOL)
    for e in experts:
        assert_close(f"dW_gate[{e}] (mxfp8)", f32(c.grads["d_w_gate"][e]), rb["dWg"][e], MX_TOL)
        assert_close(f"dW_up[{e}] (mxfp8)", f32(c.grads["d_w_up"][e]), rb["dWu"][e], MX_TOL)
        assert_close(f"dW_down[{e}] (mxfp8)", f32(c.grads["d_w_down"][e]), rb["dWd"][e], MX_TOL)
    assert_rerun_bitwise(c)


def test_forward_backward_mx_ep_share_full_size_sampled():
    """MXFP8 on one GPU's expert-parallel share (8 experts x 2560 rows, top-1)."""
    c = MXCase(si.SHAPES["e8_ep_share"])
    c.schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    from mixture_experts_layer_dispatch_amd import binding as B
    assert B.moe_check_device_error(c.ws) == 0
    idx, w, sch = c.oracle_schedule()
    assert np.array_equal(c.sched["topk_idx"].cpu().numpy(), idx)
    rng = np.random.default_rng(8)
    tokens = np.sort(rng.choice(c.shape.T, size=24, replace=False))
    x, dy = f32(c.x), f32(c.dy)
    wgv, wuv, wdv = c.expert_view(c.wg), c.expert_view(c.wu), c.expert_view(c.wd)
    ref = oracle.forward(x, wgv, wuv, wdv, idx, w, tokens=tokens, mx=True)
    assert_close("y[sampled] (mxfp8)", f32(c.y)[tokens], ref["y"], MX_TOL)
    rb = oracle.backward(x, wgv, wuv, wdv, idx, w, dy, mx=True, sched=sch, tokens=tokens,
                         experts=[0, 7])
    assert_close("dx[sampled] (mxfp8)", f32(c.dx)[tokens], rb["dx"], MX_TOL)
    assert_close("dw[sampled] (mxfp8)", c.dw.cpu().numpy()[tokens], rb["dw"], MX_TOL)
    for e in (0, 7):
        assert_close(f"dW_gate[{e}] (mxfp8)", f32(c.grads["d_w_gate"][e]), rb["dWg"][e], MX_TOL)
        assert_close(f"dW_up[{e}] (mxfp8)", f32(c.grads["d_w_up"][e]), rb["dWu"][e], MX_TOL)
        assert_close(f"dW_down[{e}] (mxfp8)", f32(c.grads["d_w_down"][e]), rb["dWd"][e], MX_TOL)


def _region(c, name, shape):
    from mixture_experts_layer_dispatch_amd import binding as B
    off, n = B.workspace_region(c.cfg, name)
    return c.ws[off:off + n].view(*shape).cpu().numpy()


def _check_activation_codes(c, which):
    """The E4M3 codes and E8M0 scales the path made of x (forward) or dy
    (backward), bit for bit against the oracle's quantiser of the same bf16
    rows along H."""
    src = c.x if which == "x" else c.dy
    T, H = c.shape.T, c.shape.H
    codes = _region(c, f"{which}_codes", (T, H))
    scales = _region(c, f"{which}_scales", (T, H // 32))
    ref_c, ref_s = oracle.mx_quantize(f32(src).astype(np.float64), axis=1)
    np.testing.assert_array_equal(scales, ref_s)
    np.testing.assert_array_equal(codes, ref_c)


def _check_wgrad_x_codes(c, experts=None):
    """The weight-gradient operand x (dW_gate, dW_up reduce over an expert's
    rows): each expert group's x rows, zero-padded to a multiple of 32 rows,
    quantised along the rows in 32-row blocks, stored transposed group after
    group; compared bit for bit with the oracle's quantiser of the same bf16
    rows (one macrobatch, no shared expert)."""
    idx, w, sch = c.oracle_schedule()
    assert sch["n_macro"] == 1 and c.shape.n_shared == 0
    E, H, k = c.shape.E, c.shape.H, c.shape.k
    counts, offsets = sch["counts"][0], sch["offsets"][0]
    nblk = -(-counts // 32)
    boff = np.concatenate([[0], np.cumsum(nblk)])
    np.testing.assert_array_equal(_region(c, "wgrad_block_offsets", (-1,)).view(np.int32), boff)
    codes = _region(c, "wgrad_x_codes", (-1,))
    scales = _region(c, "wgrad_x_scales", (-1,))
    x = f32(c.x).astype(np.float64)
    for e in (range(E) if experts is None else experts):
        n, npad = int(counts[e]), 32 * int(nblk[e])
        if n == 0:
            continue
        tok = sch["slot_of_row"][offsets[e]:offsets[e + 1]] // k
        xe = np.zeros((npad, H))
        xe[:n] = x[tok]
        rc, rs = oracle.mx_quantize(xe, axis=0)
        c0, s0 = 32 * int(boff[e]) * H, int(boff[e]) * H
        np.testing.assert_array_equal(codes[c0:c0 + H * npad].reshape(H, npad), rc.T, err_msg=f"expert {e}")
        np.testing.assert_array_equal(scales[s0:s0 + H * npad // 32].reshape(H, npad // 32), rs.T,
                                      err_msg=f"expert {e}")


@pytest.mark.parametrize("name", ["tiny", "ragged", "dense_experts", "stripes", "all_experts", "max_k",
                                  "max_e"])
def test_wgrad_operand_codes_bit_exact(name):
    c = MXCase(SHAPES[name])
    c.schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    _check_wgrad_x_codes(c)


def test_wgrad_operand_codes_bit_exact_full_size():
    c = MXCase(si.SHAPES["e512_t2048"])
    c.schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    _check_wgrad_x_codes(c, experts=[0, 1, 77, 300, 511])


@pytest.mark.parametrize("name", ["tiny", "ring_shared", "zipf_ring", "max_k"])
def test_activation_codes_bit_exact(name):
    """The dispatch gathers each routed row's codes from x quantised once per
    token, and the reverse-combine those of dy: both quantisations compared
    bit for bit with the oracle's (identical bf16 inputs on both sides)."""
    c = MXCase(SHAPES[name])
    c.schedule()
    c.forward()
    torch.cuda.synchronize()
    _check_activation_codes(c, "x")
    c.backward()
    torch.cuda.synchronize()
    _check_activation_codes(c, "dy")


def test_activation_codes_bit_exact_full_size():
    c = MXCase(si.SHAPES["e512_t2048"])
    c.schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    _check_activation_codes(c, "x")
    _check_activation_codes(c, "dy")
