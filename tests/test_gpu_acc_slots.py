"""The weight-gradient running sums of a macrobatch stream, kept only for the
experts that take rows from several macrobatches (moe_config.acc_experts).

With exactly as many accumulator slots as such experts, every output is bit
for bit the one of the full-size accumulator (the slots change where a sum is
kept, not how it is formed); with one slot fewer the layer raises the
capacity bit of the device error word, and nothing faults."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_cases import Case
from mixture_experts_layer_dispatch_amd import binding as B

pytestmark = pytest.mark.gpu

SHAPES = {
    "zipf_ring": si.custom_shape("zipf_ring_acc", T=1024, H=128, I=128, E=32, k=4, seed=15,
                                 macrobatch=256, minibatch=128, zipf=True),
    # a shared expert, whose dense gradient keeps its own running sum, and
    # wider outputs (weight-gradient slabs dealt over several blocks)
    "zipf_shared": si.custom_shape("zipf_shared_acc", T=1024, H=512, I=256, E=64, k=2, seed=16,
                                   n_shared=1, macrobatch=256, minibatch=128, zipf=True),
}


def spanning_experts(shape) -> int:
    """Experts with rows in at least two macrobatches, from the oracle's routing."""
    idx, _ = oracle.route(si.logits(shape).numpy(), shape.k)
    sch = oracle.schedule(idx, shape.E, shape.macrobatch, shape.minibatch)
    return int(((sch["counts"] > 0).sum(0) >= 2).sum())


def run(shape, precision, acc_experts):
    c = Case(shape, precision=precision, acc_experts=acc_experts)
    c.schedule()
    c.forward()
    c.backward()
    torch.cuda.synchronize()
    return c


def outputs(c):
    out = {"y": c.y, "dx": c.dx, "dw": c.dw, "d_logits": c.dlogits}
    out.update(c.grads)
    return out


@pytest.mark.parametrize("precision", [B.PREC_BF16, B.PREC_MXFP8])
@pytest.mark.parametrize("name", list(SHAPES))
def test_slots_for_spanning_experts_only_match_the_full_accumulator(name, precision):
    shape = SHAPES[name]
    need = spanning_experts(shape)
    assert 0 < need < shape.E                      # the shapes exercise a real subset
    full = run(shape, precision, 0)
    assert B.moe_check_device_error(full.ws) == 0
    part = run(shape, precision, need)
    assert B.moe_check_device_error(part.ws) == 0
    assert B.workspace_size(part.cfg) < B.workspace_size(full.cfg)
    a, b = outputs(full), outputs(part)
    for k in a:
        assert torch.equal(a[k], b[k]), f"{k} differs with {need} accumulator slots"


@pytest.mark.parametrize("precision", [B.PREC_BF16, B.PREC_MXFP8])
def test_too_few_slots_raise_the_capacity_bit(precision):
    shape = SHAPES["zipf_ring"]
    need = spanning_experts(shape)
    c = run(shape, precision, need - 1)
    assert B.moe_check_device_error(c.ws) == B.DEVERR_ACC_CAPACITY


def test_full_size_zipf_stream_with_content_sized_accumulators():
    """The 65 536-token Zipf stream (4 macrobatches, shared expert): the
    accumulators sized for the experts that span macrobatches (a few dozen of
    512) give the same bits as the full-size ones."""
    shape = si.SHAPES["e512_t65536_zipf"]
    need = spanning_experts(shape)
    assert need < shape.E // 4
    part = run(shape, B.PREC_BF16, need)
    assert B.moe_check_device_error(part.ws) == 0
    got = {k: v.clone() for k, v in outputs(part).items()}
    small = B.workspace_size(part.cfg)
    del part
    torch.cuda.empty_cache()
    full = run(shape, B.PREC_BF16, 0)
    assert B.moe_check_device_error(full.ws) == 0
    assert small < B.workspace_size(full.cfg) - 8 * 1024 ** 3
    for k, v in outputs(full).items():
        assert torch.equal(got[k], v), f"{k} differs with {need} accumulator slots"
