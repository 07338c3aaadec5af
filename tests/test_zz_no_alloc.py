"""The no-allocation schedule (moe_schedule_noalloc): its scratch lives in the
library's fixed device array, and its results must equal moe_schedule's with a
caller workspace bit for bit, on two calls in a row (the second with a
smaller input, so stale contents of the shared array would show)."""
import pytest
import torch

import synth_inputs as si
from gpu_cases import cfg_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(shape):
    from mixture_experts_layer_dispatch_amd import binding as B
    cfg = cfg_of(shape)
    logits = si.logits(shape, "cuda")
    ref = B.alloc_schedule(cfg)
    ws = B.alloc_workspace(cfg)
    B.moe_schedule(cfg, logits, ref, ws)
    got = {k: torch.full_like(v, -7) for k, v in ref.items()}
    B.moe_schedule_noalloc(cfg, logits, got)
    torch.cuda.synchronize()
    assert B.moe_check_device_error(ws) == 0
    return ref, got


def test_noalloc_schedule_equals_the_workspace_schedule():
    big = si.SHAPES["e512_t65536_zipf"]                 # 4 macrobatches x 4 minibatches
    small = si.custom_shape("ring_shared_na", T=512, H=128, I=128, E=16, k=4, seed=60,
                            macrobatch=128, minibatch=64)
    for shape in (big, small):                          # second call: a smaller input
        ref, got = _both(shape)
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"{shape.name}: {k}"
