"""No host synchronisation in the layer's calls: moe_schedule, moe_forward and
moe_backward enqueue kernels only (no copy to the host, no wait, no memset,
no allocation), so the three can be captured into one HIP graph and replayed
(arex-research.com "Cursor 放出 MoK", design section, second decision: the
ring buffer removes every CPU-GPU synchronisation from the layer).

Each case runs the step eagerly, captures it on a side stream, then replays
the graph three times.  Before every replay all outputs and the workspace are
poisoned by ordinary eager work on the default stream; every replay must
reproduce the eager outputs bit for bit."""
import pytest
import torch

import synth_inputs as si
from gpu_cases import Case

pytestmark = pytest.mark.gpu

CASES = [
    ("ring_shared", "bf16", False),
    ("ring_shared", "mxfp8", False),
    ("ring_shared", "bf16", True),
    ("ring_shared", "mxfp8", True),
    ("e512_t2048", "bf16", False),
    ("e512_t2048", "mxfp8", False),
]


def _shape(name):
    if name == "ring_shared":
        return si.custom_shape("ring_shared_graph", T=512, H=256, I=128, E=16, k=4, seed=50,
                               n_shared=1, macrobatch=128, minibatch=64)
    return si.SHAPES[name]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(c):
    out = {"y": c.y, "dx": c.dx, "dw": c.dw, "d_logits": c.dlogits}
    out.update(c.grads)
    out.update({"sched_" + k: v for k, v in c.sched.items()})
    return out


@pytest.mark.parametrize("name,prec,recompute", CASES)
def test_step_captured_in_a_graph_replays_bitwise(name, prec, recompute):
    from mixture_experts_layer_dispatch_amd import binding as B
    p = B.PREC_MXFP8 if prec == "mxfp8" else B.PREC_BF16
    c = Case(_shape(name), precision=p, recompute=recompute)

    def step():
        c.schedule()
        c.forward()
        c.backward()

    step()                                   # eager, allocates the outputs
    torch.cuda.synchronize()
    assert B.moe_check_device_error(c.ws) == 0
    eager = {k: v.clone() for k, v in _outputs(c).items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # a warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        c.poison_outputs()                   # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in _outputs(c).items():
            assert torch.equal(v, eager[k]), f"replay {r}: {k} differs from the eager run"
    del graph
