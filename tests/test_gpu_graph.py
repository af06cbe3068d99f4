"""The whole layer (forward and backward) captured once in a HIP graph and
replayed: every call of the C ABI only enqueues work on its stream (no host
synchronisation, allocation or memset, the tile schedules built on the
device), so a capture of one pass replays it.  Each replay follows eager work
that overwrites every buffer of the layer and its workspace, and its outputs
must equal, bit for bit, those of the eager pass (the kernels use no atomics:
their results do not depend on timing).
"""
import pytest
import torch

import moe_inputs as mi
from mixture_experts_layer_limited_amd.layer import MoELayer

from harness import shape_of, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # DeepSeek-V3-like: sigmoid, groups, shared expert, skewed routing with empty experts
    mi.MoEConfig("graph_bf16", T=256, d=256, E=16, k=4, f=128, f_shared=128, score="sigmoid", n_group=4,
                 topk_group=2, scale=2.5, bias="zipf", backward=True, expert_std=0.05),
    # softmax with the aux loss, gates folded into act, act formed again in the backward
    mi.MoEConfig("graph_bf16_fold_recompute", T=192, d=256, E=8, k=2, f=256, aux_coeff=1e-3, backward=True,
                 expert_std=0.05, fold_gates=True, recompute_act=True),
    # microscaled expert GEMMs (weights quantised before the capture)
    mi.MoEConfig("graph_mxfp8", T=256, d=256, E=16, k=4, f=128, f_shared=128, score="sigmoid", n_group=4,
                 topk_group=2, scale=2.5, bias="zipf", backward=True, expert_std=0.05, dtype="mxfp8"),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_layer_pass_replays_from_a_graph(cfg):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print(f"\n[graph] {cfg.name}", flush=True)
    dev = to_dev(mi.make_inputs(cfg, seed=3))
    layer = MoELayer(shape_of(cfg), "cuda", backward=True)
    args = (dev["x"], dev["w_router"], dev["bias"], dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])

    def one_pass():
        layer.forward(*args)
        layer.backward(dev["dy"], dev["x"], dev["w_router"], dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])

    # eager pass: the reference (it also quantises microscaled weights and
    # sets every kernel's LDS limit, so the capture holds only kernel launches)
    one_pass()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in layer.buf.t.items() if v is not None}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    torch.cuda.synchronize()

    for replay in range(3):
        # eager work between replays: every buffer and the workspace overwritten
        for v in layer.buf.t.values():
            if v is not None:
                v.fill_(float("nan") if v.is_floating_point() else -7)
        layer.ws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, w in want.items():
            got = layer.buf.t[k]
            assert torch.equal(got, w), f"replay {replay}: {k} differs from the eager pass"
