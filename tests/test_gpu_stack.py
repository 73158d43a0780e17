"""A model-shaped stack: several layers back to back through one workspace
(page "MoE Execution Path Analysis": per-step launches and allocations over
the model's layers, intermediates allocated once), eagerly and replayed as a
HIP graph.

* The stack gives bit-for-bit the outputs of the same layers called one by
  one with fresh workspaces and outputs (reuse leaks nothing between layers).
* A step allocates no device memory and queues the launches its dispatch
  readout reports.
* The last layer, given the GPU's own input to it, matches the oracle.
* With the residual stream, the deepest layer still routes over many
  experts.
* A captured step replayed several times, with other eager work in between,
  reproduces the eager step bit for bit each time.
"""

from __future__ import annotations

import numpy as np
import pytest

import moe_workloads as wl
from oracle import moe_oracle as mo
from tests import helpers as h

pytestmark = pytest.mark.gpu

NLAYERS = 4


def _moe():
    import mixture_experts_ffn_renorm_amd as moe
    return moe


def make_stack(name: str, M: int, n: int = NLAYERS, first: int = 1, residual: bool = True):
    from mixture_experts_ffn_renorm_amd.stack import MoEStack
    shape = wl.WORKLOADS[name]
    layers = [wl.make_device_layer(shape, M, layer=first + i, device="cuda") for i in range(n)]
    return MoEStack(layers, shape.top_k, M, shape.renormalize, residual=residual), shape, layers


def draw_x(M: int, H: int, seed: int):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((M, H), generator=g, device="cuda").to(torch.bfloat16)


def bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("residual", [True, False])
@pytest.mark.parametrize("M", [4, 64])
def test_stack_equals_layer_by_layer(M, residual):
    import torch
    moe = _moe()
    stack, shape, layers = make_stack("qwen3_decode", M, residual=residual)
    x = draw_x(M, shape.H, 7)
    y = bits(stack.step(x))
    torch.cuda.synchronize()
    src = x.clone()
    for lay in layers:
        out, _ = moe.moe_forward(src, lay["w_router"], lay["w13"], lay["w2"], shape.top_k,
                                 shape.renormalize, logit_bias=lay["logit_bias"])
        src = src + out if residual else out
    torch.cuda.synchronize()
    assert np.array_equal(y, bits(src))


def test_stack_residual_keeps_routing_spread():
    """With the residual stream the deepest layer still spreads its tokens
    over many experts (without it, shrinking activations tie the logits)."""
    import torch
    M = 64
    stack, shape, _ = make_stack("qwen3_decode", M)
    stack.step(draw_x(M, shape.H, 11))
    torch.cuda.synchronize()
    touched = torch.unique(stack.topk_ids[-1][:M]).numel()
    assert touched >= shape.E // 2


@pytest.mark.parametrize("M,per_layer", [(4, 4), (64, 5)])
def test_stack_allocates_nothing_and_counts_launches(M, per_layer):
    import torch
    moe = _moe()
    stack, shape, _ = make_stack("qwen3_decode", M)
    x = draw_x(M, shape.H, 8)
    stack.step(x)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    stack.step(x)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert stack.last_launches == NLAYERS * per_layer
    assert all(i["launches"] == per_layer for i in stack.last_infos)
    want = moe.MOE_VARIANT_PAIR_GEMV if M * shape.top_k * 4 <= shape.E else moe.MOE_VARIANT_STREAM
    assert all(i["variant"] == want for i in stack.last_infos)


def test_stack_last_layer_matches_oracle():
    """Without the residual: layer 1's input is layer 0's output (the other
    ping-pong buffer) and its output is the step's result."""
    import torch
    M = 64
    stack, shape, layers = make_stack("qwen3_decode", M, n=2, residual=False)
    x = draw_x(M, shape.H, 9)
    y = stack.step(x)
    torch.cuda.synchronize()
    x_last = stack.bufs[0][:M]
    lay = layers[-1]
    host = dict(x=bits(x_last).view(np.uint16), w_router=bits(lay["w_router"]).view(np.uint16),
                w13=bits(lay["w13"]).view(np.uint16), w2=bits(lay["w2"]).view(np.uint16),
                logit_bias=None, M=M, E=shape.E, top_k=shape.top_k, H=shape.H, I=shape.I,
                renormalize=shape.renormalize)
    toks = h.sample_tokens(M, 16, 3)
    r = mo.route(host["x"][toks], host["w_router"], shape.top_k, shape.renormalize, None)
    ids = stack.topk_ids[-1][:M].cpu().numpy()
    wts = stack.topk_weights[-1][:M].cpu().numpy().astype(np.float64)
    w_ref = h.check_routing(ids[toks], wts[toks], r, shape.renormalize)
    full_ids, full_w = h.scatter_routing(M, toks, ids[toks], w_ref)
    ref_y = mo.layer_forward(host["x"], host["w13"], host["w2"], full_ids, full_w, toks)
    got = h.host_bf16_to_f64(y)[toks]
    h.assert_close_outputs(got, ref_y, "last layer")


@pytest.mark.parametrize("name,M", [("qwen3_decode", 2), ("qwen3_decode", 16),
                                    ("qwen15", 512), ("qwen15", 2048)])
def test_stack_graph_replay_matches_eager(name, M):
    """Per-pair GEMVs, streaming kernels with the fused top-k + lists, and the
    tiled kernels with the multi-workgroup align (M = 2048: 8192 pairs)."""
    import torch
    stack, shape, layers = make_stack(name, M, n=3 if M <= 16 else 2)
    from mixture_experts_ffn_renorm_amd.stack import MoEStack
    ref_stack = MoEStack(layers, shape.top_k, M, shape.renormalize)
    inputs = [draw_x(M, shape.H, 20 + r) for r in range(3)]
    refs = [bits(ref_stack.step(xr)) for xr in inputs]
    torch.cuda.synchronize()
    x_static = torch.empty_like(inputs[0])
    x_static.copy_(inputs[0])
    graph, out = stack.capture(x_static)
    for r in range(3):
        x_static.copy_(inputs[r])
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), refs[r]), f"replay {r}"
        # eager work of the program between replays (another stack's step)
        ref_stack.step(inputs[(r + 1) % 3])
        torch.cuda.synchronize()
