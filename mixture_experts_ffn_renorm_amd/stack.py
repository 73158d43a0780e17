"""Many MoE layers back to back through one workspace, eagerly or as one
replayed HIP graph.

Page "MoE Execution Path Analysis" counts, per decode step of a model, the
MoE layer's launches and allocations over all of the model's layers, and
asks ("What we can actually change") for intermediates allocated once and
reused.  :class:`MoEStack` allocates everything when it is built -- one
workspace sized for the largest batch, a residual-stream buffer, the MoE
output buffer and the per-layer routing outputs -- so a step allocates
nothing.  Only MoE layers are stacked (no attention or norms): the stack
exists to run and measure the layer at model scale.  Between layers the
model's residual connection keeps the stream at its scale (r <- r + y_l, one
in-place torch add -- the model's glue, not a step of the MoE layer);
without it a SwiGLU-only stack shrinks its activations several-fold per
layer until every token's router logits tie and all tokens pick the same few
experts.  ``residual=False`` chains the layers directly (y_l feeds layer
l + 1).  A step can be recorded once into a HIP graph
(``torch.cuda.CUDAGraph``) and replayed, which removes the host's per-launch
cost.

Orchestration only: every layer is one ``moe_forward`` call of the C ABI.
"""

from __future__ import annotations

from typing import Sequence

from . import moe_forward, workspace


class MoEStack:
    """``layers``: sequence of dicts with device tensors ``w_router`` [E, H],
    ``w13`` [E, 2I, H], ``w2`` [E, H, I] (bf16) and ``logit_bias`` ([E] fp32
    or None), all of one shape.  ``M_max``: the largest batch a step takes."""

    def __init__(self, layers: Sequence[dict], top_k: int, M_max: int,
                 renormalize: bool = True, residual: bool = True, device=None):
        import torch

        if len(layers) == 0:
            raise ValueError("a stack needs at least one layer")
        E, two_i, H = layers[0]["w13"].shape
        for lay in layers:
            if tuple(lay["w13"].shape) != (E, two_i, H) or \
                    tuple(lay["w2"].shape) != (E, H, two_i // 2) or \
                    tuple(lay["w_router"].shape) != (E, H):
                raise ValueError("every layer of a stack must have the same shape")
        self.layers = list(layers)
        self.top_k, self.M_max, self.renormalize = top_k, M_max, renormalize
        self.residual = residual
        self.E, self.H, self.I = E, H, two_i // 2
        device = device or layers[0]["w13"].device
        self.ws = workspace(M_max, E, top_k, H, self.I, device)
        # residual: bufs[0] is the stream, bufs[1] the MoE output; otherwise
        # the two are ping-pong outputs
        self.bufs = [torch.empty((M_max, H), dtype=torch.bfloat16, device=device)
                     for _ in range(2)]
        self.topk_ids = [torch.empty((M_max, top_k), dtype=torch.int32, device=device)
                         for _ in self.layers]
        self.topk_weights = [torch.empty((M_max, top_k), dtype=torch.float32, device=device)
                             for _ in self.layers]
        self.last_launches = 0
        self.last_infos: list = []

    def step(self, x, stream=None):
        """Run every layer on x [M, H] bf16 (M <= M_max); returns the final
        residual stream (or, without the residual, the last layer's output),
        a view of one of the stack's own buffers, valid until the next step.
        MoE kernel launches of the step: ``last_launches`` (the residual adds
        are one more torch launch per layer, plus the initial copy)."""
        import torch

        M = x.shape[0]
        if M > self.M_max:
            raise ValueError(f"batch of {M} tokens exceeds the stack's M_max {self.M_max}")
        launches = 0
        infos = []
        if self.residual:
            stream_buf, y = self.bufs[0][:M], self.bufs[1][:M]
            ctx = torch.cuda.stream(stream) if stream is not None else _null()
            with ctx:
                stream_buf.copy_(x)
            src = stream_buf
        else:
            src = x
        for l, lay in enumerate(self.layers):
            dst = y if self.residual else self.bufs[l % 2][:M]
            _, info = moe_forward(src, lay["w_router"], lay["w13"], lay["w2"], self.top_k,
                                  self.renormalize, logit_bias=lay.get("logit_bias"), out=dst,
                                  topk_ids_out=self.topk_ids[l][:M],
                                  topk_weights_out=self.topk_weights[l][:M], ws=self.ws,
                                  stream=stream)
            launches += info["launches"]
            infos.append(info)
            if self.residual:
                with (torch.cuda.stream(stream) if stream is not None else _null()):
                    stream_buf.add_(y)
            else:
                src = dst
        self.last_launches = launches
        self.last_infos = infos
        return src

    def capture(self, x_static, warmup: int = 1):
        """Record one step on x_static into a HIP graph.  Returns (graph,
        out): ``graph.replay()`` reruns the step on whatever x_static then
        holds and leaves the result in ``out``."""
        import torch

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):   # library attributes are set outside the capture
                self.step(x_static)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            out = self.step(x_static)
        return graph, out


class _null:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


__all__ = ["MoEStack"]
