"""Seeded synthetic inputs for one mixture-of-experts SwiGLU layer forward.

This module only draws random numbers, rounds them to bf16 and names the
workload shapes.  It holds none of the layer's arithmetic, so both the CPU
oracle (``oracle/``) and the HIP path's tests and benchmark can take their
inputs from it without sharing any of the method's code.

Shapes follow the pages this project builds from:
  * "Mixture of Experts in vLLM -- From First Principles to fused_moe",
    section "One expert, and one token": x has H values, the stacked gate/up
    matrix W13 is [2I, H] (gate rows first), the down matrix W2 is [H, I],
    the router W_r is [E, H].
  * same page, "A batch: (token, expert) pairs": the toy batch has M=3
    tokens, 4 experts and top_k=2.
  * "MoE Execution Path Analysis", "The Real Bottleneck": 256 experts with
    top-8 routing (the wide layer below keeps that routing shape).

Value distributions (readings of the pages where they leave details open):
  x ~ N(0, 1); W13 ~ N(0, 1/H) and W2 ~ N(0, 1/I) (variance 1/fan-in);
  W_r ~ N(0, 0.02^2) for the model-shaped layers and N(0, 1/H) for the toy.
  Every tensor is drawn in float32 and rounded once, round-to-nearest-even,
  to bf16; all consumers see the same bf16 bit patterns.
  The skewed prefill layer adds a Zipf(s=1.1) prior to the router logits:
  bias[e] = -1.1 * ln(rank[e]) with rank a seeded permutation of 1..E.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

SEED_BASE = 20261202


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    index: int          # position in the workload list; enters the seed
    E: int              # experts
    top_k: int          # experts per token
    H: int              # hidden size (GEMM 1 K, GEMM 2 N)
    I: int              # expert intermediate size (GEMM 2 K)
    Ms: tuple           # token counts exercised for this shape
    router_std: Optional[float]   # None -> 1/sqrt(H)
    zipf_s: Optional[float] = None
    renormalize: bool = True
    description: str = ""


WORKLOADS = {
    "toy": LayerShape(
        "toy", 0, E=4, top_k=2, H=64, I=32, Ms=(3,), router_std=None,
        description="toy layer: M=3, E=4, top_k=2, H=64, I=32"),
    "qwen3_decode": LayerShape(
        "qwen3_decode", 1, E=128, top_k=8, H=2048, I=768, Ms=(1, 2, 8, 16, 64),
        router_std=0.02,
        description="Qwen3-30B-A3B-shaped MoE layer, decode batches M=1..64"),
    "qwen3_prefill": LayerShape(
        "qwen3_prefill", 2, E=128, top_k=8, H=2048, I=768, Ms=(4096,),
        router_std=0.02, zipf_s=1.1,
        description="Qwen3-30B-A3B-shaped MoE layer, prefill M=4096, "
                    "Zipf(1.1)-biased router"),
    "qwen15": LayerShape(
        "qwen15", 3, E=60, top_k=4, H=2048, I=1408, Ms=(1, 16, 512, 2048),
        router_std=0.02,
        description="Qwen1.5-MoE-A2.7B-shaped MoE layer (down-proj K=1408)"),
    "wide256": LayerShape(
        "wide256", 4, E=256, top_k=8, H=2048, I=512, Ms=(1, 8, 8192),
        router_std=0.02,
        description="256-expert wide layer, top-8"),
}


def seed_for(shape: LayerShape, M: int, layer: int = 0) -> int:
    """Seed of one synthetic layer; ``layer`` > 0 names extra timing layers."""
    return SEED_BASE + 100 * shape.index + M + 1_000_003 * layer


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16.  Inputs here are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16_into(out: np.ndarray, seq: np.random.SeedSequence,
                     std: float) -> None:
    """Fill ``out`` (uint16) with bf16(N(0, std^2)) drawn from stream ``seq``."""
    rng = np.random.Generator(np.random.PCG64(seq))
    v = rng.standard_normal(out.shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    u = v.view(np.uint32)
    u += ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    u >>= np.uint32(16)
    out[...] = u


def make_layer(shape: LayerShape | str, M: int, layer: int = 0,
               E: Optional[int] = None, top_k: Optional[int] = None,
               H: Optional[int] = None, I: Optional[int] = None,
               seed: Optional[int] = None) -> dict:
    """Draw one synthetic MoE layer and a batch of M tokens.

    Returns a dict with numpy arrays
      x          uint16 [M, H]       bf16 bits
      w_router   uint16 [E, H]       bf16 bits
      w13        uint16 [E, 2I, H]   bf16 bits, gate rows 0..I-1, up rows I..2I-1
      w2         uint16 [E, H, I]    bf16 bits
      logit_bias float32 [E] or None
    and the scalars M, E, top_k, H, I, renormalize.
    E/top_k/H/I may be overridden to make small cases of the same recipe.
    Streams: numpy SeedSequence(seed).spawn(2 + 2E + 1) gives one PCG64
    stream each to x, W_r, W13[e] (e = 0..E-1), W2[e], and the Zipf rank
    permutation, in that order; tensors are independent of thread order.
    """
    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    E = shape.E if E is None else E
    top_k = shape.top_k if top_k is None else top_k
    H = shape.H if H is None else H
    I = shape.I if I is None else I
    seqs = np.random.SeedSequence(
        seed_for(shape, M, layer) if seed is None else seed).spawn(2 + 2 * E + 1)
    rstd = shape.router_std if shape.router_std is not None else 1.0 / math.sqrt(H)
    x = np.empty((M, H), dtype=np.uint16)
    w_router = np.empty((E, H), dtype=np.uint16)
    w13 = np.empty((E, 2 * I, H), dtype=np.uint16)
    w2 = np.empty((E, H, I), dtype=np.uint16)
    jobs = [(x, seqs[0], 1.0), (w_router, seqs[1], rstd)]
    jobs += [(w13[e], seqs[2 + e], 1.0 / math.sqrt(H)) for e in range(E)]
    jobs += [(w2[e], seqs[2 + E + e], 1.0 / math.sqrt(I)) for e in range(E)]
    workers = max(1, min(16, os.cpu_count() or 1))
    if workers == 1 or w13.size < (1 << 20):
        for job in jobs:
            _normal_bf16_into(*job)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda j: _normal_bf16_into(*j), jobs))
    bias = None
    if shape.zipf_s is not None:
        rank = np.random.Generator(np.random.PCG64(seqs[-1])).permutation(E) + 1
        bias = (-shape.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    return dict(x=x, w_router=w_router, w13=w13, w2=w2, logit_bias=bias,
                M=M, E=E, top_k=top_k, H=H, I=I,
                renormalize=shape.renormalize, name=shape.name)


def make_topk_ids(M: int, top_k: int, E: int, seed: int,
                  pattern: str = "random") -> np.ndarray:
    """Synthetic expert choices [M, top_k] int32 for testing the align step.

    Patterns: "random" (distinct ids per token, uniform), "one_expert_heavy"
    (every token takes expert 0 in some slot), "round_robin"
    (token t takes experts (t*top_k + j) mod E), "sparse" (only a few
    experts are ever chosen, so most experts are empty).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = np.empty((M, top_k), dtype=np.int32)
    if pattern == "round_robin":
        for t in range(M):
            ids[t] = (t * top_k + np.arange(top_k)) % E
        return ids
    if pattern == "sparse":
        pool = rng.choice(E, size=min(E, max(top_k, 2 * top_k)), replace=False)
        for t in range(M):
            ids[t] = rng.choice(pool, size=top_k, replace=False)
        return ids
    for t in range(M):
        ids[t] = rng.choice(E, size=top_k, replace=False)
    if pattern == "one_expert_heavy":
        for t in range(M):
            if 0 not in ids[t]:
                ids[t, rng.integers(top_k)] = 0
    return ids


def make_device_layer(shape: LayerShape | str, M: int, layer: int, device,
                      E: Optional[int] = None, I: Optional[int] = None):
    """Draw the weights of one extra timing layer directly in device memory.

    Same distributions as :func:`make_layer` but drawn with torch's seeded
    generator on the device (a different stream of numbers), so a benchmark
    can cycle through many distinct layers without host-side generation.
    Returns a dict of torch tensors (bf16) w_router, w13, w2 and logit_bias.
    """
    import torch  # local import: the oracle side never needs torch

    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    E = shape.E if E is None else E
    I = shape.I if I is None else I
    H = shape.H
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(shape, M, layer))
    rstd = shape.router_std if shape.router_std is not None else 1.0 / math.sqrt(H)

    def draw(sz, std):
        t = torch.randn(sz, generator=g, device=device, dtype=torch.float32)
        t.mul_(std)
        return t.to(torch.bfloat16)

    w_router = draw((E, H), rstd)
    w13 = draw((E, 2 * I, H), 1.0 / math.sqrt(H))
    w2 = draw((E, H, I), 1.0 / math.sqrt(I))
    bias = None
    if shape.zipf_s is not None:
        rank = torch.randperm(E, generator=g, device=device).to(torch.float64) + 1
        bias = (-shape.zipf_s * torch.log(rank)).to(torch.float32)
    return dict(w_router=w_router, w13=w13, w2=w2, logit_bias=bias)


# ---------------------------------------------------------------------------
# group-quantized expert weights (affine, 64-element groups, 4 or 8 bits)
# ---------------------------------------------------------------------------

QUANT_GROUP = 64


def _pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [..., K] (K a multiple of 32 / bits) into uint32 words,
    element i of a row at bits [bits * (i % per), ...) of word i // per."""
    per = 32 // bits
    c = np.asarray(codes, dtype=np.uint32).reshape(*codes.shape[:-1], codes.shape[-1] // per, per)
    words = np.zeros(c.shape[:-1], dtype=np.uint32)
    for i in range(per):
        words |= c[..., i] << np.uint32(bits * i)
    return words


def _quantized_matrix(rows: int, K: int, bits: int, seq: np.random.SeedSequence):
    """Random codes, scales and biases of one expert matrix [rows, K]: codes
    uniform over [0, 2^bits); per 64-element group a scale and bias (bf16)
    that map the code range onto about [-a, a] with a = sqrt(3 / K) (a
    variance near 1/K, like the bf16 layers), each jittered by 10 %."""
    rng = np.random.Generator(np.random.PCG64(seq))
    codes = rng.integers(0, 1 << bits, size=(rows, K), dtype=np.uint32)
    ng = K // QUANT_GROUP
    a = math.sqrt(3.0 / K)
    s = (2.0 * a / ((1 << bits) - 1)) * (1.0 + 0.1 * rng.standard_normal((rows, ng)))
    b = -a * (1.0 + 0.1 * rng.standard_normal((rows, ng)))
    return (_pack_codes(codes, bits), f32_to_bf16_bits(s.astype(np.float32)),
            f32_to_bf16_bits(b.astype(np.float32)))


def make_quantized_layer(shape: LayerShape | str, M: int, bits: int, layer: int = 0,
                         E: Optional[int] = None, top_k: Optional[int] = None,
                         H: Optional[int] = None, I: Optional[int] = None,
                         seed: Optional[int] = None) -> dict:
    """One synthetic layer with group-quantized expert weights.

    x, w_router (bf16) and the Zipf prior are drawn as by :func:`make_layer`;
    W13 [E, 2I, H] and W2 [E, H, I] come as packed codes
    (``w13_q`` [E, 2I, H*bits/32] uint32), ``*_scales`` and ``*_biases``
    [E, rows, K/64] (bf16 bits).  H and I must be multiples of 64.
    """
    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    E = shape.E if E is None else E
    top_k = shape.top_k if top_k is None else top_k
    H = shape.H if H is None else H
    I = shape.I if I is None else I
    if H % QUANT_GROUP or I % QUANT_GROUP:
        raise ValueError("H and I must be multiples of 64")
    base = seed_for(shape, M, layer) + 7919 * bits if seed is None else seed
    seqs = np.random.SeedSequence(base).spawn(2 + 2 * E + 1)
    rstd = shape.router_std if shape.router_std is not None else 1.0 / math.sqrt(H)
    x = np.empty((M, H), dtype=np.uint16)
    w_router = np.empty((E, H), dtype=np.uint16)
    _normal_bf16_into(x, seqs[0], 1.0)
    _normal_bf16_into(w_router, seqs[1], rstd)
    w13 = [_quantized_matrix(2 * I, H, bits, seqs[2 + e]) for e in range(E)]
    w2 = [_quantized_matrix(H, I, bits, seqs[2 + E + e]) for e in range(E)]
    bias = None
    if shape.zipf_s is not None:
        rank = np.random.Generator(np.random.PCG64(seqs[-1])).permutation(E) + 1
        bias = (-shape.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    return dict(x=x, w_router=w_router, logit_bias=bias,
                w13_q=np.stack([m[0] for m in w13]), w13_scales=np.stack([m[1] for m in w13]),
                w13_biases=np.stack([m[2] for m in w13]),
                w2_q=np.stack([m[0] for m in w2]), w2_scales=np.stack([m[1] for m in w2]),
                w2_biases=np.stack([m[2] for m in w2]),
                M=M, E=E, top_k=top_k, H=H, I=I, bits=bits,
                renormalize=shape.renormalize, name=shape.name)


def make_device_quantized_layer(shape: LayerShape | str, M: int, bits: int, layer: int,
                                device) -> dict:
    """Draw one extra timing layer with group-quantized expert weights
    directly in device memory: uniformly random code words (int32), and per
    64-element group scales and biases drawn as by :func:`make_quantized_layer`
    (bf16), with torch's seeded generator on the device.  Returns a dict of
    torch tensors w_router, logit_bias and the ``moe_forward_quantized``
    weight dict under ``q``."""
    import torch  # local import: the oracle side never needs torch

    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    E, H, I = shape.E, shape.H, shape.I
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(shape, M, layer) + 7919 * bits)
    rstd = shape.router_std if shape.router_std is not None else 1.0 / math.sqrt(H)
    w_router = (torch.randn((E, H), generator=g, device=device) * rstd).to(torch.bfloat16)
    q = {"bits": bits}
    for name, rows, K in (("w13", 2 * I, H), ("w2", H, I)):
        q[name + "_q"] = torch.randint(-2 ** 31, 2 ** 31 - 1, (E, rows, K * bits // 32),
                                       generator=g, device=device, dtype=torch.int32)
        a = math.sqrt(3.0 / K)
        jit = torch.randn((2, E, rows, K // QUANT_GROUP), generator=g, device=device)
        q[name + "_scales"] = ((2.0 * a / ((1 << bits) - 1)) * (1.0 + 0.1 * jit[0])).to(
            torch.bfloat16)
        q[name + "_biases"] = (-a * (1.0 + 0.1 * jit[1])).to(torch.bfloat16)
    bias = None
    if shape.zipf_s is not None:
        rank = torch.randperm(E, generator=g, device=device).to(torch.float64) + 1
        bias = (-shape.zipf_s * torch.log(rank)).to(torch.float32)
    return dict(w_router=w_router, logit_bias=bias, q=q)


MX_BLOCK = 32


# E4M3 codes other than the two NaN codes (0x7F, 0xFF): zero and negative
# zero, the subnormals, every exponent field 1..15 and +-448, in code order.
MX_FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def mx_code_rms() -> float:
    """Root mean square of the E4M3 values when the code is uniform over
    MX_FINITE_CODES (codes decoded from their bit fields: bias 7, exponent 0
    subnormal with steps of 2^-9)."""
    c = MX_FINITE_CODES.astype(np.int64)
    e, m = (c >> 3) & 0xF, (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return float(np.sqrt(np.mean(mag * mag)))


def mx_scale_base(K: int) -> int:
    """E8M0 code that gives weights of uniform random finite codes a spread
    near 1/sqrt(K): 127 + round(log2(1 / (rms * sqrt(K))))."""
    return 127 + int(round(math.log2(1.0 / (mx_code_rms() * math.sqrt(K)))))


def _mx_matrix(rows: int, K: int, seq: np.random.SeedSequence):
    """Random MXFP8 codes and scales of one expert matrix [rows, K]: E4M3
    bytes uniform over every finite code (zeros, subnormals, all exponent
    fields, +-448; no NaN), and per 32-element block an E8M0 scale
    mx_scale_base(K) + {-1, 0, 1}, so that the weights spread near
    1/sqrt(K) with the heavy tail of the full E4M3 range."""
    rng = np.random.Generator(np.random.PCG64(seq))
    codes = MX_FINITE_CODES[rng.integers(0, MX_FINITE_CODES.size, size=(rows, K))]
    scales = (mx_scale_base(K) + rng.integers(-1, 2, size=(rows, K // MX_BLOCK))).astype(np.uint8)
    return codes, scales


def make_mx_layer(shape: LayerShape | str, M: int, layer: int = 0,
                  E: Optional[int] = None, top_k: Optional[int] = None,
                  H: Optional[int] = None, I: Optional[int] = None,
                  seed: Optional[int] = None) -> dict:
    """One synthetic layer with MXFP8 expert weights: x, w_router (bf16) and
    the Zipf prior drawn as by :func:`make_layer`; W13 [E, 2I, H] and W2
    [E, H, I] as E4M3 codes (``w13_codes``, uint8) and E8M0 scales per 32
    elements (``w13_scales`` [E, 2I, H/32], uint8).  H and I must be
    multiples of 32."""
    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    E = shape.E if E is None else E
    top_k = shape.top_k if top_k is None else top_k
    H = shape.H if H is None else H
    I = shape.I if I is None else I
    if H % MX_BLOCK or I % MX_BLOCK:
        raise ValueError("H and I must be multiples of 32")
    base = seed_for(shape, M, layer) + 104729 if seed is None else seed
    seqs = np.random.SeedSequence(base).spawn(2 + 2 * E + 1)
    rstd = shape.router_std if shape.router_std is not None else 1.0 / math.sqrt(H)
    x = np.empty((M, H), dtype=np.uint16)
    w_router = np.empty((E, H), dtype=np.uint16)
    _normal_bf16_into(x, seqs[0], 1.0)
    _normal_bf16_into(w_router, seqs[1], rstd)
    w13 = [_mx_matrix(2 * I, H, seqs[2 + e]) for e in range(E)]
    w2 = [_mx_matrix(H, I, seqs[2 + E + e]) for e in range(E)]
    bias = None
    if shape.zipf_s is not None:
        rank = np.random.Generator(np.random.PCG64(seqs[-1])).permutation(E) + 1
        bias = (-shape.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    return dict(x=x, w_router=w_router, logit_bias=bias,
                w13_codes=np.stack([m[0] for m in w13]), w13_scales=np.stack([m[1] for m in w13]),
                w2_codes=np.stack([m[0] for m in w2]), w2_scales=np.stack([m[1] for m in w2]),
                M=M, E=E, top_k=top_k, H=H, I=I, renormalize=shape.renormalize,
                name=shape.name)


def make_device_mx_layer(shape: LayerShape | str, M: int, layer: int, device) -> dict:
    """An MXFP8 timing layer drawn directly in device memory with torch's
    seeded generator (same recipe as :func:`make_mx_layer`).  Returns
    w_router, logit_bias and the ``moe_forward_mxfp8`` weight dict under
    ``w``."""
    import torch  # local import: the oracle side never needs torch

    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    E, H, I = shape.E, shape.H, shape.I
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(shape, M, layer) + 104729)
    rstd = shape.router_std if shape.router_std is not None else 1.0 / math.sqrt(H)
    w_router = (torch.randn((E, H), generator=g, device=device) * rstd).to(torch.bfloat16)
    w = {}
    for name, rows, K in (("w13", 2 * I, H), ("w2", H, I)):
        # uniform over the 254 finite codes: draw 0..253 and step over 0x7F
        r = torch.randint(0, 254, (E, rows, K), generator=g, device=device, dtype=torch.int32)
        w[name + "_codes"] = (r + (r >= 0x7F).to(torch.int32)).to(torch.uint8)
        base = mx_scale_base(K)
        w[name + "_scales"] = (base + torch.randint(-1, 2, (E, rows, K // MX_BLOCK), generator=g,
                                                    device=device)).to(torch.uint8)
    bias = None
    if shape.zipf_s is not None:
        rank = torch.randperm(E, generator=g, device=device).to(torch.float64) + 1
        bias = (-shape.zipf_s * torch.log(rank)).to(torch.float32)
    return dict(w_router=w_router, logit_bias=bias, w=w)
