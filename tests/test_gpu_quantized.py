"""Parity of moe_forward_quantized (group-quantized expert weights, the affine
64-element-group format of the MLX part of the page "SGLang issue #22283",
4 and 8 bits) against the oracle's forward_quantized.

Two kernel families: per-pair GEMVs up to E/2 pairs (M*top_k*2 <= E) and
for shapes whose H or I is not a multiple of 128, and weight-streaming MFMA
GEMMs over block_m 16 index lists above.

Cases: the Qwen1.5-MoE shape whose down projection has K = 1408 (not a
multiple of the kernels' 256- or 512-element passes, the case that thread
asks about), the Qwen3-30B-A3B decode shape, and small layers whose H and I
pick every per-lane unit count, several passes and ragged last passes, plus
top_k above the eight waves of GEMV 2, renormalize off, and larger batches
on both families: the streaming GEMMs at decode batches, with a K tail of
half a slice, a one-slice GEMM 2, experts spanning many blocks (Zipf
prior) and a two-segment index-list build.  Same criteria as the bf16
layer: routing ids where the top-k margin exceeds 1e-4, the weights of the
GPU's own ids to 1e-5, and every sampled token's output (near ties
included, against the oracle's layer on the GPU's ids) within 2e-2 max-abs
(relative to max |ref|) and 5e-3 mean-relative.
"""

from __future__ import annotations

import numpy as np
import pytest

import moe_workloads as wl
from oracle import moe_oracle as mo
from tests import helpers as h

pytestmark = pytest.mark.gpu

QKEYS = ("w13_q", "w13_scales", "w13_biases", "w2_q", "w2_scales", "w2_biases")


def _moe():
    import mixture_experts_ffn_renorm_amd as moe
    return moe


def quant_to_device(ql: dict) -> dict:
    import torch
    d = {"bits": ql["bits"]}
    for k in QKEYS:
        a = np.ascontiguousarray(ql[k])
        if a.dtype == np.uint32:
            d[k] = torch.from_numpy(a.view(np.int32)).to("cuda")
        else:
            d[k] = h.dev_bf16(a)
    return d


def run_quantized(ql: dict, ws=None, out=None):
    import torch
    moe = _moe()
    M, k = ql["M"], ql["top_k"]
    x = h.dev_bf16(ql["x"])
    wr = h.dev_bf16(ql["w_router"])
    lb = None if ql.get("logit_bias") is None else h.dev_f32(ql["logit_bias"])
    ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    wts = torch.full((M, k), -1.0, dtype=torch.float32, device="cuda")
    out, info = moe.moe_forward_quantized(x, wr, quant_to_device(ql), k, ql["renormalize"],
                                          logit_bias=lb, out=out, topk_ids_out=ids,
                                          topk_weights_out=wts, ws=ws)
    torch.cuda.synchronize()
    return out, ids.cpu().numpy(), wts.cpu().numpy().astype(np.float64), info


def tiles(ql: dict) -> bool:
    """Whether moe_forward_quantized takes the LDS-tiled GEMMs (block_m 128)."""
    M, E, k = ql["M"], ql["E"], ql["top_k"]
    return M * k * 2 > E and _moe().moe_pick_block_m(M, E, k) >= 64


def streams(ql: dict) -> bool:
    """Whether moe_forward_quantized takes the weight-streaming GEMMs."""
    M, E, k, H, I = ql["M"], ql["E"], ql["top_k"], ql["H"], ql["I"]
    return M * k * 2 > E and not tiles(ql) and H % 128 == 0 and I % 128 == 0


def check_dispatch(ql: dict, info: dict):
    moe = _moe()
    P = ql["M"] * ql["top_k"]
    route_launches = 2 if P <= 2048 else 4
    if tiles(ql):
        assert info["variant"] == moe.MOE_VARIANT_TILED_QUANT
        assert info["sorted"] == 1 and info["block_m"] == 128
        assert info["launches"] == route_launches + 3
        assert info["k_tail"] == 0
    elif streams(ql):
        assert info["variant"] == moe.MOE_VARIANT_STREAM_QUANT
        assert info["sorted"] == 1 and info["block_m"] == 16
        assert info["launches"] == route_launches + 3
        assert info["k_tail"] == int(ql["H"] % 256 != 0)
    else:
        assert info["variant"] == moe.MOE_VARIANT_PAIR_GEMV_QUANT
        assert info["launches"] == 4 and info["sorted"] == 0 and info["block_m"] == 1


def check_quantized(ql: dict, n_tokens: int = 64, seed: int = 0, **kw):
    print(f"quantized case {ql['name']} M={ql['M']} E={ql['E']} k={ql['top_k']} "
          f"H={ql['H']} I={ql['I']} bits={ql['bits']}", flush=True)
    out, ids, wts, info = run_quantized(ql, **kw)
    check_dispatch(ql, info)
    toks = h.sample_tokens(ql["M"], n_tokens, seed)
    r = mo.route(ql["x"][toks], ql["w_router"], ql["top_k"], ql["renormalize"],
                 ql.get("logit_bias"))
    w_ref = h.check_routing(ids[toks], wts[toks], r, ql["renormalize"])
    full_ids, full_w = h.scatter_routing(ql["M"], toks, ids[toks], w_ref)
    w13, w2 = mo.dequantized_experts(ql)
    ref_y = mo.layer_forward(ql["x"], w13, w2, full_ids, full_w, toks)
    y = h.host_bf16_to_f64(out)[toks]
    h.assert_close_outputs(y, ref_y, f"bits={ql['bits']}")
    return out


MODEL_CASES = [(n, m, b) for n, ms in (("qwen15", (1, 3)), ("qwen3_decode", (1, 4)))
               for m in ms for b in (4, 8)]


@pytest.mark.parametrize("name,M,bits", MODEL_CASES)
def test_quantized_model_shapes(name, M, bits):
    check_quantized(wl.make_quantized_layer(name, M, bits))


# (M, bits, E, top_k, H, I): units per lane per pass are min(4, ceil(units/64))
# with 32 (4-bit) or 16 (8-bit) elements per 16-byte unit; 4-bit GEMV 2 is
# capped at 2.
SMALL_CASES = [
    (5, 4, 8, 2, 576, 320),      # 18 / 10 units: one ragged pass each
    (5, 8, 8, 2, 576, 320),      # 36 / 20 units
    (3, 8, 4, 2, 2560, 2560),    # 160 units: three per lane
    (3, 4, 4, 2, 5120, 6144),    # GEMV 1 three per lane; GEMV 2 192 units in passes of 128
    (2, 8, 4, 2, 4608, 4096),    # 288 units: two passes of 256; GEMV 2 256 units
    (2, 4, 4, 2, 9216, 64),      # 288 units in 4-bit; I = 64 is two units
    (2, 4, 32, 12, 256, 128),    # top_k 12 > 8 waves: waves take two slots
    (2, 8, 32, 12, 256, 128),
]


@pytest.mark.parametrize("M,bits,E,top_k,H,I", SMALL_CASES)
def test_quantized_unit_counts_and_tails(M, bits, E, top_k, H, I):
    check_quantized(wl.make_quantized_layer("toy", M, bits, E=E, top_k=top_k, H=H, I=I,
                                            seed=1000 + H + I + bits))


def test_quantized_renormalize_off():
    ql = wl.make_quantized_layer("qwen3_decode", 2, 4)
    ql["renormalize"] = False
    check_quantized(ql)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantized_larger_batch(bits):
    """M = 64 of the Qwen3 decode shape: 512 pairs on the streaming GEMMs."""
    ql = wl.make_quantized_layer("qwen3_decode", 64, bits)
    assert streams(ql)
    check_quantized(ql, n_tokens=24)


def test_quantized_pair_gemv_at_any_batch():
    """H = 576 is not a multiple of 128: the per-pair GEMVs take every M."""
    ql = wl.make_quantized_layer("toy", 48, 4, E=16, top_k=2, H=576, I=384, seed=77)
    assert not streams(ql)
    check_quantized(ql, n_tokens=24)


# Streaming GEMMs: (name, M, bits, overrides)
STREAM_CASES = [
    ("qwen3_decode", 12, 4, {}),
    ("qwen3_decode", 16, 8, {}),
    ("qwen15", 16, 4, {}),                                      # I = 1408: 11 GEMM 2 slices
    ("qwen15", 16, 8, {}),
    ("toy", 8, 4, dict(E=8, top_k=2, H=1408, I=384)),          # K tail of half a slice
    ("toy", 8, 8, dict(E=8, top_k=2, H=1408, I=384)),
    ("toy", 40, 4, dict(E=32, top_k=4, H=256, I=128)),         # GEMM 2 in one slice
    ("qwen3_prefill", 128, 4, {}),                              # Zipf: experts over many blocks
    ("qwen3_prefill", 128, 8, {}),
]


@pytest.mark.parametrize("name,M,bits,over", STREAM_CASES,
                         ids=lambda v: str(v) if not isinstance(v, dict) else
                         "_".join(f"{k}{x}" for k, x in v.items()) or "model")
def test_quantized_streaming(name, M, bits, over):
    seed = {"seed": 3000 + M + bits} if over else {}
    ql = wl.make_quantized_layer(name, M, bits, **over, **seed)
    assert streams(ql)
    check_quantized(ql, n_tokens=32)


def test_quantized_streaming_two_segments():
    """4096 pairs: the index lists are built by the two-kernel align."""
    ql = wl.make_quantized_layer("toy", 512, 4, E=512, top_k=8, H=256, I=256, seed=3100)
    assert streams(ql) and ql["M"] * ql["top_k"] > 2048
    check_quantized(ql, n_tokens=32)


# LDS-tiled GEMMs on codes widened in LDS: (name, M, bits, overrides)
TILED_CASES = [
    ("qwen3_prefill", 256, 8, {}),                              # 16 pairs per expert: mostly pads
    ("qwen3_prefill", 1024, 4, {}),                             # Zipf: 1 .. many blocks per expert
    ("qwen3_prefill", 1024, 8, {}),
    ("qwen15", 1024, 4, {}),                                    # I = 1408: 22 k stages in GEMM 2
    ("wide256", 2048, 8, {}),                                   # 256 experts, I = 512
    ("qwen3_prefill", 4096, 4, {}),                             # the prefill batch bench.py times
    ("qwen3_prefill", 4096, 8, {}),
    ("toy", 200, 4, dict(E=8, top_k=2, H=576, I=320)),         # H, I % 64 only; N tails
    ("toy", 200, 8, dict(E=8, top_k=2, H=576, I=320)),
    ("toy", 300, 4, dict(E=4, top_k=1, H=64, I=64)),           # one k stage: one stage per tile
    ("toy", 300, 8, dict(E=4, top_k=1, H=64, I=64)),
]


@pytest.mark.parametrize("name,M,bits,over", TILED_CASES,
                         ids=lambda v: str(v) if not isinstance(v, dict) else
                         "_".join(f"{k}{x}" for k, x in v.items()) or "model")
def test_quantized_tiled(name, M, bits, over):
    seed = {"seed": 3200 + M + bits} if over else {}
    ql = wl.make_quantized_layer(name, M, bits, **over, **seed)
    assert tiles(ql)
    check_quantized(ql, n_tokens=32)


# Shapes drawn once (numpy seed 2026) among H, I multiples of 64 with more
# than 8 pairs per expert: 1 to 23 k stages (odd and even group counts), N
# tails, 1 to 64 experts, top_k 1 to 8, one- and multi-segment index lists.
RANDOM_TILED = [
    (553, 4, 64, 1, 64, 640), (1247, 8, 4, 2, 960, 384), (1288, 8, 60, 8, 1088, 192),
    (1094, 8, 4, 2, 256, 960), (184, 8, 8, 4, 896, 768), (694, 4, 32, 8, 1024, 448),
    (1281, 8, 4, 2, 256, 256), (1246, 4, 4, 2, 448, 640), (254, 4, 16, 2, 1472, 384),
    (997, 4, 16, 4, 512, 448), (1435, 8, 64, 1, 1408, 896), (699, 8, 32, 4, 320, 384),
]


@pytest.mark.parametrize("M,bits,E,top_k,H,I", RANDOM_TILED)
def test_quantized_tiled_random_shapes(M, bits, E, top_k, H, I):
    ql = wl.make_quantized_layer("toy", M, bits, E=E, top_k=top_k, H=H, I=I, seed=3500 + M)
    assert tiles(ql)
    check_quantized(ql, n_tokens=24)


def test_quantized_tiled_poisoned_workspace_repeatable():
    """Workspace and output filled with 0xFF bytes, then reused: identical
    outputs on the tiled path."""
    import torch
    moe = _moe()
    ql = wl.make_quantized_layer("toy", 256, 4, E=16, top_k=4, H=512, I=256, seed=3300)
    assert tiles(ql)
    nbytes = moe.moe_workspace_size(ql["M"], ql["E"], ql["top_k"], ql["H"], ql["I"])
    ws = torch.full((nbytes,), -1, dtype=torch.uint8, device="cuda")
    out = torch.full((ql["M"], ql["H"]), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    a, _, _, info = run_quantized(ql, ws=ws, out=out)
    assert info["variant"] == moe.MOE_VARIANT_TILED_QUANT
    a = a.clone()
    b, _, _, _ = run_quantized(ql, ws=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    check_quantized(ql, n_tokens=16, ws=ws)


def test_quantized_streaming_poisoned_workspace_repeatable():
    """Workspace filled with 0xFF bytes, then reused: identical outputs."""
    import torch
    ql = wl.make_quantized_layer("qwen3_decode", 16, 4)
    moe = _moe()
    nbytes = moe.moe_workspace_size(ql["M"], ql["E"], ql["top_k"], ql["H"], ql["I"])
    ws = torch.full((nbytes,), -1, dtype=torch.uint8, device="cuda")
    a, _, _, info = run_quantized(ql, ws=ws)
    assert info["variant"] == moe.MOE_VARIANT_STREAM_QUANT
    b, _, _, _ = run_quantized(ql, ws=ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    check_quantized(ql, n_tokens=16, ws=ws)


def test_quantized_poisoned_workspace_and_output():
    """Every workspace byte and output element the path reads or leaves is
    written first: NaN-filled workspace and output give the same result."""
    import torch
    moe = _moe()
    ql = wl.make_quantized_layer("qwen15", 3, 4)
    ref_out = check_quantized(ql).clone()
    ws = moe.workspace(3, ql["E"], ql["top_k"], ql["H"], ql["I"])
    ws.fill_(0xFF)
    out = torch.full((3, ql["H"]), float("nan"), dtype=torch.bfloat16, device="cuda")
    got, _, _, _ = run_quantized(ql, ws=ws, out=out)
    assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16))


@pytest.mark.parametrize("name,M,bits,over", [
    ("qwen3_decode", 2, 4, {}),                                  # per-pair GEMVs
    ("qwen3_decode", 16, 8, {}),                                 # streaming GEMMs
    ("toy", 300, 4, dict(E=8, top_k=2, H=576, I=320)),           # tiles, one segment
    ("toy", 1200, 8, dict(E=8, top_k=2, H=256, I=192)),          # tiles, multi-segment lists
])
def test_quantized_graph_replay_matches_eager(name, M, bits, over):
    """moe_forward_quantized captured once into a HIP graph: every replay, with
    other eager launches in between, gives the eager call's bits."""
    import torch
    seed = {"seed": 3400 + M + bits} if over else {}
    ql = wl.make_quantized_layer(name, M, bits, **over, **seed)
    moe = _moe()
    k = ql["top_k"]
    q = quant_to_device(ql)
    wr = h.dev_bf16(ql["w_router"])
    lb = None if ql.get("logit_bias") is None else h.dev_f32(ql["logit_bias"])
    inputs = [h.dev_bf16(ql["x"])]
    for r in (1, 2):   # other batches: the same rows permuted
        perm = np.random.default_rng(100 + r).permutation(M)
        inputs.append(h.dev_bf16(np.ascontiguousarray(ql["x"][perm])))
    ws = moe.workspace(M, ql["E"], k, ql["H"], ql["I"])
    eager_out = torch.empty((M, ql["H"]), dtype=torch.bfloat16, device="cuda")

    def run(x, out):
        return moe.moe_forward_quantized(x, wr, q, k, ql["renormalize"], logit_bias=lb,
                                         out=out, ws=ws)[1]

    refs = []
    for xr in inputs:
        run(xr, eager_out)
        torch.cuda.synchronize()
        refs.append(eager_out.clone())
    x_static = inputs[0].clone()
    out = torch.empty_like(eager_out)
    run(x_static, out)                       # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        info = run(x_static, out)
    print(f"quantized graph case {name} M={M} bits={bits} variant={info['variant']}", flush=True)
    for r in range(3):
        x_static.copy_(inputs[r])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), refs[r].view(torch.int16)), f"replay {r}"
        run(inputs[(r + 1) % 3], eager_out)   # eager work between replays
        torch.cuda.synchronize()


# Small-batch shapes drawn once (numpy seed 2028): the streaming quantized
# GEMMs (H and I multiples of 128) and the per-pair GEMVs (M * top_k * 2 <= E,
# H and I multiples of 64).
RANDOM_Q_SMALL = [(5, 32, 6, 256, 1024), (14, 64, 8, 128, 1792), (57, 16, 1, 1408, 1280),
                  (20, 128, 8, 640, 512), (77, 64, 4, 1024, 1408), (198, 64, 1, 1792, 768),
                  (28, 256, 1, 448, 832), (16, 256, 8, 448, 448), (8, 60, 1, 384, 832),
                  (7, 128, 1, 448, 64), (9, 64, 1, 128, 704)]


@pytest.mark.parametrize("M,E,top_k,H,I", RANDOM_Q_SMALL)
@pytest.mark.parametrize("bits", [4, 8])
def test_quantized_small_batch_random_shapes(M, E, top_k, H, I, bits):
    ql = wl.make_quantized_layer("toy", M, bits, E=E, top_k=top_k, H=H, I=I,
                                 seed=4000 + M + H + bits)
    assert not tiles(ql)
    check_quantized(ql, n_tokens=24)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantized_maximum_experts_and_top_k(bits):
    ql = wl.make_quantized_layer("toy", 256, bits, E=512, top_k=32, H=256, I=128, seed=4300 + bits)
    check_quantized(ql, n_tokens=24)


# Degenerate layers: one expert (a dense FFN) and top_k = E (every expert
# chosen, renormalized weights = the softmax), on the streaming GEMMs (few
# pairs per expert) and on the tiles.
DEGENERATE = [(3, 1, 1), (40, 1, 1), (3, 4, 4), (100, 4, 4)]


@pytest.mark.parametrize("M,E,top_k", DEGENERATE)
@pytest.mark.parametrize("bits", [4, 8])
def test_quantized_degenerate_layers(M, E, top_k, bits):
    ql = wl.make_quantized_layer("toy", M, bits, E=E, top_k=top_k, H=256, I=128,
                                 seed=4400 + M + E + bits)
    check_quantized(ql, n_tokens=24)


def test_quantized_zero_tokens():
    import torch
    moe = _moe()
    ql = wl.make_quantized_layer("toy", 3, 4, E=8, top_k=2, H=256, I=128, seed=4500)
    x0 = h.dev_bf16(ql["x"])[:0]
    out, info = moe.moe_forward_quantized(x0, h.dev_bf16(ql["w_router"]), quant_to_device(ql), 2,
                                          True)
    torch.cuda.synchronize()
    assert out.shape == (0, 256) and info["launches"] == 0
