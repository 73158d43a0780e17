"""Parity of the MXFP8 path (moe_mx_quantize, moe_forward_mxfp8) against the
oracle's mx_quantize and forward_mxfp8.

* The quantizer is integer output decided by floating point on the same
  exact values on both sides (division by a power of two), so its codes and
  scales must match bit for bit: random blocks over a wide range of
  magnitudes, all-zero blocks, negative zeros, exact ties between E4M3
  neighbours, blocks that saturate at 448, bf16-subnormal blocks.
* The layer: routing ids where the top-k margin exceeds 1e-4 (validity
  elsewhere), weights to 1e-5, outputs within 2e-2 max-abs (relative to max |ref|) and 5e-3
  mean-relative, through the weight-streaming kernels (block_m 16: small
  layers, the Qwen3-30B-A3B decode shape at 1, 8 and 64 tokens, the
  Qwen1.5-MoE shape whose I = 1408 leaves a ragged last slice, 256 experts),
  the per-pair MXFP8 GEMVs of very small batches (no index lists; x
  quantized by the top-k launch, act quantized in registers by GEMV 2)
  and the tiled kernels (a mid layer, the Qwen1.5-MoE shape at 512 and 2048
  tokens, the Qwen3 prefill shape with its Zipf prior at block_m 128), plus
  a poisoned workspace; weight codes span the whole finite E4M3 range.
  Outputs of every sampled token are compared against the oracle's MXFP8
  layer on the GPU's own ids.
* act is quantized from its bf16 value, which the GPU forms from fp32 sums
  and the oracle from fp64 ones; where an act element sits within one bf16
  step of an E4M3 rounding boundary, or its block's largest magnitude within
  one step of a power of two (the shared scale), either decision is correct.
  A token whose output misses the bound is accepted only if the oracle's
  layer with some choice of those decisions (at most four per pair) meets
  it; the mean-relative error is then taken against that choice.
"""

from __future__ import annotations

import numpy as np
import pytest

import moe_workloads as wl
from oracle import moe_oracle as mo
from tests import helpers as h

pytestmark = pytest.mark.gpu


def _moe():
    import mixture_experts_ffn_renorm_amd as moe
    return moe


def dev_u8(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def _quant_inputs(rows: int, K: int, seed: int) -> np.ndarray:
    """bf16 bits: per block a random magnitude, some zero blocks, negative
    zeros, exact ties, saturating blocks, bf16-subnormal blocks."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, K)) * np.repeat(
        np.exp2(rng.integers(-30, 30, (rows, K // 32))), 32, axis=1)
    v[0, :32] = 0.0
    v[0, 32:64] = -0.0
    bits = wl.f32_to_bf16_bits(v.astype(np.float32))
    if rows > 2 and K >= 64:
        # exact ties: block max 256 (scale 1), midpoints of E4M3 neighbours
        grid = mo.e4m3_value(np.arange(0x7F))
        mids = (grid[1:] + grid[:-1]) / 2
        row = np.concatenate([[256.0], mids[rng.integers(0, mids.size, 31)],
                              [448.0], [470.0, 500.0, -511.0], rng.standard_normal(28) * 300])
        bits[1, :64] = wl.f32_to_bf16_bits(row.astype(np.float32))
    if rows > 3 and K >= 96:
        # bf16 subnormals (below 2^-126): a block of subnormal codes of both
        # signs (scale clamps to 2^-127), a block mixing normal values near
        # 2^-120 with subnormals, a block whose largest value is 2^-118 (the
        # first unclamped scale) with subnormal neighbours
        sub = rng.integers(1, 0x80, 32).astype(np.uint16) | \
            (rng.integers(0, 2, 32).astype(np.uint16) << 15)
        bits[2, :32] = sub
        mix = wl.f32_to_bf16_bits((rng.standard_normal(32) * 2.0 ** -120).astype(np.float32))
        mix[::3] = sub[::3]
        bits[2, 32:64] = mix
        edge = sub.copy()
        edge[7] = wl.f32_to_bf16_bits(np.array([2.0 ** -118], dtype=np.float32))[0]
        bits[2, 64:96] = edge
        bits[3, :32] = rng.integers(0, 0x10000, 32).astype(np.uint16) & 0x807F   # +-0 and subnormals
    return bits


@pytest.mark.parametrize("rows,K,seed", [(37, 96, 1), (64, 2048, 2), (300, 768, 3)])
def test_mx_quantize_bit_exact(rows, K, seed):
    moe = _moe()
    bits = _quant_inputs(rows, K, seed)
    codes, scales = moe.moe_mx_quantize(h.dev_bf16(bits))
    import torch
    torch.cuda.synchronize()
    ref_c, ref_s = mo.mx_quantize(mo.widen_bf16(bits))
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != ref_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def mx_to_device(lay: dict) -> dict:
    return {k: dev_u8(lay[k]) for k in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")}


def run_mx(lay: dict, ws=None, out=None):
    import torch
    moe = _moe()
    M, k = lay["M"], lay["top_k"]
    ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    wts = torch.full((M, k), -1.0, dtype=torch.float32, device="cuda")
    lb = None if lay.get("logit_bias") is None else h.dev_f32(lay["logit_bias"])
    out, info = moe.moe_forward_mxfp8(h.dev_bf16(lay["x"]), h.dev_bf16(lay["w_router"]),
                                      mx_to_device(lay), k, lay["renormalize"], logit_bias=lb,
                                      out=out, topk_ids_out=ids, topk_weights_out=wts, ws=ws)
    torch.cuda.synchronize()
    return out, ids.cpu().numpy(), wts.cpu().numpy().astype(np.float64), info


def check_mx(lay: dict, n_tokens: int = 48, seed: int = 0, **kw):
    moe = _moe()
    print(f"mxfp8 case {lay['name']} M={lay['M']} E={lay['E']} k={lay['top_k']} "
          f"H={lay['H']} I={lay['I']}", flush=True)
    out, ids, wts, info = run_mx(lay, **kw)
    B = moe.moe_pick_block_m(lay["M"], lay["E"], lay["top_k"])
    assert info["block_m"] == B
    P = lay["M"] * lay["top_k"]
    if P * 4 <= lay["E"]:
        # router logits, top-k (+ x quantized), GEMV 1, GEMV 2 with the sum
        assert B == 1 and info["sorted"] == 0 and info["launches"] == 4
        assert info["variant"] == moe.MOE_VARIANT_PAIR_GEMV_MXFP8
    else:
        # router logits, top-k + lists + x quantized (one launch, or top-k
        # with x, count, scatter), GEMM 1 (quantizing act in its epilogue at
        # block_m 16; a separate quantize launch after the tiles), GEMM 2,
        # per-token sum
        route_launches = 2 if P <= 2048 else 4
        assert info["launches"] == route_launches + (3 if B == 16 else 4)
        assert info["sorted"] == 1
        assert info["variant"] == (moe.MOE_VARIANT_STREAM_MXFP8 if B == 16
                                   else moe.MOE_VARIANT_TILED_MXFP8)
    toks = h.sample_tokens(lay["M"], n_tokens, seed)
    r = mo.route(lay["x"][toks], lay["w_router"], lay["top_k"], lay["renormalize"],
                 lay.get("logit_bias"))
    w_ref = h.check_routing(ids[toks], wts[toks], r, lay["renormalize"])
    full_ids, full_w = h.scatter_routing(lay["M"], toks, ids[toks], w_ref)
    ref_y, _, _ = mo.mx_layer_forward(lay, full_ids, full_w, toks)
    y = h.host_bf16_to_f64(out)[toks]
    ref_y = h.mx_boundary_reference(lay, full_ids, full_w, toks, y, ref_y)
    h.assert_close_outputs(y, ref_y, "mxfp8 output")
    return out


# per-pair MXFP8 GEMVs (M*top_k*4 <= E): a small layer, H = 4224 (two
# passes of GEMV 1, the second ragged) with I = 1408 (a ragged GEMV 2 pass),
# top_k = 12 (more slots than GEMV 2's eight waves), the Qwen3 decode shape
# at 1, 2 and 4 tokens, the Qwen1.5 shape at 1 token, 256 experts at 8;
# block_m 16 (streaming): toy M=5, Qwen3 decode M=8 and 64, Qwen1.5 M=16
# (I = 1408: a ragged last slice in both streaming kernels), 256 experts
# M=8; tiled: toy M=70, Qwen1.5 M=512 (block_m 64), toy M=300 (block_m 128,
# the copy-wave tiles), Qwen1.5 M=2048 (136 pairs per expert: block_m 256,
# the eight-wave tiles with a two-stage ring), Qwen3 prefill (block_m 128).
# Weight codes are uniform over every finite E4M3 code (zeros, subnormals,
# all exponent fields, +-448).
MX_CASES = [("toy", 3, dict(E=64, top_k=2, H=256, I=128)),
            ("toy", 2, dict(E=64, top_k=2, H=4224, I=1408)),
            ("toy", 2, dict(E=128, top_k=12, H=384, I=256)),
            ("qwen3_decode", 2, {}),
            ("qwen3_decode", 4, {}),
            ("qwen15", 1, {}),
            ("toy", 5, dict(E=8, top_k=2, H=256, I=128)),
            ("toy", 6, dict(E=8, top_k=2, H=384, I=256)),      # streaming, K tail of half a slice
            ("toy", 70, dict(E=6, top_k=2, H=384, I=256)),
            ("toy", 300, dict(E=6, top_k=2, H=384, I=256)),
            ("qwen3_decode", 1, {}),
            ("qwen3_decode", 8, {}),
            ("qwen3_decode", 64, {}),
            ("qwen15", 16, {}),
            ("wide256", 8, {}),
            ("qwen15", 512, {}),
            ("qwen15", 2048, {}),
            ("qwen3_prefill", 4096, {})]


@pytest.mark.parametrize("name,M,kw", MX_CASES, ids=lambda v: str(v))
def test_forward_mxfp8(name, M, kw):
    lay = wl.make_mx_layer(name, M, seed=500 + M if kw else None, **kw)
    check_mx(lay, n_tokens=24 if M >= 512 else 48)


def test_forward_mxfp8_poisoned_workspace():
    """NaN-filled workspace and output give the same bits as a fresh call."""
    import torch
    moe = _moe()
    lay = wl.make_mx_layer("toy", 70, E=6, top_k=2, H=384, I=256, seed=77)
    ref_out = check_mx(lay).clone()
    ws = moe.mx_workspace(70, 6, 2, 384, 256)
    ws.fill_(0xFF)
    out = torch.full((70, 384), float("nan"), dtype=torch.bfloat16, device="cuda")
    got, _, _, _ = run_mx(lay, ws=ws, out=out)
    assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16))


# Tiled-path shapes drawn once (numpy seed 2027; H and I multiples of 128)
# with block_m 64, 128 and 256.
RANDOM_MX_TILED = [
    (2501, 64, 2, 1152, 128), (633, 32, 8, 1408, 256), (638, 60, 4, 256, 256),
    (2974, 60, 2, 256, 384), (518, 32, 2, 896, 128), (2632, 32, 1, 640, 384),
    (1027, 8, 4, 1152, 256), (1511, 8, 4, 256, 896),
]


@pytest.mark.parametrize("M,E,top_k,H,I", RANDOM_MX_TILED)
def test_forward_mxfp8_tiled_random_shapes(M, E, top_k, H, I):
    lay = wl.make_mx_layer("toy", M, E=E, top_k=top_k, H=H, I=I, seed=3700 + M)
    check_mx(lay, n_tokens=24)


# Small-batch shapes drawn once (numpy seed 2028; H and I multiples of 128):
# the streaming MXFP8 kernels (block_m 16) and the per-pair MXFP8 GEMVs.
RANDOM_MX_SMALL = [(36, 256, 6, 896, 256), (87, 60, 4, 3200, 384), (22, 8, 1, 3456, 384),
                   (188, 32, 1, 3968, 128), (71, 256, 2, 768, 256), (11, 16, 4, 2304, 640),
                   (1, 32, 2, 1920, 512), (3, 64, 4, 384, 1024), (1, 32, 2, 1792, 1152),
                   (5, 32, 1, 1792, 384), (14, 64, 1, 640, 1280)]


@pytest.mark.parametrize("M,E,top_k,H,I", RANDOM_MX_SMALL)
def test_forward_mxfp8_small_batch_random_shapes(M, E, top_k, H, I):
    lay = wl.make_mx_layer("toy", M, E=E, top_k=top_k, H=H, I=I, seed=3900 + M + H)
    check_mx(lay, n_tokens=24)


def test_forward_mxfp8_maximum_experts_and_top_k():
    lay = wl.make_mx_layer("toy", 256, E=512, top_k=32, H=256, I=128, seed=4200)
    check_mx(lay, n_tokens=24)


# Degenerate layers: one expert (a dense FFN) and top_k = E, on the
# streaming kernels and on the tiles.
@pytest.mark.parametrize("M,E,top_k", [(3, 1, 1), (40, 1, 1), (3, 4, 4), (100, 4, 4)])
def test_forward_mxfp8_degenerate_layers(M, E, top_k):
    lay = wl.make_mx_layer("toy", M, E=E, top_k=top_k, H=256, I=128, seed=4600 + M + E)
    check_mx(lay, n_tokens=24)


def test_forward_mxfp8_zero_tokens():
    import torch
    moe = _moe()
    lay = wl.make_mx_layer("toy", 3, E=8, top_k=2, H=256, I=128, seed=4700)
    x0 = h.dev_bf16(lay["x"])[:0]
    out, info = moe.moe_forward_mxfp8(x0, h.dev_bf16(lay["w_router"]), mx_to_device(lay), 2, True)
    torch.cuda.synchronize()
    assert out.shape == (0, 256) and info["launches"] == 0
