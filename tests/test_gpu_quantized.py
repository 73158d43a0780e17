"""Parity of moe_forward_quantized (group-quantized expert weights, the affine
64-element-group format of the MLX part of the page "SGLang issue #22283",
4 and 8 bits) against the oracle's forward_quantized.

Cases: the Qwen1.5-MoE shape whose down projection has K = 1408 (not a
multiple of the kernels' 256- or 512-element passes, the case that thread
asks about), the Qwen3-30B-A3B decode shape, and small layers whose H and I
pick every per-lane unit count, several passes and ragged last passes, plus
top_k above the eight waves of GEMV 2, renormalize off, and a larger batch
(the path is correct for any M).  Same criteria as the bf16 layer: routing
ids where the top-k margin exceeds 1e-4, weights to 1e-5, outputs within
2e-2 max-abs (relative to max |ref|) and 5e-3 mean-relative.
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


def check_quantized(ql: dict, n_tokens: int = 64, seed: int = 0, **kw):
    moe = _moe()
    print(f"quantized case {ql['name']} M={ql['M']} E={ql['E']} k={ql['top_k']} "
          f"H={ql['H']} I={ql['I']} bits={ql['bits']}", flush=True)
    out, ids, wts, info = run_quantized(ql, **kw)
    assert info["variant"] == moe.MOE_VARIANT_PAIR_GEMV_QUANT
    assert info["launches"] == 4 and info["sorted"] == 0 and info["block_m"] == 1
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
    """M = 64 of the Qwen3 decode shape: 512 pairs, each its own GEMV."""
    check_quantized(wl.make_quantized_layer("qwen3_decode", 64, bits), n_tokens=24)


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
