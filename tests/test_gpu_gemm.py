"""GPU parity of the two grouped GEMMs, teacher-forced: the GPU kernels get
the oracle's routing and index lists, so each GEMM is checked on its own
(the per-pair GEMVs, block_m = 1, the weight-streaming kernels, block_m = 16,
and the tiled kernels, block_m = 64 / 128 / 256)."""

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


def lists_to_device(a: dict, P: int, E: int, B: int):
    moe = _moe()
    cap, nbl = moe.align_capacity(P, E, B)
    s = np.full(cap, -7, dtype=np.int32)       # never read beyond num_blocks*B
    s[: a["sorted_token_ids"].size] = a["sorted_token_ids"]
    e = np.full(max(nbl, 1), -7, dtype=np.int32)
    e[: a["expert_ids"].size] = a["expert_ids"]
    return h.dev_i32(s), h.dev_i32(e), h.dev_i32(a["expert_block_offsets"])


def run_case(lay: dict, B: int, pairs_checked: int = 4096, seed: int = 0):
    import torch
    moe = _moe()
    M, k, E, H, I = lay["M"], lay["top_k"], lay["E"], lay["H"], lay["I"]
    P = M * k
    r = mo.route(lay["x"], lay["w_router"], k, lay["renormalize"], lay.get("logit_bias"))
    ids, wts = r["topk_ids"], r["topk_weights"]
    a = mo.align(ids, E, B)
    s, e, off = lists_to_device(a, P, E, B)
    d = h.layer_to_device(lay)

    # GEMM 1 + SiLU*up, pair order
    act, info = moe.moe_grouped_gemm_w13_act(d["x"], d["w13"], s, e, off, k, B)
    torch.cuda.synchronize()
    variant = {1: moe.MOE_VARIANT_PAIR_GEMV, 16: moe.MOE_VARIANT_STREAM}
    assert info["variant"] == variant.get(B, moe.MOE_VARIANT_TILED)
    toks = h.sample_tokens(M, max(1, pairs_checked // k), seed)
    ref_act = mo.pair_activations(lay["x"], lay["w13"], ids, toks)
    rows = (toks[:, None] * k + np.arange(k)).reshape(-1)
    got = h.host_bf16_to_f64(act)[rows]
    h.assert_close_outputs(got, ref_act[rows], "act")

    # GEMM 2 + combine, from the oracle's activations rounded to bf16
    act_ref_full = mo.pair_activations(lay["x"], lay["w13"], ids) if M <= 4096 // k else None
    if act_ref_full is not None:
        act_bits = wl.f32_to_bf16_bits(act_ref_full.astype(np.float32))
        act_in = h.dev_bf16(act_bits)
        out, info2 = moe.moe_grouped_gemm_w2_combine(
            act_in, d["w2"], h.dev_f32(wts.reshape(-1)), s, e, off, M, k, B)
        torch.cuda.synchronize()
        ref_out = mo.combine_from_act(act_bits, lay["w2"], ids, wts, toks)
        h.assert_close_outputs(h.host_bf16_to_f64(out)[toks], ref_out, "gemm2 out")
    return info


# mid-size shapes: several tiles in every direction plus ragged tails
# (H = 520 is not a multiple of 64 or 256; I = 200 not a multiple of 16 or 64)
MID = [dict(M=70, E=6, top_k=2, H=520, I=200, seed=31),
       dict(M=300, E=5, top_k=3, H=256, I=128, seed=32),
       dict(M=257, E=9, top_k=4, H=1032, I=136, seed=33),
       dict(M=3, E=4, top_k=2, H=64, I=32, seed=34)]


@pytest.mark.parametrize("B", [1, 16, 64, 128, 256])
@pytest.mark.parametrize("case", MID, ids=lambda c: f"M{c['M']}E{c['E']}H{c['H']}I{c['I']}")
def test_gemms_mid_shapes(case, B):
    lay = wl.make_layer("qwen15", case["M"], E=case["E"], top_k=case["top_k"], H=case["H"],
                        I=case["I"], seed=case["seed"])
    run_case(lay, B)


@pytest.mark.parametrize("B", [1, 16, 128])
def test_gemms_renormalize_off(B):
    lay = wl.make_layer("qwen15", 40, E=8, top_k=3, H=256, I=64, seed=41)
    lay["renormalize"] = False
    run_case(lay, B)


@pytest.mark.parametrize("name,M,B", [("qwen3_decode", 1, 1), ("qwen3_decode", 4, 1),
                                      ("wide256", 8, 1), ("qwen15", 3, 1),
                                      ("qwen3_decode", 64, 16), ("qwen15", 16, 16),
                                      ("qwen15", 512, 64), ("wide256", 8, 16),
                                      ("qwen3_decode", 64, 64), ("qwen15", 512, 256),
                                      ("qwen3_prefill", 4096, 256), ("qwen3_prefill", 4096, 128),
                                      ("qwen15", 2048, 256), ("wide256", 8192, 128)])
def test_gemms_full_shapes(name, M, B):
    lay = wl.make_layer(name, M)
    run_case(lay, B, pairs_checked=512)
