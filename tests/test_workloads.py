"""The seeded input recipe (CPU only): bf16 rounding, determinism, value
distributions and the skew of the Zipf-biased prefill router."""

import math

import numpy as np
import torch

import moe_workloads as wl
from oracle import moe_oracle as mo


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0,
                                  3.0e38, 1e-40], dtype=np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.f32_to_bf16_bits(v), want)
    assert np.array_equal(wl.bf16_bits_to_f32(want), torch.from_numpy(want.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_layer_is_deterministic_and_shaped():
    a = wl.make_layer("qwen15", 16, E=6, I=64, H=128)
    b = wl.make_layer("qwen15", 16, E=6, I=64, H=128)
    for key in ("x", "w_router", "w13", "w2"):
        assert np.array_equal(a[key], b[key])
    assert a["x"].shape == (16, 128) and a["w13"].shape == (6, 128, 128)
    assert a["w2"].shape == (6, 128, 64) and a["w_router"].shape == (6, 128)
    c = wl.make_layer("qwen15", 17, E=6, I=64, H=128)
    assert not np.array_equal(a["w13"], c["w13"])


def test_value_distributions():
    lay = wl.make_layer("qwen3_decode", 8, E=8)     # full H, I; 8 experts
    H, I = lay["H"], lay["I"]
    x = mo.widen_bf16(lay["x"])
    assert abs(x.std() - 1.0) < 0.02
    assert abs(mo.widen_bf16(lay["w13"]).std() * math.sqrt(H) - 1.0) < 0.01
    assert abs(mo.widen_bf16(lay["w2"]).std() * math.sqrt(I) - 1.0) < 0.01
    assert abs(mo.widen_bf16(lay["w_router"]).std() / 0.02 - 1.0) < 0.02


def test_zipf_prefill_router_has_empty_experts():
    """The Zipf(1.1) prior makes the prefill routing skewed: some experts get
    no pair at all and the hottest expert serves most tokens."""
    s = wl.WORKLOADS["qwen3_prefill"]
    lay = wl.make_layer(s, 4096, E=s.E, H=s.H, I=8)    # only routing matters
    r = mo.route(lay["x"], lay["w_router"], s.top_k, True, lay["logit_bias"])
    counts = np.bincount(r["topk_ids"].reshape(-1), minlength=s.E)
    assert (counts == 0).sum() >= 1
    assert counts.max() > 0.5 * 4096
    rank = np.round(np.exp(-lay["logit_bias"] / 1.1)).astype(int)
    assert sorted(rank.tolist()) == list(range(1, s.E + 1))


def test_mx_weights_cover_every_finite_e4m3_code():
    """MXFP8 weight codes are uniform over the 254 finite E4M3 codes (zeros,
    subnormals, exponent fields 1..15, +-448) and never NaN; the weights
    spread near 1/sqrt(K)."""
    from oracle import moe_oracle as mo
    lay = wl.make_mx_layer("toy", 3, E=2, top_k=1, H=512, I=256, seed=5)
    codes = np.concatenate([lay["w13_codes"].ravel(), lay["w2_codes"].ravel()])
    present = set(np.unique(codes).tolist())
    assert present == set(range(256)) - {0x7F, 0xFF}
    for c in (0x00, 0x80, 0x01, 0x07, 0x08, 0x7E, 0xFE):
        assert c in present
    w = mo.mx_dequantize(lay["w13_codes"][0], lay["w13_scales"][0])
    assert np.all(np.isfinite(w))
    assert 0.5 < w.std() * np.sqrt(512) < 2.0
