"""Pins of the oracle's MXFP8 functions (CPU only).

The MLX part of the page "SGLang issue #22283" names MXFP8; the format is
the OCP Microscaling one (32-element blocks, one E8M0 power-of-two scale
each, FP8 E4M3 elements).  Each oracle function is pinned to something
other than itself:
  * E4M3 decoding against torch's float8_e4m3fn (a library routine) on all
    256 codes;
  * E4M3 rounding against torch's float32 -> float8_e4m3fn cast (round to
    nearest even) on random values, grid points and exact midpoints, and
    the saturation rule in closed form;
  * fp32-then-bf16 rounding against torch's casts;
  * block quantization against closed forms (a block whose largest value is
    1 gets the scale code 119 and 1.0 -> 0x78; an all-zero block gets scale
    code 0; values on the scaled E4M3 grid round-trip exactly, block by
    block with different scales; tiny blocks clamp the scale; the error
    bound of round to nearest);
  * the layer against the pinned bf16 oracle functions (pair_activations,
    combine_from_act) fed with the MX-dequantized x and weights, which bf16
    holds exactly;
and planted mistakes (scale exponent off by one, ties away from even, a
bias-8 E4M3 decoding, the scales of the wrong block, act not re-quantized)
are each caught by the battery.
"""

from __future__ import annotations

import numpy as np
import pytest

import moe_workloads as wl
from oracle import moe_oracle as mo


def _torch():
    import torch
    return torch


def check_decode_matches_torch():
    torch = _torch()
    c = np.arange(256, dtype=np.uint8)
    v = mo.e4m3_value(c)
    t = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(v), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(v[ok], t[ok])
    # a few values by hand: 1.0, 448, the smallest subnormal, -2
    assert mo.e4m3_value(np.array([0x38, 0x7E, 0x01, 0xC0])).tolist() == [1.0, 448.0, 2.0 ** -9, -2.0]


def _round_inputs():
    rng = np.random.default_rng(11)
    r = (rng.standard_normal(20000) * np.exp2(rng.integers(-14, 9, 20000))).astype(np.float32)
    r = np.clip(r, -448, 448)
    grid = mo.e4m3_value(np.arange(0x7F)).astype(np.float32)
    mids = ((grid[1:].astype(np.float64) + grid[:-1]) / 2).astype(np.float32)   # exact in fp32
    return np.concatenate([r, grid, -grid, mids, -mids]).astype(np.float64)


def check_round_matches_torch():
    torch = _torch()
    v = _round_inputs()
    ours = mo.e4m3_round(v)
    theirs = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)
    # saturation: anything at or beyond 448 in magnitude is +-448
    assert mo.e4m3_round(np.array([448.0, 460.0, 1e6, -500.0])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    # sign kept when rounding to zero
    assert mo.e4m3_round(np.array([-1e-9, 1e-9])).tolist() == [0x80, 0x00]


def check_bf16_rounding_matches_torch():
    torch = _torch()
    rng = np.random.default_rng(12)
    v = rng.standard_normal(5000) * np.exp2(rng.integers(-20, 20, 5000))
    ours = mo.round_to_bf16_via_f32(v)
    theirs = torch.from_numpy(v).float().bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def check_quantize_closed_forms():
    # largest value 1: scale 2^(0 - 8), code 119; 1.0 / 2^-8 = 256 -> 0x78
    v = np.zeros(32)
    v[0], v[5] = 1.0, -0.5
    q, s = mo.mx_quantize(v)
    assert s.tolist() == [119] and q[0] == 0x78 and q[5] == 0xF0 and np.all(q[[1, 2, 31]] == 0)
    # all-zero block
    q, s = mo.mx_quantize(np.zeros(64))
    assert s.tolist() == [0, 0] and np.all(q == 0)
    # values on the scaled grid round-trip, with a different scale per block
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 0x7F, size=(3, 128)).astype(np.uint8) | \
        (rng.integers(0, 2, size=(3, 128)).astype(np.uint8) << 7)
    codes[:, ::32] = 0x7E                             # each block reaches 448
    scales = rng.integers(100, 150, size=(3, 4)).astype(np.uint8)
    vals = mo.mx_dequantize(codes, scales)
    q, s = mo.mx_quantize(vals)
    assert np.array_equal(s, scales)
    assert np.array_equal(mo.mx_dequantize(q, s), vals)
    # tiny block: the scale clamps at 2^-127
    _, s = mo.mx_quantize(np.full(32, 2.0 ** -140))
    assert s.tolist() == [0]
    # round to nearest: error at most half an E4M3 step (1/16 relative in
    # the normal range, 2^-10 scale units below it), plus what saturation at
    # 448 scale units cuts off the block's largest values (the scale puts
    # them in [256, 512) units)
    v = rng.standard_normal((40, 256))
    q, s = mo.mx_quantize(v)
    d = mo.mx_dequantize(q, s)
    X = np.repeat(mo.e8m0_value(s), 32, axis=-1)
    tol = np.maximum(np.abs(v) / 16, X * 2.0 ** -10) + np.maximum(0.0, np.abs(v) - 448 * X)
    assert np.all(np.abs(d - v) <= tol * (1 + 1e-12))
    assert np.all(np.abs(d) <= 448 * X)


def _bf16_bits_exact(v):
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)                    # exactly a bf16 value
    return (b >> 16).astype(np.uint16)


def check_layer_against_bf16_oracle():
    lay = wl.make_mx_layer("toy", 5, E=4, top_k=2, H=64, I=64, seed=21)
    res = mo.forward_mxfp8(lay)
    r = res["route"]
    xd = mo.mx_dequantize(*mo.mx_quantize(mo.widen_bf16(lay["x"])))
    w13 = _bf16_bits_exact(mo.mx_dequantize(lay["w13_codes"], lay["w13_scales"]))
    w2 = _bf16_bits_exact(mo.mx_dequantize(lay["w2_codes"], lay["w2_scales"]))
    ids, wts = r["topk_ids"], r["topk_weights"]
    act = mo.pair_activations(_bf16_bits_exact(xd), w13, ids)
    act16 = mo.widen_bf16(mo.round_to_bf16_via_f32(act))
    actd = mo.mx_dequantize(*mo.mx_quantize(act16))
    y = mo.combine_from_act(_bf16_bits_exact(actd), w2, ids, wts)
    assert np.allclose(res["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


CHECKS = (check_decode_matches_torch, check_round_matches_torch, check_bf16_rounding_matches_torch,
          check_quantize_closed_forms, check_layer_against_bf16_oracle)


def _battery() -> bool:
    for c in CHECKS:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


_orig_quant = mo.mx_quantize
_orig_round = mo.e4m3_round
_orig_value = mo.e4m3_value
_orig_deq = mo.mx_dequantize


def _quant_scale_off_by_one(v, block=32):
    # scale exponent floor(log2 amax) - 7: twice the spec's scale
    v = np.asarray(v, dtype=np.float64)
    _, s = _orig_quant(v, block)
    s2 = (s.astype(np.int64) + 1).clip(0, 254).astype(np.uint8)
    return mo.e4m3_round(v / np.repeat(mo.e8m0_value(s2), block, axis=-1)), s2


def _round_ties_away(v):
    v = np.asarray(v, dtype=np.float64)
    grid = mo._E4M3_GRID
    a = np.abs(v)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 1, 0x7E)
    lo = hi - 1
    mag = np.where(grid[hi] - a <= a - grid[lo], hi, lo)
    mag = np.where(a >= grid[0x7E], 0x7E, mag)
    return (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _value_bias8(codes):
    return _orig_value(codes) / 2.0


def _deq_wrong_block(codes, scales, block=32):
    s = np.asarray(scales)
    return _orig_deq(codes, np.roll(s, 1, axis=-1), block)


def _forward_act_not_requantized(layer, tokens=None):
    saved = mo.mx_quantize
    calls = {"n": 0}

    def q(v, block=32):
        calls["n"] += 1
        if calls["n"] > 1:                      # every call after x's: act left as is
            v = np.asarray(v, dtype=np.float64)
            return _orig_quant(v, block)[0] * 0 + mo.e4m3_round(v / 2.0 ** -6), \
                np.full(v.shape[:-1] + (v.shape[-1] // block,), 121, np.uint8)
        return _orig_quant(v, block)
    mo.mx_quantize = q
    try:
        return _orig_forward(layer, tokens)
    finally:
        mo.mx_quantize = saved


_orig_forward = mo.forward_mxfp8

MUTANTS = {
    "scale_exponent_off_by_one": ("mx_quantize", _quant_scale_off_by_one),
    "ties_away_from_even": ("e4m3_round", _round_ties_away),
    "e4m3_bias_8": ("e4m3_value", _value_bias8),
    "scales_of_the_wrong_block": ("mx_dequantize", _deq_wrong_block),
    "act_not_requantized": ("forward_mxfp8", _forward_act_not_requantized),
}


def test_battery_passes_on_oracle():
    assert _battery()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(mo, attr, fn)
    if attr == "e4m3_value":
        monkeypatch.setattr(mo, "_E4M3_ALL", fn(np.arange(256)))
        monkeypatch.setattr(mo, "_E4M3_GRID", fn(np.arange(0x7F)))
    assert not _battery(), f"planted mistake {name} passed every pin"


# ---------------------------------------------------------------------------
# The GPU tests' acceptance of act quantization decisions that either side
# could take (tests.helpers.mx_ambiguous_act_choices / mx_boundary_reference):
# it must find exactly the decisions one rounding step could flip, and it
# must not accept an output that no such decision explains.

def test_ambiguous_act_choices_finds_the_flippable_element():
    from tests import helpers as h
    rng = np.random.default_rng(5)
    a = rng.normal(size=64)
    a[0] = 4.0                                    # block 0's scale: 2^(2 - 8)
    # 68.25 scale units: just above the midpoint of bf16 1.0625 (68 units, a
    # tie of E4M3 64 and 72 that goes to the even code 64) and 1.0703125
    # (68.5 units -> 72); one fp32 step either way decides the code
    a[5] = 1.06640625 * (1.0 + 2.0 ** -20)
    base_bits = mo.round_to_bf16_via_f32(a)
    choices = h.mx_ambiguous_act_choices(a)
    assert choices is not None and len(choices) >= 2
    flips = [np.flatnonzero(c != mo.widen_bf16(base_bits)) for c in choices[1:]]
    assert any(list(f) == [5] for f in flips)
    five = [c[5] for c in choices]
    assert set(five) == {1.0703125, 1.0625}
    # the two decisions give different codes
    assert mo.mx_quantize(choices[0])[0][5] != mo.mx_quantize(choices[1])[0][5]


def test_ambiguous_act_choices_ignores_values_far_from_midpoints():
    from tests import helpers as h
    v = np.full(32, 1.0)                         # bf16-exact, far from every midpoint
    v[3] = 2.0
    assert len(h.mx_ambiguous_act_choices(v)) == 1


def test_boundary_reference_rejects_a_planted_error():
    from tests import helpers as h
    lay = wl.make_mx_layer("toy", 6, E=4, top_k=2, H=128, I=128, seed=41)
    toks = np.arange(6)
    r = mo.route(lay["x"], lay["w_router"], 2, lay["renormalize"], lay.get("logit_bias"))
    ids, w = r["topk_ids"], r["topk_weights"]
    ref, _, _ = mo.mx_layer_forward(lay, ids, w, toks)
    y = ref.copy()
    y[2, 17] += 0.05 * np.abs(ref).max()        # a wrong element no act decision explains
    got = h.mx_boundary_reference(lay, ids, w, toks, y, ref)
    assert np.array_equal(got, ref)
    with pytest.raises(AssertionError):
        h.assert_close_outputs(y, got, "planted")
    # the exact oracle output passes untouched
    assert np.array_equal(h.mx_boundary_reference(lay, ids, w, toks, ref, ref), ref)
