"""Pins of the oracle's group-quantized weights (CPU only).

The oracle reads the affine group format that the MLX part of the page
"SGLang issue #22283" names (64-element
groups, 4 or 8 bits; w = s * q + b per group, codes packed least significant
first into 32-bit words).  Each function is pinned to something other than
itself:
  * code unpacking against an independent bit-stream decode (the words as
    one little-endian integer, element i = bits [bits*i, bits*(i+1)));
  * dequantization against closed forms (zero codes give the biases, unit
    scales and zero biases give the codes, the scale changes exactly at a
    64-element group boundary);
  * the quantized layer against the bf16 layer (already pinned by
    ``test_oracle_pins``) on weights that the quantized format represents
    exactly, bit for bit;
and planted mistakes (most significant code first, groups shifted by one
element, scale and bias swapped, the wrong expert's matrix) are each
caught by the battery.
"""

from __future__ import annotations

import numpy as np
import pytest

import moe_workloads as wl
from oracle import moe_oracle as mo


def bitstream_decode(words: np.ndarray, bits: int, K: int) -> np.ndarray:
    out = np.empty(words.shape[:-1] + (K,), dtype=np.int64)
    mask = (1 << bits) - 1
    for idx in np.ndindex(*words.shape[:-1]):
        big = int.from_bytes(np.ascontiguousarray(words[idx], dtype="<u4").tobytes(), "little")
        for i in range(K):
            out[idx + (i,)] = (big >> (bits * i)) & mask
    return out


def check_unpack_bitstream():
    rng = np.random.default_rng(3)
    for bits in (4, 8):
        per = 32 // bits
        words = rng.integers(0, 2 ** 32, size=(3, 5), dtype=np.uint64).astype(np.uint32)
        K = 5 * per
        assert np.array_equal(mo.unpack_codes(words, bits, K), bitstream_decode(words, bits, K))


def _bf16(v: float) -> int:
    return int(wl.f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])


def check_dequant_closed_forms():
    rng = np.random.default_rng(4)
    for bits in (4, 8):
        K = 128
        codes = rng.integers(0, 1 << bits, size=(2, K), dtype=np.uint32)
        words = wl._pack_codes(codes, bits)
        # zero codes: every weight is its group's bias
        zero = wl._pack_codes(np.zeros_like(codes), bits)
        s = np.full((2, 2), _bf16(0.5), dtype=np.uint16)
        b = np.array([[_bf16(-0.25), _bf16(0.75)], [_bf16(1.5), _bf16(-2.0)]], dtype=np.uint16)
        w0 = mo.dequantize_affine(zero, s, b, bits, K)
        assert np.array_equal(w0[:, :64], np.repeat(mo.widen_bf16(b)[:, :1], 64, axis=1))
        assert np.array_equal(w0[:, 64:], np.repeat(mo.widen_bf16(b)[:, 1:], 64, axis=1))
        # unit scales, zero biases: the weights are the codes
        one = np.full((2, 2), _bf16(1.0), dtype=np.uint16)
        zb = np.zeros((2, 2), dtype=np.uint16)
        assert np.array_equal(mo.dequantize_affine(words, one, zb, bits, K), codes)
        # the scale switches exactly between elements 63 and 64
        s2 = np.array([[_bf16(1.0), _bf16(2.0)]] * 2, dtype=np.uint16)
        w2 = mo.dequantize_affine(words, s2, zb, bits, K)
        assert np.array_equal(w2[:, :64], codes[:, :64]) and np.array_equal(w2[:, 64:], 2 * codes[:, 64:])


def exact_pair(M=3, E=4, top_k=2, H=128, I=64, seed=8):
    """A quantized layer whose weights w = (q - 128) / 128 are exact in bf16,
    and the bf16 layer holding those same weights."""
    lay = wl.make_layer("toy", M, E=E, top_k=top_k, H=H, I=I, seed=seed)
    rng = np.random.default_rng(seed)
    s = _bf16(1.0 / 128.0)
    b = _bf16(-1.0)
    q = {}
    for name, rows, K in (("w13", 2 * I, H), ("w2", H, I)):
        codes = rng.integers(0, 256, size=(E, rows, K), dtype=np.uint32)
        q[name] = codes
        lay[name] = wl.f32_to_bf16_bits(((codes.astype(np.float64) - 128.0) / 128.0).astype(np.float32))
    ql = dict(lay)
    for name, K in (("w13", H), ("w2", I)):
        codes = q[name]
        ql[name + "_q"] = wl._pack_codes(codes, 8)
        ql[name + "_scales"] = np.full(codes.shape[:2] + (K // 64,), s, dtype=np.uint16)
        ql[name + "_biases"] = np.full(codes.shape[:2] + (K // 64,), b, dtype=np.uint16)
    ql["bits"] = 8
    return ql, lay


def check_quantized_layer_equals_bf16_layer():
    ql, lay = exact_pair()
    rq = mo.forward_quantized(ql)
    rb = mo.forward(lay)
    assert np.array_equal(rq["route"]["topk_ids"], rb["route"]["topk_ids"])
    assert np.array_equal(rq["y"], rb["y"])


def _battery() -> bool:
    for c in (check_unpack_bitstream, check_dequant_closed_forms,
              check_quantized_layer_equals_bf16_layer):
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


def test_unpack_matches_bitstream():
    check_unpack_bitstream()


def test_dequantize_closed_forms():
    check_dequant_closed_forms()


def test_quantized_layer_equals_bf16_layer():
    check_quantized_layer_equals_bf16_layer()


def test_generator_scale_and_format():
    """The seeded quantized layers: codes in range, groups of 64, weights
    with a variance near 1/K."""
    ql = wl.make_quantized_layer("qwen15", 2, 4, E=4, H=256, I=192, seed=5)
    assert ql["w13_q"].shape == (4, 384, 256 * 4 // 32)
    assert ql["w2_scales"].shape == (4, 256, 3)
    W = mo.dequantize_affine(ql["w13_q"][1], ql["w13_scales"][1], ql["w13_biases"][1], 4, 256)
    assert 0.7 < W.std() * np.sqrt(256) < 1.4


_orig_unpack = mo.unpack_codes
_orig_dequant = mo.dequantize_affine
_orig_dq_experts = mo.DequantizedExperts


def _unpack_msb_first(words, bits, K):
    per = 32 // bits
    q = _orig_unpack(words, bits, (np.asarray(words).shape[-1]) * per)
    q = q.reshape(*q.shape[:-1], -1, per)[..., ::-1].reshape(q.shape)
    return q[..., :K]


def _dequant_groups_shifted(words, scales, biases, bits, K, group=64):
    q = mo.unpack_codes(words, bits, K).astype(np.float64)
    S = np.roll(np.repeat(mo.widen_bf16(scales), group, axis=-1)[..., :K], 1, axis=-1)
    B = np.roll(np.repeat(mo.widen_bf16(biases), group, axis=-1)[..., :K], 1, axis=-1)
    return S * q + B


def _dequant_scale_bias_swapped(words, scales, biases, bits, K, group=64):
    return _orig_dequant(words, biases, scales, bits, K, group)


class _ExpertsOffByOne(_orig_dq_experts):
    def __getitem__(self, e):
        return super().__getitem__((e + 1) % self.words.shape[0])


MUTANTS = {
    "codes_msb_first": ("unpack_codes", _unpack_msb_first),
    "groups_shifted_by_one": ("dequantize_affine", _dequant_groups_shifted),
    "scale_bias_swapped": ("dequantize_affine", _dequant_scale_bias_swapped),
    "expert_index_off_by_one": ("DequantizedExperts", _ExpertsOffByOne),
}


def test_battery_passes_on_oracle():
    assert _battery()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(mo, attr, fn)
    assert not _battery(), f"planted mistake {name} passed every pin"
