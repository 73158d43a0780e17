"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and its host-side logic (workspace sizes, tile table, argument
checks) behaves as documented.  No call here reaches the GPU: every call
either computes on the host or is rejected before any launch."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def _moe():
    import mixture_experts_ffn_renorm_amd as moe
    return moe


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    moe = _moe()
    lib = moe.library()
    names = declared_functions()
    assert set(names) >= {"moe_route", "moe_align", "moe_grouped_gemm_w13_act",
                          "moe_grouped_gemm_w2_combine", "moe_forward", "moe_workspace_size",
                          "moe_strerror", "moe_pick_block_m"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    # binding signatures cover exactly the declared calls
    assert set(moe._SIGNATURES) == set(names)


def test_strerror():
    moe = _moe()
    assert moe.moe_strerror(0) == "ok"
    assert "workspace" in moe.moe_strerror(-3)
    assert moe.moe_strerror(12345) == "unknown status"


def test_tile_table():
    moe = _moe()
    # per-pair GEMVs while M*top_k*4 <= E
    assert moe.moe_pick_block_m(1, 128, 8) == 1
    assert moe.moe_pick_block_m(4, 128, 8) == 1
    assert moe.moe_pick_block_m(5, 128, 8) == 16
    assert moe.moe_pick_block_m(3, 60, 4) == 1
    assert moe.moe_pick_block_m(0, 60, 4) == 16
    assert moe.moe_pick_block_m(64, 128, 8) == 16
    assert moe.moe_pick_block_m(16, 60, 4) == 16
    assert moe.moe_pick_block_m(512, 60, 4) == 64
    assert moe.moe_pick_block_m(1024, 60, 4) == 128
    assert moe.moe_pick_block_m(2048, 60, 4) == 256
    assert moe.moe_pick_block_m(4096, 128, 8) == 128
    assert moe.moe_pick_block_m(8192, 256, 8) == 128
    assert moe.moe_pick_block_m(8, 256, 8) == 1
    assert moe.moe_pick_block_m(9, 256, 8) == 16


def test_workspace_size_monotone_and_bounded():
    moe = _moe()
    prev = 0
    for M in (1, 2, 8, 64, 512, 4096, 8192):
        n = moe.moe_workspace_size(M, 256, 8, 2048, 512)
        assert n >= prev
        prev = n
    # act [P, I] bf16 + fp32 partial rows [P, H] dominate: ~604 MB at M = 8192
    n = moe.moe_workspace_size(8192, 256, 8, 2048, 512)
    P = 8192 * 8
    big = P * 512 * 2 + P * 2048 * 4
    assert big <= n <= 1.05 * big + (16 << 20)
    assert moe.moe_workspace_size(1, 600, 8, 2048, 512) == 0     # E > 512
    assert moe.moe_workspace_size(1, 128, 8, 2044, 512) == 0     # H % 8 != 0


NULL = None


@pytest.mark.parametrize("args,status", [
    ((NULL, NULL, NULL, NULL, NULL, -1, 128, 8, 2048, 768, 1), -1),     # M < 0
    ((NULL, NULL, NULL, NULL, NULL, 4, 128, 0, 2048, 768, 1), -1),      # top_k = 0
    ((NULL, NULL, NULL, NULL, NULL, 4, 4, 8, 2048, 768, 1), -1),        # top_k > E
    ((NULL, NULL, NULL, NULL, NULL, 4, 600, 8, 2048, 768, 1), -2),      # E > 512
    ((NULL, NULL, NULL, NULL, NULL, 4, 128, 40, 2048, 768, 1), -2),     # top_k > 32
    ((NULL, NULL, NULL, NULL, NULL, 4, 128, 8, 2044, 768, 1), -2),      # H % 8
    ((NULL, NULL, NULL, NULL, NULL, 4, 128, 8, 2048, 770, 1), -2),      # I % 8
    ((NULL, NULL, NULL, NULL, NULL, 4, 128, 8, 2048, 768, 2), -1),      # renormalize flag
    ((NULL, NULL, NULL, NULL, NULL, 4, 128, 8, 2048, 768, 1), -1),      # null pointers
    ((NULL, NULL, NULL, NULL, NULL, 0, 128, 8, 2048, 768, 1), 0),       # M = 0: no launch
])
def test_forward_argument_checks(args, status):
    lib = _moe().library()
    st = lib.moe_forward(*args, NULL, NULL, NULL, NULL, 0, NULL, NULL)
    assert st == status


def test_forward_workspace_too_small():
    lib = _moe().library()
    fake = ctypes.c_void_p(0x10000)      # never dereferenced: the size check fails first
    st = lib.moe_forward(fake, fake, NULL, fake, fake, 4, 128, 8, 2048, 768, 1, fake, NULL,
                         NULL, fake, 1024, NULL, NULL)
    assert st == -3
    st = lib.moe_forward(fake, fake, NULL, fake, fake, 4, 128, 8, 2048, 768, 1, fake, NULL,
                         NULL, NULL, 1 << 30, NULL, NULL)
    assert st == -3


def test_other_calls_argument_checks():
    moe = _moe()
    lib = moe.library()
    fake = ctypes.c_void_p(0x10000)
    info = moe.DispatchInfo()
    # align: block_m out of range, null outputs, M = 0
    assert lib.moe_align(fake, 4, 2, 8, 0, fake, fake, fake, NULL, NULL, 0, NULL) == -2
    assert lib.moe_align(fake, 4, 2, 8, 300, fake, fake, fake, NULL, NULL, 0, NULL) == -2
    assert lib.moe_align(fake, 4, 2, 8, 16, NULL, fake, fake, NULL, NULL, 0, NULL) == -1
    assert lib.moe_align(fake, 0, 2, 8, 16, NULL, NULL, NULL, NULL, NULL, 0, NULL) == 0
    # large batches need align scratch; small ones need none
    assert moe.moe_align_workspace_size(4, 2, 8) == 0
    assert moe.moe_align_workspace_size(8192, 8, 256) > 0
    assert lib.moe_align(fake, 8192, 8, 256, 16, fake, fake, fake, NULL, NULL, 0, NULL) == -3
    # GEMMs: block_m must be 1, 16, 64, 128 or 256
    assert lib.moe_grouped_gemm_w13_act(fake, fake, fake, fake, fake, 4, 2, 8, 64, 32, 32,
                                        fake, ctypes.byref(info), NULL) == -2
    assert lib.moe_grouped_gemm_w13_act(fake, fake, fake, fake, fake, 0, 2, 8, 64, 32, 16,
                                        fake, ctypes.byref(info), NULL) == 0
    assert info.variant == moe.MOE_VARIANT_STREAM and info.block_m == 16 and info.launches == 0
    assert lib.moe_grouped_gemm_w2_combine(fake, fake, fake, fake, fake, fake, 4, 2, 8, 64, 32,
                                           64, fake, fake, 16, ctypes.byref(info), NULL) == -3
    assert lib.moe_grouped_gemm_w2_combine(fake, fake, fake, fake, fake, fake, 0, 2, 8, 64, 32,
                                           64, fake, NULL, 0, ctypes.byref(info), NULL) == 0
    assert info.variant == moe.MOE_VARIANT_TILED and info.block_k == 64
    # route: needs a logits buffer or a workspace
    assert lib.moe_route(fake, fake, NULL, 4, 64, 8, 2, 1, fake, fake, NULL, NULL, 0, NULL) == -3
    assert lib.moe_route(fake, fake, NULL, 4, 64, 8, 9, 1, fake, fake, NULL, NULL, 0, NULL) == -1


def test_dispatch_info_forward_readout():
    moe = _moe()
    lib = moe.library()
    info = moe.DispatchInfo()
    assert lib.moe_forward(NULL, NULL, NULL, NULL, NULL, 0, 60, 4, 2048, 1408, 1, NULL, NULL,
                           NULL, NULL, 0, ctypes.byref(info), NULL) == 0
    assert info.variant == moe.MOE_VARIANT_STREAM and info.k_tail == 1


@pytest.mark.parametrize("bits,group,H,I,M,status", [
    (5, 64, 2048, 768, 4, -2),        # bits must be 4 or 8
    (4, 32, 2048, 768, 4, -2),        # groups of 64 only
    (4, 64, 2048 + 8, 768, 4, -2),    # H % 64
    (8, 64, 2048, 768 + 8, 4, -2),    # I % 64
    (4, 64, 2048, 768, 4, -1),        # null pointers
    (8, 64, 2048, 768, 0, 0),         # M = 0: no launch
])
def test_forward_quantized_argument_checks(bits, group, H, I, M, status):
    moe = _moe()
    lib = moe.library()
    qw = moe.QuantizedWeights(bits, group)
    info = moe.DispatchInfo()
    st = lib.moe_forward_quantized(NULL, NULL, NULL, ctypes.byref(qw), M, 128, 8, H, I, 1,
                                   NULL, NULL, NULL, NULL, 0, ctypes.byref(info), NULL)
    assert st == status
    if status == 0:
        assert info.launches == 0
        assert info.variant in (moe.MOE_VARIANT_PAIR_GEMV_QUANT, moe.MOE_VARIANT_STREAM_QUANT)


@pytest.mark.parametrize("M,H,I,variant,launches", [
    (1, 2048, 768, "pair", 4),          # M*top_k*4 <= E: per-pair GEMVs
    (64, 2048, 768, "stream", 5),       # router, fused top-k + lists, GEMM 1, GEMM 2, sum
    (128, 2048, 768, "stream", 5),      # 8 pairs per expert: still streaming
    (256, 2048, 768, "tiled", 5),       # 16 pairs per expert: tiles
    (512, 4096, 768, "tiled", 7),       # 4096 pairs: top-k, count, scatter launches
    (64, 2048 + 64, 768, "pair", 4),    # H % 128 != 0: per-pair GEMVs at any M
    (64, 2048, 768 + 64, "pair", 4),
    (1024, 2048, 768, "tiled", 7),      # 64 pairs per expert: bf16 tiles widened in LDS
    (4096, 2048, 768, "tiled", 7),
    (1024, 2048 + 64, 768 + 64, "tiled", 7),   # the tiles take H, I % 64
])
def test_forward_quantized_dispatch(M, H, I, variant, launches):
    """The dispatch report is filled before any pointer is looked at."""
    moe = _moe()
    lib = moe.library()
    qw = moe.QuantizedWeights(4, 64)
    info = moe.DispatchInfo()
    st = lib.moe_forward_quantized(NULL, NULL, NULL, ctypes.byref(qw), M, 128, 8, H, I, 1,
                                   NULL, NULL, NULL, NULL, 0, ctypes.byref(info), NULL)
    assert st == -1
    want = {"stream": moe.MOE_VARIANT_STREAM_QUANT, "tiled": moe.MOE_VARIANT_TILED_QUANT,
            "pair": moe.MOE_VARIANT_PAIR_GEMV_QUANT}[variant]
    assert info.variant == want and info.launches == launches
    assert info.block_m == {"stream": 16, "tiled": 128, "pair": 1}[variant]
    assert info.sorted == int(variant != "pair")


def test_forward_quantized_null_struct_and_workspace():
    moe = _moe()
    lib = moe.library()
    assert lib.moe_forward_quantized(NULL, NULL, NULL, NULL, 4, 128, 8, 2048, 768, 1, NULL, NULL,
                                     NULL, NULL, 0, NULL, NULL) == -1
    fake = ctypes.c_void_p(0x10000)      # never dereferenced: the size check fails first
    qw = moe.QuantizedWeights(4, 64, *([0x10000] * 6))
    assert lib.moe_forward_quantized(fake, fake, NULL, ctypes.byref(qw), 4, 128, 8, 2048, 768, 1,
                                     fake, NULL, NULL, fake, 1024, NULL, NULL) == -3


@pytest.mark.parametrize("H,I,M,status", [
    (2048, 768, 4, -1),          # null pointers
    (2048 + 64, 768, 4, -2),     # H % 128
    (2048, 768 + 32, 4, -2),     # I % 128
    (2048, 768, 0, 0),           # M = 0: no launch
])
def test_forward_mxfp8_argument_checks(H, I, M, status):
    moe = _moe()
    lib = moe.library()
    w = moe.MxWeights()
    info = moe.DispatchInfo()
    st = lib.moe_forward_mxfp8(NULL, NULL, NULL, ctypes.byref(w), M, 128, 8, H, I, 1, NULL, NULL,
                               NULL, NULL, 0, ctypes.byref(info), NULL)
    assert st == status
    if status == 0:
        assert info.variant == moe.MOE_VARIANT_STREAM_MXFP8 and info.launches == 0
        assert info.block_m == 16


def test_mx_workspace_and_quantize_checks():
    moe = _moe()
    lib = moe.library()
    assert moe.moe_mx_workspace_size(64, 128, 8, 2048, 768) >= moe.moe_workspace_size(64, 128, 8, 2048, 768)
    assert moe.moe_mx_workspace_size(64, 128, 8, 2048 + 64, 768) == 0
    fake = ctypes.c_void_p(0x10000)
    assert lib.moe_mx_quantize(fake, 4, 48, fake, fake, NULL) == -2        # K % 32
    assert lib.moe_mx_quantize(NULL, 4, 64, fake, fake, NULL) == -1
    assert lib.moe_mx_quantize(NULL, 0, 64, NULL, NULL, NULL) == 0
    assert lib.moe_forward_mxfp8(NULL, NULL, NULL, NULL, 4, 128, 8, 2048, 768, 1, NULL, NULL,
                                 NULL, NULL, 0, NULL, NULL) == -1
    w = moe.MxWeights(*([0x10000] * 4))
    assert lib.moe_forward_mxfp8(fake, fake, NULL, ctypes.byref(w), 4, 128, 8, 2048, 768, 1, fake,
                                 NULL, NULL, fake, 1024, NULL, NULL) == -3


def test_forward_list_offsets():
    """Where moe_forward leaves its index lists: inside the workspace,
    non-overlapping, at the tile table's block size; no lists for the
    per-pair batches."""
    moe = _moe()
    E, k, H, I = 128, 8, 2048, 768
    o = moe.moe_forward_list_offsets(1, E, k, H, I)
    assert o["sorted"] == 0 and o["block_m"] == 1
    for M in (16, 64, 512, 4096):
        o = moe.moe_forward_list_offsets(M, E, k, H, I)
        B = moe.moe_pick_block_m(M, E, k)
        assert o["sorted"] == 1 and o["block_m"] == B
        cap, nbl = moe.align_capacity(M * k, E, B)
        spans = sorted([(o["sorted_token_ids"], 4 * cap), (o["expert_ids"], 4 * nbl),
                        (o["expert_block_offsets"], 4 * (E + 1)), (o["expert_counts"], 4 * E)])
        for (a, n), (b, _) in zip(spans, spans[1:]):
            assert a + n <= b
        assert spans[-1][0] + spans[-1][1] <= moe.moe_workspace_size(M, E, k, H, I)
        assert all(off % 16 == 0 for off, _ in spans)
    import ctypes
    assert moe.library().moe_forward_list_offsets(4, E, k, H, I, None) == -1
    lists = moe.ForwardLists()
    assert moe.library().moe_forward_list_offsets(4, E, 0, H, I, ctypes.byref(lists)) == -1
