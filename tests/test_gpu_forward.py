"""GPU parity of the whole layer (moe_forward) against the CPU oracle on
every workload shape, plus the layer's special cases and robustness checks.

Routing ids are compared bit-exactly on tokens whose top-k logit margin
exceeds 1e-4 and checked for validity on the others; the outputs of every
sampled token are compared, with the max-abs and mean-relative criteria,
against the oracle's expert layer run on the GPU's own ids with the oracle's
weights for those ids (so near-tie tokens are checked too).  At the large
batch sizes the oracle checks a seeded sample of tokens (it computes them one
expert group at a time)."""

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


def run_forward(lay: dict, ws=None, out=None):
    import torch
    moe = _moe()
    d = h.layer_to_device(lay)
    M, k = lay["M"], lay["top_k"]
    ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    wts = torch.full((M, k), -1.0, dtype=torch.float32, device="cuda")
    out, info = moe.moe_forward(d["x"], d["w_router"], d["w13"], d["w2"], k,
                                lay["renormalize"], logit_bias=d["logit_bias"], out=out,
                                topk_ids_out=ids, topk_weights_out=wts, ws=ws)
    torch.cuda.synchronize()
    return out, ids.cpu().numpy(), wts.cpu().numpy().astype(np.float64), info


def check_forward(lay: dict, n_tokens: int = 256, seed: int = 0, **kw):
    out, ids, wts, info = run_forward(lay, **kw)
    M = lay["M"]
    toks = h.sample_tokens(M, n_tokens, seed)
    r = mo.route(lay["x"][toks], lay["w_router"], lay["top_k"], lay["renormalize"],
                 lay.get("logit_bias"))
    w_ref = h.check_routing(ids[toks], wts[toks], r, lay["renormalize"])
    full_ids, full_w = h.scatter_routing(M, toks, ids[toks], w_ref)
    ref_y = mo.layer_forward(lay["x"], lay["w13"], lay["w2"], full_ids, full_w, toks)
    y = h.host_bf16_to_f64(out)[toks]
    h.assert_close_outputs(y, ref_y)
    return info, out


FORWARD_CASES = [("toy", 3)] + [("qwen3_decode", m) for m in (1, 2, 4, 8, 16, 64)] + \
    [("qwen3_prefill", 4096)] + [("qwen15", m) for m in (1, 16, 512, 2048)] + \
    [("wide256", m) for m in (1, 8, 8192)]


@pytest.mark.parametrize("name,M", FORWARD_CASES)
def test_forward_workloads(name, M):
    moe = _moe()
    lay = wl.make_layer(name, M)
    info, _ = check_forward(lay)
    check_dispatch(lay, info)
    if (name, M) in (("qwen3_decode", 1), ("qwen3_decode", 4), ("wide256", 1), ("wide256", 8),
                     ("qwen15", 1)):
        assert info["variant"] == moe.MOE_VARIANT_PAIR_GEMV
    if (name, M) in (("qwen3_decode", 8), ("qwen3_decode", 64), ("qwen15", 16)):
        assert info["variant"] == moe.MOE_VARIANT_STREAM
    if (name, M) in (("qwen3_prefill", 4096), ("wide256", 8192)):
        assert info["variant"] == moe.MOE_VARIANT_TILED
    if name == "qwen15" and info["block_m"] == 16:
        assert info["k_tail"] == 1       # I = 1408 is not a multiple of 256


def check_dispatch(lay: dict, info: dict):
    """What moe_forward reports it ran: small batches (M*top_k*4 <= E) skip
    the sort and run per-pair GEMVs (four launches, no index lists); the
    others use the tile table's block size."""
    moe = _moe()
    M, E, k = lay["M"], lay["E"], lay["top_k"]
    if M * k * 4 <= E:
        assert info["variant"] == moe.MOE_VARIANT_PAIR_GEMV
        assert info["sorted"] == 0 and info["block_m"] == 1 and info["launches"] == 4
    else:
        B = moe.moe_pick_block_m(M, E, k)
        assert info["block_m"] == B and info["sorted"] == 1
        assert info["variant"] == (moe.MOE_VARIANT_STREAM if B == 16 else moe.MOE_VARIANT_TILED)
    bk = info["block_k"]
    assert info["k_tail"] == int(lay["H"] % bk != 0 or lay["I"] % bk != 0)


# Per-pair GEMV shapes beyond the workloads: K over several 2048-element
# passes with a ragged last pass (H = 4104), I not a multiple of the 16
# features of a GEMM 1 workgroup, top_k above the 8 waves of GEMM 2 (slots
# loop), the largest top_k, and top_k = 1.
PAIR_GEMV_CASES = [
    dict(M=2, E=64, top_k=2, H=4104, I=520, seed=21),
    dict(M=2, E=128, top_k=12, H=256, I=136, seed=22),
    dict(M=1, E=512, top_k=32, H=1032, I=64, seed=23),
    dict(M=3, E=16, top_k=1, H=64, I=32, seed=24),
    dict(M=4, E=32, top_k=2, H=2048, I=1416, seed=25),
]


@pytest.mark.parametrize("case", PAIR_GEMV_CASES, ids=lambda c: "M{M}_E{E}_k{top_k}_H{H}_I{I}".format(**c))
def test_forward_pair_gemv_shapes(case):
    c = dict(case)
    M = c.pop("M")
    lay = wl.make_layer("toy", M, **c)
    info, _ = check_forward(lay)
    check_dispatch(lay, info)
    assert info["variant"] == _moe().MOE_VARIANT_PAIR_GEMV


@pytest.mark.parametrize("M", [16, 64])
def test_forward_exact_ties_across_lane_blocks(M):
    """Ties through the fused top-k + index-list launch (one and several
    workgroups)."""
    from tests.test_gpu_route_align import check_tied_order, tie_layer
    lay = tie_layer(M)
    _, ids, wts, _ = run_forward(lay)
    ref = mo.route(lay["x"], lay["w_router"], lay["top_k"], True, None)
    assert check_tied_order(ids, ref["topk_ids"]) >= 2
    ok = ref["margin"] > h.MARGIN
    assert np.array_equal(ids[ok], ref["topk_ids"][ok])
    assert np.abs(wts[ok] - ref["topk_weights"][ok]).max() <= h.WEIGHT_TOL


def test_forward_exact_ties_in_pair_gemv():
    """Ties through the per-pair path (router, top-k launch, GEMVs reading
    the top-k ids directly)."""
    from tests.test_gpu_route_align import check_tied_order, tie_layer
    lay = tie_layer(4)
    out, ids, wts, info = run_forward(lay)
    assert info["variant"] == _moe().MOE_VARIANT_PAIR_GEMV
    ref = mo.route(lay["x"], lay["w_router"], lay["top_k"], True, None)
    assert check_tied_order(ids, ref["topk_ids"]) >= 2
    w_ref = h.check_routing(ids, wts, ref, True)
    y_ref = mo.layer_forward(lay["x"], lay["w13"], lay["w2"], ids, w_ref)
    h.assert_close_outputs(h.host_bf16_to_f64(out), y_ref)


def test_forward_pair_gemv_renormalize_off():
    lay = wl.make_layer("toy", 2, E=64, top_k=4, H=256, I=128, seed=26)
    lay["renormalize"] = False
    info, _ = check_forward(lay)
    assert info["variant"] == _moe().MOE_VARIANT_PAIR_GEMV


def test_forward_all_logits_equal():
    """Zero router: every token keeps experts 0..k-1 with weight 1/k, so the
    layer equals the mean of those experts' FFNs."""
    lay = wl.make_layer("qwen3_decode", 16)
    lay["w_router"][:] = 0
    _, ids, wts, _ = run_forward(lay)
    k = lay["top_k"]
    assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (16, 1)))
    assert np.abs(wts - 1.0 / k).max() <= 1e-6
    out, _, _, _ = run_forward(lay)
    xw = mo.widen_bf16(lay["x"])
    ref = sum(mo.expert_ffn(xw, lay["w13"][e], lay["w2"][e]) for e in range(k)) / k
    h.assert_close_outputs(h.host_bf16_to_f64(out), ref)


def test_forward_zipf_prefill_has_empty_experts():
    """The skewed prefill layer routes no pair to some experts and very many
    to a few; the layer output still matches."""
    lay = wl.make_layer("qwen3_prefill", 4096)
    _, ids, _, _ = run_forward(lay)
    counts = np.bincount(ids.reshape(-1), minlength=lay["E"])
    assert (counts == 0).sum() >= 1 and counts.max() > 2048


def test_forward_dense_single_expert():
    """E = 1, top_k = 1: a dense SwiGLU FFN."""
    lay = wl.make_layer("toy", 33, E=1, top_k=1, H=128, I=64, seed=9)
    check_forward(lay)


def test_forward_identical_experts():
    lay = wl.make_layer("toy", 40, E=8, top_k=3, H=128, I=64, seed=10)
    lay["w13"][:] = lay["w13"][0]
    lay["w2"][:] = lay["w2"][0]
    out, _, _, _ = run_forward(lay)
    f = mo.expert_ffn(mo.widen_bf16(lay["x"]), lay["w13"][0], lay["w2"][0])
    h.assert_close_outputs(h.host_bf16_to_f64(out), f)


def test_forward_renormalize_off_and_k_equals_E():
    lay = wl.make_layer("toy", 3)
    lay["renormalize"] = False
    check_forward(lay)
    lay = wl.make_layer("toy", 5, top_k=4, seed=12)
    check_forward(lay)


def test_forward_zero_tokens():
    import torch
    moe = _moe()
    lay = wl.make_layer("toy", 3)
    d = h.layer_to_device(lay)
    x0 = d["x"][:0]
    out, info = moe.moe_forward(x0, d["w_router"], d["w13"], d["w2"], 2, True)
    torch.cuda.synchronize()
    assert out.shape == (0, 64) and info["launches"] == 0


@pytest.mark.parametrize("M", [16, 2])
def test_forward_poisoned_workspace_and_guard_bands(M):
    """Workspace filled with NaN bytes before the call; output rows written
    through a view with canary rows on both sides (sorted path and per-pair
    GEMVs)."""
    import torch
    moe = _moe()
    lay = wl.make_layer("qwen3_decode", M)
    M, H = lay["M"], lay["H"]
    ws = moe.workspace(M, lay["E"], lay["top_k"], H, lay["I"])
    ws.fill_(0xFF)
    buf = torch.full((M + 2, H), 7.0, dtype=torch.bfloat16, device="cuda")
    check_forward(lay, ws=ws, out=buf[1:M + 1])
    assert torch.all(buf[0] == 7.0) and torch.all(buf[M + 1] == 7.0)
    # the same workspace again, now holding the last call's contents
    check_forward(lay, ws=ws, out=buf[1:M + 1])


def test_forward_workspace_reuse_across_sizes():
    """One workspace sized for the largest batch serves smaller ones."""
    moe = _moe()
    big = wl.make_layer("qwen15", 512)
    ws = moe.workspace(512, big["E"], big["top_k"], big["H"], big["I"])
    check_forward(big, ws=ws)
    small = wl.make_layer("qwen15", 16)
    check_forward(small, ws=ws)


def test_forward_repeatable():
    """Routing is bitwise repeatable; outputs agree to the bf16 rounding of
    fp32 sums added in a different order."""
    lay = wl.make_layer("wide256", 8)
    o1, i1, w1, _ = run_forward(lay)
    o2, i2, w2, _ = run_forward(lay)
    assert np.array_equal(i1, i2) and np.array_equal(w1, w2)
    a, b = h.host_bf16_to_f64(o1), h.host_bf16_to_f64(o2)
    assert np.abs(a - b).max() <= 2 ** -7 * np.abs(a).max()


# Long K in every kernel family: H = 7168 (not a multiple of 2048: the
# per-pair GEMV 1 takes four passes, the last one ragged), I = 2048.
# M = 1 runs the per-pair GEMVs, M = 24 the streaming kernels (6 pairs per
# expert), M = 512 the tiled kernels (128 pairs per expert).
@pytest.fixture(scope="module")
def long_k_layer():
    return wl.make_layer("toy", 512, E=16, top_k=4, H=7168, I=2048, seed=61)


@pytest.mark.parametrize("M,variant", [(1, "pair"), (24, "stream"), (512, "tiled")])
def test_forward_long_k(long_k_layer, M, variant):
    moe = _moe()
    lay = dict(long_k_layer)
    lay["x"] = lay["x"][:M]
    lay["M"] = M
    info, _ = check_forward(lay, n_tokens=12, seed=5)
    check_dispatch(lay, info)
    want = {"pair": moe.MOE_VARIANT_PAIR_GEMV, "stream": moe.MOE_VARIANT_STREAM,
            "tiled": moe.MOE_VARIANT_TILED}[variant]
    assert info["variant"] == want


# Tiled-path shapes drawn once (numpy seed 2027) with block_m 64, 128 and
# 256: 1 to 23 k stages, N tails, 4 to 128 experts, top_k 1 to 8, one- and
# multi-segment index lists; the last two have K tails (H and I multiples
# of 8 only).
RANDOM_TILED = [
    (860, 60, 1, 256, 384), (1350, 4, 2, 768, 896), (379, 60, 4, 960, 320),
    (276, 60, 4, 832, 128), (2172, 64, 1, 832, 384), (2884, 128, 4, 64, 832),
    (1612, 128, 4, 576, 704), (2151, 8, 1, 896, 832), (2593, 128, 8, 896, 64),
    (2389, 4, 1, 1472, 320), (900, 16, 2, 200, 136), (1500, 32, 4, 1000, 520),
]


@pytest.mark.parametrize("M,E,top_k,H,I", RANDOM_TILED)
def test_forward_tiled_random_shapes(M, E, top_k, H, I):
    moe = _moe()
    assert moe.moe_pick_block_m(M, E, top_k) >= 64
    lay = wl.make_layer("toy", M, E=E, top_k=top_k, H=H, I=I, seed=3600 + M)
    check_forward(lay, n_tokens=32)


# Small-batch shapes drawn once (numpy seed 2028; E*H*I <= 1e8, H and I
# multiples of 8): the weight-streaming kernels (block_m 16) and the
# per-pair GEMVs (M * top_k * 4 <= E).
RANDOM_STREAM = [(15, 60, 8, 1600, 472), (16, 32, 1, 2824, 560), (119, 32, 1, 1968, 936),
                 (111, 16, 1, 584, 1424), (136, 60, 2, 448, 1688), (165, 32, 1, 3984, 24),
                 (165, 64, 1, 1544, 272), (11, 32, 8, 1368, 1368)]
RANDOM_PAIR = [(1, 64, 4, 496, 1176), (14, 128, 2, 120, 136), (2, 128, 4, 24, 1040),
               (5, 256, 2, 1088, 328), (1, 16, 1, 1448, 128), (32, 256, 1, 320, 728)]


@pytest.mark.parametrize("M,E,top_k,H,I", RANDOM_STREAM + RANDOM_PAIR)
def test_forward_small_batch_random_shapes(M, E, top_k, H, I):
    moe = _moe()
    B = moe.moe_pick_block_m(M, E, top_k)
    assert B == (1 if M * top_k * 4 <= E else 16)
    lay = wl.make_layer("toy", M, E=E, top_k=top_k, H=H, I=I, seed=3800 + M + H)
    check_forward(lay, n_tokens=32)


def test_forward_maximum_experts_and_top_k():
    """E = 512 and top_k = 32, the largest the entry points take: the top-k
    threshold over eight 64-expert blocks, 32 slots per token in the lists and
    in the per-token sum (256 tokens: 8192 pairs, 16 per expert, block_m 64)."""
    lay = wl.make_layer("toy", 256, E=512, top_k=32, H=256, I=128, seed=4100)
    check_forward(lay, n_tokens=32)


def test_forward_largest_batch():
    """65536 tokens of the Qwen3 prefill shape: 524288 pairs, the index lists
    cut into the maximum number of segments, ~4100 block tiles per GEMM."""
    lay = wl.make_layer("qwen3_prefill", 65536)
    check_forward(lay, n_tokens=24)
