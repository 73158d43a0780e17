"""GPU parity of the routing (moe_route) and index-list (moe_align) calls
against the CPU oracle, through the C ABI."""

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


# ---------------------------------------------------------------------------
# align on fixed topk_ids: bit-exact
# ---------------------------------------------------------------------------

def run_align(ids: np.ndarray, E: int, B: int):
    import torch
    moe = _moe()
    s, e, off, cnt = moe.moe_align(h.dev_i32(ids), E, B)
    torch.cuda.synchronize()
    off = off.cpu().numpy()
    nb = int(off[E])
    return (s.cpu().numpy()[: nb * B], e.cpu().numpy()[:nb], off, cnt.cpu().numpy())


def check_align(ids: np.ndarray, E: int, B: int):
    ref = mo.align(ids, E, B)
    s, e, off, cnt = run_align(ids, E, B)
    assert np.array_equal(off, ref["expert_block_offsets"])
    assert np.array_equal(cnt, ref["expert_counts"])
    assert np.array_equal(e, ref["expert_ids"])
    assert np.array_equal(s, ref["sorted_token_ids"])


def test_align_page_toy():
    """The page's toy batch (M=3, E=4, top_k=2, BLOCK_SIZE_M=4), completed."""
    ids = np.array([[2, 0], [0, 3], [1, 2]], dtype=np.int32)
    s, e, off, cnt = run_align(ids, 4, 4)
    assert s[:4].tolist() == [1, 2, 6, 6] and e[0] == 0
    assert s.tolist() == [1, 2, 6, 6, 4, 6, 6, 6, 0, 5, 6, 6, 3, 6, 6, 6]
    assert e.tolist() == [0, 1, 2, 3] and off.tolist() == [0, 1, 2, 3, 4]
    check_align(ids, 4, 4)


SHAPES = [(3, 2, 4), (1, 8, 128), (64, 8, 128), (37, 4, 60), (16, 4, 60),
          (4096, 8, 128), (8192, 8, 256), (1, 1, 1), (100, 3, 7)]


@pytest.mark.parametrize("pattern", ["random", "round_robin", "sparse", "one_expert_heavy"])
@pytest.mark.parametrize("M,k,E", SHAPES)
def test_align_patterns(pattern, M, k, E):
    if k > E:
        pytest.skip("top_k > E")
    ids = wl.make_topk_ids(M, k, E, seed=1000 + M + E, pattern=pattern)
    for B in (1, 4, 16, 32, 64, 128, 256):
        check_align(ids, E, B)


def test_align_all_pairs_one_expert():
    ids = np.zeros((1000, 1), dtype=np.int32)
    for B in (1, 16, 128):
        check_align(ids, 8, B)
    ids = np.full((777, 1), 59, dtype=np.int32)
    check_align(ids, 60, 16)


def test_align_max_size():
    """512 experts, 524,288 pairs (the largest expert count supported)."""
    ids = wl.make_topk_ids(65536, 8, 512, seed=7)
    for B in (16, 128):
        check_align(ids, 512, B)


def test_align_deterministic():
    ids = wl.make_topk_ids(8192, 8, 256, seed=3)
    a = run_align(ids, 256, 128)
    b = run_align(ids, 256, 128)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def run_route(lay, renormalize=None, top_k=None):
    import torch
    moe = _moe()
    k = lay["top_k"] if top_k is None else top_k
    ren = lay["renormalize"] if renormalize is None else renormalize
    x, wr = h.dev_bf16(lay["x"]), h.dev_bf16(lay["w_router"])
    bias = None if lay.get("logit_bias") is None else h.dev_f32(lay["logit_bias"])
    M, E = lay["x"].shape[0], lay["w_router"].shape[0]
    logits = torch.empty((M, E), dtype=torch.float32, device="cuda")
    ids, wts = moe.moe_route(x, wr, k, ren, logit_bias=bias, logits_out=logits)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), wts.cpu().numpy().astype(np.float64), logits.cpu().numpy()


def check_route(lay, renormalize=None, top_k=None, min_pass=0.9):
    k = lay["top_k"] if top_k is None else top_k
    ren = lay["renormalize"] if renormalize is None else renormalize
    ids, wts, logits = run_route(lay, ren, k)
    ref = mo.route(lay["x"], lay["w_router"], k, ren, lay.get("logit_bias"))
    lref = ref["logits"]
    assert np.abs(logits - lref).max() <= 1e-4 * max(1.0, np.abs(lref).max())
    ok = ref["margin"] > h.MARGIN
    assert ok.mean() >= min_pass
    assert np.array_equal(ids[ok], ref["topk_ids"][ok])
    assert np.abs(wts[ok] - ref["topk_weights"][ok]).max() <= h.WEIGHT_TOL
    if ren:
        assert np.abs(wts.sum(axis=1) - 1.0).max() <= 1e-6 * k
    # every token: distinct ids in range, weights non-increasing
    assert np.all((ids >= 0) & (ids < lay["w_router"].shape[0]))
    assert all(len(set(r)) == k for r in ids.tolist())
    assert np.all(np.diff(wts, axis=1) <= 1e-7)
    # near-tie tokens: every chosen id is within the margin of the k-th logit
    if (~ok).any():
        kth = -np.sort(-ref["logits_f32"][~ok], axis=1)[:, k - 1]
        chosen = np.take_along_axis(ref["logits_f32"][~ok], ids[~ok].astype(np.int64), axis=1)
        assert np.all(chosen >= kth[:, None] - 2 * h.MARGIN)


ROUTE_CASES = [("toy", 3), ("qwen3_decode", 1), ("qwen3_decode", 64), ("qwen3_prefill", 4096),
               ("qwen15", 16), ("qwen15", 2048), ("wide256", 8), ("wide256", 8192)]


@pytest.mark.parametrize("name,M", ROUTE_CASES)
def test_route_workloads(name, M):
    lay = wl.make_layer(name, M, I=8)   # same x and router as the full layer
    check_route(lay)


@pytest.mark.parametrize("M,E,k,H", [(300, 60, 4, 520), (777, 200, 8, 1032), (2100, 6, 2, 64)])
def test_route_large_batch_ragged(M, E, k, H):
    """Batches above 256 tokens take the LDS-tiled router GEMM: partial token
    and expert tiles and a K tail (H not a multiple of 64)."""
    lay = wl.make_layer("qwen15", M, E=E, top_k=k, H=H, I=8, seed=M + E)
    check_route(lay)


def test_route_no_renormalize():
    check_route(wl.make_layer("qwen15", 512, I=8), renormalize=False)
    check_route(wl.make_layer("toy", 3), renormalize=False)


def test_route_k_equals_E_and_k1():
    lay = wl.make_layer("toy", 3)
    check_route(lay, top_k=4)
    check_route(lay, top_k=1)
    check_route(wl.make_layer("wide256", 64, I=8), top_k=1)


def test_route_exact_ties_lower_id():
    lay = wl.make_layer("toy", 9, E=6, top_k=3, H=64, I=8, seed=5)
    lay["w_router"][4] = lay["w_router"][1]
    lay["w_router"][5] = lay["w_router"][1]
    ids, wts, logits = run_route(lay, True, 3)
    assert np.array_equal(logits[:, 1], logits[:, 4]) and np.array_equal(logits[:, 1], logits[:, 5])
    for t in range(9):
        row = ids[t].tolist()
        tied = [e for e in row if e in (1, 4, 5)]
        assert tied == sorted(tied)     # lower id first among equal logits
        order = np.lexsort((np.arange(6), -logits[t]))[:3]
        assert row == order.tolist()


def tie_layer(M: int):
    """wide256 layer whose experts 0, 5, 63, 64, 130, 200, 255 share one
    router row (4x row 17, exact in bf16): their logits tie exactly, inside
    one 64-expert block and across blocks, and often fill the top 7."""
    lay = wl.make_layer("wide256", M, I=8)
    row = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(lay["w_router"][17]) * 4.0)
    for e in TIED:
        lay["w_router"][e] = row
    return lay


TIED = [0, 5, 63, 64, 130, 200, 255]


def check_tied_order(ids: np.ndarray, ref_ids: np.ndarray) -> int:
    """Tied experts appear in ascending id order in every token; tokens whose
    top 7 are the tied group match the oracle exactly.  Returns how many."""
    full = 0
    for t in range(ids.shape[0]):
        row = ids[t].tolist()
        tied = [e for e in row if e in TIED]
        assert tied == sorted(tied)
        if row[:7] == TIED:
            full += 1
            assert ref_ids[t][:7].tolist() == TIED
    return full


def test_route_exact_ties_across_lane_blocks():
    lay = tie_layer(64)
    ids, _, logits = run_route(lay)
    assert len({logits[0, e] for e in TIED}) == 1
    ref = mo.route(lay["x"], lay["w_router"], lay["top_k"], True, None)
    assert check_tied_order(ids, ref["topk_ids"]) >= 8
    ok = ref["margin"] > h.MARGIN
    assert np.array_equal(ids[ok], ref["topk_ids"][ok])


TIED128 = [3, 63, 64, 100, 127]


@pytest.mark.parametrize("M", [1, 8, 64, 300])
def test_route_exact_ties_two_logits_a_lane(M):
    """Up to 128 experts the top-k searches order-preserving keys with wave
    ballots; experts 3, 63, 64, 100 and 127 share one router row (inside one
    64-expert block and across the two), so their logits tie exactly and
    must come out in ascending id order, with the oracle's ids where the
    margin is clear.  M = 300 reaches the tiled router."""
    lay = wl.make_layer("qwen3_decode", M, I=8)
    row = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(lay["w_router"][17]) * 4.0)
    for e in TIED128:
        lay["w_router"][e] = row
    ids, _, logits = run_route(lay)
    assert len({logits[0, e] for e in TIED128}) == 1
    ref = mo.route(lay["x"], lay["w_router"], lay["top_k"], True, None)
    full = 0
    for t in range(M):
        r = ids[t].tolist()
        tied = [e for e in r if e in TIED128]
        assert tied == sorted(tied)
        if r[:5] == TIED128:
            full += 1
            assert ref["topk_ids"][t][:5].tolist() == TIED128
    if M >= 8:
        assert full >= M // 8
    ok = ref["margin"] > h.MARGIN
    assert np.array_equal(ids[ok], ref["topk_ids"][ok])


@pytest.mark.parametrize("E", [63, 64, 65, 127, 128, 129])
def test_route_expert_counts_at_the_top_k_split(E):
    """Expert counts on both sides of the one- and two-logits-a-lane forms
    and of the lane-maxima form above 128 experts."""
    for M in (3, 40):
        check_route(wl.make_layer("qwen15", M, E=E, top_k=8, H=256, I=8, seed=E * 7 + M))
        check_route(wl.make_layer("qwen15", M, E=E, top_k=8, H=256, I=8, seed=E * 7 + M),
                    renormalize=False)


@pytest.mark.parametrize("name,M", [("wide256", 16), ("qwen3_decode", 8), ("toy", 3)])
def test_route_all_logits_equal(name, M):
    """A zero router makes every logit 0: the kept experts are 0..k-1 in
    order, with equal weights (1/k renormalized, 1/E without)."""
    lay = wl.make_layer(name, M, I=8)
    lay["w_router"][:] = 0
    E, k = lay["E"], lay["top_k"]
    for ren in (True, False):
        ids, wts, _ = run_route(lay, ren)
        assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (M, 1)))
        assert np.abs(wts - (1.0 / k if ren else 1.0 / E)).max() <= 1e-6


def test_route_deterministic():
    lay = wl.make_layer("qwen3_prefill", 4096, I=8)
    a = run_route(lay)
    b = run_route(lay)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------------------
# the index lists moe_forward builds from its own routing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M", [5, 16, 17, 64, 256, 512])
def test_forward_index_lists_bit_exact(M):
    """The lists moe_forward leaves in its workspace equal oracle.align of
    the GPU's own topk_ids, bit for bit: the fused top-k + index-list launch
    with two workgroups of four tokens (5 tokens, the second short), several
    (16, 17: five workgroups with the last one short, 64), the most a
    one-segment batch takes (256 tokens = 2048 pairs), and the two-kernel
    align of a multi-segment batch (512)."""
    import torch
    moe = _moe()
    lay = wl.make_layer("qwen3_decode", M)
    M, E, k, H, I = lay["M"], lay["E"], lay["top_k"], lay["H"], lay["I"]
    d = h.layer_to_device(lay)
    ws = moe.workspace(M, E, k, H, I)
    ws.fill_(0xFF)
    ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    print(f"index lists case M={M}", flush=True)
    _, info = moe.moe_forward(d["x"], d["w_router"], d["w13"], d["w2"], k, True,
                              topk_ids_out=ids, ws=ws)
    torch.cuda.synchronize()
    s, e, off, cnt, B = moe.forward_lists(ws, M, E, k, H, I)
    assert B == info["block_m"]
    ref = mo.align(ids.cpu().numpy(), E, B)
    off = off.cpu().numpy()
    nb = int(off[E])
    assert np.array_equal(off, ref["expert_block_offsets"])
    assert np.array_equal(cnt.cpu().numpy(), ref["expert_counts"])
    assert np.array_equal(e.cpu().numpy()[:nb], ref["expert_ids"])
    assert np.array_equal(s.cpu().numpy()[:nb * B], ref["sorted_token_ids"])


def _random_list_cases(n: int = 14, seed: int = 2024):
    """(M, E, top_k) drawn so the lists are built (M * top_k * 4 > E), half of
    them one-segment batches (the fused top-k + lists launch, P <= 2048) and
    half multi-segment ones, over every top-k form (E up to 512, k up to 32)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([2, 7, 60, 64, 65, 128, 129, 200, 256, 512]))
        k = int(rng.integers(1, min(E, 32) + 1))
        lo = E // (4 * k) + 1
        if i % 2 == 0:
            M = int(rng.integers(lo, max(lo, 2048 // k) + 1))
        else:
            M = int(rng.integers(2048 // k + 1, 2048 // k + 600))
        cases.append((M, E, k))
    return cases


@pytest.mark.parametrize("M,E,k", _random_list_cases())
def test_forward_index_lists_random_shapes(M, E, k):
    """moe_forward's own lists against oracle.align of its topk_ids, bit for
    bit, on random expert counts, top_k and batch sizes."""
    import torch
    moe = _moe()
    lay = wl.make_layer("qwen15", M, E=E, top_k=k, H=64, I=64, seed=M * 131 + E * 7 + k)
    H, I = lay["H"], lay["I"]
    d = h.layer_to_device(lay)
    ws = moe.workspace(M, E, k, H, I)
    ws.fill_(0xFF)
    ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    print(f"index lists case M={M} E={E} k={k}", flush=True)
    _, info = moe.moe_forward(d["x"], d["w_router"], d["w13"], d["w2"], k, True,
                              topk_ids_out=ids, ws=ws)
    torch.cuda.synchronize()
    assert info["sorted"] == 1
    s, e, off, cnt, B = moe.forward_lists(ws, M, E, k, H, I)
    assert B == info["block_m"]
    ref = mo.align(ids.cpu().numpy(), E, B)
    off = off.cpu().numpy()
    nb = int(off[E])
    assert np.array_equal(off, ref["expert_block_offsets"])
    assert np.array_equal(cnt.cpu().numpy(), ref["expert_counts"])
    assert np.array_equal(e.cpu().numpy()[:nb], ref["expert_ids"])
    assert np.array_equal(s.cpu().numpy()[:nb * B], ref["sorted_token_ids"])


def test_route_zero_logits_from_signed_zero_rows():
    """Router rows of -0 and of +0 weights both score zero: the GPU keeps the
    lower expert id first, in either order of the rows, as the oracle does."""
    H = 64
    x = wl.f32_to_bf16_bits(np.full((3, H), 0.5, dtype=np.float32))
    rows = np.array([[-0.0] * H, [0.0] * H, [-1.0] * H, [-2.0] * H], dtype=np.float32)
    for perm in ([0, 1, 2, 3], [1, 0, 2, 3]):
        lay = {"x": x, "w_router": wl.f32_to_bf16_bits(rows[perm]), "top_k": 2,
               "renormalize": True}
        ids, wts, logits = run_route(lay)
        assert np.all(logits[:, :2] == 0.0)
        assert ids.tolist() == [[0, 1]] * 3
        assert np.abs(wts - 0.5).max() <= 1e-6
