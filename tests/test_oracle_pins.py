"""Pins of the CPU oracle to things other than itself (CPU only).

Each pin comes from the pages, from mathematics, or from an independent
implementation:
  * the page's toy worked example of the index lists (tests/golden/);
  * hand-derived closed forms of SwiGLU and of softmax-top-k-renormalize;
  * a pure-Python dense brute force (tests/bruteforce.py);
  * library special cases (scipy softmax / expit, numpy stable argsort);
  * the grouping invariants the page states (sum of group sizes, one expert
    per block, padding with the id M*top_k).
The last test plants plausible mistakes in the oracle and checks that the
pins catch every one of them.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import moe_workloads as wl
from oracle import moe_oracle as mo
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(values) -> np.ndarray:
    """Exactly representable float values -> bf16 bit patterns."""
    a = np.asarray(values, dtype=np.float32)
    b = wl.f32_to_bf16_bits(a)
    assert np.array_equal(wl.bf16_bits_to_f32(b), a), "value not exact in bf16"
    return b


def tiny_layer(seed, M=3, E=5, top_k=2, H=12, I=6, renormalize=True, bias=False):
    lay = wl.make_layer("toy", M, E=E, top_k=top_k, H=H, I=I, seed=seed)
    lay["renormalize"] = renormalize
    if bias:
        rng = np.random.default_rng(seed)
        lay["logit_bias"] = rng.normal(0, 0.5, E).astype(np.float32)
    return lay


# ---------------------------------------------------------------------------
# the page's worked example
# ---------------------------------------------------------------------------

def _toy_completions(fx):
    """All topk_ids consistent with what the page prints."""
    E, k = fx["E"], fx["top_k"]
    t0 = fx["known_choices"]["t0"]
    s0 = fx["known_choices"]["t1_slot0"]
    nonzero = [e for e in range(E) if e != 0]
    for t1s1 in nonzero:
        if t1s1 == s0:
            continue
        for t2 in itertools.permutations(nonzero, k):
            yield np.array([t0, [s0, t1s1], list(t2)], dtype=np.int32)


def check_page_toy():
    with open(os.path.join(GOLDEN, "page_toy_align.json")) as f:
        fx = json.load(f)
    ex = fx["expect"]
    n = 0
    for ids in _toy_completions(fx):
        n += 1
        a = mo.align(ids, fx["E"], fx["block_m"])
        B = fx["block_m"]
        assert a["pad_id"] == ex["pad_id"] == ex["num_valid_tokens"]
        assert a["expert_ids"][0] == ex["block0_expert"]
        blk0 = a["sorted_token_ids"][:B].tolist()
        assert blk0 == ex["block0_sorted_token_ids"]
        real = [p for p in blk0 if p < a["pad_id"]]
        assert [p // fx["top_k"] for p in real] == ex["block0_tokens_of_real_pairs"]
        # pair p0 sits in a block of expert 2 and reads token row 0
        pos = a["sorted_token_ids"].tolist().index(0)
        assert a["expert_ids"][pos // B] == ex["pair_p0_expert"]
        assert 0 // fx["top_k"] == ex["pair_p0_token"]
    assert n > 0


def test_page_toy_example():
    check_page_toy()


# ---------------------------------------------------------------------------
# hand-derived closed forms
# ---------------------------------------------------------------------------

def check_swiglu_hand():
    # One expert, H=2, I=1: gate row (1, 0), up row (2, 0), W2 = [[1], [-0.5]].
    # For x = (1, 0): g = 1, u = 2, a = SiLU(1) * 2 = 2 / (1 + e^-1),
    # y = (a, -a/2).
    w13 = bits([[[1.0, 0.0], [2.0, 0.0]]])
    w2 = bits([[[1.0], [-0.5]]])
    x = bits([[1.0, 0.0]])
    a = 2.0 / (1.0 + math.exp(-1.0))
    y = mo.expert_ffn(mo.widen_bf16(x), w13[0], w2[0])
    assert y.shape == (1, 2)
    assert abs(y[0, 0] - a) < 1e-14 and abs(y[0, 1] + 0.5 * a) < 1e-14
    # negative gate: x = (-1, 0): g = -1, u = -2, a = SiLU(-1) * (-2)
    #                = (-1 / (1 + e)) * (-2) = 2 / (1 + e)
    y = mo.expert_ffn(mo.widen_bf16(bits([[-1.0, 0.0]])), w13[0], w2[0])
    a = 2.0 / (1.0 + math.e)
    assert abs(y[0, 0] - a) < 1e-14 and abs(y[0, 1] + 0.5 * a) < 1e-14


def check_route_hand():
    # E=3, H=2, x=(1,0), W_r rows (1,0), (0,0), (-1,0) -> logits (1, 0, -1).
    # softmax p = (e, 1, 1/e) / (e + 1 + 1/e); top-2 = experts 0, 1.
    wr = bits([[1.0, 0.0], [0.0, 0.0], [-1.0, 0.0]])
    x = bits([[1.0, 0.0]])
    z = math.e + 1.0 + 1.0 / math.e
    r = mo.route(x, wr, 2, renormalize=False)
    assert r["topk_ids"].tolist() == [[0, 1]]
    assert np.allclose(r["topk_weights"], [[math.e / z, 1.0 / z]], rtol=0, atol=1e-15)
    r = mo.route(x, wr, 2, renormalize=True)
    assert r["topk_ids"].tolist() == [[0, 1]]
    assert np.allclose(r["topk_weights"], [[math.e / (math.e + 1), 1 / (math.e + 1)]],
                       rtol=0, atol=1e-15)
    # a bias of +3 on expert 2 makes its logit 2: order becomes 2, 0.
    r = mo.route(x, wr, 2, renormalize=True,
                 logit_bias=np.array([0, 0, 3], dtype=np.float32))
    assert r["topk_ids"].tolist() == [[2, 0]]
    assert np.allclose(r["topk_weights"], [[math.e / (math.e + 1), 1 / (math.e + 1)]],
                       rtol=0, atol=1e-15)


def check_combine_hand():
    # Two experts that output constant-direction vectors; token picks both.
    # E=2, k=2, H=2, I=1, x=(1,0).  Expert 0: gate (1,0), up (1,0), W2 (1,0)^T
    # -> y0 = (SiLU(1), 0).  Expert 1: gate (1,0), up (1,0), W2 (0,1)^T
    # -> y1 = (0, SiLU(1)).  Router rows (1,0),(0,0): logits (1, 0).
    # Renormalized weights (e/(e+1), 1/(e+1)) -> y = SiLU(1) * w.
    w13 = bits([[[1.0, 0.0], [1.0, 0.0]], [[1.0, 0.0], [1.0, 0.0]]])
    w2 = bits([[[1.0], [0.0]], [[0.0], [1.0]]])
    wr = bits([[1.0, 0.0], [0.0, 0.0]])
    x = bits([[1.0, 0.0]])
    lay = dict(x=x, w_router=wr, w13=w13, w2=w2, logit_bias=None, M=1, E=2,
               top_k=2, H=2, I=1, renormalize=True)
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    want = [s1 * math.e / (math.e + 1), s1 / (math.e + 1)]
    y = mo.forward(lay)["y"]
    assert np.allclose(y, [want], rtol=0, atol=1e-14)


def test_swiglu_closed_form():
    check_swiglu_hand()


def test_route_closed_form():
    check_route_hand()


def test_combine_closed_form():
    check_combine_hand()


# ---------------------------------------------------------------------------
# independent brute force
# ---------------------------------------------------------------------------

BF_CASES = [
    dict(seed=1, M=3, E=4, top_k=2, H=8, I=4),
    dict(seed=2, M=4, E=5, top_k=3, H=12, I=6, renormalize=False),
    dict(seed=3, M=2, E=6, top_k=6, H=10, I=3),
    dict(seed=4, M=5, E=3, top_k=1, H=8, I=5),
    dict(seed=5, M=3, E=6, top_k=2, H=16, I=8, bias=True),
    dict(seed=6, M=4, E=4, top_k=4, H=6, I=2, renormalize=False, bias=True),
]


def check_against_bruteforce(case):
    lay = tiny_layer(**case)
    ids_b, w_b, y_b = bf.layer(lay)
    o = mo.forward(lay)
    r = o["route"]
    assert r["topk_ids"].tolist() == ids_b
    assert np.allclose(r["topk_weights"], w_b, rtol=1e-12, atol=1e-14)
    assert np.allclose(o["y"], y_b, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("case", BF_CASES, ids=lambda c: f"seed{c['seed']}")
def test_oracle_matches_bruteforce(case):
    check_against_bruteforce(case)


def test_toy_workload_matches_bruteforce():
    """The toy workload itself (M=3, E=4, top_k=2, H=64, I=32)."""
    lay = wl.make_layer("toy", 3)
    ids_b, w_b, y_b = bf.layer(lay)
    o = mo.forward(lay, block_m=4)
    assert o["route"]["topk_ids"].tolist() == ids_b
    assert np.allclose(o["route"]["topk_weights"], w_b, rtol=1e-12)
    assert np.allclose(o["y"], y_b, rtol=1e-10, atol=1e-12)


# Teacher-forced halves of the layer (what the per-step GEMM tests compare
# against): the activation rows of every pair in pair order, the output from
# given activation rows, and the router weights of given (not necessarily
# top-k) experts, each against the brute force on random routings that
# repeat experts across tokens and need not be any router's top-k.

TF_CASES = [
    dict(seed=31, M=4, E=5, top_k=3, H=8, I=4),
    dict(seed=32, M=3, E=3, top_k=2, H=12, I=6, bias=True),
    dict(seed=33, M=5, E=7, top_k=1, H=6, I=3),
]


def _random_ids(M, E, k, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32)


def check_pair_activations_bruteforce(case):
    lay = tiny_layer(**case)
    X, _, W13, _ = bf.to_lists(lay)
    ids = _random_ids(lay["M"], lay["E"], lay["top_k"], case["seed"])
    want = np.asarray(bf.pair_rows(X, W13, ids.tolist()))
    got = mo.pair_activations(lay["x"], lay["w13"], ids)
    assert got.shape == want.shape
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def check_combine_from_act_bruteforce(case):
    lay = tiny_layer(**case)
    _, _, _, W2 = bf.to_lists(lay)
    M, k, I = lay["M"], lay["top_k"], lay["I"]
    ids = _random_ids(M, lay["E"], k, case["seed"] + 1)
    rng = np.random.default_rng(case["seed"])
    act = wl.f32_to_bf16_bits(rng.standard_normal((M * k, I)).astype(np.float32))
    wts = rng.uniform(0.05, 1.0, (M, k))
    A = [[bf.bf16_to_float(v) for v in row] for row in act]
    want = np.asarray(bf.combine(A, W2, ids.tolist(), wts.tolist()))
    got = mo.combine_from_act(act, lay["w2"], ids, wts)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def check_weights_of_bruteforce(case):
    lay = tiny_layer(**case)
    X, WR, _, _ = bf.to_lists(lay)
    ids = _random_ids(lay["M"], lay["E"], lay["top_k"], case["seed"] + 2)
    bias = lay.get("logit_bias")
    logits = mo.router_logits(lay["x"], lay["w_router"], bias)
    for renorm in (True, False):
        want = [bf.weights_of_ids(xv, WR, row, renorm, bias) for xv, row in zip(X, ids.tolist())]
        assert np.allclose(mo.weights_of(logits, ids, renorm), want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("case", TF_CASES, ids=lambda c: f"seed{c['seed']}")
def test_pair_activations_match_bruteforce(case):
    check_pair_activations_bruteforce(case)


@pytest.mark.parametrize("case", TF_CASES, ids=lambda c: f"seed{c['seed']}")
def test_combine_from_act_matches_bruteforce(case):
    check_combine_from_act_bruteforce(case)


@pytest.mark.parametrize("case", TF_CASES, ids=lambda c: f"seed{c['seed']}")
def test_weights_of_given_ids_match_bruteforce(case):
    check_weights_of_bruteforce(case)


# ---------------------------------------------------------------------------
# library special cases
# ---------------------------------------------------------------------------

def test_topk_all_experts_is_softmax():
    """k = E with renormalize: the weights are the full softmax, sorted."""
    lay = tiny_layer(11, M=4, E=7, top_k=7, H=16, I=4)
    r = mo.route(lay["x"], lay["w_router"], 7, True)
    sm = scipy.special.softmax(r["logits"], axis=1)
    want = -np.sort(-sm, axis=1)
    assert np.allclose(r["topk_weights"], want, rtol=1e-13, atol=0)
    want_ids = np.argsort(-r["logits_f32"], axis=1, kind="stable")
    assert np.array_equal(r["topk_ids"], want_ids)


def test_top1_is_argmax_weight_one():
    lay = tiny_layer(12, M=6, E=9, top_k=1, H=16, I=4)
    r = mo.route(lay["x"], lay["w_router"], 1, True)
    assert np.array_equal(r["topk_ids"][:, 0], np.argmax(r["logits_f32"], axis=1))
    assert np.array_equal(r["topk_weights"], np.ones((6, 1)))
    r = mo.route(lay["x"], lay["w_router"], 1, False)
    assert np.allclose(r["topk_weights"][:, 0],
                       scipy.special.softmax(r["logits"], axis=1).max(axis=1))


def check_ties():
    # rows 1 and 3 of W_r are equal -> equal logits; the lower id comes first
    wr = bits([[0.0, 0.0], [1.0, 1.0], [-1.0, 0.5], [1.0, 1.0]])
    x = bits([[1.0, 1.0], [2.0, 2.0]])
    r = mo.route(x, wr, 2, True)
    assert r["topk_ids"].tolist() == [[1, 3], [1, 3]]
    assert np.allclose(r["topk_weights"], 0.5)
    assert np.all(r["margin"] == 0.0)


def test_exact_ties_go_to_lower_expert():
    check_ties()


def test_single_expert_is_dense_swiglu():
    """E = 1, k = 1: the layer is one dense SwiGLU FFN."""
    lay = tiny_layer(13, M=5, E=1, top_k=1, H=16, I=8)
    y = mo.forward(lay)["y"]
    X = wl.bf16_bits_to_f32(lay["x"]).astype(np.float64)
    W13 = wl.bf16_bits_to_f32(lay["w13"][0]).astype(np.float64)
    W2 = wl.bf16_bits_to_f32(lay["w2"][0]).astype(np.float64)
    g = X @ W13[:8].T
    u = X @ W13[8:].T
    want = (g * scipy.special.expit(g) * u) @ W2.T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-13)


def test_identical_experts_any_routing():
    """All experts equal and weights renormalized: y = f(x) whatever the
    router picks."""
    lay = tiny_layer(14, M=4, E=6, top_k=3, H=16, I=8)
    lay["w13"][:] = lay["w13"][0]
    lay["w2"][:] = lay["w2"][0]
    y = mo.forward(lay)["y"]
    f = mo.expert_ffn(mo.widen_bf16(lay["x"]), lay["w13"][0], lay["w2"][0])
    assert np.allclose(y, f, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# grouping invariants and closed forms
# ---------------------------------------------------------------------------

def check_align_invariants(ids, E, B):
    a = mo.align(ids, E, B)
    P = ids.size
    s = a["sorted_token_ids"]
    nb = a["num_blocks"]
    assert s.size == nb * B and a["expert_ids"].size == nb
    assert int(a["expert_counts"].sum()) == P                  # sum n_e = M*k
    real = s[s < P]
    assert np.array_equal(np.sort(real), np.arange(P))         # each pair once
    assert np.all(s[s >= P] == P)                              # pad id = M*k
    flat = ids.reshape(-1)
    for b in range(nb):                                        # one expert per block
        blk = s[b * B:(b + 1) * B]
        assert np.all(flat[blk[blk < P]] == a["expert_ids"][b])
    assert np.all(np.diff(a["expert_ids"]) >= 0)
    off = a["expert_block_offsets"]
    assert off[0] == 0 and off[-1] == nb
    assert np.array_equal(np.diff(off), -(-a["expert_counts"] // B))
    # ascending pair id inside each expert: equals a stable argsort by expert
    want = np.argsort(flat, kind="stable")
    assert np.array_equal(real, want)
    return a


@pytest.mark.parametrize("pattern", ["random", "one_expert_heavy", "round_robin", "sparse"])
@pytest.mark.parametrize("B", [1, 4, 16, 64])
def test_align_invariants(pattern, B):
    for (M, k, E) in [(3, 2, 4), (37, 4, 60), (64, 8, 128), (9, 8, 256)]:
        ids = wl.make_topk_ids(M, k, E, seed=M * 7 + E, pattern=pattern)
        check_align_invariants(ids, E, B)


def test_align_empty_experts_get_no_block():
    ids = np.array([[3, 1], [3, 1]], dtype=np.int32)
    a = mo.align(ids, 6, 4)
    assert a["expert_counts"].tolist() == [0, 2, 0, 2, 0, 0]
    assert a["expert_block_offsets"].tolist() == [0, 0, 1, 1, 2, 2, 2]
    assert a["expert_ids"].tolist() == [1, 3]
    assert a["sorted_token_ids"].tolist() == [1, 3, 4, 4, 0, 2, 4, 4]


def test_closed_form_expert_weight_count():
    """Each Qwen3-30B-A3B-shaped expert holds 4,718,592 weights
    (gate + up + down = 3 * 768 * 2048), per the page's statement that a
    decode-time expert reads all 4,718,592 of its weights for one row."""
    s = wl.WORKLOADS["qwen3_decode"]
    assert 2 * s.I * s.H + s.H * s.I == 4_718_592
    assert wl.WORKLOADS["qwen3_prefill"].H == s.H and wl.WORKLOADS["qwen3_prefill"].I == s.I


def test_closed_form_mean_rows():
    """Mean group size = M*top_k/E (= M/16 for 128 experts, top-8)."""
    s = wl.WORKLOADS["qwen3_decode"]
    for M in (1, 16, 64):
        ids = wl.make_topk_ids(M, s.top_k, s.E, seed=M)
        a = mo.align(ids, s.E, 16)
        assert a["expert_counts"].mean() == M / 16


def test_margin_definition():
    l = np.array([[3.0, 1.0, 2.5, 0.0]], dtype=np.float32)
    # sorted 3, 2.5, 1, 0: k=1 -> gap(3,2.5)=0.5; k=2 -> min(0.5, 1.5) = 0.5
    assert mo.topk_margin(l, 1)[0] == 0.5
    assert mo.topk_margin(l, 2)[0] == 0.5
    assert mo.topk_margin(l, 3)[0] == 0.5
    l2 = np.array([[3.0, 2.0, 1.9, 0.0]], dtype=np.float32)
    assert abs(mo.topk_margin(l2, 2)[0] - 0.1) < 1e-6


# ---------------------------------------------------------------------------
# planted mistakes must be caught
# ---------------------------------------------------------------------------

def _battery():
    """Run the pins; return True only if all pass."""
    checks = [check_page_toy, check_swiglu_hand, check_route_hand, check_combine_hand,
              check_ties]
    checks += [lambda c=c: check_against_bruteforce(c) for c in BF_CASES]
    checks += [lambda c=c, f=f: f(c) for c in TF_CASES
               for f in (check_pair_activations_bruteforce, check_combine_from_act_bruteforce,
                         check_weights_of_bruteforce)]
    checks += [lambda: check_align_invariants(
        wl.make_topk_ids(37, 4, 60, seed=5, pattern="random"), 60, 4)]
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


def _swap_gate_up(h, I):
    g, u = h[..., I:], h[..., :I]
    return g / (1.0 + np.exp(-g)) * u


def _silu_wrong_sign(h, I):
    g, u = h[..., :I], h[..., I:]
    return g / (1.0 + np.exp(g)) * u


def _sigmoid_not_silu(h, I):
    g, u = h[..., :I], h[..., I:]
    return 1.0 / (1.0 + np.exp(-g)) * u


_orig_align = mo.align
_orig_route = mo.route
_orig_router_logits = mo.router_logits
_orig_pairs = mo._pairs_by_expert


def _align_column_major(topk_ids, num_experts, block_m):
    return _orig_align(np.ascontiguousarray(np.asarray(topk_ids).T), num_experts, block_m)


def _align_pad_zero(topk_ids, num_experts, block_m):
    a = _orig_align(topk_ids, num_experts, block_m)
    s = a["sorted_token_ids"]
    s[s == a["pad_id"]] = 0
    return a


def _align_descending_in_group(topk_ids, num_experts, block_m):
    a = _orig_align(topk_ids, num_experts, block_m)
    s = a["sorted_token_ids"]
    off = a["expert_block_offsets"]
    for e in range(num_experts):
        n = a["expert_counts"][e]
        st = off[e] * block_m
        s[st:st + n] = s[st:st + n][::-1].copy()
    return a


def _route_no_renorm(x, w_router, top_k, renormalize, logit_bias=None):
    return _orig_route(x, w_router, top_k, False, logit_bias)


def _route_ties_high(x, w_router, top_k, renormalize, logit_bias=None):
    r = _orig_route(x, w_router, top_k, renormalize, logit_bias)
    E = r["logits_f32"].shape[1]
    idx = np.broadcast_to(np.arange(E), r["logits_f32"].shape)
    order = np.lexsort((-idx, -r["logits_f32"]), axis=1)
    r["topk_ids"] = order[:, :top_k].astype(np.int32)
    return r


def _route_ascending_slots(x, w_router, top_k, renormalize, logit_bias=None):
    r = _orig_route(x, w_router, top_k, renormalize, logit_bias)
    r["topk_ids"] = r["topk_ids"][:, ::-1].copy()
    r["topk_weights"] = r["topk_weights"][:, ::-1].copy()
    return r


def _logits_drop_bias(x, w_router, logit_bias=None):
    return _orig_router_logits(x, w_router, None)


def _logits_transposed_weights(x, w_router, logit_bias=None):
    X = mo.widen_bf16(x)
    W = mo.widen_bf16(w_router)
    out = X @ W[::-1].T
    if logit_bias is not None:
        out = out + np.asarray(logit_bias, np.float64)
    return out


def _pairs_wrong_slot(topk_ids, tokens):
    for e, ts, js in _orig_pairs(topk_ids, tokens):
        yield e, ts, (js + 1) % topk_ids.shape[1]


def _expert_w2_transposed(x_rows, w13_e, w2_e, return_act=False):
    W13 = mo.widen_bf16(w13_e)
    W2 = mo.widen_bf16(w2_e)
    I = W2.shape[1]
    a = mo.swiglu(x_rows @ W13.T, I)
    y = a @ W2.reshape(W2.shape[1], W2.shape[0])   # wrong operand layout
    return (y, a) if return_act else y


def _pair_activations_slot_major(x, w13, topk_ids, tokens=None):
    M, k = topk_ids.shape
    I = w13.shape[1] // 2
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    X = mo.widen_bf16(x)
    act = np.full((M * k, I), np.nan)
    for e, ts, js in _orig_pairs(topk_ids, tokens):
        act[js * M + ts] = mo.swiglu(X[ts] @ mo.widen_bf16(w13[e]).T, I)   # wrong row
    return act


def _combine_rows_slot_major(act_bits, w2, topk_ids, topk_weights, tokens=None):
    M, k = topk_ids.shape
    H = w2.shape[1]
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    pos = np.full(M, -1)
    pos[tokens] = np.arange(tokens.size)
    A = mo.widen_bf16(act_bits)
    slots = np.zeros((tokens.size, k, H))
    for e, ts, js in _orig_pairs(topk_ids, tokens):
        slots[pos[ts], js] = A[js * M + ts] @ mo.widen_bf16(w2[e]).T   # wrong row
    return np.einsum("tk,tkh->th", np.asarray(topk_weights, np.float64)[tokens], slots)


_orig_combine = mo.combine_from_act


def _combine_weight_of_next_slot(act_bits, w2, topk_ids, topk_weights, tokens=None):
    w = np.roll(np.asarray(topk_weights, np.float64), 1, axis=1)
    return _orig_combine(act_bits, w2, topk_ids, w, tokens)


_orig_weights_of = mo.weights_of


def _weights_softmax_over_kept_only(logits, ids, renormalize):
    kept = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(ids, np.int64), axis=1)
    ex = np.exp(kept - kept.max(axis=1, keepdims=True))
    return ex / ex.sum(axis=1, keepdims=True)


MUTANTS = {
    "swap_gate_up": ("swiglu", _swap_gate_up),
    "silu_wrong_sign": ("swiglu", _silu_wrong_sign),
    "sigmoid_not_silu": ("swiglu", _sigmoid_not_silu),
    "pair_id_column_major": ("align", _align_column_major),
    "pad_id_zero": ("align", _align_pad_zero),
    "group_order_descending": ("align", _align_descending_in_group),
    "no_renormalize": ("route", _route_no_renorm),
    "ties_to_higher_id": ("route", _route_ties_high),
    "slots_ascending": ("route", _route_ascending_slots),
    "bias_dropped": ("router_logits", _logits_drop_bias),
    "router_rows_permuted": ("router_logits", _logits_transposed_weights),
    "combine_wrong_slot_weight": ("_pairs_by_expert", _pairs_wrong_slot),
    "w2_wrong_layout": ("expert_ffn", _expert_w2_transposed),
    "pair_rows_slot_major": ("pair_activations", _pair_activations_slot_major),
    "combine_reads_slot_major_rows": ("combine_from_act", _combine_rows_slot_major),
    "combine_weight_of_next_slot": ("combine_from_act", _combine_weight_of_next_slot),
    "softmax_over_kept_experts_only": ("weights_of", _weights_softmax_over_kept_only),
}


def test_battery_passes_on_oracle():
    assert _battery()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(mo, attr, fn)
    assert not _battery(), f"planted mistake {name} passed every pin"


def test_route_zero_logits_from_signed_zero_rows_tie_by_lower_id():
    """A router row of -0 weights and a row of +0 weights both score a token
    exactly zero (the sum of signed-zero products is a zero), so the two
    experts tie and the lower id comes first, in either order of the rows;
    experts 2 and 3 score below zero."""
    H = 8
    x = wl.f32_to_bf16_bits(np.full((1, H), 0.5, dtype=np.float32))
    rows = np.array([[-0.0] * H, [0.0] * H, [-1.0] * H, [-2.0] * H], dtype=np.float32)
    for perm in ([0, 1, 2, 3], [1, 0, 2, 3]):
        r = mo.route(x, wl.f32_to_bf16_bits(rows[perm]), 2, True)
        assert r["logits_f32"][0, 0] == 0.0 and r["logits_f32"][0, 1] == 0.0
        assert r["topk_ids"][0].tolist() == [0, 1]
        assert np.allclose(r["topk_weights"][0], [0.5, 0.5])
