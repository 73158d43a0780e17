"""Plain, slow, obviously correct CPU oracle of one MoE SwiGLU layer forward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the HIP library never
calls this module, and this module never imports the HIP library.

All floating point is float64 on bf16 inputs widened exactly.  The one place
where floating point decides an integer -- which experts a token keeps -- is
taken on float32 logits, the precision the GPU kernel decides in; the
probabilities and weights themselves are computed in float64.

Sources (page title, then section):
  [MoE-vLLM] "Mixture of Experts in vLLM - From First Principles to fused_moe"
  [Exec]     "MoE Execution Path Analysis"
"""

from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half
    of an IEEE float32)."""
    b = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# routing: [MoE-vLLM] "One expert, and one token", sub-section
# "One token uses only 8 experts"
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray,
                  logit_bias: np.ndarray | None = None) -> np.ndarray:
    """Router scores: one linear layer W_r [E, H] applied to each token,
    logits[t, e] = sum_h x[t, h] * W_r[e, h]  (+ bias[e] when a per-expert
    prior is given).  Returns float64 [M, E]."""
    X = widen_bf16(x)
    W = widen_bf16(w_router)
    logits = X @ W.T
    if logit_bias is not None:
        logits = logits + np.asarray(logit_bias, dtype=np.float32).astype(np.float64)
    return logits


def topk_margin(logits_f32: np.ndarray, top_k: int) -> np.ndarray:
    """Smallest gap between consecutive sorted logits that decides a token's
    ordered top-k: min over j = 1..k of (l_(j) - l_(j+1)) (the (k+1)-th only
    when k < E).  A token whose margin is tiny may be routed differently by
    any implementation whose logits differ in the last bits."""
    s = -np.sort(-np.asarray(logits_f32, dtype=np.float64), axis=1)
    last = min(top_k + 1, s.shape[1])
    if last < 2:
        return np.full(s.shape[0], np.inf)
    gaps = s[:, :last - 1] - s[:, 1:last]
    return gaps.min(axis=1)


def route(x: np.ndarray, w_router: np.ndarray, top_k: int, renormalize: bool,
          logit_bias: np.ndarray | None = None) -> dict:
    """The router steps in the page's order:
      1. softmax over all E scores;
      2. keep the top_k largest -> top_k expert ids and weights, slot 0 the
         largest (exact ties go to the lower expert id);
      3. if renormalize, rescale the kept weights to sum to 1.

    Returns dict(topk_ids int32 [M, k], topk_weights float64 [M, k],
    logits float64 [M, E], logits_f32 float32 [M, E], margin float64 [M]).
    """
    logits = router_logits(x, w_router, logit_bias)
    M, E = logits.shape
    assert 1 <= top_k <= E
    logits_f32 = logits.astype(np.float32)
    # 2. the k largest, descending; ties -> lower id.  Softmax is strictly
    #    increasing, so ordering the float32 logits orders the probabilities.
    idx = np.broadcast_to(np.arange(E), (M, E))
    order = np.lexsort((idx, -logits_f32), axis=1)
    topk_ids = order[:, :top_k].astype(np.int32)
    # 1. and 3.: softmax over all experts, the kept probabilities, renormalize
    w = weights_of(logits, topk_ids, renormalize)
    return dict(topk_ids=topk_ids, topk_weights=w, logits=logits,
                logits_f32=logits_f32, margin=topk_margin(logits_f32, top_k))


def softmax_probs(logits: np.ndarray) -> np.ndarray:
    """Softmax over all E experts of each row of float64 logits."""
    shifted = logits - logits.max(axis=1, keepdims=True)
    ex = np.exp(shifted)
    return ex / ex.sum(axis=1, keepdims=True)


def weights_of(logits: np.ndarray, ids: np.ndarray, renormalize: bool) -> np.ndarray:
    """Router weights of the experts `ids` [M, k] of each token: their
    softmax probabilities (softmax over all E), rescaled to sum 1 when
    renormalize is set.  For the top-k ids this is the router's output; for
    other ids (another implementation's choice among near-tied experts) it
    is what the same router step gives those experts."""
    prob = softmax_probs(np.asarray(logits, dtype=np.float64))
    w = np.take_along_axis(prob, np.asarray(ids, dtype=np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w


# ---------------------------------------------------------------------------
# grouping: [MoE-vLLM] "A batch: (token, expert) pairs" (pair id p = t*k + j),
# "Group the pairs by expert, and the GEMM shapes", and
# "How vLLM runs the layer: two index lists and no copies", sub-section
# "The two index lists" (moe_align_block_size)
# ---------------------------------------------------------------------------

def align(topk_ids: np.ndarray, num_experts: int, block_m: int) -> dict:
    """The two index lists built from topk_ids.

    Pair p is cell p of topk_ids read row by row (p = t*top_k + j).
    sorted_token_ids lists the pair ids grouped by expert, experts in
    ascending order; each group is padded with the id P = M*top_k (not a real
    pair) up to a multiple of block_m; empty experts get no block.  Inside a
    group the pages leave the order free; this oracle uses ascending pair id.
    expert_ids holds the expert of every block of block_m entries.
    expert_block_offsets[e] is the first block of expert e (length E+1, the
    last entry is the number of blocks); expert_counts[e] = n_e.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    P = flat.size
    E = num_experts
    sorted_ids: list[int] = []
    expert_ids: list[int] = []
    offsets = [0]
    counts = []
    for e in range(E):
        members = np.nonzero(flat == e)[0]          # ascending pair ids
        n_e = members.size
        counts.append(n_e)
        nblk = -(-n_e // block_m)
        sorted_ids.extend(int(p) for p in members)
        sorted_ids.extend([P] * (nblk * block_m - n_e))
        expert_ids.extend([e] * nblk)
        offsets.append(offsets[-1] + nblk)
    return dict(sorted_token_ids=np.asarray(sorted_ids, dtype=np.int32),
                expert_ids=np.asarray(expert_ids, dtype=np.int32),
                expert_block_offsets=np.asarray(offsets, dtype=np.int32),
                expert_counts=np.asarray(counts, dtype=np.int32),
                num_blocks=offsets[-1], pad_id=P)


# ---------------------------------------------------------------------------
# one expert: [MoE-vLLM] "One expert, and one token", sub-section
# "An expert is a small SwiGLU MLP"
# ---------------------------------------------------------------------------

def swiglu(h: np.ndarray, I: int) -> np.ndarray:
    """a = SiLU(h_gate) * h_up with h_gate = the first I values of h and
    h_up = the last I; SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    g = h[..., :I]
    u = h[..., I:]
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return silu * u


def _weights(w: np.ndarray) -> np.ndarray:
    """An expert's weight matrix as float64: bf16 bit patterns are widened,
    real-valued matrices (dequantized weights) are taken as they are."""
    w = np.asarray(w)
    return widen_bf16(w) if w.dtype == np.uint16 else w.astype(np.float64)


def expert_ffn(x_rows: np.ndarray, w13_e: np.ndarray, w2_e: np.ndarray,
               return_act: bool = False):
    """f_e on a stack of rows: h = x W13_e^T ([n, 2I]), a = SwiGLU(h),
    y = a W2_e^T ([n, H]).  x_rows float64 [n, H]; weights bf16 bits (or
    real-valued matrices)."""
    W13 = _weights(w13_e)
    W2 = _weights(w2_e)
    I = W2.shape[1]
    h = x_rows @ W13.T
    a = swiglu(h, I)
    y = a @ W2.T
    return (y, a) if return_act else y


# ---------------------------------------------------------------------------
# the layer: group by expert -> one GEMM pair per expert -> put each result
# back into its pair slot [M, k, H] -> weighted sum over the k slots.
# [MoE-vLLM] "Group the pairs by expert, and the GEMM shapes",
# "Put the results back, and combine them per token".
# ---------------------------------------------------------------------------

def _pairs_by_expert(topk_ids: np.ndarray, tokens: np.ndarray):
    """For the given tokens, yield (expert, token array, slot array)."""
    k = topk_ids.shape[1]
    sub = np.asarray(topk_ids)[tokens]                       # [T, k]
    t_of = np.repeat(tokens, k)
    j_of = np.tile(np.arange(k), tokens.size)
    e_of = sub.reshape(-1)
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        yield int(e), t_of[sel], j_of[sel]


def pair_activations(x: np.ndarray, w13: np.ndarray, topk_ids: np.ndarray,
                     tokens: np.ndarray | None = None) -> np.ndarray:
    """GEMM 1 + SiLU-and-mul for every pair, in pair order: row p = t*k + j
    holds a = SwiGLU(W13_{id} x_t).  Returns float64 [M*k, I] (rows of tokens
    not asked for are left as NaN)."""
    M, k = topk_ids.shape
    I = w13.shape[1] // 2
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    X = widen_bf16(x)
    act = np.full((M * k, I), np.nan)
    for e, ts, js in _pairs_by_expert(topk_ids, tokens):
        W13 = widen_bf16(w13[e])
        act[ts * k + js] = swiglu(X[ts] @ W13.T, I)
    return act


def layer_forward(x: np.ndarray, w13: np.ndarray, w2: np.ndarray,
                  topk_ids: np.ndarray, topk_weights: np.ndarray,
                  tokens: np.ndarray | None = None) -> np.ndarray:
    """y_t = sum_j w[t, j] * f_{id[t, j]}(x_t) for the requested tokens.

    Steps as the pages give them: group the pairs by expert, run expert e on
    its rows, send each output row back to its pair slot, then multiply each
    slot by its router weight and add the top_k slots of each token.
    Returns float64 [len(tokens), H] (all tokens when tokens is None)."""
    M, k = topk_ids.shape
    H = x.shape[1]
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    pos = np.full(M, -1)
    pos[tokens] = np.arange(tokens.size)
    X = widen_bf16(x)
    slots = np.zeros((tokens.size, k, H))
    for e, ts, js in _pairs_by_expert(topk_ids, tokens):
        slots[pos[ts], js] = expert_ffn(X[ts], w13[e], w2[e])
    wts = np.asarray(topk_weights, dtype=np.float64)[tokens]
    return np.einsum("tk,tkh->th", wts, slots)


def combine_from_act(act_bits: np.ndarray, w2: np.ndarray,
                     topk_ids: np.ndarray, topk_weights: np.ndarray,
                     tokens: np.ndarray | None = None) -> np.ndarray:
    """Second half of the layer from given activations: for each pair p,
    y_p = W2_{id_p} a_p, then out_t = sum_j w[t, j] y_{t*k+j}.
    act_bits: bf16 bits [M*k, I] in pair order.  Returns float64 [T, H]."""
    M, k = topk_ids.shape
    H = w2.shape[1]
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    pos = np.full(M, -1)
    pos[tokens] = np.arange(tokens.size)
    A = widen_bf16(act_bits)
    slots = np.zeros((tokens.size, k, H))
    for e, ts, js in _pairs_by_expert(topk_ids, tokens):
        W2 = widen_bf16(w2[e])
        slots[pos[ts], js] = A[ts * k + js] @ W2.T
    wts = np.asarray(topk_weights, dtype=np.float64)[tokens]
    return np.einsum("tk,tkh->th", wts, slots)


def forward(layer: dict, block_m: int | None = None,
            tokens: np.ndarray | None = None) -> dict:
    """Whole layer for a dict made by ``moe_workloads.make_layer``:
    routing, (optionally) the index lists, and the output of the requested
    tokens (routing is computed for those tokens only)."""
    x = layer["x"]
    M = x.shape[0]
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    r = route(x[tokens], layer["w_router"], layer["top_k"],
              layer["renormalize"], layer.get("logit_bias"))
    ids = np.zeros((M, layer["top_k"]), dtype=np.int32)
    wts = np.zeros((M, layer["top_k"]))
    ids[tokens] = r["topk_ids"]
    wts[tokens] = r["topk_weights"]
    out = dict(route=r, tokens=tokens)
    if block_m is not None and tokens.size == M:
        out["align"] = align(ids, layer["E"], block_m)
    out["y"] = layer_forward(x, layer["w13"], layer["w2"], ids, wts, tokens)
    return out


# ---------------------------------------------------------------------------
# group-quantized expert weights.  In the MLX part of the page "SGLang issue
# #22283" (GitHub thread) the kernels read weights in the affine group format
# (kernel names affine_qmv ... gs_64_b_4: group size 64, 4 bits; 6 and 8
# bits are discussed too) and the thread's open question is a kernel that
# tolerates a K that is not a multiple of its block (K = 1408).
# Readings (the thread names the format, not its layout): each row of a weight
# matrix holds K codes q in [0, 2^bits); codes are packed little-end first
# into 32-bit words (element i of a row is bits [bits*i, bits*(i+1)) of the
# row's bit stream); each group of 64 consecutive elements of a row has one
# scale s and one bias b (bf16), and the weight is w = s * q + b.
# ---------------------------------------------------------------------------

QUANT_GROUP = 64


def unpack_codes(words: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Codes of a packed weight array [..., K * bits / 32] uint32 ->
    [..., K] integers (element i: bits [bits*(i % per), ...) of word
    i // per, least significant first; per = 32 / bits)."""
    per = 32 // bits
    w = np.asarray(words, dtype=np.uint32)
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))
    q = (w[..., :, None] >> shifts) & np.uint32((1 << bits) - 1)
    return q.reshape(*w.shape[:-1], w.shape[-1] * per)[..., :K].astype(np.int64)


def dequantize_affine(words: np.ndarray, scales: np.ndarray, biases: np.ndarray,
                      bits: int, K: int, group: int = QUANT_GROUP) -> np.ndarray:
    """w[..., i] = s[..., i // group] * q[..., i] + b[..., i // group], in
    float64 (scales and biases are bf16 bit patterns, widened exactly)."""
    q = unpack_codes(words, bits, K).astype(np.float64)
    S = np.repeat(widen_bf16(scales), group, axis=-1)[..., :K]
    B = np.repeat(widen_bf16(biases), group, axis=-1)[..., :K]
    return S * q + B


class DequantizedExperts:
    """Expert e's weight matrix on demand, dequantized (float64)."""

    def __init__(self, words, scales, biases, bits: int, K: int):
        self.words, self.scales, self.biases = words, scales, biases
        self.bits, self.K = bits, K

    def __getitem__(self, e: int) -> np.ndarray:
        return dequantize_affine(self.words[e], self.scales[e], self.biases[e], self.bits,
                                 self.K)

    @property
    def shape(self):
        return (self.words.shape[0], self.words.shape[1], self.K)


def forward_quantized(layer: dict, tokens: np.ndarray | None = None) -> dict:
    """The layer with group-quantized expert weights (a dict made by
    ``moe_workloads.make_quantized_layer``): routing exactly as ``forward``
    (the router stays bf16), then the same grouped expert FFNs and weighted
    sum on the dequantized W13 and W2."""
    x = layer["x"]
    M = x.shape[0]
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    r = route(x[tokens], layer["w_router"], layer["top_k"], layer["renormalize"],
              layer.get("logit_bias"))
    ids = np.zeros((M, layer["top_k"]), dtype=np.int32)
    wts = np.zeros((M, layer["top_k"]))
    ids[tokens] = r["topk_ids"]
    wts[tokens] = r["topk_weights"]
    w13, w2 = dequantized_experts(layer)
    return dict(route=r, tokens=tokens, y=layer_forward(x, w13, w2, ids, wts, tokens))


def dequantized_experts(layer: dict):
    """(W13, W2) of a group-quantized layer as on-demand dequantized expert
    matrices, for ``layer_forward``."""
    H, I, bits = layer["H"], layer["I"], layer["bits"]
    return (DequantizedExperts(layer["w13_q"], layer["w13_scales"], layer["w13_biases"], bits, H),
            DequantizedExperts(layer["w2_q"], layer["w2_scales"], layer["w2_biases"], bits, I))


# ---------------------------------------------------------------------------
# MXFP8 experts and activations.  The MLX part of the page "SGLang issue
# #22283" names MXFP8 next to the affine formats; the format is the OCP
# Microscaling (MX) one: blocks of 32 consecutive elements along K, each
# block one E8M0 scale (a power of two, 2^(code - 127)) and 32 FP8 E4M3
# elements (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
# is subnormal, m * 2^-9; 0x7F and 0xFF are NaN; no infinities; largest
# finite 448).  The page [MoE-vLLM] "The two index lists" names the FP8
# GEMM 1 input qhidden, a quantized copy of x.
# Readings: x (GEMM 1 input) and act (GEMM 2 input) are both quantized to
# MXFP8 by the layer; act is the bf16 activation (fp32 value rounded to
# bf16, as the bf16 layer stores it) before it is quantized; the router stays
# bf16.  Quantizing a block: amax = max |v|; the scale is 2^(floor(log2
# amax) - 8) (8 = the exponent of E4M3's largest power of two), clamped to
# E8M0's range [2^-127, 2^127], code 0 for an all-zero block; an element is
# v / scale rounded to the nearest E4M3 value, ties to the even code,
# saturating at +-448; the sign of v is kept, also when it rounds to zero.
# ---------------------------------------------------------------------------

MX_BLOCK = 32


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """E4M3 code bytes -> float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e8m0_value(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> 2^(code - 127) (NaN for 0xFF)."""
    c = np.asarray(codes).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


_E4M3_GRID = e4m3_value(np.arange(0x7F))          # the 127 finite non-negative values, ascending


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each finite float64 value, ties to the even
    code, saturating at +-448, sign kept (also for a zero result)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    hi = np.clip(np.searchsorted(_E4M3_GRID, a, side="left"), 1, 0x7E)
    lo = hi - 1
    dlo = a - _E4M3_GRID[lo]
    dhi = _E4M3_GRID[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a >= _E4M3_GRID[0x7E], 0x7E, mag)
    return (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def mx_quantize(v: np.ndarray, block: int = MX_BLOCK) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 codes [..., K] (uint8 E4M3) and scales [..., K/32] (uint8 E8M0)
    of float64 values [..., K] (K a multiple of 32)."""
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(*v.shape[:-1], v.shape[-1] // block, block)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                      # amax = f * 2^ex, f in [0.5, 1)
    shared = np.clip(ex - 1 - 8, -127, 127)     # floor(log2 amax) - 8
    shared = np.where(amax == 0, -127, shared)
    codes = e4m3_round(blocks / np.exp2(shared.astype(np.float64))[..., None])
    return codes.reshape(v.shape), (shared + 127).astype(np.uint8)


_E4M3_ALL = e4m3_value(np.arange(256))         # every code's value (a table of the same definition)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, block: int = MX_BLOCK) -> np.ndarray:
    """float64 values of MXFP8 codes [..., K] with scales [..., K/32]."""
    c = _E4M3_ALL[np.asarray(codes, dtype=np.uint8)]
    s = np.repeat(e8m0_value(scales), block, axis=-1)
    return c * s


def round_to_bf16_via_f32(v: np.ndarray) -> np.ndarray:
    """bf16 bits of float64 values rounded first to float32 and then to
    bf16, both to nearest even (an fp32 value stored as bf16)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def forward_mxfp8(layer: dict, tokens: np.ndarray | None = None) -> dict:
    """The layer with MXFP8 experts and activations (a dict made by
    ``moe_workloads.make_mx_layer``): routing as ``forward`` (bf16 router),
    x quantized to MXFP8, per pair h = W13_e deq(q(x_t)), act = SwiGLU(h)
    stored as bf16 then quantized to MXFP8, y_p = W2_e deq(q(act_p)), and
    the weighted top-k sum."""
    x = layer["x"]
    M, H = x.shape
    I, k = layer["I"], layer["top_k"]
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    r = route(x[tokens], layer["w_router"], k, layer["renormalize"], layer.get("logit_bias"))
    ids = np.zeros((M, k), dtype=np.int32)
    wts = np.zeros((M, k))
    ids[tokens] = r["topk_ids"]
    wts[tokens] = r["topk_weights"]
    y, xq, xs = mx_layer_forward(layer, ids, wts, tokens)
    return dict(route=r, tokens=tokens, y=y, x_codes=xq, x_scales=xs)


def mx_layer_forward(layer: dict, topk_ids: np.ndarray, topk_weights: np.ndarray,
                     tokens: np.ndarray | None = None):
    """The expert part of the MXFP8 layer for given routing (ids and
    weights [M, k]): x quantized to MXFP8, per pair h = W13_e deq(q(x_t)),
    act = SwiGLU(h) stored as bf16 then quantized, y_p = W2_e deq(q(act_p)),
    and the weighted top-k sum of the requested tokens.  Returns
    (y float64 [T, H], x codes, x scales)."""
    x = layer["x"]
    M, H = x.shape
    I, k = layer["I"], layer["top_k"]
    tokens = np.arange(M) if tokens is None else np.asarray(tokens)
    xq, xs = mx_quantize(widen_bf16(x))
    X = mx_dequantize(xq, xs)
    pos = np.full(M, -1)
    pos[tokens] = np.arange(tokens.size)
    slots = np.zeros((tokens.size, k, H))
    for e, ts, js in _pairs_by_expert(topk_ids, tokens):
        W13 = mx_dequantize(layer["w13_codes"][e], layer["w13_scales"][e])
        W2 = mx_dequantize(layer["w2_codes"][e], layer["w2_scales"][e])
        act = widen_bf16(round_to_bf16_via_f32(swiglu(X[ts] @ W13.T, I)))
        aq, asc = mx_quantize(act)
        slots[pos[ts], js] = mx_dequantize(aq, asc) @ W2.T
    y = np.einsum("tk,tkh->th", np.asarray(topk_weights, dtype=np.float64)[tokens], slots)
    return y, xq, xs
