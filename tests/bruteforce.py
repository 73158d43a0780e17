"""Pure-Python dense brute force of the MoE layer, for pinning the oracle.

Written separately from ``oracle/`` (no numpy in the arithmetic, a different
structure): every expert is run on every token, and the output is the sum of
all expert outputs gated by a vector that holds the token's routed weight at
its chosen experts and 0 elsewhere.  Only for tiny shapes.

Definitions followed ("Mixture of Experts in vLLM - From First Principles to
fused_moe", section "One expert, and one token"):
  logits = W_r x; probabilities = softmax over all experts; keep the top_k
  largest (slot 0 = largest, exact ties -> lower id); optionally rescale the
  kept weights to sum to 1; f_e(x) = W2_e (SiLU(W_gate,e x) * (W_up,e x)),
  gate = first I rows of W13_e, up = last I rows; y = sum_j w_j f_{id_j}(x).
"""

from __future__ import annotations

import math
import struct


def bf16_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def to_lists(layer: dict):
    """numpy bf16 arrays of a layer -> nested Python float lists."""
    def conv(a):
        if a.ndim == 1:
            return [bf16_to_float(v) for v in a]
        return [conv(r) for r in a]
    return (conv(layer["x"]), conv(layer["w_router"]), conv(layer["w13"]),
            conv(layer["w2"]))


def dot(a, b):
    return math.fsum(p * q for p, q in zip(a, b))


def sigmoid(z):
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    ez = math.exp(z)
    return ez / (1.0 + ez)


def expert(xv, w13_e, w2_e):
    I = len(w13_e) // 2
    gate = [dot(w13_e[n], xv) for n in range(I)]
    up = [dot(w13_e[I + n], xv) for n in range(I)]
    a = [gate[n] * sigmoid(gate[n]) * up[n] for n in range(I)]
    return [dot(row, a) for row in w2_e]


def route_token(xv, wr, top_k, renormalize, bias=None):
    E = len(wr)
    logits = [dot(wr[e], xv) + (0.0 if bias is None else float(bias[e]))
              for e in range(E)]
    mx = max(logits)
    ex = [math.exp(l - mx) for l in logits]
    s = math.fsum(ex)
    prob = [v / s for v in ex]
    # rank by float32-rounded logit (the precision the decision is taken in)
    f32 = [struct.unpack("<f", struct.pack("<f", l))[0] for l in logits]
    ranked = sorted(range(E), key=lambda e: (-f32[e], e))
    ids = ranked[:top_k]
    w = [prob[e] for e in ids]
    if renormalize:
        tot = math.fsum(w)
        w = [v / tot for v in w]
    return ids, w, logits


def layer(layer_np: dict):
    """Dense brute force of the whole layer. Returns (ids, weights, y)."""
    X, WR, W13, W2 = to_lists(layer_np)
    k = layer_np["top_k"]
    E = len(WR)
    bias = layer_np.get("logit_bias")
    ids_all, w_all, y_all = [], [], []
    for xv in X:
        ids, w, _ = route_token(xv, WR, k, layer_np["renormalize"], bias)
        gatevec = [0.0] * E
        for e, wt in zip(ids, w):
            gatevec[e] = wt
        outs = [expert(xv, W13[e], W2[e]) for e in range(E)]
        H = len(xv)
        y = [math.fsum(gatevec[e] * outs[e][h] for e in range(E)) for h in range(H)]
        ids_all.append(ids)
        w_all.append(w)
        y_all.append(y)
    return ids_all, w_all, y_all


def expert_act(xv, w13_e):
    """The activation row of one (token, expert) pair: SiLU(gate) * up."""
    I = len(w13_e) // 2
    gate = [dot(w13_e[n], xv) for n in range(I)]
    up = [dot(w13_e[I + n], xv) for n in range(I)]
    return [gate[n] * sigmoid(gate[n]) * up[n] for n in range(I)]


def weights_of_ids(xv, wr, ids, renormalize, bias=None):
    """Router weights of the given experts (not necessarily the top-k):
    their softmax probabilities over all experts, optionally rescaled to
    sum 1."""
    E = len(wr)
    logits = [dot(wr[e], xv) + (0.0 if bias is None else float(bias[e])) for e in range(E)]
    mx = max(logits)
    ex = [math.exp(l - mx) for l in logits]
    s = math.fsum(ex)
    w = [ex[e] / s for e in ids]
    if renormalize:
        tot = math.fsum(w)
        w = [v / tot for v in w]
    return w


def pair_rows(X, W13, ids):
    """Activation rows of every pair, listed by pair id: for token t (rows
    of X in order) and slot j (columns of ids[t] in order), the row
    SiLU(gate) * up of expert ids[t][j] on x_t.  Returns a list of rows."""
    rows = []
    for t, xv in enumerate(X):
        for e in ids[t]:
            rows.append(expert_act(xv, W13[e]))
    return rows


def combine(A, W2, ids, weights):
    """Per-token output from given activation rows A (listed by pair id):
    out_t = sum over slots j of weights[t][j] * (W2 of expert ids[t][j]) a,
    with a the row of pair number t * len(ids[t]) + j."""
    out = []
    for t, (row_ids, row_w) in enumerate(zip(ids, weights)):
        k = len(row_ids)
        H = len(W2[row_ids[0]])
        ys = [[dot(W2[e][h], A[t * k + j]) for h in range(H)] for j, e in enumerate(row_ids)]
        out.append([math.fsum(row_w[j] * ys[j][h] for j in range(k)) for h in range(H)])
    return out
