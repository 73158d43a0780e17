"""Shared helpers of the GPU tests: moving seeded inputs to the device and
the comparison protocol against the CPU oracle."""

from __future__ import annotations

import itertools

import numpy as np

from oracle import moe_oracle as mo

# Layer outputs: bf16 inputs, fp32 accumulation, bf16 activations and output.
MAX_ABS_REL = 2e-2       # max |y - ref| <= 2e-2 * max |ref|
MEAN_REL = 5e-3          # sum |y - ref| <= 5e-3 * sum |ref|
MARGIN = 1e-4            # routing ids compared where the top-k logit margin exceeds this
WEIGHT_TOL = 1e-5        # |w_gpu - w_ref| on margin-passing tokens


def dev_bf16(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def dev_i32(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def dev_f32(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_bf16_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def layer_to_device(lay: dict, device="cuda") -> dict:
    d = dict(x=dev_bf16(lay["x"], device), w_router=dev_bf16(lay["w_router"], device),
             w13=dev_bf16(lay["w13"], device), w2=dev_bf16(lay["w2"], device), logit_bias=None)
    if lay.get("logit_bias") is not None:
        d["logit_bias"] = dev_f32(lay["logit_bias"], device)
    return d


def assert_close_outputs(y: np.ndarray, ref: np.ndarray, what: str = "output"):
    """The layer-output criteria: max-abs and mean-relative error."""
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite values"
    err = np.abs(y - ref)
    mx = np.abs(ref).max()
    assert err.max() <= MAX_ABS_REL * mx, \
        f"{what}: max|err| {err.max():.4e} > {MAX_ABS_REL} * max|ref| ({mx:.4e})"
    rel = err.sum() / max(np.abs(ref).sum(), 1e-30)
    assert rel <= MEAN_REL, f"{what}: mean-rel error {rel:.4e} > {MEAN_REL}"
    return err.max() / mx, rel


def sample_tokens(M: int, n: int, seed: int) -> np.ndarray:
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    t = rng.choice(M, size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, M - 1], t]))


def check_routing(ids: np.ndarray, wts: np.ndarray, r: dict, renormalize: bool) -> np.ndarray:
    """Routing of the sampled tokens against the oracle's route `r` of the
    same tokens.  Ids are unique where the top-k logit margin exceeds MARGIN
    and must match there bit for bit; on every token the choice must be a
    valid ordered top-k up to near ties (distinct ids in range, each chosen
    expert's oracle logit within 2*MARGIN of the k-th largest, every expert
    clearly above the k-th chosen, slots in descending logit order up to
    2*MARGIN).  The weights of every token must equal, within WEIGHT_TOL,
    what the oracle's router step gives the GPU's own ids.  Returns those
    oracle weights (float64 [T, k]) for the output reference."""
    ids = np.asarray(ids)
    T, k = ids.shape
    lf = np.asarray(r["logits_f32"], dtype=np.float64)
    E = lf.shape[1]
    ok = r["margin"] > MARGIN
    assert np.array_equal(ids[ok], r["topk_ids"][ok]), "routing ids differ on margin tokens"
    assert np.all((ids >= 0) & (ids < E)), "expert id out of range"
    assert all(len(set(row)) == k for row in ids.tolist()), "repeated expert id"
    chosen = np.take_along_axis(lf, ids.astype(np.int64), axis=1)
    kth = -np.sort(-lf, axis=1)[:, k - 1]
    assert np.all(chosen >= kth[:, None] - 2 * MARGIN), "a chosen expert is not near the top-k"
    mask = np.zeros((T, E), dtype=bool)
    np.put_along_axis(mask, ids.astype(np.int64), True, axis=1)
    clearly_in = lf > chosen.min(axis=1, keepdims=True) + 2 * MARGIN
    assert not np.any(clearly_in & ~mask), "an expert clearly above the chosen ones was dropped"
    assert np.all(np.diff(chosen, axis=1) <= 2 * MARGIN), "slots not in descending order"
    w_ref = mo.weights_of(r["logits"], ids, renormalize)
    assert np.abs(np.asarray(wts, dtype=np.float64) - w_ref).max() <= WEIGHT_TOL, \
        "routing weights differ from the oracle's weights of the same experts"
    return w_ref


def scatter_routing(M: int, toks: np.ndarray, ids: np.ndarray, wts: np.ndarray):
    """[M, k] id and weight arrays holding the sampled tokens' rows."""
    k = ids.shape[1]
    full_ids = np.zeros((M, k), dtype=np.int32)
    full_w = np.zeros((M, k))
    full_ids[toks] = ids
    full_w[toks] = wts
    return full_ids, full_w


# relative distance of an fp64 act value from a bf16 rounding midpoint below
# which the GPU's fp32 sums (K terms, fp32 accumulation, fast exp) may round
# it the other way
ACT_ROUNDING_TOL = 2.0 ** -13


def mx_ambiguous_act_choices(act64: np.ndarray):
    """act values (float64, bf16-exact) of one pair for every combination of
    the quantization decisions that could go either way: elements whose fp64
    value lies within ACT_ROUNDING_TOL of a bf16 rounding midpoint and whose
    E4M3 code or block scale changes on the other side of it.  None if more
    than four such elements."""
    bits = mo.round_to_bf16_via_f32(act64)
    a = mo.widen_bf16(bits)
    codes0, scales0 = mo.mx_quantize(a)
    options = []
    for i in range(a.size):
        if (bits[i] & 0x7FFF) == 0:
            continue
        # the bf16 neighbour on the side of the fp64 value (bits -1 / +1 step
        # the magnitude down / up)
        toward_larger_mag = abs(act64[i]) > abs(a[i])
        nb = int(bits[i]) + (1 if toward_larger_mag else -1)
        if (nb & 0x7F80) == 0x7F80:
            continue
        nv = mo.widen_bf16(np.array([nb], dtype=np.uint16))[0]
        if abs(act64[i] - 0.5 * (a[i] + nv)) > ACT_ROUNDING_TOL * abs(act64[i]):
            continue
        blk = i // mo.MX_BLOCK
        sl = slice(blk * mo.MX_BLOCK, (blk + 1) * mo.MX_BLOCK)
        alt = a[sl].copy()
        alt[i - blk * mo.MX_BLOCK] = nv
        c, sc = mo.mx_quantize(alt)
        if not (np.array_equal(c, codes0[sl]) and sc[0] == scales0[blk]):
            options.append((i, nv))
    if len(options) > 4:
        return None
    out = []
    for mask in range(1 << len(options)):
        v = a.copy()
        for bit, (i, val) in enumerate(options):
            if mask >> bit & 1:
                v[i] = val
        out.append(v)
    return out


def mx_boundary_reference(lay, full_ids, full_w, toks, y, ref_y):
    """ref_y with the rows of tokens over the max-abs bound replaced by the
    closest oracle output among the act decisions one bf16 step could flip
    (unchanged where no choice meets the bound)."""
    bad = np.flatnonzero(np.abs(y - ref_y).max(axis=1) > MAX_ABS_REL * np.abs(ref_y).max())
    if bad.size == 0:
        return ref_y
    I = lay["I"]
    xq, xs = mo.mx_quantize(mo.widen_bf16(lay["x"][toks]))
    X = mo.mx_dequantize(xq, xs)
    ref = ref_y.copy()
    bound = MAX_ABS_REL * np.abs(ref_y).max()
    for r in bad:
        per_pair = []
        for j in range(lay["top_k"]):
            e = full_ids[toks[r], j]
            W13 = mo.mx_dequantize(lay["w13_codes"][e], lay["w13_scales"][e])
            W2 = mo.mx_dequantize(lay["w2_codes"][e], lay["w2_scales"][e])
            choices = mx_ambiguous_act_choices(mo.swiglu(X[r] @ W13.T, I))
            if choices is None:
                per_pair = None
                break
            per_pair.append([full_w[toks[r], j] * (mo.mx_dequantize(*mo.mx_quantize(c)) @ W2.T)
                             for c in choices])
        if per_pair is None:
            continue
        best, best_err = None, np.inf
        for combo in itertools.product(*per_pair):
            cand = np.sum(combo, axis=0)
            err = np.abs(y[r] - cand).max()
            if err < best_err:
                best, best_err = cand, err
        if best_err <= bound:
            ref[r] = best
    return ref
