"""Shared helpers of the GPU tests: moving seeded inputs to the device and
the comparison protocol against the CPU oracle."""

from __future__ import annotations

import numpy as np

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
