"""Python binding of the MI355X MoE layer-forward library (libmoe_mi355x.so).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/moe_mi355x.h``.  torch supplies device
memory and the current stream; nothing here computes any part of the layer,
and there is no CPU fallback -- if the library is missing, importing the
binding works but every call raises.

Function names match the C ABI: moe_route, moe_align,
moe_grouped_gemm_w13_act, moe_grouped_gemm_w2_combine, moe_forward,
moe_forward_quantized, moe_forward_mxfp8, moe_mx_quantize, plus
moe_workspace_size, moe_mx_workspace_size, moe_pick_block_m,
moe_forward_list_offsets and moe_strerror.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoe_mi355x.so")

MOE_VARIANT_TILED = 0
MOE_VARIANT_STREAM = 1
MOE_VARIANT_PAIR_GEMV = 2
MOE_VARIANT_PAIR_GEMV_QUANT = 3
MOE_VARIANT_TILED_MXFP8 = 4
MOE_VARIANT_STREAM_MXFP8 = 5
MOE_VARIANT_PAIR_GEMV_MXFP8 = 6
MOE_VARIANT_STREAM_QUANT = 7
MOE_VARIANT_TILED_QUANT = 8

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size_t = ctypes.c_size_t


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} failed: {moe_strerror(status)} (status {status})")
        self.status = status


class DispatchInfo(ctypes.Structure):
    _fields_ = [("variant", _c_int), ("block_m", _c_int), ("block_n", _c_int),
                ("block_k", _c_int), ("k_tail", _c_int), ("launches", _c_int),
                ("sorted", _c_int)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class ForwardLists(ctypes.Structure):
    """moe_forward_lists: where moe_forward leaves its index lists."""
    _fields_ = [("block_m", _c_int), ("sorted", _c_int), ("sorted_token_ids", _c_size_t),
                ("expert_ids", _c_size_t), ("expert_block_offsets", _c_size_t),
                ("expert_counts", _c_size_t)]


class MxWeights(ctypes.Structure):
    """moe_mx_weights: four device pointers (E4M3 codes and E8M0 scales)."""
    _fields_ = [("w13_codes", _c_void_p), ("w13_scales", _c_void_p),
                ("w2_codes", _c_void_p), ("w2_scales", _c_void_p)]


class QuantizedWeights(ctypes.Structure):
    """moe_quantized_weights: bits, group size and six device pointers."""
    _fields_ = [("bits", _c_int), ("group_size", _c_int),
                ("w13_q", _c_void_p), ("w13_scales", _c_void_p), ("w13_biases", _c_void_p),
                ("w2_q", _c_void_p), ("w2_scales", _c_void_p), ("w2_biases", _c_void_p)]


_SIGNATURES = {
    "moe_workspace_size": (_c_size_t, [_c_int] * 5),
    "moe_strerror": (ctypes.c_char_p, [_c_int]),
    "moe_pick_block_m": (_c_int, [_c_int] * 3),
    "moe_route": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                           _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t,
                           _c_void_p]),
    "moe_align_workspace_size": (_c_size_t, [_c_int] * 3),
    "moe_align": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                           _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "moe_grouped_gemm_w13_act": (_c_int, [_c_void_p] * 5 + [_c_int] * 6 +
                                 [_c_void_p, ctypes.POINTER(DispatchInfo), _c_void_p]),
    "moe_grouped_gemm_w2_combine": (_c_int, [_c_void_p] * 6 + [_c_int] * 6 +
                                    [_c_void_p, _c_void_p, _c_size_t,
                                     ctypes.POINTER(DispatchInfo), _c_void_p]),
    "moe_forward": (_c_int, [_c_void_p] * 5 + [_c_int] * 6 +
                    [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t,
                     ctypes.POINTER(DispatchInfo), _c_void_p]),
    "moe_forward_noalloc": (_c_int, [_c_void_p] * 5 + [_c_int] * 6 +
                            [_c_void_p, _c_void_p, _c_void_p, ctypes.POINTER(DispatchInfo),
                             _c_void_p]),
    "moe_forward_list_offsets": (_c_int, [_c_int] * 5 + [ctypes.POINTER(ForwardLists)]),
    "moe_mx_quantize": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "moe_mx_workspace_size": (_c_size_t, [_c_int] * 5),
    "moe_forward_mxfp8": (_c_int, [_c_void_p] * 3 + [ctypes.POINTER(MxWeights)] + [_c_int] * 6 +
                          [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t,
                           ctypes.POINTER(DispatchInfo), _c_void_p]),
    "moe_forward_quantized": (_c_int, [_c_void_p] * 3 + [ctypes.POINTER(QuantizedWeights)] +
                              [_c_int] * 6 +
                              [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t,
                               ctypes.POINTER(DispatchInfo), _c_void_p]),
}

_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """Load libmoe_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -c "
                "'import __graft_entry__ as g; g.build()'); there is no fallback path")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def moe_workspace_size(M_max: int, E: int, top_k: int, H: int, I: int) -> int:
    return int(library().moe_workspace_size(M_max, E, top_k, H, I))


def moe_strerror(status: int) -> str:
    return library().moe_strerror(status).decode()


def moe_pick_block_m(M: int, E: int, top_k: int) -> int:
    return int(library().moe_pick_block_m(M, E, top_k))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t, name, dtypes, shape=None):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.data_ptr() % 16 != 0:
        raise ValueError(f"{name} must be 16-byte aligned")
    del torch


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _raise(call: str, st: int):
    if st != 0:
        raise MoeError(call, st)


def workspace(M_max: int, E: int, top_k: int, H: int, I: int, device=None):
    """Allocate a workspace tensor (uint8) large enough for every call with
    M <= M_max and these layer sizes."""
    torch = _torch()
    n = moe_workspace_size(M_max, E, top_k, H, I)
    if n == 0:
        raise MoeError("moe_workspace_size", -2)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def moe_route(x, w_router, top_k: int, renormalize: bool = True, logit_bias=None,
              topk_ids=None, topk_weights=None, logits_out=None, ws=None, stream=None):
    torch = _torch()
    M, H = x.shape
    E = w_router.shape[0]
    _check(x, "x", _bf16_types())
    _check(w_router, "w_router", _bf16_types(), (E, H))
    if logit_bias is not None:
        _check(logit_bias, "logit_bias", (torch.float32,), (E,))
    if topk_ids is None:
        topk_ids = torch.empty((M, top_k), dtype=torch.int32, device=x.device)
    if topk_weights is None:
        topk_weights = torch.empty((M, top_k), dtype=torch.float32, device=x.device)
    _check(topk_ids, "topk_ids", (torch.int32,), (M, top_k))
    _check(topk_weights, "topk_weights", (torch.float32,), (M, top_k))
    if logits_out is not None:
        _check(logits_out, "logits_out", (torch.float32,), (M, E))
    elif ws is None:
        ws = torch.empty(max(M * E * 4, 16), dtype=torch.uint8, device=x.device)
    st = library().moe_route(_ptr(x), _ptr(w_router), _ptr(logit_bias), M, H, E, top_k,
                             int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_weights),
                             _ptr(logits_out), _ptr(ws), 0 if ws is None else ws.numel(),
                             _stream(stream))
    _raise("moe_route", st)
    return topk_ids, topk_weights


def align_capacity(P: int, E: int, block_m: int) -> tuple:
    """(sorted_token_ids length, expert_ids length) that moe_align needs."""
    nz = min(E, P)
    return P + nz * (block_m - 1), -(-P // block_m) + nz


def moe_align_workspace_size(M: int, top_k: int, E: int) -> int:
    return int(library().moe_align_workspace_size(M, top_k, E))


def moe_align(topk_ids, E: int, block_m: int, sorted_token_ids=None, expert_ids=None,
              expert_block_offsets=None, expert_counts=None, ws=None, stream=None):
    torch = _torch()
    M, top_k = topk_ids.shape
    _check(topk_ids, "topk_ids", (torch.int32,))
    P = M * top_k
    cap, nbl = align_capacity(P, E, block_m)
    dev = topk_ids.device
    if sorted_token_ids is None:
        sorted_token_ids = torch.empty(max(cap, 4), dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(max(nbl, 4), dtype=torch.int32, device=dev)
    if expert_block_offsets is None:
        expert_block_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if expert_counts is None:
        expert_counts = torch.empty(E, dtype=torch.int32, device=dev)
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (expert_block_offsets, "expert_block_offsets"),
                 (expert_counts, "expert_counts")):
        _check(t, n, (torch.int32,))
    if sorted_token_ids.numel() < cap or expert_ids.numel() < nbl or \
            expert_block_offsets.numel() < E + 1 or expert_counts.numel() < E:
        raise ValueError("moe_align output buffers are too small")
    need = moe_align_workspace_size(M, top_k, E)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = library().moe_align(_ptr(topk_ids), M, top_k, E, block_m, _ptr(sorted_token_ids),
                             _ptr(expert_ids), _ptr(expert_block_offsets),
                             _ptr(expert_counts), _ptr(ws), 0 if ws is None else ws.numel(),
                             _stream(stream))
    _raise("moe_align", st)
    return sorted_token_ids, expert_ids, expert_block_offsets, expert_counts


def moe_grouped_gemm_w13_act(x, w13, sorted_token_ids, expert_ids, expert_block_offsets,
                             top_k: int, block_m: int, act=None, stream=None):
    torch = _torch()
    M, H = x.shape
    E, two_i, H2 = w13.shape
    I = two_i // 2
    _check(x, "x", _bf16_types())
    _check(w13, "w13", _bf16_types(), (E, 2 * I, H))
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (expert_block_offsets, "expert_block_offsets")):
        _check(t, n, (torch.int32,))
    if act is None:
        act = torch.empty((M * top_k, I), dtype=torch.bfloat16, device=x.device)
    _check(act, "act", _bf16_types(), (M * top_k, I))
    info = DispatchInfo()
    st = library().moe_grouped_gemm_w13_act(
        _ptr(x), _ptr(w13), _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(expert_block_offsets), M, top_k, E, H, I, block_m, _ptr(act),
        ctypes.byref(info), _stream(stream))
    _raise("moe_grouped_gemm_w13_act", st)
    return act, info.as_dict()


def moe_grouped_gemm_w2_combine(act, w2, topk_weights, sorted_token_ids, expert_ids,
                                expert_block_offsets, M: int, top_k: int, block_m: int,
                                out=None, ws=None, stream=None):
    torch = _torch()
    E, H, I = w2.shape
    _check(act, "act", _bf16_types(), (M * top_k, I))
    _check(w2, "w2", _bf16_types())
    _check(topk_weights, "topk_weights", (torch.float32,))
    if topk_weights.numel() != M * top_k:
        raise ValueError("topk_weights must hold M*top_k values")
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (expert_block_offsets, "expert_block_offsets")):
        _check(t, n, (torch.int32,))
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=act.device)
    _check(out, "out", _bf16_types(), (M, H))
    if ws is None:
        ws = workspace(M, E, top_k, H, I, act.device)
    info = DispatchInfo()
    st = library().moe_grouped_gemm_w2_combine(
        _ptr(act), _ptr(w2), _ptr(topk_weights), _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(expert_block_offsets), M, top_k, E, H, I, block_m, _ptr(out), _ptr(ws),
        ws.numel(), ctypes.byref(info), _stream(stream))
    _raise("moe_grouped_gemm_w2_combine", st)
    return out, info.as_dict()


def moe_forward(x, w_router, w13, w2, top_k: int, renormalize: bool = True,
                logit_bias=None, out=None, topk_ids_out=None, topk_weights_out=None,
                ws=None, stream=None):
    """The whole layer.  Returns (out [M, H] bf16, dispatch info dict)."""
    torch = _torch()
    M, H = x.shape
    E, two_i, _ = w13.shape
    I = two_i // 2
    _check(x, "x", _bf16_types())
    _check(w_router, "w_router", _bf16_types(), (E, H))
    _check(w13, "w13", _bf16_types(), (E, 2 * I, H))
    _check(w2, "w2", _bf16_types(), (E, H, I))
    if logit_bias is not None:
        _check(logit_bias, "logit_bias", (torch.float32,), (E,))
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", _bf16_types(), (M, H))
    if topk_ids_out is not None:
        _check(topk_ids_out, "topk_ids_out", (torch.int32,), (M, top_k))
    if topk_weights_out is not None:
        _check(topk_weights_out, "topk_weights_out", (torch.float32,), (M, top_k))
    if ws is None:
        ws = workspace(M, E, top_k, H, I, x.device)
    info = DispatchInfo()
    st = library().moe_forward(
        _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(w13), _ptr(w2), M, E, top_k, H, I,
        int(bool(renormalize)), _ptr(out), _ptr(topk_ids_out), _ptr(topk_weights_out),
        _ptr(ws), ws.numel(), ctypes.byref(info), _stream(stream))
    _raise("moe_forward", st)
    return out, info.as_dict()


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(x, w_router, w13, w2, top_k: int, renormalize: bool = True,
                        logit_bias=None, out=None, topk_ids_out=None, topk_weights_out=None,
                        stream=None):
    """moe_forward with the library's own device scratch array (no workspace
    argument; allocates no device memory when ``out`` is given).  Returns
    (out [M, H] bf16, dispatch info dict)."""
    torch = _torch()
    M, H = x.shape
    E, two_i, _ = w13.shape
    I = two_i // 2
    _check(x, "x", _bf16_types())
    _check(w_router, "w_router", _bf16_types(), (E, H))
    _check(w13, "w13", _bf16_types(), (E, 2 * I, H))
    _check(w2, "w2", _bf16_types(), (E, H, I))
    if logit_bias is not None:
        _check(logit_bias, "logit_bias", (torch.float32,), (E,))
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", _bf16_types(), (M, H))
    if topk_ids_out is not None:
        _check(topk_ids_out, "topk_ids_out", (torch.int32,), (M, top_k))
    if topk_weights_out is not None:
        _check(topk_weights_out, "topk_weights_out", (torch.float32,), (M, top_k))
    info = DispatchInfo()
    st = library().moe_forward_noalloc(
        _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(w13), _ptr(w2), M, E, top_k, H, I,
        int(bool(renormalize)), _ptr(out), _ptr(topk_ids_out), _ptr(topk_weights_out),
        ctypes.byref(info), _stream(stream))
    _raise("moe_forward_noalloc", st)
    return out, info.as_dict()


def moe_forward_list_offsets(M: int, E: int, top_k: int, H: int, I: int) -> dict:
    """Byte offsets in moe_forward's workspace of the index lists it builds
    for a batch of M tokens, with their block size (``sorted`` 0: none)."""
    lists = ForwardLists()
    _raise("moe_forward_list_offsets",
           library().moe_forward_list_offsets(M, E, top_k, H, I, ctypes.byref(lists)))
    return {f: getattr(lists, f) for f, _ in lists._fields_}


def forward_lists(ws, M: int, E: int, top_k: int, H: int, I: int):
    """The index lists moe_forward left in workspace tensor ``ws`` (after a
    completed call with these sizes), as int32 views: (sorted_token_ids,
    expert_ids, expert_block_offsets, expert_counts, block_m).  Only the
    first num_blocks*block_m / num_blocks entries of the first two hold
    data (num_blocks = expert_block_offsets[E])."""
    torch = _torch()
    o = moe_forward_list_offsets(M, E, top_k, H, I)
    if not o["sorted"]:
        raise ValueError("moe_forward builds no index lists for this batch size")
    cap, nbl = align_capacity(M * top_k, E, o["block_m"])

    def view(off, n):
        return ws[off:off + 4 * n].view(torch.int32)

    return (view(o["sorted_token_ids"], cap), view(o["expert_ids"], nbl),
            view(o["expert_block_offsets"], E + 1), view(o["expert_counts"], E), o["block_m"])


def moe_forward_quantized(x, w_router, qweights: dict, top_k: int, renormalize: bool = True,
                          logit_bias=None, out=None, topk_ids_out=None, topk_weights_out=None,
                          ws=None, stream=None):
    """The layer with group-quantized expert weights.  ``qweights`` holds
    ``bits`` (4 or 8), ``w13_q`` [E, 2I, H*bits/32] and ``w2_q``
    [E, H, I*bits/32] (int32 or uint32 words of packed codes), and
    ``w13_scales``, ``w13_biases`` [E, 2I, H/64], ``w2_scales``,
    ``w2_biases`` [E, H, I/64] (bf16).  Returns (out [M, H] bf16, dispatch
    info dict)."""
    torch = _torch()
    M, H = x.shape
    E = w_router.shape[0]
    bits = int(qweights["bits"])
    I = qweights["w2_q"].shape[2] * 32 // bits if bits in (4, 8) else 0
    words = (torch.int32, getattr(torch, "uint32", torch.int32))
    _check(x, "x", _bf16_types())
    _check(w_router, "w_router", _bf16_types(), (E, H))
    if bits in (4, 8):
        for name, shape, types in (("w13_q", (E, 2 * I, H * bits // 32), words),
                                   ("w13_scales", (E, 2 * I, H // 64), _bf16_types()),
                                   ("w13_biases", (E, 2 * I, H // 64), _bf16_types()),
                                   ("w2_q", (E, H, I * bits // 32), words),
                                   ("w2_scales", (E, H, I // 64), _bf16_types()),
                                   ("w2_biases", (E, H, I // 64), _bf16_types())):
            _check(qweights[name], name, types, shape)
    if logit_bias is not None:
        _check(logit_bias, "logit_bias", (torch.float32,), (E,))
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", _bf16_types(), (M, H))
    if topk_ids_out is not None:
        _check(topk_ids_out, "topk_ids_out", (torch.int32,), (M, top_k))
    if topk_weights_out is not None:
        _check(topk_weights_out, "topk_weights_out", (torch.float32,), (M, top_k))
    if ws is None:
        ws = workspace(M, E, top_k, H, max(I, 1), x.device)
    qw = QuantizedWeights(bits, int(qweights.get("group_size", 64)),
                          *(_ptr(qweights.get(n)) for n in ("w13_q", "w13_scales", "w13_biases",
                                                            "w2_q", "w2_scales", "w2_biases")))
    info = DispatchInfo()
    st = library().moe_forward_quantized(
        _ptr(x), _ptr(w_router), _ptr(logit_bias), ctypes.byref(qw), M, E, top_k, H, I,
        int(bool(renormalize)), _ptr(out), _ptr(topk_ids_out), _ptr(topk_weights_out),
        _ptr(ws), ws.numel(), ctypes.byref(info), _stream(stream))
    _raise("moe_forward_quantized", st)
    return out, info.as_dict()


def moe_mx_workspace_size(M_max: int, E: int, top_k: int, H: int, I: int) -> int:
    return int(library().moe_mx_workspace_size(M_max, E, top_k, H, I))


def mx_workspace(M_max: int, E: int, top_k: int, H: int, I: int, device=None):
    """Workspace tensor (uint8) for every moe_forward_mxfp8 call with M <= M_max."""
    torch = _torch()
    n = moe_mx_workspace_size(M_max, E, top_k, H, I)
    if n == 0:
        raise MoeError("moe_mx_workspace_size", -2)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def moe_mx_quantize(src, codes=None, scales=None, stream=None):
    """MXFP8 codes [rows, K] (uint8 E4M3) and scales [rows, K/32] (uint8
    E8M0) of bf16 rows src [rows, K]."""
    torch = _torch()
    rows, K = src.shape
    _check(src, "src", _bf16_types())
    if codes is None:
        codes = torch.empty((rows, K), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=src.device)
    _check(codes, "codes", (torch.uint8,), (rows, K))
    _check(scales, "scales", (torch.uint8,), (rows, K // 32))
    st = library().moe_mx_quantize(_ptr(src), rows, K, _ptr(codes), _ptr(scales), _stream(stream))
    _raise("moe_mx_quantize", st)
    return codes, scales


def moe_forward_mxfp8(x, w_router, mxw: dict, top_k: int, renormalize: bool = True,
                      logit_bias=None, out=None, topk_ids_out=None, topk_weights_out=None,
                      ws=None, stream=None):
    """The layer with MXFP8 experts and GEMM inputs.  ``mxw`` holds
    ``w13_codes`` [E, 2I, H], ``w13_scales`` [E, 2I, H/32], ``w2_codes``
    [E, H, I] and ``w2_scales`` [E, H, I/32] (uint8).  Returns (out [M, H]
    bf16, dispatch info dict)."""
    torch = _torch()
    M, H = x.shape
    E = w_router.shape[0]
    I = mxw["w2_codes"].shape[2]
    _check(x, "x", _bf16_types())
    _check(w_router, "w_router", _bf16_types(), (E, H))
    for name, shape in (("w13_codes", (E, 2 * I, H)), ("w13_scales", (E, 2 * I, H // 32)),
                        ("w2_codes", (E, H, I)), ("w2_scales", (E, H, I // 32))):
        _check(mxw[name], name, (torch.uint8,), shape)
    if logit_bias is not None:
        _check(logit_bias, "logit_bias", (torch.float32,), (E,))
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _check(out, "out", _bf16_types(), (M, H))
    if topk_ids_out is not None:
        _check(topk_ids_out, "topk_ids_out", (torch.int32,), (M, top_k))
    if topk_weights_out is not None:
        _check(topk_weights_out, "topk_weights_out", (torch.float32,), (M, top_k))
    if ws is None:
        ws = mx_workspace(M, E, top_k, H, I, x.device)
    w = MxWeights(*(_ptr(mxw[n]) for n in ("w13_codes", "w13_scales", "w2_codes", "w2_scales")))
    info = DispatchInfo()
    st = library().moe_forward_mxfp8(
        _ptr(x), _ptr(w_router), _ptr(logit_bias), ctypes.byref(w), M, E, top_k, H, I,
        int(bool(renormalize)), _ptr(out), _ptr(topk_ids_out), _ptr(topk_weights_out),
        _ptr(ws), ws.numel(), ctypes.byref(info), _stream(stream))
    _raise("moe_forward_mxfp8", st)
    return out, info.as_dict()
