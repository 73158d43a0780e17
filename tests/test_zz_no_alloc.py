"""moe_forward_noalloc (the library's own device scratch array instead of a
caller workspace) against moe_forward on the same inputs, through the C
ABI: two calls in a row, the second with a smaller batch (the array keeps
the first call's contents), then a per-pair batch; outputs and routing
must equal moe_forward's bit for bit and meet the oracle criteria; no
device memory is allocated by the calls; a batch whose workspace would
exceed the array is rejected before any launch."""

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


def _forward_pair(lay, d):
    """(moe_forward out/ids/wts, moe_forward_noalloc out/ids/wts, info of each,
    device bytes allocated during the no-alloc call)."""
    import torch
    moe = _moe()
    M, k, H = lay["M"], lay["top_k"], lay["H"]
    outs = []
    for noalloc in (False, True):
        out = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
        wts = torch.full((M, k), -1.0, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        if noalloc:
            _, info = moe.moe_forward_noalloc(d["x"], d["w_router"], d["w13"], d["w2"], k,
                                              lay["renormalize"], logit_bias=d["logit_bias"],
                                              out=out, topk_ids_out=ids, topk_weights_out=wts)
        else:
            _, info = moe.moe_forward(d["x"], d["w_router"], d["w13"], d["w2"], k,
                                      lay["renormalize"], logit_bias=d["logit_bias"], out=out,
                                      topk_ids_out=ids, topk_weights_out=wts)
        torch.cuda.synchronize()
        grown = torch.cuda.memory_allocated() - before
        outs.append((out, ids.cpu().numpy(), wts.cpu().numpy().astype(np.float64), info, grown))
    return outs


@pytest.fixture(scope="module")
def big_layer():
    return wl.make_layer("qwen3_decode", 64)


def _check(lay):
    import torch
    d = h.layer_to_device(lay)
    (o_ref, i_ref, w_ref, info_ref, _), (o, i, w, info, grown) = _forward_pair(lay, d)
    print(f"no-alloc case M={lay['M']} block_m={info['block_m']}", flush=True)
    assert grown == 0
    assert info == info_ref
    assert np.array_equal(i, i_ref) and np.array_equal(w, w_ref)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    # ... and the oracle criteria on the GPU's own ids
    M = lay["M"]
    toks = h.sample_tokens(M, 32, 1)
    r = mo.route(lay["x"][toks], lay["w_router"], lay["top_k"], lay["renormalize"], None)
    wr = h.check_routing(i[toks], w[toks], r, lay["renormalize"])
    full_ids, full_w = h.scatter_routing(M, toks, i[toks], wr)
    ref_y = mo.layer_forward(lay["x"], lay["w13"], lay["w2"], full_ids, full_w, toks)
    h.assert_close_outputs(h.host_bf16_to_f64(o)[toks], ref_y, "no-alloc output")


def test_noalloc_two_calls_second_smaller(big_layer):
    """64 tokens (streaming kernels, four-workgroup fused top-k + lists), then
    16 tokens of the same layer (the array still holds the first call's
    lists and rows), then 2 tokens (per-pair GEMVs, no lists)."""
    for M in (64, 16, 2):
        lay = dict(big_layer)
        lay["x"] = big_layer["x"][:M]
        lay["M"] = M
        _check(lay)


def test_noalloc_rejects_batches_beyond_the_array():
    import torch
    moe = _moe()
    E, k, H, I = 128, 8, 2048, 768
    M = 1
    while moe.moe_workspace_size(M, E, k, H, I) <= moe.MOE_NOALLOC_SCRATCH_BYTES:
        M *= 2
    x = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((E, H), dtype=torch.bfloat16, device="cuda")
    w13 = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((E, H, I), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as exc:
        moe.moe_forward_noalloc(x, wr, w13, w2, k, True)
    assert exc.value.status == -3      # MOE_ERR_WORKSPACE, nothing launched
