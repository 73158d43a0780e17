#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

A step is one moe_forward call (route -> align -> GEMM 1 + SiLU*up -> GEMM 2 +
combine) on one batch of M tokens.  Steps cycle through L distinct synthetic
layers held in HBM (weights drawn on the device), so the 256 MB Infinity
Cache cannot serve the weights from one step to the next.  Inputs are
resident in HBM before the timed region starts.

Prints ONE JSON line:
  value            tokens/s of the whole layer (M * steps / elapsed)
  roofline         the dominant kernel's algorithmic bytes (or flops) per
                   launch / its mean launch time (HIP events on the stream it
                   runs on), against the MI355X peak
  cpu_baseline     the CPU oracle on a bounded sample of the same workload
                   (all BLAS threads, and one thread), with the host CPU model
  kernels_us       mean duration of every per-step call (events)
  prefill          the Zipf-routed Qwen3-shaped layer at 4096 tokens timed
                   the same way, with its own roofline (GEMM 1 flops / its
                   mean launch time against the bf16 MFMA peak), and the
                   same batch on 4- and 8-bit group-quantized experts
                   (expert flops / layer time against the bf16 MFMA peak)
  mxfp8            context: moe_forward_mxfp8 (MXFP8 experts and GEMM inputs)
                   on the same shape and batch, the L layers drawn as MXFP8
                   (mxfp8_M1: the same at one token, the per-pair GEMVs)
  quantized        context: moe_forward_quantized (affine 64-element groups,
                   4 and 8 bits) on the same shape at M = 1, 4 (per-pair GEMVs)
                   and 64 (streaming GEMMs), one captured HIP graph of the L
                   layers replayed
Default workload: the Qwen3-30B-A3B-shaped decode layer (E=128, top_k=8,
H=2048, I=768) at M=64 tokens.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5033.2       # MI355X dense fp8 MFMA, TFLOP/s

DEFAULT_WORKLOAD = ("qwen3_decode", 64)
PREFILL_WORKLOAD = ("qwen3_prefill", 4096)


VARIANT_NAMES = {0: "tiled", 1: "stream", 2: "pair_gemv", 3: "pair_gemv_quant", 4: "tiled_mxfp8",
                 5: "stream_mxfp8", 6: "pair_gemv_mxfp8", 7: "stream_quant", 8: "tiled_quant"}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="name:M, e.g. qwen3_prefill:4096 (default qwen3_decode:64)")
    ap.add_argument("--layers", type=int, default=16, help="distinct layers cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the many-layer stack (eager and HIP-graph replay) figures")
    ap.add_argument("--no-quant", action="store_true",
                    help="skip the group-quantized (4- and 8-bit) figures")
    ap.add_argument("--quant-sizes", default="4:1,4:4,4:64,8:1,8:4,8:64",
                    help="bits:M pairs of the quantized figures (default 4:1,4:4,4:64,8:1,8:4,8:64)")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the MXFP8 figures")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill object (the Zipf-routed Qwen3-shaped layer at 4096 "
                         "tokens, timed like the headline)")
    ap.add_argument("--prefill-layers", type=int, default=4,
                    help="distinct layers cycled by the prefill object (each 1.2 GB)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration runs)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (what the method must move / compute)
# ---------------------------------------------------------------------------

def algorithmic(shape, M, touched):
    """Per-forward algorithmic bytes and flops, and those of each GEMM.

    touched = number of experts with at least one pair.
      layer bytes  = touched*6*H*I (W13 + W2, bf16) + 2*E*H (router) + 4*M*H (x in, out)
      GEMM 1 bytes = touched*4*H*I (W13) + 2*M*H (x) + 2*P*I (act out)
      GEMM 2 bytes = touched*2*H*I (W2) + 2*P*I (act in) + 4*P (weights) + 2*M*H (out)
      layer flops  = 6*H*I*P + 2*M*H*E;  GEMM 1 flops = 4*H*I*P;  GEMM 2 flops = 2*H*I*P
    """
    E, k, H, I = shape.E, shape.top_k, shape.H, shape.I
    P = M * k
    return dict(
        layer_bytes=touched * 6 * H * I + 2 * E * H + 4 * M * H,
        layer_flops=6 * H * I * P + 2 * M * H * E,
        gemm1_bytes=touched * 4 * H * I + 2 * M * H + 2 * P * I,
        gemm1_flops=4 * H * I * P,
        gemm2_bytes=touched * 2 * H * I + 2 * P * I + 4 * P + 2 * M * H,
        gemm2_flops=2 * H * I * P,
    )


def kernel_source_hash():
    """Hash of the HIP sources; a stored counter profile is valid only for it."""
    import glob
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mixture_experts_ffn_renorm_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload_key, kernel):
    """HBM traffic per launch of `kernel` from the committed counter summary
    (profiles/counters_<workload>.md), or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload_key}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_hash:\s*(\w+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"traffic_bytes_per_launch\[{kernel}\]:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


# ---------------------------------------------------------------------------
# the run
# ---------------------------------------------------------------------------

def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding over several GPUs is a design, not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_workloads as wl
    import mixture_experts_ffn_renorm_amd as moe

    name, M = DEFAULT_WORKLOAD
    if args.workload:
        name, m = args.workload.split(":")
        M = int(m)
    shape = wl.WORKLOADS[name]
    E, k, H, I = shape.E, shape.top_k, shape.H, shape.I
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.library()
    stream = torch.cuda.current_stream()

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    L = max(1, args.layers)
    m = measure_layer(shape, M, L, args.steps, args.warmup, dev, stream)
    layers, x, ws, info = m.pop("_layers"), m.pop("_x"), m.pop("_ws"), m.pop("_info")
    result = {
        "metric": "MoE-layer tokens/s",
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_layer"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": m["config"],
        "layer": m["layer"],
        "kernels_us": m["kernels_us"],
        "roofline": m["roofline"],
    }

    # ---- the prefill half of the metric: the Zipf-routed Qwen3-shaped layer
    #      at 4096 tokens, timed the same way, with its own MFMA roofline ----
    if not args.no_prefill and (name, M) != PREFILL_WORKLOAD:
        pname, pM = PREFILL_WORKLOAD
        pm = measure_layer(wl.WORKLOADS[pname], pM, max(1, min(L, args.prefill_layers)),
                           args.steps, args.warmup, dev, stream)
        px = pm["_x"]
        for key in ("_layers", "_x", "_ws", "_info"):
            pm.pop(key)
        result["prefill"] = {"workload": pname, "M": pM, "ms_per_layer": pm["ms_per_layer"],
                             "tokens_per_s": pm["tokens_per_s"],
                             "mfma_frac": pm["layer"]["mfma_frac"],
                             "hbm_frac": pm["layer"]["hbm_frac"], "layer": pm["layer"],
                             "kernels_us": pm["kernels_us"], "roofline": pm["roofline"],
                             "config": pm["config"]}
        torch.cuda.empty_cache()
        if not args.no_quant:
            # the same batch on 4- and 8-bit group-quantized experts (tiles
            # with the codes widened in LDS), MFMA fraction as the bf16 layer's
            pshape = wl.WORKLOADS[pname]
            pq = quantized_figures(pshape, 2, px, dev, max(5, min(args.steps, 20)),
                                   [(4, pM), (8, pM)])
            for v in pq.values():
                fl = 6.0 * pshape.H * pshape.I * pM * pshape.top_k
                v["mfma_frac"] = round(fl / (v["us_per_layer"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
            result["prefill"]["quantized"] = pq
        del px
        torch.cuda.empty_cache()

    # ---- decode sweep (same shape, smaller batches) ----
    if not args.no_sweep and name == "qwen3_decode":
        sweep = {}
        for Ms in (1, 8):
            xs = x[:Ms].contiguous()
            outs = torch.empty((Ms, H), dtype=torch.bfloat16, device=dev)
            for i in range(args.warmup):
                lay = layers[i % L]
                _, sinfo = moe.moe_forward(xs, lay["w_router"], lay["w13"], lay["w2"], k, True,
                                           out=outs, ws=ws, stream=stream)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                lay = layers[i % L]
                moe.moe_forward(xs, lay["w_router"], lay["w13"], lay["w2"], k, True,
                                out=outs, ws=ws, stream=stream)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / args.steps
            sweep[f"M={Ms}"] = {"tokens_per_s": round(Ms / dt, 1), "us_per_layer": round(1e6 * dt, 2),
                                "variant": VARIANT_NAMES[sinfo["variant"]]}
        result["decode_sweep"] = sweep

    # ---- the cycled layers as one model-shaped stack: layer l's output is
    #      layer l + 1's input, one workspace, eager steps and one captured
    #      HIP graph replayed (context figures; `value` above is the layer) ----
    if not args.no_stack:
        from mixture_experts_ffn_renorm_amd.stack import MoEStack
        stack = MoEStack(layers, k, M, shape.renormalize)
        nst = max(2, min(args.steps, 20))
        stack.step(x)
        torch.cuda.synchronize()
        mem0 = torch.cuda.memory_allocated()
        t0 = time.perf_counter()
        for _ in range(nst):
            stack.step(x)
        torch.cuda.synchronize()
        eager_s = (time.perf_counter() - t0) / nst
        alloc_delta = torch.cuda.memory_allocated() - mem0
        x_static = x.clone()
        graph, _ = stack.capture(x_static)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(nst):
            graph.replay()
        torch.cuda.synchronize()
        graph_s = (time.perf_counter() - t0) / nst
        result["stack"] = {"layers": L, "launches_per_step": stack.last_launches,
                           "device_bytes_allocated_per_step": int(alloc_delta),
                           "us_per_layer_eager": round(1e6 * eager_s / L, 2),
                           "us_per_layer_graph": round(1e6 * graph_s / L, 2),
                           "layer_tokens_per_s_graph": round(M * L / graph_s, 1)}
        del graph, stack

    # ---- MXFP8 experts and GEMM inputs at the same batch (context) ----
    if not args.no_mx and H % 128 == 0 and I % 128 == 0:
        result["mxfp8"] = mxfp8_figures(shape, M, L, x, dev, max(5, min(args.steps, 50)))
        if M > 1 and name == "qwen3_decode":
            # one token: the per-pair MXFP8 GEMVs, beside decode_sweep's bf16 M=1
            result["mxfp8_M1"] = mxfp8_figures(shape, 1, L, x[:1].contiguous(), dev,
                                               max(5, min(args.steps, 50)))

    # ---- group-quantized expert weights at small batches (context) ----
    sizes = [tuple(int(v) for v in p.split(":")) for p in args.quant_sizes.split(",") if p]
    if not args.no_quant and sizes and shape.H % 64 == 0 and shape.I % 64 == 0 and M <= 64:
        result["quantized"] = quantized_figures(shape, L, x, dev, max(10, min(args.steps, 50)),
                                                sizes)

    # ---- the oracle on the host, on a bounded sample ----
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(shape, M, layers[0], x)

    print(json.dumps(result), flush=True)


def measure_layer(shape, M, L, steps, warmup, dev, stream):
    """Time moe_forward on one batch of M tokens over L device-resident
    layers cycled step by step, then each per-step C-ABI call on its own
    (launched `steps` times back to back between two HIP events on the
    launch stream, each with its own layer's routing and index lists).
    Returns tokens/s, ms per layer, the layer's algorithmic fractions, the
    per-call times and the dominant kernel's (GEMM 1) roofline."""
    import numpy as np
    import torch

    import moe_workloads as wl
    import mixture_experts_ffn_renorm_amd as moe

    name = shape.name
    E, k, H, I = shape.E, shape.top_k, shape.H, shape.I
    # ---- inputs resident in HBM: L distinct layers, one batch of x ----
    layers = [wl.make_device_layer(shape, M, layer=i + 1, device=dev) for i in range(L)]
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed_for(shape, M))
    x = torch.randn((M, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((M, k), dtype=torch.int32, device=dev)
    wts = torch.empty((M, k), dtype=torch.float32, device=dev)
    ws = moe.workspace(M, E, k, H, I, dev)
    torch.cuda.synchronize()

    def step(i):
        lay = layers[i % L]
        return moe.moe_forward(x, lay["w_router"], lay["w13"], lay["w2"], k,
                               shape.renormalize, logit_bias=lay["logit_bias"], out=out,
                               topk_ids_out=ids, topk_weights_out=wts, ws=ws, stream=stream)

    # touched experts per layer (from each layer's own routing)
    touched = []
    for i in range(L):
        _, info = step(i)
        touched.append(int(torch.unique(ids).numel()))
    torch.cuda.synchronize()
    mean_touched = float(np.mean(touched))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / steps
    tokens_per_s = M * steps / elapsed

    # ---- per-kernel times: the same work as separate C-ABI calls ----
    B = moe.moe_pick_block_m(M, E, k)
    cap, nbl = moe.align_capacity(M * k, E, B)
    act = torch.empty((M * k, I), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((M, E), dtype=torch.float32, device=dev)
    align_ws = torch.empty(max(moe.moe_align_workspace_size(M, k, E), 16), dtype=torch.uint8,
                           device=dev)
    routed = []
    for i in range(L):
        lay = layers[i]
        r_ids = torch.empty((M, k), dtype=torch.int32, device=dev)
        r_wts = torch.empty((M, k), dtype=torch.float32, device=dev)
        moe.moe_route(x, lay["w_router"], k, shape.renormalize, logit_bias=lay["logit_bias"],
                      topk_ids=r_ids, topk_weights=r_wts, logits_out=logits, stream=stream)
        lists = (torch.empty(cap, dtype=torch.int32, device=dev),
                 torch.empty(max(nbl, 1), dtype=torch.int32, device=dev),
                 torch.empty(E + 1, dtype=torch.int32, device=dev),
                 torch.empty(E, dtype=torch.int32, device=dev))
        moe.moe_align(r_ids, E, B, *lists, ws=align_ws, stream=stream)
        routed.append((r_ids, r_wts, lists))
    scratch_lists = tuple(torch.empty_like(t) for t in routed[0][2])

    def stage(sname, i):
        lay = layers[i % L]
        r_ids, r_wts, (s_ids, e_ids, b_off, cnt) = routed[i % L]
        if sname == "route":
            moe.moe_route(x, lay["w_router"], k, shape.renormalize, logit_bias=lay["logit_bias"],
                          topk_ids=ids, topk_weights=wts, logits_out=logits, stream=stream)
        elif sname == "align":
            moe.moe_align(r_ids, E, B, *scratch_lists, ws=align_ws, stream=stream)
        elif sname == "gemm1":
            moe.moe_grouped_gemm_w13_act(x, lay["w13"], s_ids, e_ids, b_off, k, B, act=act,
                                         stream=stream)
        else:
            moe.moe_grouped_gemm_w2_combine(act, lay["w2"], r_wts, s_ids, e_ids, b_off, M, k, B,
                                            out=out, ws=ws, stream=stream)

    kern_us = {}
    for n in ("route", "align", "gemm1", "gemm2"):
        for i in range(min(warmup, 10)):
            stage(n, i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            stage(n, i)
        e1.record(stream)
        torch.cuda.synchronize()
        kern_us[n] = 1e3 * e0.elapsed_time(e1) / steps
    del routed, scratch_lists, act

    work = algorithmic(shape, M, mean_touched)
    # the staged calls run the forward's kernel family at the same block size;
    # at block_m 1 GEMM 1 is the forward's own GEMV (in index-list order),
    # while the forward's GEMM 2 reads topk_ids and sums in the same launch
    variant = {1: "pair_gemv", 16: "stream"}.get(B, "tiled")
    # dominant kernel: GEMM 1 (2/3 of the weight bytes and of the flops)
    mfma_bound = variant == "tiled" and work["gemm1_flops"] / work["gemm1_bytes"] > \
        1e3 * BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 0.5
    t_g1 = kern_us["gemm1"] * 1e-6
    workload_key = f"{name}_M{M}"
    if mfma_bound:
        achieved = work["gemm1_flops"] / t_g1 / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
        roof["algorithmic_flops_per_launch"] = int(work["gemm1_flops"])
    else:
        achieved = work["gemm1_bytes"] / t_g1 / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = f"gemm1_{variant}"
    roof["mean_launch_us"] = round(kern_us["gemm1"], 2)
    roof["algorithmic_bytes_per_launch"] = int(work["gemm1_bytes"])
    roof["traffic"] = stored_traffic(workload_key, f"gemm1_{variant}")

    layer_s = ms_per_step * 1e-3
    return {
        "tokens_per_s": round(tokens_per_s, 1),
        "ms_per_layer": round(ms_per_step, 5),
        "config": {"workload": name, "description": shape.description, "M": M, "E": E,
                   "top_k": k, "H": H, "I": I, "renormalize": shape.renormalize,
                   "layers_cycled": L, "block_m": B, "variant": variant,
                   "forward_variant": VARIANT_NAMES[info["variant"]],
                   "mean_touched_experts": mean_touched},
        "layer": {"alg_bytes": int(work["layer_bytes"]), "alg_flops": int(work["layer_flops"]),
                  "hbm_frac": round(work["layer_bytes"] / layer_s / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(work["layer_flops"] / layer_s / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "kernels_us": {n: round(v, 2) for n, v in kern_us.items()},
        "roofline": roof,
        "_layers": layers, "_x": x, "_ws": ws, "_info": info,
    }


def quantized_alg_bytes(shape, M, bits, touched):
    """Per-forward algorithmic bytes with group-quantized expert weights:
    per touched expert the 3*H*I codes (bits/8 bytes each) and 4 bytes of
    bf16 scale and bias per 64-element group; plus the bf16 router and x in
    and out."""
    E, H, I = shape.E, shape.H, shape.I
    per_expert = 3 * H * I * bits // 8 + (3 * H * I // 64) * 4
    return touched * per_expert + 2 * E * H + 4 * M * H


def mxfp8_figures(shape, M, L, x, dev, reps):
    """moe_forward_mxfp8 on the workload's batch over L device-drawn MXFP8
    layers, the L calls captured once into a HIP graph and replayed `reps`
    times.  Algorithmic bytes: per touched expert 3*H*I E4M3 bytes and
    3*H*I/32 scale bytes, the bf16 router, x in and out; flops as the bf16
    layer (the GEMMs run at the fp8 rate)."""
    import numpy as np
    import torch

    import moe_workloads as wl
    import mixture_experts_ffn_renorm_amd as moe

    E, k, H, I = shape.E, shape.top_k, shape.H, shape.I
    layers = [wl.make_device_mx_layer(shape, M, layer=i + 1, device=dev) for i in range(L)]
    ws = moe.mx_workspace(M, E, k, H, I, dev)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ids = [torch.empty((M, k), dtype=torch.int32, device=dev) for _ in range(L)]

    def run_all():
        for i, lay in enumerate(layers):
            _, info = moe.moe_forward_mxfp8(x, lay["w_router"], lay["w"], k, shape.renormalize,
                                            logit_bias=lay["logit_bias"], out=out,
                                            topk_ids_out=ids[i], ws=ws)
        return info

    info = run_all()
    torch.cuda.synchronize()
    touched = float(np.mean([torch.unique(t).numel() for t in ids]))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / (reps * L)
    alg = touched * (3 * H * I + 3 * H * I // 32) + 2 * E * H + 4 * M * H
    flops = 6 * H * I * M * k
    del graph, layers
    return {"M": M, "us_per_layer": round(us, 2), "tokens_per_s": round(M / (us * 1e-6), 1),
            "alg_bytes": int(alg), "alg_flops": int(flops),
            "hbm_frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac_fp8": round(flops / (us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4),
            "mean_touched_experts": touched, "variant": VARIANT_NAMES[info["variant"]],
            "block_m": info["block_m"], "launches": info["launches"]}


def quantized_figures(shape, L, x, dev, reps, sizes):
    """moe_forward_quantized at the (bits, M) pairs of `sizes` over L
    device-drawn quantized layers: the L calls captured once into a HIP
    graph, replayed `reps` times (host marshalling out of the timed
    region)."""
    import numpy as np
    import torch

    import moe_workloads as wl
    import mixture_experts_ffn_renorm_amd as moe

    E, k, H, I = shape.E, shape.top_k, shape.H, shape.I
    res = {}
    ws = moe.workspace(max(m for _, m in sizes), E, k, H, I, dev)
    for bits in sorted({b for b, _ in sizes}):
        qlayers = [wl.make_device_quantized_layer(shape, 4, bits, layer=i + 1, device=dev)
                   for i in range(L)]
        for Ms in sorted(m for b, m in sizes if b == bits):
            xs = x[:Ms].contiguous() if x.shape[0] >= Ms else \
                torch.randn((Ms, H), device=dev).to(torch.bfloat16)
            out = torch.empty((Ms, H), dtype=torch.bfloat16, device=dev)
            ids = [torch.empty((Ms, k), dtype=torch.int32, device=dev) for _ in range(L)]

            def run_all():
                for i, ql in enumerate(qlayers):
                    _, info = moe.moe_forward_quantized(
                        xs, ql["w_router"], ql["q"], k, shape.renormalize,
                        logit_bias=ql["logit_bias"], out=out, topk_ids_out=ids[i], ws=ws)
                return info

            info = run_all()
            torch.cuda.synchronize()
            touched = float(np.mean([torch.unique(t).numel() for t in ids]))
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                run_all()
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / (reps * L)
            alg = quantized_alg_bytes(shape, Ms, bits, touched)
            res[f"b{bits}_M{Ms}"] = {
                "bits": bits, "M": Ms, "us_per_layer": round(us, 2),
                "tokens_per_s": round(Ms / (us * 1e-6), 1),
                "alg_bytes": int(alg), "hbm_frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "mean_touched_experts": touched, "variant": VARIANT_NAMES[info["variant"]],
                "launches": info["launches"]}
            del graph
        del qlayers
    return res


def cpu_model_name() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, M, lay, x, min_s=8.0, max_reps=40):
    """Time the CPU oracle (as it stands) on a bounded sample of the same
    workload: layer 0 of the cycle, the first S <= 64 tokens of the batch,
    the whole forward repeated until about `min_s` seconds of CPU work have
    run (at most `max_reps` times); tokens/s = reps * S / wall time.  Timed
    twice: with numpy's BLAS on all its threads (`value`, `cores`) and
    limited to one thread (`value_1thread`)."""
    import numpy as np
    import torch

    from oracle import moe_oracle as mo

    def bits(t):
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    S = min(M, 64)
    host = dict(x=bits(x[:S]), w_router=bits(lay["w_router"]), w13=bits(lay["w13"]),
                w2=bits(lay["w2"]),
                logit_bias=None if lay["logit_bias"] is None else lay["logit_bias"].cpu().numpy(),
                M=S, E=shape.E, top_k=shape.top_k, H=shape.H, I=shape.I,
                renormalize=shape.renormalize)

    def timed():
        reps = 0
        t0 = time.perf_counter()
        while True:
            mo.forward(host)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_s or reps >= max_reps:
                return reps, dt

    threads = None
    limits = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((p.get("num_threads") or 1) for p in threadpool_info()) or None
        limits = threadpool_limits
    except Exception:
        pass
    reps, dt = timed()
    res = {"value": round(reps * S / dt, 3), "unit": "tokens/s",
           "cores": threads or os.cpu_count(), "kind": "oracle",
           "sample": f"{S} tokens of layer 0 ({shape.name}, M={M}), the whole oracle forward "
                     f"run {reps} times; numpy float64, {dt:.2f} s wall",
           "host_cpus": os.cpu_count(), "cpu_model": cpu_model_name()}
    if limits is not None:
        with limits(limits=1):
            reps1, dt1 = timed()
        res["value_1thread"] = round(reps1 * S / dt1, 3)
        res["sample_1thread"] = f"the same sample run {reps1} times on one thread, {dt1:.2f} s wall"
    return res


if __name__ == "__main__":
    main()
