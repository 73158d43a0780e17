"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the
algorithmic byte and flop counts the roofline fractions divide by, and the
rule that counter-derived traffic is reported only for the kernel sources it
was recorded on."""

from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

import pytest

import moe_workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_counts_qwen3_shapes():
    """Per-expert bf16 weights 6*H*I = 9,437,184 bytes at the Qwen3 shape;
    GEMM 1 at the 4096-token prefill is 4*P*H*I = 206,158,430,208 flops."""
    b = _bench()
    shape = wl.WORKLOADS["qwen3_prefill"]
    w = b.algorithmic(shape, 4096, touched=1)
    P = 4096 * 8
    assert w["gemm1_flops"] == 206_158_430_208
    assert w["gemm2_flops"] == w["gemm1_flops"] // 2
    assert w["layer_flops"] == 3 * w["gemm2_flops"] + 2 * 4096 * 2048 * 128
    # one touched expert: its weights, the router, x in and out
    assert w["layer_bytes"] == 9_437_184 + 2 * 128 * 2048 + 4 * 4096 * 2048
    # the two GEMMs' weight bytes add up to the layer's
    w2 = b.algorithmic(shape, 4096, touched=2)
    assert (w2["gemm1_bytes"] - w["gemm1_bytes"]) + (w2["gemm2_bytes"] - w["gemm2_bytes"]) == 9_437_184
    assert w["gemm1_bytes"] == 4 * 2048 * 768 + 2 * 4096 * 2048 + 2 * P * 768


@pytest.mark.parametrize("bits", [4, 8])
def test_quantized_bytes(bits):
    b = _bench()
    shape = wl.WORKLOADS["qwen3_decode"]
    H, I = 2048, 768
    per = 3 * H * I * bits // 8 + 3 * H * I // 64 * 4
    assert b.quantized_alg_bytes(shape, 64, bits, touched=10) == \
        10 * per + 2 * 128 * H + 4 * 64 * H


def test_traffic_only_for_the_recorded_sources(tmp_path, monkeypatch):
    b = _bench()
    (tmp_path / "profiles").mkdir()
    f = tmp_path / "profiles" / "counters_demo.md"
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    cur = b.kernel_source_hash()
    f.write_text(f"source_hash: {cur}\ntraffic_bytes_per_launch[gemm1_stream]: 1234.5\n")
    assert b.stored_traffic("demo", "gemm1_stream") == 1234.5
    assert b.stored_traffic("demo", "gemm2_stream") is None
    f.write_text("source_hash: 0000000000000000\ntraffic_bytes_per_launch[gemm1_stream]: 1234.5\n")
    assert b.stored_traffic("demo", "gemm1_stream") is None
    assert b.stored_traffic("absent", "gemm1_stream") is None
