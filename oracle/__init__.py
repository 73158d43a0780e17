"""CPU oracle for the mixture-of-experts SwiGLU layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The HIP library never uses it, and it shares no code with the HIP path: its
only common dependency with the GPU side is the seeded input generator in
``moe_workloads`` (which holds none of the layer's arithmetic).

Every function is pinned by ``tests/test_oracle_pins.py`` to something other
than itself (the pages' toy example, hand-computed closed forms, a pure-Python
dense brute force, library special cases, invariants).  No function of this
oracle is "parity unpinned".
"""

from .moe_oracle import (  # noqa: F401
    widen_bf16,
    router_logits,
    route,
    softmax_probs,
    weights_of,
    topk_margin,
    align,
    swiglu,
    expert_ffn,
    pair_activations,
    layer_forward,
    combine_from_act,
    forward,
    unpack_codes,
    dequantize_affine,
    forward_quantized,
    dequantized_experts,
    QUANT_GROUP,
    MX_BLOCK,
    e4m3_value,
    e8m0_value,
    e4m3_round,
    mx_quantize,
    mx_dequantize,
    round_to_bf16_via_f32,
    forward_mxfp8,
    mx_layer_forward,
)
