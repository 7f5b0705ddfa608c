"""CPU oracle for the quantized routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link
or execute this package; only the tests, the smoke check in
__graft_entry__.py and the cpu_baseline leg of bench.py use it.

It is a plain, slow, obviously correct fp64 implementation of what the layer
computes, written from the method's definition. It shares no code, header,
table or constant generator with the HIP library; both sides only read the
same seeded inputs from the `synth` package.
"""
from .moe import (  # noqa: F401
    bf16_bits_to_f64,
    f16_bits_to_f64,
    dequant_blocks,
    expert_weights,
    shared_weights,
    router_logits,
    softmax,
    select_topk,
    route,
    swiglu_ffn,
    moe_forward,
    rmsnorm,
    round_to_bf16_bits,
    DenseExperts,
)
