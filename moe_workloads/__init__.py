"""Seeded synthetic inputs for the decode-time quantized-expert MoE block.

This module is shared by the oracle tests and by the HIP path's tests and
benchmark.  It holds *no* arithmetic of the method itself (no dequantisation,
no routing, no GEMV, no combine): only the shapes of the workloads and the
generators of their inputs, i.e. activations, router logits and
affine-4-bit-quantised expert weights.

Workload shapes follow the qwen3-30b-a3b-4bit description on the page
"perf(moe): batched decode scales 1.55x against 3.25x on dense" (section
"Current Behavior": 48 all-MoE layers, 128 experts, top_k 8, expert
intermediate size 768, 4-bit group 64) and the "256-expert top-6" checkpoints
of the page "perf(moe): attribute the MoE decode gap at the M = 1 expert
gather" (section "Corroborating observation").  Hidden sizes, value
distributions, the sharing and Zipf routing recipes, the scale sidecar and the
clamp limit are readings of the configuration list that accompanies this
project (the pages state none of them).
"""

from .gen import (  # noqa: F401
    Shape,
    SHAPES,
    Layer,
    POISON_F16,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    pack_bits,
    quantize_affine,
    quantize_affine4,
    make_layer,
    make_x,
    make_logits,
    make_router,
    make_layer_device,
    rng_for,
)
