"""CPU oracle of the DiffusionGemma 26B-A4B MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark. The GPU library never uses it.
"""
from .binding import (  # noqa: F401
    load, moe_forward, route, permute, expert_ffn, dequant_i4, dequant_q8_0, dequant_mxfp4, dequant_mxfp8,
    gelu_tanh_f32,
    gelu_tanh_f64, half_to_float, float_to_bf16_bits, canvas_head,
)
