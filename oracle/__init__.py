"""Float64 CPU oracle for the W4 g128 sparse MoE layer.

Test infrastructure only: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.
"""
from .moe_oracle import (  # noqa: F401
    GROUP, rn16, group_quantize, pack_w4, unpack_w4, unpack_plain_w4, pack_w8, unpack_w8, dequant_w8, pack_scales,
    unpack_scales, dequant, router_logits,
    softmax, topk_order, route, permute, gather_rows, silu, swiglu_ffn,
    expert_ffn_w4, combine, rmsnorm, moe_layer, tie_excused,
)
