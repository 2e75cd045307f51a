"""Beam-1.0 mixture-of-experts block on one AMD Instinct MI355X (gfx950).

The block ("Welcome Beam: a 501B open model you can own, customize, and
scale", section "Mixture of Experts"): FP32 router GEMM, sigmoid scores,
group-limited top-8 selection (8 groups of 32, 4 groups kept by the sum of
their two best scores), token permutation, bf16 SwiGLU expert grouped GEMMs
and a weighted combine scaled by 2.5, with no shared expert.

All computation happens in the HIP kernels of ``libbeam_moe.so`` (C ABI in
include/beam_moe.h); this package only marshals torch tensors into it.
"""
from ._lib import (  # noqa: F401
    ENTRY_EXPERT_FFN, ENTRY_EXPERT_FFN_LORA, ENTRY_EXPERT_STAGE, ENTRY_LAYER, ENTRY_LAYER_LORA,
    ENTRY_PERMUTE, ENTRY_ROUTE, EXPORTS, LoraWeights, MoeLora, expert_ffn_lora, layer_forward_lora,
    LAYOUT_FP8_PACKED, LAYOUT_PACKED, LAYOUT_ROW_MAJOR, LIB_PATH, Fp8Weights, MoeConfig,
    MoeError, Workspace, combine, expert_down, expert_down_fp8, expert_ffn, expert_ffn_fp8,
    expert_gate_up, expert_gate_up_fp8, layer_forward, layer_forward_fp8,
    layer_forward_noalloc, lib, make_config,
    pack_weights, permute, quantize_fp8, route, route_replay, status_string, workspace_bytes,
    LIB_CHECKED_PATH, CHECK_BITS, check_flags, use_library,
)
