"""Fused grouped W4A16 mixture-of-experts layer for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``lib/libw4a16moe.so`` (C ABI in
include/w4a16_moe.h); this package is its argument-marshalling binding.  The
library has to be built in-tree first (``w4a16_grouped_expert_amd._build.build``);
there is no fallback implementation.
"""
from .api import (MODE_AUTO, active_experts, MODE_DECODE, MODE_PREFILL, AlignOut, MoELayer, RouteOut, SlotCache,  # noqa: F401
                  alloc_align, alloc_counter, alloc_route, alloc_workspace, expert_layout, ffn_workspace_bytes,
                  moe_align, moe_align_into, moe_route, moe_route_align_into, moe_route_into, moe_w4a16_grouped_ffn,
                  moe_w4a16_grouped_ffn_into, moe_w4a16_grouped_ffn_noalloc_into, NOALLOC_SCRATCH_BYTES,
                  pack_experts, pack_w4_g128, timing_enable, timing_read,
                  timing_reset, bf16_expert_bytes, pack_bf16_experts, moe_bf16_grouped_ffn, moe_bf16_grouped_ffn_into,
                  mat_layout, mat_from_w4, moe_mat_grouped_ffn_into, alloc_layer_counters, layer_routing_timed_out,
                  decode_layer_workspace_bytes, moe_decode_layer, moe_decode_layer_into,
                  moe_mat_decode_layer_into)
from ._lib import LIB_PATH, MoeError, lib  # noqa: F401
