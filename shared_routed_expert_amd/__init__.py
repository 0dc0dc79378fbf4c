"""Fused shared + routed MoE layer (GLM4-MoE Shared Experts Fusion) for AMD MI355X / gfx950.

The compute lives in libsrmoe.so (hand-written HIP kernels behind a C ABI,
declared in include/srmoe.h); this package is its thin ctypes binding plus
buffer plumbing. Build the library with `python -m shared_routed_expert_amd.build`.
The binding is loaded on first attribute access, so building never needs an
already built library; using it without one raises ImportError.
"""
_BINDING = ("lib", "LIB_PATH", "SrmoeError", "SCALE_PER_CHANNEL", "SCALE_BLOCK128",
            "moe_route_topk_plus_shared", "moe_align_by_expert", "moe_fused_ffn", "moe_ffn_quant_x",
            "moe_ffn_gate_up", "moe_ffn_down", "moe_ffn_experts", "moe_ffn_experts_one_kernel",
            "moe_combine", "moe_layer_forward", "moe_sorted_capacity", "moe_align_workspace_bytes",
            "moe_route_topk", "moe_combine_unfused", "moe_router_logits", "moe_router_workspace_bytes",
            "moe_ffn_workspace_bytes", "moe_ffn_workspace_offsets", "moe_qk_norm_rope", "moe_rope_cos_sin_table",
            "moe_route_from_x", "moe_route_from_x_workspace_bytes", "moe_layer_forward_from_x",
            "moe_workspace_bytes", "moe_status_string", "moe_layer_forward_staged",
            "moe_layer_forward_noalloc", "NOALLOC_SCRATCH_BYTES")
_LAYER = ("FusedMoE", "UnfusedMoE", "DeviceWeights")


def __getattr__(name):
    if name in _BINDING:
        from . import _lib
        return getattr(_lib, name)
    if name in _LAYER:
        from . import layer
        return getattr(layer, name)
    raise AttributeError(name)
