"""ctypes binding of libsrmoe.so: argument marshalling only.

Every function here has the name of the C entry point it calls and only turns
torch tensors into device pointers (and the current torch stream into a
hipStream_t). All computation happens in the library's HIP kernels. If the
library has not been built, or was built from other sources than the ones beside
it, the import fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsrmoe.so")

SRMOE_OK = 0
SCALE_PER_CHANNEL = 0
SCALE_BLOCK128 = 1


class SrmoeError(RuntimeError):
    def __init__(self, name, status, lib):
        msg = lib.srmoe_status_string(status).decode()
        hip = lib.srmoe_last_hip_error() if status == -4 else 0
        super().__init__(f"{name} failed: {msg} (status {status}, hip error {hip})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m shared_routed_expert_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sigs = {
        "moe_route_topk_plus_shared": ([P, I, I, I, F, P, P, P], I),
        "moe_align_by_expert": ([P, I, I, I, I, P, P, P, P, P, P, Z, P], I),
        "moe_fused_ffn": ([P, P, P, P, P, I, I, I, I, I, I, I, P, P, P, P, P, Z, P], I),
        "moe_ffn_quant_x": ([P, I, I, I, I, I, I, I, P, Z, P], I),
        "moe_ffn_gate_up": ([P, P, I, I, I, I, I, I, I, P, P, P, P, Z, P], I),
        "moe_ffn_down": ([P, P, I, I, I, I, I, I, I, P, P, P, P, P, Z, P], I),
        "moe_ffn_experts": ([P, P, P, P, I, I, I, I, I, I, I, P, P, P, P, P, Z, P], I),
        "moe_ffn_experts_one_kernel": ([I, I, I], I),
        "moe_combine": ([P, I, I, I, P, Z, P, P], I),
        "moe_route_topk": ([P, I, I, I, P, P, P], I),
        "moe_router_logits": ([P, P, P, I, I, I, P, P, Z, P], I),
        "moe_router_workspace_bytes": ([I, I, I], Z),
        "moe_combine_unfused": ([I, I, I, P, Z, P, Z, P, P], I),
        "moe_layer_forward": ([P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, P, P, P, P, P, Z, P, Z, P, P], I),
        "moe_layer_forward_staged": ([P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, P, P, P, P, P, Z, P, Z, P,
                                      P, P, I, P, P], I),
        "moe_workspace_bytes": ([I, I, I, I, I, I, I], Z),
        "moe_layer_forward_noalloc": ([P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P], I),
        "moe_status_string": ([I], ctypes.c_char_p),
        "moe_qk_norm_rope": ([P, I, I, I, I, I, I, P, P, F, P, P, I, I, P], I),
        "moe_route_from_x": ([P, P, P, I, I, I, I, F, P, P, P, Z, P], I),
        "moe_route_from_x_workspace_bytes": ([I, I, I], Z),
        "moe_layer_forward_from_x": ([P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, P, P, P, P, P, Z, P, Z,
                                      P, Z, P, P], I),
        "moe_rope_cos_sin_table": ([P, I, I, ctypes.c_double, P], I),
        "moe_sorted_capacity": ([I, I, I, I], Z),
        "moe_align_workspace_bytes": ([I, I, I], Z),
        "moe_ffn_workspace_bytes": ([I, I, I, I, I, I, I], Z),
        "moe_ffn_workspace_offsets": ([I, I, I, I, I, I, I, P], I),
        "srmoe_status_string": ([I], ctypes.c_char_p),
        "srmoe_last_hip_error": ([], I),
        "srmoe_source_hash": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    from .build import source_hash
    stamp, want = lib.srmoe_source_hash().decode(), source_hash()
    if stamp != want:
        raise ImportError(f"{LIB_PATH} was built from other sources (stamp {stamp}, sources {want}): "
                          "rebuild it with `python -m shared_routed_expert_amd.build`")
    return lib


lib = _load()

EXPORTED = ("moe_route_topk_plus_shared", "moe_align_by_expert", "moe_fused_ffn", "moe_ffn_quant_x",
            "moe_ffn_gate_up", "moe_ffn_down", "moe_ffn_experts", "moe_ffn_experts_one_kernel",
            "moe_combine", "moe_layer_forward", "moe_route_topk", "moe_combine_unfused", "moe_router_logits",
            "moe_router_workspace_bytes", "moe_qk_norm_rope", "moe_rope_cos_sin_table", "moe_route_from_x",
            "moe_route_from_x_workspace_bytes", "moe_layer_forward_from_x", "moe_sorted_capacity",
            "moe_align_workspace_bytes", "moe_ffn_workspace_bytes", "moe_ffn_workspace_offsets",
            "srmoe_status_string", "srmoe_last_hip_error", "moe_workspace_bytes", "moe_status_string",
            "moe_layer_forward_staged", "moe_layer_forward_noalloc", "srmoe_source_hash")


def _ptr(t):
    """Device pointer of a tensor, or an int / None passed through (raw pointers in tests)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name, status):
    if status != SRMOE_OK:
        raise SrmoeError(name, status, lib)
    return status


def moe_sorted_capacity(T, K1, E1, block_m):
    return lib.moe_sorted_capacity(T, K1, E1, block_m)


def moe_align_workspace_bytes(T, K1, E1):
    return lib.moe_align_workspace_bytes(T, K1, E1)


def moe_ffn_workspace_bytes(T, H, I, E1, K1, block_m, scale_mode):
    return lib.moe_ffn_workspace_bytes(T, H, I, E1, K1, block_m, scale_mode)


def moe_workspace_bytes(T, H, I, E1, K1, block_m, scale_mode):
    return lib.moe_workspace_bytes(T, H, I, E1, K1, block_m, scale_mode)


def moe_status_string(status):
    return lib.moe_status_string(status).decode()


def moe_ffn_workspace_offsets(T, H, I, E1, K1, block_m, scale_mode):
    """Returns a dict of byte offsets: slot_out, xq, sx, a, aq, sa, rs, total."""
    arr = (ctypes.c_size_t * 8)()
    _check("moe_ffn_workspace_offsets",
           lib.moe_ffn_workspace_offsets(T, H, I, E1, K1, block_m, scale_mode, arr))
    return dict(zip(("slot_out", "xq", "sx", "a", "aq", "sa", "rs", "total"), list(arr)))


def moe_route_topk_plus_shared(logits, T, E, K, shared_weight, topk_ids, topk_w, stream=None, check=True):
    st = lib.moe_route_topk_plus_shared(_ptr(logits), T, E, K, shared_weight, _ptr(topk_ids),
                                        _ptr(topk_w), _stream(stream))
    return _check("moe_route_topk_plus_shared", st) if check else st


def moe_align_by_expert(topk_ids, T, K1, E1, block_m, sorted_slot_ids, block_expert, expert_counts,
                        expert_offsets, num_padded, workspace, ws_bytes, stream=None, check=True):
    st = lib.moe_align_by_expert(_ptr(topk_ids), T, K1, E1, block_m, _ptr(sorted_slot_ids),
                                 _ptr(block_expert), _ptr(expert_counts), _ptr(expert_offsets),
                                 _ptr(num_padded), _ptr(workspace), ws_bytes, _stream(stream))
    return _check("moe_align_by_expert", st) if check else st


def moe_fused_ffn(x, w13, s13, w2, s2, scale_mode, T, H, I, E1, K1, block_m, sorted_slot_ids,
                  block_expert, num_padded, topk_w, workspace, ws_bytes, stream=None, check=True):
    st = lib.moe_fused_ffn(_ptr(x), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), scale_mode, T, H, I, E1,
                           K1, block_m, _ptr(sorted_slot_ids), _ptr(block_expert), _ptr(num_padded),
                           _ptr(topk_w), _ptr(workspace), ws_bytes, _stream(stream))
    return _check("moe_fused_ffn", st) if check else st


def moe_ffn_quant_x(x, scale_mode, T, H, I, E1, K1, block_m, workspace, ws_bytes, stream=None, check=True):
    st = lib.moe_ffn_quant_x(_ptr(x), scale_mode, T, H, I, E1, K1, block_m, _ptr(workspace), ws_bytes,
                             _stream(stream))
    return _check("moe_ffn_quant_x", st) if check else st


def moe_ffn_gate_up(w13, s13, scale_mode, T, H, I, E1, K1, block_m, sorted_slot_ids, block_expert,
                    num_padded, workspace, ws_bytes, stream=None, check=True):
    st = lib.moe_ffn_gate_up(_ptr(w13), _ptr(s13), scale_mode, T, H, I, E1, K1, block_m,
                             _ptr(sorted_slot_ids), _ptr(block_expert), _ptr(num_padded),
                             _ptr(workspace), ws_bytes, _stream(stream))
    return _check("moe_ffn_gate_up", st) if check else st


def moe_ffn_down(w2, s2, scale_mode, T, H, I, E1, K1, block_m, sorted_slot_ids, block_expert,
                 num_padded, topk_w, workspace, ws_bytes, stream=None, check=True):
    st = lib.moe_ffn_down(_ptr(w2), _ptr(s2), scale_mode, T, H, I, E1, K1, block_m,
                          _ptr(sorted_slot_ids), _ptr(block_expert), _ptr(num_padded), _ptr(topk_w),
                          _ptr(workspace), ws_bytes, _stream(stream))
    return _check("moe_ffn_down", st) if check else st


def moe_ffn_experts(w13, s13, w2, s2, scale_mode, T, H, I, E1, K1, block_m, sorted_slot_ids, block_expert,
                    num_padded, topk_w, workspace, ws_bytes, stream=None, check=True):
    st = lib.moe_ffn_experts(_ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), scale_mode, T, H, I, E1, K1, block_m,
                             _ptr(sorted_slot_ids), _ptr(block_expert), _ptr(num_padded), _ptr(topk_w),
                             _ptr(workspace), ws_bytes, _stream(stream))
    return _check("moe_ffn_experts", st) if check else st


def moe_ffn_experts_one_kernel(H, I, block_m):
    return bool(lib.moe_ffn_experts_one_kernel(H, I, block_m))


def moe_combine(topk_w, T, K1, H, workspace, ws_bytes, out, stream=None, check=True):
    st = lib.moe_combine(_ptr(topk_w), T, K1, H, _ptr(workspace), ws_bytes, _ptr(out), _stream(stream))
    return _check("moe_combine", st) if check else st


def moe_router_workspace_bytes(T, H, E):
    return lib.moe_router_workspace_bytes(T, H, E)


def moe_router_logits(x, w_router, bias, T, H, E, logits, workspace, ws_bytes, stream=None, check=True):
    st = lib.moe_router_logits(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, _ptr(logits), _ptr(workspace),
                               ws_bytes, _stream(stream))
    return _check("moe_router_logits", st) if check else st


def moe_route_topk(logits, T, E, K, topk_ids, topk_w, stream=None, check=True):
    st = lib.moe_route_topk(_ptr(logits), T, E, K, _ptr(topk_ids), _ptr(topk_w), _stream(stream))
    return _check("moe_route_topk", st) if check else st


def moe_combine_unfused(T, K, H, routed_ws, routed_ws_bytes, shared_ws, shared_ws_bytes, out, stream=None,
                        check=True):
    st = lib.moe_combine_unfused(T, K, H, _ptr(routed_ws), routed_ws_bytes, _ptr(shared_ws), shared_ws_bytes,
                                 _ptr(out), _stream(stream))
    return _check("moe_combine_unfused", st) if check else st


def moe_layer_forward(x, logits, w13, s13, w2, s2, scale_mode, T, H, I, E, K, shared_weight, block_m,
                      topk_ids, topk_w, sorted_slot_ids, block_expert, expert_counts, expert_offsets,
                      num_padded, align_ws, align_ws_bytes, ffn_ws, ffn_ws_bytes, out, stream=None,
                      check=True):
    st = lib.moe_layer_forward(_ptr(x), _ptr(logits), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
                               scale_mode, T, H, I, E, K, shared_weight, block_m, _ptr(topk_ids),
                               _ptr(topk_w), _ptr(sorted_slot_ids), _ptr(block_expert),
                               _ptr(expert_counts), _ptr(expert_offsets), _ptr(num_padded),
                               _ptr(align_ws), align_ws_bytes, _ptr(ffn_ws), ffn_ws_bytes, _ptr(out),
                               _stream(stream))
    return _check("moe_layer_forward", st) if check else st


def moe_layer_forward_staged(x, logits, w13, s13, w2, s2, scale_mode, T, H, I, E, K, shared_weight, block_m,
                             topk_ids, topk_w, sorted_slot_ids, block_expert, expert_counts, expert_offsets,
                             num_padded, align_ws, align_ws_bytes, ffn_ws, ffn_ws_bytes, out, events,
                             stream=None, check=True):
    """moe_layer_forward with the given torch.cuda.Events (already created: recorded once)
    recorded between its stages. Returns the list of stage names, one per recorded interval."""
    n = len(events)
    ev = (ctypes.c_void_p * max(n, 1))(*[e.cuda_event for e in events])
    names = (ctypes.c_char_p * max(n, 1))()
    rec = ctypes.c_int(0)
    st = lib.moe_layer_forward_staged(_ptr(x), _ptr(logits), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
                                      scale_mode, T, H, I, E, K, shared_weight, block_m, _ptr(topk_ids),
                                      _ptr(topk_w), _ptr(sorted_slot_ids), _ptr(block_expert),
                                      _ptr(expert_counts), _ptr(expert_offsets), _ptr(num_padded),
                                      _ptr(align_ws), align_ws_bytes, _ptr(ffn_ws), ffn_ws_bytes, _ptr(out),
                                      _stream(stream), ev, n, names, ctypes.byref(rec))
    if check:
        _check("moe_layer_forward_staged", st)
    return [names[i].decode() for i in range(max(rec.value - 1, 0))]


def moe_layer_forward_noalloc(x, logits, w13, s13, w2, s2, scale_mode, T, H, I, E, K, shared_weight, block_m, out,
                              stream=None, check=True):
    st = lib.moe_layer_forward_noalloc(_ptr(x), _ptr(logits), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), scale_mode,
                                       T, H, I, E, K, shared_weight, block_m, _ptr(out), _stream(stream))
    return _check("moe_layer_forward_noalloc", st) if check else st


NOALLOC_SCRATCH_BYTES = 64 << 20   # SRMOE_NOALLOC_SCRATCH_BYTES


def moe_qk_norm_rope(qkv, T, num_q_heads, num_kv_heads, head_dim, rotary_dim, neox, q_norm_w, k_norm_w, eps,
                     positions, cos_sin, max_pos, fused=True, stream=None, check=True):
    st = lib.moe_qk_norm_rope(_ptr(qkv), T, num_q_heads, num_kv_heads, head_dim, rotary_dim, int(neox),
                              _ptr(q_norm_w), _ptr(k_norm_w), eps, _ptr(positions), _ptr(cos_sin), max_pos,
                              int(fused), _stream(stream))
    return _check("moe_qk_norm_rope", st) if check else st


def moe_rope_cos_sin_table(cos_sin, max_pos, rotary_dim, theta, stream=None, check=True):
    st = lib.moe_rope_cos_sin_table(_ptr(cos_sin), max_pos, rotary_dim, float(theta), _stream(stream))
    return _check("moe_rope_cos_sin_table", st) if check else st


def moe_route_from_x_workspace_bytes(T, H, E):
    return lib.moe_route_from_x_workspace_bytes(T, H, E)


def moe_route_from_x(x, w_router, bias, T, H, E, K, shared_weight, topk_ids, topk_w, workspace, ws_bytes,
                     stream=None, check=True):
    st = lib.moe_route_from_x(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, K, shared_weight, _ptr(topk_ids),
                              _ptr(topk_w), _ptr(workspace), ws_bytes, _stream(stream))
    return _check("moe_route_from_x", st) if check else st


def moe_layer_forward_from_x(x, w_router, bias, w13, s13, w2, s2, scale_mode, T, H, I, E, K, shared_weight,
                             block_m, topk_ids, topk_w, sorted_slot_ids, block_expert, expert_counts,
                             expert_offsets, num_padded, router_ws, router_ws_bytes, align_ws, align_ws_bytes,
                             ffn_ws, ffn_ws_bytes, out, stream=None, check=True):
    st = lib.moe_layer_forward_from_x(
        _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), scale_mode, T, H, I, E, K,
        shared_weight, block_m, _ptr(topk_ids), _ptr(topk_w), _ptr(sorted_slot_ids), _ptr(block_expert),
        _ptr(expert_counts), _ptr(expert_offsets), _ptr(num_padded), _ptr(router_ws), router_ws_bytes,
        _ptr(align_ws), align_ws_bytes, _ptr(ffn_ws), ffn_ws_bytes, _ptr(out), _stream(stream))
    return _check("moe_layer_forward_from_x", st) if check else st
