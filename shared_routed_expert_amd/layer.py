"""Buffers and call sequence for one fused shared + routed MoE layer on the GPU.

Torch provides device memory and the stream; every step of the layer runs in
libsrmoe.so's HIP kernels through the four C calls (route, align, fused FFN,
combine).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L


@dataclass
class DeviceWeights:
    w13: torch.Tensor   # uint8 [E1, 2I, H]
    s13: torch.Tensor   # float32
    w2: torch.Tensor    # uint8 [E1, H, I]
    s2: torch.Tensor    # float32
    scale_mode: int

    @staticmethod
    def from_numpy(w13_q, s13, w2_q, s2, device="cuda"):
        mode = L.SCALE_PER_CHANNEL if s13.ndim == 2 else L.SCALE_BLOCK128
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return DeviceWeights(up(w13_q), up(s13), up(w2_q), up(s2), mode)


class FusedMoE:
    """One layer's routing tables, sort arrays, workspaces and output for fixed sizes."""

    def __init__(self, T, H, I, E, K, block_m, scale_mode, device="cuda"):
        self.T, self.H, self.I, self.E, self.K = T, H, I, E, K
        self.E1, self.K1 = E + 1, K + 1
        self.block_m, self.scale_mode = block_m, scale_mode
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.P_max = L.moe_sorted_capacity(T, self.K1, self.E1, block_m)
        self.topk_ids = torch.empty((T, self.K1), **i32)
        self.topk_w = torch.empty((T, self.K1), dtype=torch.float32, device=dev)
        self.sorted_slot_ids = torch.empty(self.P_max, **i32)
        self.block_expert = torch.empty(self.P_max // block_m, **i32)
        self.expert_counts = torch.empty(self.E1, **i32)
        self.expert_offsets = torch.empty(self.E1 + 1, **i32)
        self.num_padded = torch.empty(1, **i32)
        self.align_ws_bytes = L.moe_align_workspace_bytes(T, self.K1, self.E1)
        self.align_ws = torch.empty(self.align_ws_bytes, dtype=torch.uint8, device=dev)
        self.ws_bytes = L.moe_ffn_workspace_bytes(T, H, I, self.E1, self.K1, block_m, scale_mode)
        if self.ws_bytes == 0:
            raise ValueError("unsupported FFN shape")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.offsets = L.moe_ffn_workspace_offsets(T, H, I, self.E1, self.K1, block_m, scale_mode)

    def dims(self):
        return (self.T, self.H, self.I, self.E1, self.K1, self.block_m)

    def route(self, logits, shared_weight=1.0, stream=None):
        L.moe_route_topk_plus_shared(logits, self.T, self.E, self.K, shared_weight, self.topk_ids,
                                     self.topk_w, stream)

    def align(self, stream=None):
        L.moe_align_by_expert(self.topk_ids, self.T, self.K1, self.E1, self.block_m,
                              self.sorted_slot_ids, self.block_expert, self.expert_counts,
                              self.expert_offsets, self.num_padded, self.align_ws,
                              self.align_ws_bytes, stream)

    def ffn(self, x, W: DeviceWeights, stream=None):
        T, H, I, E1, K1, bm = self.dims()
        L.moe_fused_ffn(x, W.w13, W.s13, W.w2, W.s2, self.scale_mode, T, H, I, E1, K1, bm,
                        self.sorted_slot_ids, self.block_expert, self.num_padded, self.topk_w,
                        self.ws, self.ws_bytes, stream)

    def one_kernel_experts(self):
        """True when moe_ffn_experts runs gate/up, SwiGLU, a's quantisation and down as one kernel."""
        return L.moe_ffn_experts_one_kernel(self.H, self.I, self.block_m)

    def ffn_stage_names(self, split=False):
        return ["quant_x", "gate_up", "down"] if split or not self.one_kernel_experts() else ["quant_x", "experts"]

    def ffn_stages(self, x, W: DeviceWeights, stream=None, between=None, split=False):
        """The FFN as separate C stages (ffn_stage_names); `between(name)` is called after each
        launch. split=True always takes moe_ffn_gate_up + moe_ffn_down for the expert GEMMs."""
        T, H, I, E1, K1, bm = self.dims()
        L.moe_ffn_quant_x(x, self.scale_mode, T, H, I, E1, K1, bm, self.ws, self.ws_bytes, stream)
        if between:
            between("quant_x")
        if not split and self.one_kernel_experts():
            L.moe_ffn_experts(W.w13, W.s13, W.w2, W.s2, self.scale_mode, T, H, I, E1, K1, bm,
                              self.sorted_slot_ids, self.block_expert, self.num_padded, self.topk_w,
                              self.ws, self.ws_bytes, stream)
            if between:
                between("experts")
            return
        L.moe_ffn_gate_up(W.w13, W.s13, self.scale_mode, T, H, I, E1, K1, bm, self.sorted_slot_ids,
                          self.block_expert, self.num_padded, self.ws, self.ws_bytes, stream)
        if between:
            between("gate_up")
        L.moe_ffn_down(W.w2, W.s2, self.scale_mode, T, H, I, E1, K1, bm, self.sorted_slot_ids,
                       self.block_expert, self.num_padded, self.topk_w, self.ws, self.ws_bytes, stream)
        if between:
            between("down")

    def combine(self, stream=None):
        L.moe_combine(self.topk_w, self.T, self.K1, self.H, self.ws, self.ws_bytes, self.out, stream)

    def forward(self, x, logits, W: DeviceWeights, shared_weight=1.0, stream=None):
        self.route(logits, shared_weight, stream)
        self.align(stream)
        self.ffn(x, W, stream)
        self.combine(stream)
        return self.out

    def forward_fused(self, x, logits, W: DeviceWeights, shared_weight=1.0, stream=None):
        """The same layer through moe_layer_forward (one C call; fewer launches for small batches)."""
        T, H, I, E1, K1, bm = self.dims()
        L.moe_layer_forward(x, logits, W.w13, W.s13, W.w2, W.s2, self.scale_mode, T, H, I, self.E, self.K,
                            shared_weight, bm, self.topk_ids, self.topk_w, self.sorted_slot_ids,
                            self.block_expert, self.expert_counts, self.expert_offsets, self.num_padded,
                            self.align_ws, self.align_ws_bytes, self.ws, self.ws_bytes, self.out, stream)
        return self.out

    def forward_staged(self, x, logits, W: DeviceWeights, shared_weight=1.0, events=(), stream=None):
        """moe_layer_forward_staged: the same layer with `events` (torch.cuda.Event, already
        created) recorded between its stages; returns the stage names."""
        T, H, I, E1, K1, bm = self.dims()
        return L.moe_layer_forward_staged(x, logits, W.w13, W.s13, W.w2, W.s2, self.scale_mode, T, H, I, self.E,
                                          self.K, shared_weight, bm, self.topk_ids, self.topk_w,
                                          self.sorted_slot_ids, self.block_expert, self.expert_counts,
                                          self.expert_offsets, self.num_padded, self.align_ws, self.align_ws_bytes,
                                          self.ws, self.ws_bytes, self.out, list(events), stream)

    def forward_from_x(self, x, w_router, bias, W: DeviceWeights, shared_weight=1.0, stream=None):
        """The layer from x and the router weight (moe_layer_forward_from_x: the router gate
        in front, its partial sums folded into the routing)."""
        T, H, I, E1, K1, bm = self.dims()
        if not hasattr(self, "router_ws"):
            self.router_ws_bytes = L.moe_route_from_x_workspace_bytes(T, H, self.E)
            self.router_ws = torch.empty(max(self.router_ws_bytes, 16), dtype=torch.uint8, device=self.out.device)
        L.moe_layer_forward_from_x(x, w_router, bias, W.w13, W.s13, W.w2, W.s2, self.scale_mode, T, H, I, self.E,
                                   self.K, shared_weight, bm, self.topk_ids, self.topk_w, self.sorted_slot_ids,
                                   self.block_expert, self.expert_counts, self.expert_offsets, self.num_padded,
                                   self.router_ws, self.router_ws_bytes, self.align_ws, self.align_ws_bytes,
                                   self.ws, self.ws_bytes, self.out, stream)
        return self.out

    # views into the workspace, for inspecting the stages
    def ws_view(self, name, dtype, shape):
        off = self.offsets[name]
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        return self.ws[off:off + n].view(dtype).view(*shape)


class _Pass:
    """Routing tables, sort arrays and FFN workspace of one grouped expert pass over E1
    experts with K1 slots per token."""

    def __init__(self, T, H, I, E1, K1, block_m, scale_mode, dev):
        i32 = dict(dtype=torch.int32, device=dev)
        self.E1, self.K1 = E1, K1
        self.P_max = L.moe_sorted_capacity(T, K1, E1, block_m)
        self.topk_ids = torch.zeros((T, K1), **i32)
        self.topk_w = torch.empty((T, K1), dtype=torch.float32, device=dev)
        self.sorted_slot_ids = torch.empty(self.P_max, **i32)
        self.block_expert = torch.empty(self.P_max // block_m, **i32)
        self.expert_counts = torch.empty(E1, **i32)
        self.expert_offsets = torch.empty(E1 + 1, **i32)
        self.num_padded = torch.empty(1, **i32)
        self.align_ws_bytes = L.moe_align_workspace_bytes(T, K1, E1)
        self.align_ws = torch.empty(self.align_ws_bytes, dtype=torch.uint8, device=dev)
        self.ws_bytes = L.moe_ffn_workspace_bytes(T, H, I, E1, K1, block_m, scale_mode)
        if self.ws_bytes == 0:
            raise ValueError("unsupported FFN shape")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)

    def align(self, T, block_m, stream):
        L.moe_align_by_expert(self.topk_ids, T, self.K1, self.E1, block_m, self.sorted_slot_ids,
                              self.block_expert, self.expert_counts, self.expert_offsets, self.num_padded,
                              self.align_ws, self.align_ws_bytes, stream)

    def ffn(self, x, w13, s13, w2, s2, scale_mode, T, H, I, block_m, stream, split=False):
        if not split:
            L.moe_fused_ffn(x, w13, s13, w2, s2, scale_mode, T, H, I, self.E1, self.K1, block_m,
                            self.sorted_slot_ids, self.block_expert, self.num_padded, self.topk_w, self.ws,
                            self.ws_bytes, stream)
            return
        args = (scale_mode, T, H, I, self.E1, self.K1, block_m, self.sorted_slot_ids, self.block_expert,
                self.num_padded)
        L.moe_ffn_quant_x(x, scale_mode, T, H, I, self.E1, self.K1, block_m, self.ws, self.ws_bytes, stream)
        L.moe_ffn_gate_up(w13, s13, *args, self.ws, self.ws_bytes, stream)
        L.moe_ffn_down(w2, s2, *args, self.topk_w, self.ws, self.ws_bytes, stream)


class UnfusedMoE:
    """The same layer without the shared-experts fusion, for the fused-vs-unfused comparison:
    a top-K pass over the E routed experts (route without the shared slot, align, FFN) and a
    separate pass of the shared expert over all T tokens (FFN only: its layout does not depend
    on the routing and is built once), added by moe_combine_unfused in the fused combine's
    order. Same kernels as FusedMoE; outputs equal its outputs bit for bit."""

    def __init__(self, T, H, I, E, K, block_m, scale_mode, device="cuda"):
        self.T, self.H, self.I, self.E, self.K = T, H, I, E, K
        self.block_m, self.scale_mode = block_m, scale_mode
        dev = torch.device(device)
        self.routed = _Pass(T, H, I, E, K, block_m, scale_mode, dev)
        self.shared = _Pass(T, H, I, 1, 1, block_m, scale_mode, dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self._shared_weight = None   # the coefficient the shared pass's tables hold

    def _shared_tables(self, shared_weight, stream):
        if self._shared_weight != shared_weight:
            self.shared.topk_ids.zero_()
            self.shared.topk_w.fill_(shared_weight)
            self.shared.align(self.T, self.block_m, stream)
            self._shared_weight = shared_weight

    def forward(self, x, logits, W: DeviceWeights, shared_weight=1.0, stream=None, shared_split=False):
        """shared_split: run the shared pass through the split stages (gate_up, down), which
        spread its few row blocks over more workgroups; results then differ from the fused
        layer's by float rounding only."""
        T, H, I, E, K, bm = self.T, self.H, self.I, self.E, self.K, self.block_m
        r, s = self.routed, self.shared
        self._shared_tables(shared_weight, stream)
        L.moe_route_topk(logits, T, E, K, r.topk_ids, r.topk_w, stream)
        r.align(T, bm, stream)
        # the routed pass reads the first E experts of the stacked weights, the shared pass the last
        r.ffn(x, W.w13, W.s13, W.w2, W.s2, self.scale_mode, T, H, I, bm, stream)
        s.ffn(x, W.w13[E:], W.s13[E:], W.w2[E:], W.s2[E:], self.scale_mode, T, H, I, bm, stream,
              split=shared_split)
        L.moe_combine_unfused(T, K, H, r.ws, r.ws_bytes, s.ws, s.ws_bytes, self.out, stream)
        return self.out
