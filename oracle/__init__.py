"""CPU oracle for the fused shared + routed MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU library never calls it, and it
shares no code, table or helper with the GPU path; the two meet only in the
seeded input generator (``workloads``), which holds none of the layer's
arithmetic.

What it computes (the pages' definition, written out plainly in float64):

* The unfused layer: the shared expert's output for every token, plus the
  routed experts' outputs weighted by the router and summed over each
  token's top-8 (intelliparadigm, "GLM4-MoE production optimisation",
  section 2.1 Shared Experts Fusion, the "traditional" pseudo-code;
  Optimizing GLM4-MoE for production, Novita AI, section 1).
* The fused layer: the shared expert becomes expert number E (the 161st of
  161), each token takes top-9 = its top-8 routed experts plus the shared one
  forced into the 9th position, and one weighted sum over the 9 slots gives the
  output (same sections; SGLang Optimizes GLM4-MoE Production Deployment,
  winzheng review, section 1).
* The pieces both need: the OCP FP8 E4M3FN codec, the softmax top-k router,
  the align/sort/pad of (token, slot) entries by expert, the per-token (or
  per-128-group) activation fake-quantisation and the SwiGLU expert FFN on
  dequantised weights.

Readings where the pages are silent (router scoring, tie rule, FFN form,
activation quantisation, sort order) are listed in ``moe.py``'s docstrings.

Pins: every function is checked in ``tests/test_oracle_*.py`` against
something other than itself -- brute force on tiny inputs, library routines
(numpy sort, scipy softmax, torch's float8 cast), closed forms and the pages'
own fused == unfused check. No function here is "parity unpinned".
"""
from .fp8 import e4m3_decode, e4m3_encode, E4M3_MAX
from .moe import (router_logits, route_topk, route_topk_plus_shared, align_by_expert, sorted_capacity,
                  quantize_act, dequant_weight, expert_ffn, moe_unfused, moe_fused,
                  slot_outputs, combine_slots, dense_shared_ffn)

from .attn import qk_norm_rope, head_rms_norm, rope_half, rope_interleaved, rope_angles

__all__ = ["qk_norm_rope", "head_rms_norm", "rope_half", "rope_interleaved", "rope_angles", "e4m3_decode", "e4m3_encode", "E4M3_MAX", "router_logits", "route_topk", "route_topk_plus_shared",
           "align_by_expert", "sorted_capacity", "quantize_act", "dequant_weight",
           "expert_ffn", "moe_unfused", "moe_fused", "slot_outputs", "combine_slots",
           "dense_shared_ffn"]
