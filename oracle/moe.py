"""Plain float64 CPU oracle of the shared + routed MoE layer (test infrastructure).

Notation: T tokens, hidden H, E routed experts plus one shared expert with id E
(E1 = E + 1 ids), K routed slots per token plus the shared slot K (K1 = K + 1
slots), expert intermediate size I. Weights come as an FP8 checkpoint:
w13_q [E1, 2I, H] (rows 0..I-1 gate, I..2I-1 up), w2_q [E1, H, I], with fp32
scales per output channel (s13 [E1, 2I], s2 [E1, H]) or per 128x128 block
(s13 [E1, 2I/128, H/128], s2 [E1, H/128, I/128]).

Readings of what the pages leave open (each is also listed with its reason in
the design notes):

* Router scoring: softmax over the E routed logits; the K best are kept and
  their probabilities renormalised to sum to 1. The pages only say each token
  selects its top-8 of 160 routed experts (Optimizing GLM4-MoE for production,
  section 1).
* Order and ties: routed slots are ordered by logit, highest first; equal
  logits go to the lower expert id.
* Shared slot: id E in slot K (the 9th of 9), coefficient ``shared_weight``
  = 1.0, because the unfused form adds the shared output unweighted
  (intelliparadigm, section 2.1: shared_output + routed_output).
* Expert FFN: SwiGLU, down(silu(gate(v)) * up(v)), silu(z) = z / (1 + e^-z).
* FP8 activations: both expert GEMMs take FP8 inputs. x is fake-quantised per
  token (per token and 128-wide group in block mode), the SwiGLU product ``a``
  per (token, slot) row over I (per 128-wide group in block mode):
  s = amax / 448 (1 if amax == 0), q = e4m3(v / s), v' = s * decode(q). The
  quantisation decision is taken in float32 (scale, division, rounding), the
  precision of the GPU kernels; everything else here is float64.
"""
from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode, e4m3_encode, E4M3_MAX

GROUP = 128


# ----------------------------------------------------------------------------- router gate
def router_logits(x_f32: np.ndarray, router_w: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """The router gate upstream of the routing: logits[t, e] = sum_h x[t, h] * W_r[e, h]
    (+ bias[e]) for the E routed experts, in float64. Each token scores the 160 routed
    experts and keeps its top-8 (Optimizing GLM4-MoE for production, section 1); the
    gate itself is the plain linear router over the hidden state.

    x_f32 [T, H], router_w [E, H], bias [E] or None. Returns float64 [T, E].
    """
    lg = np.asarray(x_f32, np.float64) @ np.asarray(router_w, np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, np.float64)[None, :]
    return lg


# ----------------------------------------------------------------------------- routing
def route_topk(logits: np.ndarray, K: int):
    """Top-K routed experts per token, ordered by (logit desc, id asc), with weights
    p_k / sum_{j in top-K} p_j where p = softmax over all E logits (float64).

    Returns ids int32 [T,K], weights float64 [T,K].
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    eid = np.arange(E)
    for t in range(T):
        row = lg[t].astype(np.float64)
        order = np.lexsort((eid, -row))      # primary: -logit ascending; secondary: id ascending
        top = order[:K]
        p = np.exp(row - row.max())
        p = p / p.sum()                      # full softmax over the E routed experts
        ids[t] = top
        w[t] = p[top] / p[top].sum() if K > 0 else p[top]
    return ids, w


def route_topk_plus_shared(logits: np.ndarray, K: int, shared_weight: float = 1.0):
    """The fused routing table [T, K+1]: the K routed slots, then the shared expert
    (id E) forced into the last slot with coefficient ``shared_weight``
    (intelliparadigm, section 2.1: shared expert becomes routed expert 161, every
    token takes top-9; Optimizing GLM4-MoE for production, section 1: the shared
    expert always holds the 9th position)."""
    T, E = np.asarray(logits).shape
    ids, w = route_topk(logits, K)
    ids9 = np.concatenate([ids, np.full((T, 1), E, np.int32)], axis=1)
    w9 = np.concatenate([w, np.full((T, 1), float(np.float32(shared_weight)))], axis=1)
    return ids9, w9


# ----------------------------------------------------------------------------- align
def sorted_capacity(T: int, K1: int, E1: int, block_m: int) -> int:
    """Upper bound on the padded row count: every expert pads by at most block_m - 1."""
    n = T * K1 + E1 * (block_m - 1)
    return (n + block_m - 1) // block_m * block_m


def align_by_expert(ids: np.ndarray, E1: int, block_m: int):
    """Group the flat (token, slot) entries s = t*K1 + k by expert id.

    Experts in ascending id; inside an expert, ascending s; each expert's
    segment padded with the sentinel T*K1 to a multiple of block_m (an expert
    with no entries takes no rows); the array is filled with the sentinel up to
    ``sorted_capacity``. block_expert[b] is the expert owning rows
    b*block_m..(b+1)*block_m-1, or -1 past the used rows.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, K1 = ids.shape
    flat = ids.reshape(-1)
    sentinel = T * K1
    cap = sorted_capacity(T, K1, E1, block_m)
    counts = np.zeros(E1, np.int32)
    offsets = np.zeros(E1 + 1, np.int32)
    rows = []
    for e in range(E1):
        members = [s for s in range(flat.size) if flat[s] == e] if flat.size <= 4096 else \
            list(np.nonzero(flat == e)[0])
        counts[e] = len(members)
        padded = -(-len(members) // block_m) * block_m
        rows.extend(int(s) for s in members)
        rows.extend([sentinel] * (padded - len(members)))
        offsets[e + 1] = offsets[e] + padded
    num_padded = int(offsets[E1])
    sorted_ids = np.full(cap, sentinel, np.int32)
    sorted_ids[:num_padded] = np.array(rows, dtype=np.int32)
    block_expert = np.full(cap // block_m, -1, np.int32)
    for e in range(E1):
        block_expert[offsets[e] // block_m: offsets[e + 1] // block_m] = e
    return sorted_ids, block_expert, counts, offsets, num_padded


# ----------------------------------------------------------------------------- quantisation
def quantize_act(v: np.ndarray, group: int | None):
    """Absmax FP8 quantisation of activation rows, decision taken in float32.

    group=None: one scale per row; group=128: one scale per 128 consecutive
    columns. Returns (codes uint8, scales float32 [rows] or [rows, cols/128]).
    """
    v32 = np.asarray(v, dtype=np.float32)
    n, c = v32.shape
    g = c if group is None else group
    blocks = v32.reshape(n, c // g, g)
    amax = np.abs(blocks).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    scaled = (blocks / s[:, :, None]).astype(np.float32)   # float32 division, as on the GPU
    q = e4m3_encode(scaled).reshape(n, c)
    return q, (s[:, 0] if group is None else s)


def dequant_act(q: np.ndarray, s: np.ndarray, group: int | None) -> np.ndarray:
    n, c = q.shape
    d = e4m3_decode(q)
    if group is None:
        return d * s.astype(np.float64)[:, None]
    return (d.reshape(n, c // group, group) * s.astype(np.float64)[:, :, None]).reshape(n, c)


def dequant_weight(wq: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W = scale * decode(code), float64. s is per row [N] or per 128x128 block [N/128, K/128]."""
    d = e4m3_decode(wq)
    s = np.asarray(s, dtype=np.float64)
    if s.ndim == 1:
        return d * s[:, None]
    n, k = d.shape
    return (d.reshape(n // GROUP, GROUP, k // GROUP, GROUP) * s[:, None, :, None]).reshape(n, k)


def _act_group(s13: np.ndarray):
    return None if s13.ndim == 2 else GROUP


# ----------------------------------------------------------------------------- expert FFN
def expert_ffn(xd: np.ndarray, w13: np.ndarray, w2: np.ndarray, group: int | None) -> np.ndarray:
    """SwiGLU expert on dequantised rows xd [n,H] with dequantised w13 [2I,H], w2 [H,I]:
    g = xd W_gate^T, u = xd W_up^T, a = silu(g) * u, a fake-quantised to FP8,
    y = a' W2^T. float64 apart from the float32 quantisation decision."""
    I = w13.shape[0] // 2
    g = xd @ w13[:I].T
    u = xd @ w13[I:].T
    a = g / (1.0 + np.exp(-g)) * u
    aq, sa = quantize_act(a.astype(np.float32), group)
    return dequant_act(aq, sa, group) @ w2.T


def _expert_weights(inp_w13, inp_s13, inp_w2, inp_s2, e):
    return dequant_weight(inp_w13[e], inp_s13[e]), dequant_weight(inp_w2[e], inp_s2[e])


def _quantized_x(x_f32: np.ndarray, group: int | None) -> np.ndarray:
    xq, sx = quantize_act(x_f32, group)
    return dequant_act(xq, sx, group)


def slot_outputs(x_f32, ids, w13_q, s13, w2_q, s2, tokens=None):
    """Per-(token, slot) expert outputs y [n, K1, H] (float64) for the tokens listed
    (all by default): y[t,k] = FFN_{ids[t,k]}(q(x_t)). Each expert runs once over
    all of its (token, slot) rows, in ascending flat slot order."""
    group = _act_group(s13)
    ids = np.asarray(ids)
    tok = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    sub = ids[tok]
    xd = _quantized_x(np.asarray(x_f32, np.float32)[tok], group)
    n, K1 = sub.shape
    H = xd.shape[1]
    y = np.zeros((n, K1, H), np.float64)
    flat = sub.reshape(-1)
    for e in np.unique(flat):
        members = np.nonzero(flat == e)[0]
        w13, w2 = _expert_weights(w13_q, s13, w2_q, s2, int(e))
        ye = expert_ffn(xd[members // K1], w13, w2, group)
        y[members // K1, members % K1] = ye
    return y


def combine_slots(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum_k w[t,k] * y[t,k,:] accumulated in slot order 0..K1-1 (the pages' weighted aggregation)."""
    out = np.zeros((y.shape[0], y.shape[2]), np.float64)
    for k in range(y.shape[1]):
        out += np.asarray(w, np.float64)[:, k, None] * y[:, k]
    return out


def dense_shared_ffn(x_f32, w13_q, s13, w2_q, s2, tokens=None) -> np.ndarray:
    """The shared expert (id E, the last) applied to every token as one dense FFN."""
    group = _act_group(s13)
    xs = np.asarray(x_f32, np.float32)
    if tokens is not None:
        xs = xs[np.asarray(tokens)]
    E = w13_q.shape[0] - 1
    w13, w2 = _expert_weights(w13_q, s13, w2_q, s2, E)
    return expert_ffn(_quantized_x(xs, group), w13, w2, group)


def moe_unfused(x_f32, logits, K, w13_q, s13, w2_q, s2, tokens=None) -> np.ndarray:
    """The pages' original form: shared_out + sum over the top-K routed experts of
    w_k * expert_k(x), with the shared expert run as its own dense pass
    (intelliparadigm, section 2.1, "traditional implementation")."""
    ids, w = route_topk(logits, K)
    tok = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    shared = dense_shared_ffn(x_f32, w13_q, s13, w2_q, s2, tokens=tok)
    y = slot_outputs(x_f32, ids, w13_q, s13, w2_q, s2, tokens=tok) if K > 0 else \
        np.zeros((len(tok), 0, shared.shape[1]))
    routed = combine_slots(y, w[tok])
    return shared + routed


def moe_fused(x_f32, logits, K, w13_q, s13, w2_q, s2, shared_weight=1.0, tokens=None,
              return_slots=False):
    """The fused form: top-K routed + the shared expert as id E in slot K, all K+1
    slots run as one grouped expert pass, then one weighted sum in slot order
    (intelliparadigm, section 2.1, steps 1-3; Optimizing GLM4-MoE for production,
    section 1)."""
    ids, w = route_topk_plus_shared(logits, K, shared_weight)
    tok = np.arange(ids.shape[0]) if tokens is None else np.asarray(tokens)
    y = slot_outputs(x_f32, ids, w13_q, s13, w2_q, s2, tokens=tok)
    out = combine_slots(y, w[tok])
    return (out, y, ids, w) if return_slots else out
