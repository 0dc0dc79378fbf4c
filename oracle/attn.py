"""Plain float64 CPU oracle of the attention-side QK-Norm + RoPE step (test
infrastructure, like the rest of this package).

The pages describe fusing the per-head normalisation of q and k with the rotary
position embedding into one kernel, both being computations on one attention head
at a time, and note that in GLM4-MoE the rotation covers only half of each head's
dimensions (intelliparadigm, section 2.2; Optimizing GLM4-MoE for production,
section 2). Readings of what they leave open:

* Norm: RMS normalisation over the head dimension with a learned weight per
  dimension (separate weights for q and k), y = x / sqrt(mean(x^2) + eps) * w --
  the head norm of the Qwen-MoE models the pages name as the source.
* Rotation: the first ``rotary_dim`` dimensions of each head are rotated, the rest
  pass through; angle(pos, i) = pos * theta^(-2i / rotary_dim) for frequency i <
  rotary_dim/2. The pages do not say how dimensions pair up, so both usual
  arrangements are here: rotate-half (dimension i with i + rotary_dim/2, the default)
  and interleaved (2i with 2i + 1).
"""
from __future__ import annotations

import numpy as np


def rope_angles(positions: np.ndarray, rotary_dim: int, theta: float) -> np.ndarray:
    """angle[t, i] = positions[t] * theta^(-2 i / rotary_dim), i < rotary_dim / 2 (float64)."""
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / rotary_dim)
    return np.asarray(positions, np.float64)[:, None] * inv[None, :]


def head_rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x [..., D] -> x / sqrt(mean(x^2) + eps) * w over the last axis (float64)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, np.float64)


def rope_half(x: np.ndarray, angle: np.ndarray, rotary_dim: int) -> np.ndarray:
    """Rotate the first rotary_dim dims of x [T, heads, D] in the rotate-half pairing by
    angle [T, rotary_dim/2]; the other dims pass through (float64)."""
    x = np.asarray(x, np.float64)
    h = rotary_dim // 2
    c = np.cos(angle)[:, None, :]
    s = np.sin(angle)[:, None, :]
    out = x.copy()
    x1, x2 = x[..., :h], x[..., h:rotary_dim]
    out[..., :h] = x1 * c - x2 * s
    out[..., h:rotary_dim] = x2 * c + x1 * s
    return out


def rope_interleaved(x: np.ndarray, angle: np.ndarray, rotary_dim: int) -> np.ndarray:
    """Rotate the pairs (2i, 2i+1), i < rotary_dim/2, of x [T, heads, D] by angle [T, rotary_dim/2];
    the other dims pass through (float64)."""
    x = np.asarray(x, np.float64)
    c = np.cos(angle)[:, None, :]
    s = np.sin(angle)[:, None, :]
    out = x.copy()
    a, b = x[..., 0:rotary_dim:2], x[..., 1:rotary_dim:2]
    out[..., 0:rotary_dim:2] = a * c - b * s
    out[..., 1:rotary_dim:2] = b * c + a * s
    return out


def qk_norm_rope(qkv: np.ndarray, num_q_heads: int, num_kv_heads: int, head_dim: int, rotary_dim: int,
                 q_norm_w: np.ndarray, k_norm_w: np.ndarray, eps: float, positions: np.ndarray,
                 theta: float, neox: bool = True) -> np.ndarray:
    """qkv [T, (Hq + 2 Hkv) * D] (q heads, k heads, v heads) -> the same layout with the q
    and k heads normalised and rotated (rotate-half if neox, else interleaved); v
    unchanged. float64."""
    qkv = np.asarray(qkv, np.float64)
    T = qkv.shape[0]
    D = head_dim
    heads = qkv.reshape(T, num_q_heads + 2 * num_kv_heads, D).copy()
    ang = rope_angles(positions, rotary_dim, theta)
    rope = rope_half if neox else rope_interleaved
    q = heads[:, :num_q_heads]
    k = heads[:, num_q_heads:num_q_heads + num_kv_heads]
    heads[:, :num_q_heads] = rope(head_rms_norm(q, q_norm_w, eps), ang, rotary_dim)
    heads[:, num_q_heads:num_q_heads + num_kv_heads] = rope(head_rms_norm(k, k_norm_w, eps), ang, rotary_dim)
    return heads.reshape(T, -1)
