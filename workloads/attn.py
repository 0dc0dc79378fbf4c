"""Seeded synthetic inputs for the attention-side QK-Norm + RoPE step.

Inputs only (test and benchmark infrastructure): no normalisation, rotation or
table arithmetic here. Shapes are one GPU's share of GLM4-MoE attention under TP8:
the pages give the model and the fact that only half of each head's dimensions are
rotated (intelliparadigm section 2.2); the head counts (96 q, 8 kv heads -> 12 and 1
per GPU), head_dim 128, theta 1e6, eps 1e-5 and the 131072-position table come from
the model's public configuration, not from the pages.

qkv rows are drawn as the output of a projection: standard normal values times a
per-dimension spread (log-normal, sigma 0.5) so heads have uneven magnitudes; norm
weights are uniform in [0.5, 1.5]. Positions: decode tokens each come from a
different sequence (uniform over the table), prefill tokens are one or more
sequences starting at 0.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

from .synth import bf16_bits_from_f32


@dataclass(frozen=True)
class QKConfig:
    name: str
    T: int
    num_q_heads: int = 12
    num_kv_heads: int = 1
    head_dim: int = 128
    rotary_dim: int = 64
    neox: bool = True
    eps: float = 1e-5
    theta: float = 1e6
    max_pos: int = 131072
    positions: str = "decode"   # "decode": uniform over [0, max_pos); "prefill": sequences from 0
    seq_len: int = 4096         # prefill sequence length (tokens wrap into a new sequence)
    seed: int = 2000

    def replace(self, **kw) -> "QKConfig":
        return dataclasses.replace(self, **kw)

    @property
    def row(self) -> int:
        return (self.num_q_heads + 2 * self.num_kv_heads) * self.head_dim


QK_CONFIGS = {
    "decode": QKConfig("decode", T=64, positions="decode", seed=2001),
    "prefill": QKConfig("prefill", T=4096, positions="prefill", seed=2002),
    "prefill16k": QKConfig("prefill16k", T=16384, positions="prefill", seq_len=4096, seed=2003),
    "tiny": QKConfig("tiny", T=5, num_q_heads=3, num_kv_heads=1, max_pos=64, positions="decode", seed=2004),
}


@dataclass
class QKInputs:
    cfg: QKConfig
    qkv_bf16: np.ndarray    # uint16 [T, row] bfloat16 bits
    q_norm_w: np.ndarray    # float32 [head_dim]
    k_norm_w: np.ndarray    # float32 [head_dim]
    positions: np.ndarray   # int32 [T]


def generate_qk(cfg: QKConfig) -> QKInputs:
    rng = np.random.default_rng(cfg.seed)
    spread = np.exp(0.5 * rng.standard_normal(cfg.row)).astype(np.float32)
    qkv = rng.standard_normal((cfg.T, cfg.row), dtype=np.float32) * spread
    qw = rng.uniform(0.5, 1.5, cfg.head_dim).astype(np.float32)
    kw = rng.uniform(0.5, 1.5, cfg.head_dim).astype(np.float32)
    if cfg.positions == "decode":
        pos = rng.integers(0, cfg.max_pos, cfg.T)
    else:
        pos = np.arange(cfg.T) % min(cfg.seq_len, cfg.max_pos)
    return QKInputs(cfg, bf16_bits_from_f32(qkv), qw, kw, pos.astype(np.int32))
