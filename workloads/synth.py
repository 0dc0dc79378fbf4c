"""Seeded synthetic inputs for the fused shared + routed MoE layer.

Test and benchmark infrastructure. Both the CPU oracle's tests and the GPU
path's tests/benchmark draw their inputs from here, so this module holds none
of the layer's own arithmetic (no routing, no sorting, no FFN, no activation
quantisation). What it does:

* draws the random tensors in a fixed order from ``numpy.random.default_rng``;
* rounds the activations to bfloat16 with torch's CPU cast;
* synthesises an FP8 "checkpoint": each weight matrix is quantised once, with
  torch's own ``float8_e4m3fn`` cast, using an absmax scale per output channel
  (or per 128x128 block) -- the pages serve the model as FP8 (E4M3) weights
  (Optimizing GLM4-MoE for production, Novita AI: "Benchmark configuration";
  intelliparadigm, GLM4-MoE production optimisation, section 3.1);
* computes the router logits that the routing step consumes, once, on the
  host in float64 and rounds them to float32, so both sides see the same bytes.

Shapes follow the pages: 160 routed experts plus one shared expert, top-8
routed per token, and a per-GPU expert intermediate size of 192 under TP8/FP8
(Optimizing GLM4-MoE for production, section 1 "Shared Experts Fusion").
The shared expert's weights are stored as expert id E (the last one).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0  # largest finite OCP E4M3FN magnitude
BLOCK = 128      # block edge of the 128x128 weight-scale / 128-wide activation groups


@dataclass(frozen=True)
class MoEConfig:
    """One synthetic layer shape. E routed experts, one shared (id E); K routed slots per token."""
    name: str
    T: int
    H: int
    E: int
    K: int
    I: int
    scale_mode: str = "channel"   # "channel" (per output channel) or "block128"
    zipf_s: Optional[float] = None  # per-expert Zipf bias on the router logits
    seed: int = 1000
    router_std: float = 0.02

    @property
    def E1(self) -> int:
        return self.E + 1

    @property
    def K1(self) -> int:
        return self.K + 1

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny self-check layer, then the TP8 shard (H=5120,
# I=192) at decode (64 tokens), prefill (4096 tokens, the pages' input length),
# a 16384-token chunked-prefill batch with Zipf-skewed routing, and the
# unsharded expert width (I=1536) with 128x128 block scales.
CONFIGS = {
    "tiny": MoEConfig("tiny", T=16, H=128, E=8, K=2, I=32, seed=1000),
    "decode": MoEConfig("decode", T=64, H=5120, E=160, K=8, I=192, seed=1001),
    "prefill": MoEConfig("prefill", T=4096, H=5120, E=160, K=8, I=192, seed=1002),
    "prefill16k_zipf": MoEConfig("prefill16k_zipf", T=16384, H=5120, E=160, K=8, I=192,
                                 zipf_s=1.1, seed=1003),
    "unsharded_block": MoEConfig("unsharded_block", T=4096, H=5120, E=160, K=8, I=1536,
                                 scale_mode="block128", seed=1004),
}


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x_bf16: np.ndarray      # uint16 [T,H], bfloat16 bit patterns
    logits: np.ndarray      # float32 [T,E]
    w13_q: np.ndarray       # uint8 [E1, 2I, H]; rows 0..I-1 gate, I..2I-1 up
    s13: np.ndarray         # float32 [E1, 2I] or [E1, 2I/128, H/128]
    w2_q: np.ndarray        # uint8 [E1, H, I]
    s2: np.ndarray          # float32 [E1, H] or [E1, H/128, I/128]
    router_w: np.ndarray    # float32 [E,H]
    bias: np.ndarray        # float32 [E] (zeros unless Zipf)
    w13_master: Optional[np.ndarray] = None  # float32 originals (only when asked)
    w2_master: Optional[np.ndarray] = None


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (torch's round-to-nearest-even cast); return the bits as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def _quantize_checkpoint(w: np.ndarray, mode: str):
    """FP8 checkpoint synthesis with torch's float8_e4m3fn cast (round to nearest even).

    mode "channel": one absmax scale per row (output channel); "block128": one
    per 128x128 block. scale = amax / 448, or 1 where amax == 0.
    """
    t = torch.from_numpy(w)
    n, k = t.shape
    if mode == "channel":
        amax = t.abs().amax(dim=1)
        s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        scaled = t / s[:, None]
    elif mode == "block128":
        tb = t.reshape(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
        amax = tb.abs().amax(dim=(1, 3))
        s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        scaled = (tb / s[:, None, :, None]).reshape(n, k)
    else:
        raise ValueError(mode)
    q = scaled.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), s.to(torch.float32).numpy().copy()


def zipf_bias(E: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Per-expert additive router bias: expert e gets a random rank r_e in 1..E and
    bias ln(r_e^-s / sum_r r^-s), so hot experts take a Zipf(s) share of tokens."""
    perm = rng.permutation(E)
    ranks = perm.astype(np.float64) + 1.0
    norm = np.sum(np.arange(1, E + 1, dtype=np.float64) ** (-s))
    return np.log(ranks ** (-s) / norm).astype(np.float32)


def generate(cfg: MoEConfig, weight_set: int = 0, keep_master: bool = False,
             with_weights: bool = True) -> MoEInputs:
    """Build one seeded input set. The draw order is fixed:
    x, router weight, (Zipf permutation), then per expert 0..E-1 and the shared
    expert E: W_gate, W_up (N(0,1)/sqrt(H), [I,H]), W_down (N(0,1)/sqrt(I), [H,I]).
    weight_set j uses seed + 100*j (bench cycles several independent weight sets).
    """
    T, H, E, I = cfg.T, cfg.H, cfg.E, cfg.I
    E1 = cfg.E1
    rng = np.random.default_rng(cfg.seed + 100 * weight_set)
    x = rng.standard_normal((T, H), dtype=np.float32)
    x_bf16 = bf16_bits_from_f32(x)
    del x
    router_w = (cfg.router_std * rng.standard_normal((E, H), dtype=np.float32)).astype(np.float32)
    bias = zipf_bias(E, cfg.zipf_s, rng) if cfg.zipf_s else np.zeros(E, np.float32)
    xf = f32_from_bf16_bits(x_bf16).astype(np.float64)
    logits = (xf @ router_w.astype(np.float64).T + bias.astype(np.float64)).astype(np.float32)
    del xf

    if cfg.scale_mode == "channel":
        s13_shape, s2_shape = (E1, 2 * I), (E1, H)
    else:
        assert H % BLOCK == 0 and I % BLOCK == 0
        s13_shape, s2_shape = (E1, 2 * I // BLOCK, H // BLOCK), (E1, H // BLOCK, I // BLOCK)
    if not with_weights:
        z = np.zeros((0,), np.uint8)
        return MoEInputs(cfg, x_bf16, logits, z, np.zeros((0,), np.float32), z,
                         np.zeros((0,), np.float32), router_w, bias)
    w13_q = np.empty((E1, 2 * I, H), np.uint8)
    w2_q = np.empty((E1, H, I), np.uint8)
    s13 = np.empty(s13_shape, np.float32)
    s2 = np.empty(s2_shape, np.float32)
    w13_m = np.empty((E1, 2 * I, H), np.float32) if keep_master else None
    w2_m = np.empty((E1, H, I), np.float32) if keep_master else None
    inv_sh, inv_si = np.float32(1.0 / math.sqrt(H)), np.float32(1.0 / math.sqrt(I))
    for e in range(E1):
        w13 = rng.standard_normal((2 * I, H), dtype=np.float32)  # gate rows then up rows
        w13 *= inv_sh
        wd = rng.standard_normal((H, I), dtype=np.float32)
        wd *= inv_si
        w13_q[e], s13[e] = _quantize_checkpoint(w13, cfg.scale_mode)
        w2_q[e], s2[e] = _quantize_checkpoint(wd, cfg.scale_mode)
        if keep_master:
            w13_m[e], w2_m[e] = w13, wd
    return MoEInputs(cfg, x_bf16, logits, w13_q, s13, w2_q, s2, router_w, bias, w13_m, w2_m)


def random_logits(T: int, E: int, seed: int, ties: bool = False) -> np.ndarray:
    """Plain N(0,1) float32 logits; with ties=True values are drawn from a coarse grid
    so equal logits are common (exercises the lower-id tie rule)."""
    rng = np.random.default_rng(seed)
    if ties:
        return rng.integers(-3, 4, size=(T, E)).astype(np.float32) * np.float32(0.5)
    return rng.standard_normal((T, E), dtype=np.float32)
