"""GPU router gate (moe_router_logits) against the oracle's float64 gate.

Bar: exact where the arithmetic is exact (integer-valued x, weights on a 2^-8 grid: every
partial sum is exact in float32, so any indexing slip shows as a wrong value); otherwise
within the float32 bound |gpu - ref| <= (3H + 1) * 2^-24 * sum_h |x_h w_h| (3H exact
products -- three bf16 parts per weight -- summed in float32, plus one ulp for the split);
and the routing taken from the GPU logits equals the oracle's, except where the oracle's
logits of the two experts concerned lie within twice the measured logit error (either
order is then correct).
"""
import numpy as np
import pytest
import torch

import oracle
from shared_routed_expert_amd import _lib as L
from tests.gpu_util import note, bf16_dev, to_dev, small_cfg
from workloads import CONFIGS, generate, f32_from_bf16_bits, bf16_bits_from_f32

pytestmark = pytest.mark.gpu


def gpu_logits(x_bits, w, bias):
    T, H = x_bits.shape
    E = w.shape[0]
    out = torch.empty((T, E), dtype=torch.float32, device="cuda")
    wsb = L.moe_router_workspace_bytes(T, H, E)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    L.moe_router_logits(bf16_dev(x_bits), to_dev(w), None if bias is None else to_dev(bias), T, H, E, out, ws,
                        wsb)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("T,H,E", [(64, 5120, 160), (77, 384, 12), (1, 128, 1), (300, 1024, 255), (4096, 512, 33)])
def test_router_exact_on_exact_arithmetic(T, H, E):
    rng = np.random.default_rng(T + H + E)
    x = rng.integers(-3, 4, size=(T, H)).astype(np.float32)            # exact in bf16
    w = (rng.integers(-256, 257, size=(E, H)) / 256.0).astype(np.float32)   # exact in bf16 (hi part only)
    b = (rng.integers(-64, 65, size=E) / 8.0).astype(np.float32)
    got = gpu_logits(bf16_bits_from_f32(x), w, b)
    ref = oracle.router_logits(x, w, b)
    assert np.array_equal(got.astype(np.float64), ref), np.argwhere(got != ref)[:5]


def _bound(x, w):
    H = x.shape[1]
    return (3 * H + 1) * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T)


@pytest.mark.parametrize("name", ["decode", "prefill", "prefill16k_zipf", "tiny"])
def test_router_logits_and_routing(name):
    cfg = CONFIGS[name]
    if name == "prefill16k_zipf":
        cfg = cfg.replace(T=2048)   # its router bias, fewer tokens
    inp = generate(cfg)
    x = f32_from_bf16_bits(inp.x_bf16)
    bias = inp.bias if np.any(inp.bias) else None
    got = gpu_logits(inp.x_bf16, inp.router_w, bias)
    ref = oracle.router_logits(x, inp.router_w, bias)
    err = np.abs(got - ref)
    bound = _bound(x, inp.router_w)
    assert np.all(err <= bound), float((err / bound).max())
    e_max = float(err.max())
    note(f"  router {name}: max |err| {e_max:.3e}, max |logit| {np.abs(ref).max():.3f}")
    ids_g, w_g = oracle.route_topk(got, cfg.K)
    ids_r, _ = oracle.route_topk(ref.astype(np.float32), cfg.K)
    bad = np.nonzero(np.any(ids_g != ids_r, axis=1))[0]
    for t in bad:   # a difference is only allowed between experts whose logits are within 2 e_max
        diff = np.nonzero(ids_g[t] != ids_r[t])[0]
        for k in diff:
            gap = abs(ref[t, ids_g[t, k]] - ref[t, ids_r[t, k]])
            assert gap <= 2 * e_max + 1e-12, (t, k, gap)
    note(f"  router {name}: {len(bad)} of {cfg.T} tokens route differently, all within the near-tie margin")


def test_router_deterministic():
    inp = generate(CONFIGS["decode"])
    a = gpu_logits(inp.x_bf16, inp.router_w, None)
    b = gpu_logits(inp.x_bf16, inp.router_w, None)
    assert np.array_equal(a, b)
