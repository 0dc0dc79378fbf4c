"""The oracle against its pins (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import moe as om
from tests import pins
from workloads import CONFIGS, generate, random_logits, f32_from_bf16_bits


def torch_quant_a(a):
    """Row quantisation of a list of floats with torch's float8 cast (independent of the oracle codec)."""
    t = torch.tensor(a, dtype=torch.float32)
    s = t.abs().max() / torch.tensor(448.0)
    if float(s) == 0:
        s = torch.tensor(1.0)
    q = (t / s).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * s.to(torch.float64)).tolist()


@pytest.fixture(scope="module")
def tiny():
    return generate(CONFIGS["tiny"], keep_master=True)


def test_e4m3_decode():
    pins.check_e4m3_decode(oracle.e4m3_decode)


def test_e4m3_encode():
    pins.check_e4m3_encode(oracle.e4m3_encode, oracle.e4m3_decode)


def test_route_golden():
    pins.check_route_golden(oracle.route_topk_plus_shared)


@pytest.mark.parametrize("E,K,ties", [(8, 2, False), (8, 2, True), (8, 3, True), (6, 1, False), (7, 7, True)])
def test_route_bruteforce(E, K, ties):
    lg = random_logits(24, E, seed=10 + E + K, ties=ties)
    pins.check_route_bruteforce(oracle.route_topk_plus_shared, lg, K)


def test_route_bruteforce_tiny_config(tiny):
    pins.check_route_bruteforce(oracle.route_topk_plus_shared, tiny.logits, tiny.cfg.K)


@pytest.mark.parametrize("T,E,K,ties", [(300, 160, 8, False), (200, 160, 8, True), (64, 16, 4, True)])
def test_route_lexsort(T, E, K, ties):
    lg = random_logits(T, E, seed=T + E, ties=ties)
    pins.check_route_lexsort(oracle.route_topk_plus_shared, lg, K)


def test_route_k_equals_e():
    pins.check_route_k_equals_e(oracle.route_topk_plus_shared, random_logits(20, 8, seed=3))


def test_route_shared_weight_passthrough():
    ids, w = oracle.route_topk_plus_shared(random_logits(5, 8, seed=4), 2, 0.25)
    assert np.all(ids[:, 2] == 8) and np.all(w[:, 2] == 0.25)


@pytest.mark.parametrize("bm", [1, 4, 16, 64])
@pytest.mark.parametrize("T,E,K", [(16, 8, 2), (37, 16, 4), (5, 3, 3), (1, 8, 2)])
def test_align_bruteforce(T, E, K, bm):
    ids, _ = oracle.route_topk_plus_shared(random_logits(T, E, seed=T * 7 + bm, ties=True), K)
    pins.check_align_bruteforce(oracle.align_by_expert, ids, E + 1, bm)


def test_align_skewed_and_empty_experts():
    rng = np.random.default_rng(5)
    T, E, K = 50, 12, 3
    # hot expert 0 and 1 everywhere, several experts with no tokens
    lg = np.full((T, E), -5.0, np.float32)
    lg[:, 0] = 5
    lg[:, 1] = 4
    lg[:, 2 + rng.integers(0, 3, T)] = 3
    ids, _ = oracle.route_topk_plus_shared(lg, K)
    for bm in (16, 32, 128):
        pins.check_align_bruteforce(oracle.align_by_expert, ids, E + 1, bm)


def test_align_empty():
    ids = np.zeros((0, 3), np.int32)
    s, b, c, o, n = oracle.align_by_expert(ids, 9, 16)
    assert n == 0 and np.all(c == 0) and np.all(o == 0)
    assert len(s) == oracle.sorted_capacity(0, 3, 9, 16) and np.all(s == 0) and np.all(b == -1)


@pytest.mark.parametrize("group", [None, 128])
def test_quantize_act_vs_torch(group):
    rng = np.random.default_rng(11)
    v = rng.standard_normal((33, 512)).astype(np.float32) * np.exp(rng.uniform(-8, 8, (33, 1))).astype(np.float32)
    v[3] = 0.0           # all-zero row -> scale 1
    v[4, :200] = 0.0
    pins.check_quantize_act(oracle.quantize_act, v, group)


def test_quantize_x_tiny_config(tiny):
    pins.check_quantize_act(oracle.quantize_act, f32_from_bf16_bits(tiny.x_bf16), None)


@pytest.mark.parametrize("n,H,I", [(3, 128, 32), (2, 64, 16)])
def test_expert_ffn_triple_loop(n, H, I):
    pins.check_expert_ffn(oracle.expert_ffn, np.random.default_rng(n + H), n=n, H=H, I=I,
                          quant_a=torch_quant_a)


def test_expert_ffn_closed_form():
    pins.check_ffn_closed_form(oracle.expert_ffn, oracle.e4m3_decode, oracle.e4m3_encode)


def test_dequant_weight_block_vs_channel():
    """A block-scale tensor whose 128x128 blocks share a row scale equals the per-channel form."""
    rng = np.random.default_rng(2)
    q = rng.integers(0, 256, (256, 384)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    s_row = rng.uniform(0.5, 2, 256).astype(np.float32)
    s_row = np.repeat(s_row[::128], 128)
    s_blk = np.repeat(s_row[::128][:, None], 3, axis=1)
    a = oracle.dequant_weight(q, s_row)
    b = oracle.dequant_weight(q, s_blk)
    assert np.array_equal(a, b)
    assert np.array_equal(a, oracle.e4m3_decode(q) * s_row[:, None].astype(np.float64))


def test_fused_equals_unfused_tiny(tiny):
    d = pins.check_fused_equals_unfused(oracle.moe_fused, oracle.moe_unfused, tiny)
    assert d == 0.0  # same per-expert row sets and slot order: bit-exact


def test_fused_equals_unfused_block_mode():
    cfg = CONFIGS["tiny"].replace(H=256, I=128, scale_mode="block128", T=12, E=6, K=2, seed=77)
    pins.check_fused_equals_unfused(oracle.moe_fused, oracle.moe_unfused, generate(cfg))


def test_zero_routed_weights_dense_shared(tiny):
    pins.check_zero_routed_is_dense_shared(oracle.moe_fused, oracle.combine_slots,
                                           oracle.dense_shared_ffn, tiny)


def test_dense_shared_vs_torch_matmul(tiny):
    """The dense shared FFN against a torch SwiGLU (library matmul and silu) with the same
    quantisation points computed through torch's float8 cast."""
    x = torch.from_numpy(f32_from_bf16_bits(tiny.x_bf16))
    E = tiny.cfg.E
    dec = lambda q: torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64)
    w13 = dec(tiny.w13_q[E]) * torch.from_numpy(tiny.s13[E]).double()[:, None]
    w2 = dec(tiny.w2_q[E]) * torch.from_numpy(tiny.s2[E]).double()[:, None]

    def fq(v):
        s = v.abs().amax(dim=1, keepdim=True) / torch.tensor(448.0)
        s = torch.where(s > 0, s, torch.ones_like(s))
        return (v / s).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64) * s.double()

    xd = fq(x.float())
    I = tiny.cfg.I
    g, u = xd @ w13[:I].T, xd @ w13[I:].T
    a = torch.nn.functional.silu(g) * u
    want = fq(a.float()) @ w2.T
    got = oracle.dense_shared_ffn(f32_from_bf16_bits(tiny.x_bf16), tiny.w13_q, tiny.s13, tiny.w2_q, tiny.s2)
    assert np.allclose(got, want.numpy(), rtol=0, atol=1e-12 * float(want.abs().max()))


def _all_experts(inp):
    def f(x):
        group = None if inp.s13.ndim == 2 else 128
        xq, sx = om.quantize_act(x, group)
        xd = om.dequant_act(xq, sx, group)
        return np.stack([om.expert_ffn(xd, *om._expert_weights(inp.w13_q, inp.s13, inp.w2_q, inp.s2, e), group)
                         for e in range(inp.cfg.E1)])
    return f


def test_k_equals_e_mixture(tiny):
    pins.check_k_equals_e_mixture(oracle.moe_fused, _all_experts(tiny), tiny)


def test_permutation_equivariance(tiny):
    pins.check_permutation_equivariance(oracle.moe_fused, tiny, np.random.default_rng(1).permutation(tiny.cfg.T))


def test_fp32_masters_close_to_fp8(tiny):
    """Information, loosely bounded: the fp8 layer tracks the fp32-weight, fp32-activation layer."""
    x = f32_from_bf16_bits(tiny.x_bf16).astype(np.float64)
    ids, w = oracle.route_topk_plus_shared(tiny.logits, tiny.cfg.K)
    ref = np.zeros_like(x)
    I = tiny.cfg.I
    for t in range(tiny.cfg.T):
        for k in range(tiny.cfg.K1):
            e = ids[t, k]
            g = tiny.w13_master[e][:I].astype(np.float64) @ x[t]
            u = tiny.w13_master[e][I:].astype(np.float64) @ x[t]
            ref[t] += w[t, k] * (tiny.w2_master[e].astype(np.float64) @ (g / (1 + np.exp(-g)) * u))
    got = oracle.moe_fused(f32_from_bf16_bits(tiny.x_bf16), tiny.logits, tiny.cfg.K, tiny.w13_q,
                           tiny.s13, tiny.w2_q, tiny.s2)
    rel = np.max(np.abs(got - ref), axis=1) / np.max(np.abs(ref), axis=1)
    assert rel.max() < 0.15


# ---------------------------------------------------------------------------- router gate
def test_router_logits_bruteforce():
    pins.check_router_bruteforce(oracle.router_logits)


def test_router_logits_one_hot_rows():
    pins.check_router_one_hot(oracle.router_logits)


@pytest.mark.parametrize("name", ["tiny", "prefill16k_zipf"])
def test_router_logits_reproduce_the_workload_logits(name):
    """Consistency of the input recipe, not a pin: the workloads' logits are the oracle's router
    gate of their x and router weight, rounded to fp32 (router_logits itself is pinned by the
    brute-force and one-hot tests above)."""
    cfg = CONFIGS[name]
    if name != "tiny":
        cfg = cfg.replace(T=64)
    inp = generate(cfg)
    lg = oracle.router_logits(f32_from_bf16_bits(inp.x_bf16), inp.router_w, inp.bias)
    assert np.array_equal(lg.astype(np.float32), inp.logits)


# ---------------------------------------------------------------------------- QK-Norm + half RoPE
def test_head_rms_norm_closed_forms():
    pins.check_head_rms_norm(oracle.head_rms_norm)


def test_rope_angles_hand_values():
    pins.check_rope_angles(oracle.rope_angles)


def test_rope_half_properties():
    pins.check_rope_half(oracle.rope_half, oracle.rope_angles)


def test_qk_norm_rope_layout():
    pins.check_qk_layout(oracle.qk_norm_rope, oracle.head_rms_norm)


def test_rope_interleaved_is_a_permuted_rope_half():
    pins.check_rope_interleaved(oracle.rope_interleaved, oracle.rope_half, oracle.rope_angles)
