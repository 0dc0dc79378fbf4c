"""Plant a plausible mistake in the oracle (on the CPU) and check that a pin catches it."""
import numpy as np
import pytest

from oracle import fp8 as of
from oracle import moe as om
from tests import pins
from tests.test_oracle_pins import torch_quant_a
from workloads import CONFIGS, generate, random_logits


@pytest.fixture(scope="module")
def tiny():
    return generate(CONFIGS["tiny"])


def _route_ties_high(logits, K):
    lg = np.asarray(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K))
    for t in range(T):
        order = np.lexsort((-np.arange(E), -lg[t].astype(np.float64)))[:K]
        p = np.exp(lg[t] - lg[t].max())
        ids[t], w[t] = order, p[order] / p[order].sum()
    return ids, w


def _mut_route_no_renorm(orig):
    def f(logits, K):
        ids, w = orig(logits, K)
        p = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return f


def _mut_shared_first(orig):
    def f(logits, K, shared_weight=1.0):
        ids, w = orig(logits, K, shared_weight)
        return np.roll(ids, 1, axis=1), np.roll(w, 1, axis=1)
    return f


def _mut_shared_weight(orig, value):
    def f(logits, K, shared_weight=1.0):
        return orig(logits, K, value)
    return f


def _mut_align_unstable(orig):
    def f(ids, E1, bm):
        s, b, c, o, n = orig(ids, E1, bm)
        s = s.copy()
        for e in range(E1):
            seg = s[o[e]:o[e] + c[e]]
            s[o[e]:o[e] + c[e]] = seg[::-1]
        return s, b, c, o, n
    return f


def _mut_align_nopad(orig):
    def f(ids, E1, bm):
        return orig(ids, E1, 1)
    return f


def _mut_encode_half_away(v):
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), 448.0)
    mags = of._MAGS
    hi = np.minimum(np.searchsorted(mags, a), 126)
    lo = np.maximum(hi - 1, 0)
    code = np.where(mags[hi] - a <= a - mags[lo], hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def _mut_decode_bias8(codes):
    return of.e4m3_decode(codes) / 2.0


def _mut_ffn(kind):
    def f(xd, w13, w2, group):
        I = w13.shape[0] // 2
        g, u = xd @ w13[:I].T, xd @ w13[I:].T
        if kind == "silu_sign":
            a = g / (1.0 + np.exp(g)) * u
        elif kind == "gate_up_swapped":
            a = u / (1.0 + np.exp(-u)) * g
        elif kind == "no_act_quant":
            return (g / (1.0 + np.exp(-g)) * u) @ w2.T
        aq, sa = om.quantize_act(a.astype(np.float32), group)
        return om.dequant_act(aq, sa, group) @ w2.T
    return f


def _mut_quant_scale(v, group):
    v32 = np.asarray(v, np.float32)
    n, c = v32.shape
    amax = np.abs(v32).max(axis=1)
    s = np.where(amax > 0, amax / np.float32(240.0), 1).astype(np.float32)
    return of.e4m3_encode(v32 / s[:, None]), s


def _mut_combine_drop_last(y, w):
    out = np.zeros((y.shape[0], y.shape[2]))
    for k in range(y.shape[1] - 1):
        out += w[:, k, None] * y[:, k]
    return out


def _fails(check, *args):
    with pytest.raises((pins.PinFailure, AssertionError)):
        check(*args)


def test_mut_route_ties_to_higher_id(monkeypatch):
    monkeypatch.setattr(om, "route_topk", _route_ties_high)
    lg = random_logits(24, 8, seed=3, ties=True)
    _fails(pins.check_route_bruteforce, om.route_topk_plus_shared, lg, 2)


def test_mut_route_without_renormalisation(monkeypatch):
    monkeypatch.setattr(om, "route_topk", _mut_route_no_renorm(om.route_topk))
    _fails(pins.check_route_lexsort, om.route_topk_plus_shared, random_logits(40, 16, seed=2), 4)
    _fails(pins.check_route_golden, om.route_topk_plus_shared)


def test_mut_shared_in_first_slot():
    _fails(pins.check_route_bruteforce, _mut_shared_first(om.route_topk_plus_shared),
           random_logits(8, 8, seed=1), 2)


@pytest.mark.parametrize("value", [0.0, 0.5])
def test_mut_shared_coefficient(monkeypatch, tiny, value):
    monkeypatch.setattr(om, "route_topk_plus_shared", _mut_shared_weight(om.route_topk_plus_shared, value))
    _fails(pins.check_fused_equals_unfused, om.moe_fused, om.moe_unfused, tiny)


def test_mut_align_unstable():
    ids, _ = om.route_topk_plus_shared(random_logits(40, 8, seed=9, ties=True), 2)
    _fails(pins.check_align_bruteforce, _mut_align_unstable(om.align_by_expert), ids, 9, 16)


def test_mut_align_missing_padding():
    ids, _ = om.route_topk_plus_shared(random_logits(40, 8, seed=9), 2)
    _fails(pins.check_align_bruteforce, _mut_align_nopad(om.align_by_expert), ids, 9, 16)


def test_mut_encode_ties_away_from_zero():
    _fails(pins.check_e4m3_encode, _mut_encode_half_away, of.e4m3_decode)


def test_mut_decode_wrong_bias():
    _fails(pins.check_e4m3_decode, _mut_decode_bias8)


@pytest.mark.parametrize("kind", ["silu_sign", "gate_up_swapped", "no_act_quant"])
def test_mut_expert_ffn(kind):
    _fails(pins.check_expert_ffn, _mut_ffn(kind), np.random.default_rng(1), 3, 128, 32, None, torch_quant_a)


def test_mut_activation_scale():
    v = np.random.default_rng(3).standard_normal((8, 256)).astype(np.float32)
    _fails(pins.check_quantize_act, _mut_quant_scale, v, None)


def test_mut_combine_drops_shared_slot(monkeypatch, tiny):
    monkeypatch.setattr(om, "combine_slots", _mut_combine_drop_last)
    _fails(pins.check_fused_equals_unfused, om.moe_fused, om.moe_unfused, tiny)
    _fails(pins.check_zero_routed_is_dense_shared, om.moe_fused, om.combine_slots, om.dense_shared_ffn, tiny)


# ----------------------------------------------------------------------------- router gate
def _router_no_bias(x, w, bias=None):
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def _router_fp32(x, w, bias=None):
    out = np.asarray(x, np.float32) @ np.asarray(w, np.float32).T
    return (out + (0 if bias is None else np.asarray(bias, np.float32))).astype(np.float64)


def test_mut_router_drops_bias():
    _fails(pins.check_router_bruteforce, _router_no_bias)
    _fails(pins.check_router_one_hot, _router_no_bias)


def test_mut_router_float32_sums():
    _fails(pins.check_router_bruteforce, _router_fp32)


# ----------------------------------------------------------------------------- QK-Norm + RoPE
from oracle import attn as oa   # noqa: E402


def _norm_no_eps(x, w, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * w


def _norm_mean_abs(x, w, eps):
    x = np.asarray(x, np.float64)
    return x / (np.mean(np.abs(x), axis=-1, keepdims=True) + eps) * w


def _angles_wrong_exponent(positions, rd, theta):
    i = np.arange(rd // 2, dtype=np.float64)
    return np.asarray(positions, np.float64)[:, None] * (theta ** (-i / rd))[None, :]


def _rope_reversed(x, angle, rd):
    return oa.rope_half(x, -np.asarray(angle), rd)


def _rope_adjacent_pairs(x, angle, rd):
    return oa.rope_interleaved(x, angle, rd)


def _qk_norms_v_too(qkv, Hq, Hkv, D, rd, qw, kw, eps, positions, theta, neox=True):
    out = oa.qk_norm_rope(qkv, Hq, Hkv, D, rd, qw, kw, eps, positions, theta, neox).reshape(qkv.shape[0], -1, D)
    v = out[:, Hq + Hkv:]
    out[:, Hq + Hkv:] = oa.head_rms_norm(v, kw, eps)
    return out.reshape(qkv.shape[0], -1)


def _qk_k_weight_for_q(qkv, Hq, Hkv, D, rd, qw, kw, eps, positions, theta, neox=True):
    return oa.qk_norm_rope(qkv, Hq, Hkv, D, rd, kw, kw, eps, positions, theta, neox)


@pytest.mark.parametrize("mut", [_norm_no_eps, _norm_mean_abs])
def test_mut_head_norm(mut):
    _fails(pins.check_head_rms_norm, mut)


def test_mut_rope_frequency_exponent():
    _fails(pins.check_rope_angles, _angles_wrong_exponent)
    _fails(pins.check_rope_half, oa.rope_half, _angles_wrong_exponent)


@pytest.mark.parametrize("mut", [_rope_reversed, _rope_adjacent_pairs])
def test_mut_rope_rotation(mut):
    _fails(pins.check_rope_half, mut, oa.rope_angles)


def test_mut_rope_interleaved_as_rotate_half():
    _fails(pins.check_rope_interleaved, oa.rope_half, oa.rope_half, oa.rope_angles)


@pytest.mark.parametrize("mut", [_qk_norms_v_too, _qk_k_weight_for_q])
def test_mut_qk_layout(mut):
    _fails(pins.check_qk_layout, mut, oa.head_rms_norm)
