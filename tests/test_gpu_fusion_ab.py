"""The layer with and without the shared-experts fusion (intelliparadigm, section 2.1: the
unfused form computes the shared expert apart and adds it to the weighted routed sum; the
fused form routes it as expert E in slot K of one top-(K+1) pass).

Bar: the two layers agree bit for bit (the pages check allclose with atol 1e-5; the same
kernels on the same rows in the same summation order leave no difference at all), the
routed-only router matches the oracle's top-K exactly, and captured graphs of either layer
replay to the eager bits (the benchmark times the comparison on graph replays).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import note, to_dev, bf16_dev, bf16_to_np, make_layer, small_cfg, x_f32, check_rows_with_ties
from workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu

CASES = [
    (CONFIGS["tiny"], 16),
    (CONFIGS["decode"], 16),
    (small_cfg("ragged", T=77, H=384, I=96, E=12, K=3, seed=11), 32),
    (small_cfg("block", T=50, H=384, I=256, E=6, K=2, mode="block128", seed=15), 16),
    (small_cfg("multigroup", T=64, H=256, I=128, E=4, K=2, seed=24), 16),
    (small_cfg("prefill_like", T=300, H=256, I=64, E=16, K=4, seed=29), 128),
]


def _unfused(inp, bm, W):
    from shared_routed_expert_amd import UnfusedMoE
    c = inp.cfg
    return UnfusedMoE(c.T, c.H, c.I, c.E, c.K, bm, W.scale_mode, device="cuda")


@pytest.mark.parametrize("cfg,bm", CASES, ids=[f"{c.name}-{bm}" for c, bm in CASES])
def test_unfused_equals_fused(cfg, bm):
    inp = generate(cfg)
    note(f"fusion A/B {cfg.name} bm={bm}")
    x, lg = bf16_dev(inp.x_bf16), to_dev(inp.logits)
    fused, W = make_layer(inp, bm)
    fused.forward(x, lg, W, 1.0)
    unf = _unfused(inp, bm, W)
    unf.forward(x, lg, W, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(unf.out.view(torch.int16), fused.out.view(torch.int16))
    assert torch.equal(unf.routed.topk_ids, fused.topk_ids[:, :cfg.K])
    assert torch.equal(unf.routed.topk_w.view(torch.int32), fused.topk_w[:, :cfg.K].contiguous().view(torch.int32))


@pytest.mark.parametrize("cfg,bm", CASES, ids=[f"{c.name}-{bm}" for c, bm in CASES])
def test_unfused_against_oracle(cfg, bm):
    """The unfused GPU layer (routed top-K pass + separate shared pass + add) against the
    oracle's unfused form, the pages' "traditional" formulation (intelliparadigm, section
    2.1): every token within 2e-2 (inf-norm relative), with the FP8 tie allowance."""
    inp = generate(cfg)
    c = inp.cfg
    note(f"unfused vs oracle {cfg.name} bm={bm}")
    x, lg = bf16_dev(inp.x_bf16), to_dev(inp.logits)
    _, W = make_layer(inp, bm)
    unf = _unfused(inp, bm, W)
    unf.forward(x, lg, W, 1.0)
    torch.cuda.synchronize()
    ids_r, _ = oracle.route_topk(inp.logits, c.K)
    assert np.array_equal(unf.routed.topk_ids.cpu().numpy(), ids_r)
    ref = oracle.moe_unfused(x_f32(inp), inp.logits, c.K, inp.w13_q, inp.s13, inp.w2_q, inp.s2)
    got = bf16_to_np(unf.out)
    # the tie allowance walks the token's slots: the routed ones and the shared expert (weight 1)
    ids9, w9 = oracle.route_topk_plus_shared(inp.logits, c.K)
    e, n_tie = check_rows_with_ties(got, ref, inp, [[(t, k) for k in range(c.K1)] for t in range(c.T)], ids9, w9)
    note(f"  unfused {cfg.name}: max per-token rel err {e:.3e}, tokens on the tie allowance {n_tie}")


def test_unfused_split_shared_pass_within_tolerance():
    """The shared pass through the split stages (the benchmark's other unfused baseline): same
    layer up to float rounding, checked against the fused output at the parity tolerance."""
    from tests.gpu_util import TOL, token_rel_err, bf16_to_np
    inp = generate(CONFIGS["decode"])
    x, lg = bf16_dev(inp.x_bf16), to_dev(inp.logits)
    fused, W = make_layer(inp, 16)
    fused.forward(x, lg, W, 1.0)
    unf = _unfused(inp, 16, W)
    unf.forward(x, lg, W, 1.0, shared_split=True)
    torch.cuda.synchronize()
    err = token_rel_err(bf16_to_np(unf.out), bf16_to_np(fused.out))
    note(f"  split shared pass: max per-token rel diff to the fused layer {err.max():.3e}")
    assert err.max() < TOL


def test_route_topk_matches_oracle():
    inp = generate(CONFIGS["prefill"])
    c = inp.cfg
    fused, W = make_layer(inp, 128)
    unf = _unfused(inp, 128, W)
    from shared_routed_expert_amd import _lib as L
    L.moe_route_topk(to_dev(inp.logits), c.T, c.E, c.K, unf.routed.topk_ids, unf.routed.topk_w)
    torch.cuda.synchronize()
    ids, _ = oracle.route_topk(inp.logits, c.K)
    assert np.array_equal(unf.routed.topk_ids.cpu().numpy(), ids)


def test_shared_weight_in_unfused():
    inp = generate(small_cfg("sw", T=40, H=256, I=64, E=8, K=2, seed=30))
    x, lg = bf16_dev(inp.x_bf16), to_dev(inp.logits)
    fused, W = make_layer(inp, 16)
    unf = _unfused(inp, 16, W)
    for sw in (0.375, 1.0):
        fused.forward(x, lg, W, sw)
        unf.forward(x, lg, W, sw)
        torch.cuda.synchronize()
        assert torch.equal(unf.out.view(torch.int16), fused.out.view(torch.int16)), sw


@pytest.mark.parametrize("which", ["fused_four_calls", "fused_one_call", "unfused"])
def test_graph_replay_matches_eager(which):
    inp = generate(CONFIGS["decode"])
    x, lg = bf16_dev(inp.x_bf16), to_dev(inp.logits)
    fused, W = make_layer(inp, 16)
    layer = _unfused(inp, 16, W) if which == "unfused" else fused
    step = {"fused_four_calls": lambda s: fused.forward(x, lg, W, 1.0, s),
            "fused_one_call": lambda s: fused.forward_fused(x, lg, W, 1.0, s),
            "unfused": lambda s: layer.forward(x, lg, W, 1.0, s)}[which]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step(side)   # eager reference (and one-time setup) on the capture stream
    torch.cuda.synchronize()
    ref = layer.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(side)
    for rep in range(3):
        layer.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out.view(torch.int16), ref.view(torch.int16)), rep
        step(torch.cuda.current_stream())   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(layer.out.view(torch.int16), ref.view(torch.int16)), rep
