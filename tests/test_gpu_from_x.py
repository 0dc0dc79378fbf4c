"""Routing and the whole layer straight from x (moe_route_from_x, moe_layer_forward_from_x).

- Bit for bit equal to the router gate call followed by the logits-taking call
  (moe_router_logits + moe_route_topk_plus_shared, or + moe_layer_forward): the gate's
  partial tiles are summed inside the routing with the same float32 operations in the
  same order as the gate's own reduction.
- Against the oracle: the routing ids equal the oracle's routing of its float64 gate
  (rounded to float32, the logits every other test uses) except between experts whose
  logits lie within twice the gate's float32 error bound (either order is then correct);
  where a token's ids agree, the layer output is within the 2e-2 bar (with the FP8 tie
  allowance of the other layer tests).
"""
import numpy as np
import pytest
import torch

import oracle
from shared_routed_expert_amd import _lib as L
from tests.gpu_util import (DEV, note, to_dev, bf16_dev, bf16_to_np, make_layer, small_cfg, x_f32,
                            check_rows_with_ties, token_rel_err)
from tests.test_gpu_layer_forward import _outputs
from workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu

ROUTE_CASES = [
    CONFIGS["decode"],
    CONFIGS["prefill"],
    CONFIGS["tiny"],
    small_cfg("ragged", T=77, H=384, I=96, E=12, K=3, seed=11),
    small_cfg("edge_e255", T=30, H=256, I=64, E=255, K=15, seed=21),
    small_cfg("one_token", T=1, H=640, I=64, E=20, K=4, seed=29),
    small_cfg("zipf_bias", T=300, H=512, I=64, E=40, K=8, seed=30, zipf=1.1),
]


def _bias(inp):
    return to_dev(inp.bias) if np.any(inp.bias) else None


def _gate_bound(inp):
    x = x_f32(inp).astype(np.float64)
    H = x.shape[1]
    return (3 * H + 1) * 2.0 ** -24 * (np.abs(x) @ np.abs(inp.router_w.astype(np.float64)).T)


@pytest.mark.parametrize("cfg", ROUTE_CASES, ids=lambda c: c.name)
def test_route_from_x(cfg):
    inp = generate(cfg)
    T, H, E, K = cfg.T, cfg.H, cfg.E, cfg.K
    note(f"route_from_x {cfg.name} T={T} H={H} E={E} K={K}")
    x, w, b = bf16_dev(inp.x_bf16), to_dev(inp.router_w), _bias(inp)
    # the two calls
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    wsb = L.moe_router_workspace_bytes(T, H, E)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    L.moe_router_logits(x, w, b, T, H, E, lg, ws, wsb)
    ids_a = torch.empty((T, K + 1), dtype=torch.int32, device=DEV)
    w_a = torch.empty((T, K + 1), dtype=torch.float32, device=DEV)
    L.moe_route_topk_plus_shared(lg, T, E, K, 0.625, ids_a, w_a)
    # the folded call
    rwb = L.moe_route_from_x_workspace_bytes(T, H, E)
    rws = torch.empty(rwb, dtype=torch.uint8, device=DEV)
    ids_b = torch.full((T, K + 1), -1, dtype=torch.int32, device=DEV)
    w_b = torch.full((T, K + 1), -1.0, dtype=torch.float32, device=DEV)
    L.moe_route_from_x(x, w, b, T, H, E, K, 0.625, ids_b, w_b, rws, rwb)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b)
    assert torch.equal(w_a.view(torch.int32), w_b.view(torch.int32))
    # against the oracle's routing of its own gate
    ref = oracle.router_logits(x_f32(inp), inp.router_w, inp.bias if np.any(inp.bias) else None)
    ids_r, w_r = oracle.route_topk_plus_shared(ref.astype(np.float32), K, shared_weight=0.625)
    ids_g = ids_b.cpu().numpy()
    e_max = float(_gate_bound(inp).max())
    bad = np.nonzero(np.any(ids_g != ids_r, axis=1))[0]
    for t in bad:
        for k in np.nonzero(ids_g[t] != ids_r[t])[0]:
            gap = abs(ref[t, ids_g[t, k]] - ref[t, ids_r[t, k]])
            assert gap <= 2 * e_max, (t, k, gap)
    good = np.setdiff1d(np.arange(T), bad)
    wg = w_b.cpu().numpy()
    assert np.allclose(wg[good], w_r[good], rtol=1e-5, atol=1e-7)
    note(f"  {len(bad)} of {T} tokens route differently, all within the near-tie margin")


@pytest.mark.parametrize("cfg,bm", [
    (CONFIGS["decode"], 16),
    (CONFIGS["prefill"], 128),
    (CONFIGS["tiny"], 16),
    (small_cfg("ragged", T=77, H=384, I=96, E=12, K=3, seed=11), 32),
    (small_cfg("zipf_bias", T=300, H=512, I=64, E=40, K=8, seed=30, zipf=1.1), 64),
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_layer_from_x_matches_two_calls(cfg, bm):
    inp = generate(cfg)
    T, H, E = cfg.T, cfg.H, cfg.E
    note(f"layer_from_x {cfg.name} bm={bm}")
    x, w, b = bf16_dev(inp.x_bf16), to_dev(inp.router_w), _bias(inp)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    wsb = L.moe_router_workspace_bytes(T, H, E)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    L.moe_router_logits(x, w, b, T, H, E, lg, ws, wsb)
    a, W = make_layer(inp, bm)
    a.forward_fused(x, lg, W, 1.0)
    torch.cuda.synchronize()
    ref = _outputs(a)
    c_, _ = make_layer(inp, bm)
    c_.forward_from_x(x, w, b, W, 1.0)
    torch.cuda.synchronize()
    got = _outputs(c_)
    for k in ref:
        assert np.array_equal(ref[k], got[k]), k


def test_layer_from_x_decode_against_oracle():
    inp = generate(CONFIGS["decode"])
    c = inp.cfg
    note("layer_from_x decode vs oracle")
    x, w = bf16_dev(inp.x_bf16), to_dev(inp.router_w)
    layer, W = make_layer(inp, 16)
    layer.forward_from_x(x, w, None, W, 1.0)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.route_topk_plus_shared(inp.logits, c.K)
    ids = layer.topk_ids.cpu().numpy()
    same = np.all(ids == ids_ref, axis=1)
    ref = oracle.router_logits(x_f32(inp), inp.router_w)
    e_max = float(_gate_bound(inp).max())
    for t in np.nonzero(~same)[0]:
        for k in np.nonzero(ids[t] != ids_ref[t])[0]:
            assert abs(ref[t, ids[t, k]] - ref[t, ids_ref[t, k]]) <= 2 * e_max
    tok = np.nonzero(same)[0]
    out_ref = oracle.moe_fused(x_f32(inp), inp.logits, c.K, inp.w13_q, inp.s13, inp.w2_q, inp.s2, tokens=tok)
    out = bf16_to_np(layer.out)[tok]
    e, n_tie = check_rows_with_ties(out, out_ref, inp, [[(int(t), k) for k in range(c.K1)] for t in tok],
                                    ids_ref, w_ref)
    note(f"  {len(tok)} of {c.T} tokens compared; max per-token rel err {e:.3e}; on the tie allowance: {n_tie}")
    assert len(tok) >= c.T - 2
