"""GPU parity of the routing (step 1) and align (step 2) calls against the oracle:
bit-exact ids, sort order, padding, counts, offsets; routing weights to 1e-6."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, note, to_dev
from workloads import CONFIGS, generate, random_logits

pytestmark = pytest.mark.gpu


def gpu_route(logits, K, shared_weight=1.0):
    import shared_routed_expert_amd as m
    T, E = logits.shape
    ids = torch.full((T, K + 1), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, K + 1), -7.0, dtype=torch.float32, device=DEV)
    m.moe_route_topk_plus_shared(to_dev(logits), T, E, K, shared_weight, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check_route(logits, K, shared_weight=1.0):
    ids, w = gpu_route(logits, K, shared_weight)
    rid, rw = oracle.route_topk_plus_shared(logits, K, shared_weight)
    assert np.array_equal(ids, rid), f"ids differ at {np.argwhere(ids != rid)[:5]}"
    rel = np.abs(w.astype(np.float64) - rw) / np.maximum(np.abs(rw), 1e-30)
    assert rel.max() <= 1e-6, rel.max()
    return ids, w


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "prefill16k_zipf"])
def test_route_configs(name):
    inp = generate(CONFIGS[name], with_weights=False)
    note(f"route {name} T={inp.cfg.T}")
    check_route(inp.logits, inp.cfg.K)


@pytest.mark.parametrize("T,E,K", [(1000, 160, 8), (300, 8, 2), (77, 255, 15), (50, 8, 8), (33, 5, 0),
                                   (1, 160, 8), (129, 64, 4)])
def test_route_ties_and_shapes(T, E, K):
    note(f"route ties T={T} E={E} K={K}")
    check_route(random_logits(T, E, seed=T + E, ties=True), K)
    check_route(random_logits(T, E, seed=T * E), K)


def test_route_shared_weight_and_signed_zero():
    lg = random_logits(40, 16, seed=5)
    lg[:, 3] = 0.0
    lg[:, 4] = -0.0   # equal to +0: the lower id (3) must win the tie
    lg[:, 5:] = -1.0
    ids, w = check_route(lg, 4, shared_weight=0.375)
    assert np.all(w[:, 4] == np.float32(0.375)) and np.all(ids[:, 4] == 16)


def test_route_empty_untouched():
    import shared_routed_expert_amd as m
    ids = torch.full((4, 9), -7, dtype=torch.int32, device=DEV)
    w = torch.full((4, 9), -7.0, dtype=torch.float32, device=DEV)
    m.moe_route_topk_plus_shared(torch.zeros((4, 160), device=DEV), 0, 160, 8, 1.0, ids, w)
    torch.cuda.synchronize()
    assert torch.all(ids == -7) and torch.all(w == -7.0)


def gpu_align(ids, E1, bm):
    import shared_routed_expert_amd as m
    T, K1 = ids.shape
    P = m.moe_sorted_capacity(T, K1, E1, bm)
    i32 = dict(dtype=torch.int32, device=DEV)
    out = dict(sorted=torch.full((P,), -9, **i32), block_expert=torch.full((P // bm,), -9, **i32),
               counts=torch.full((E1,), -9, **i32), offsets=torch.full((E1 + 1,), -9, **i32),
               num_padded=torch.full((1,), -9, **i32))
    wsb = m.moe_align_workspace_bytes(T, K1, E1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    m.moe_align_by_expert(to_dev(ids.astype(np.int32)), T, K1, E1, bm, out["sorted"], out["block_expert"],
                          out["counts"], out["offsets"], out["num_padded"], ws, wsb)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check_align(ids, E1, bm):
    g = gpu_align(ids, E1, bm)
    s, b, c, o, n = oracle.align_by_expert(ids, E1, bm)
    assert g["num_padded"][0] == n
    assert np.array_equal(g["counts"], c)
    assert np.array_equal(g["offsets"], o)
    assert np.array_equal(g["block_expert"], b), np.argwhere(g["block_expert"] != b)[:5]
    assert np.array_equal(g["sorted"], s), np.argwhere(g["sorted"] != s)[:5]
    return g


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "prefill16k_zipf"])
def test_align_configs(name, bm):
    inp = generate(CONFIGS[name], with_weights=False)
    ids, _ = oracle.route_topk_plus_shared(inp.logits, inp.cfg.K)
    note(f"align {name} bm={bm}")
    check_align(ids, inp.cfg.E1, bm)


@pytest.mark.parametrize("T,E,K,bm", [(455, 160, 8, 16), (455, 160, 8, 128), (1, 8, 2, 16), (4096 // 9, 9, 8, 32),
                                      (3000, 20, 3, 64), (2000, 255, 15, 16), (5000, 1, 1, 128)])
def test_align_ragged_and_limits(T, E, K, bm):
    ids, _ = oracle.route_topk_plus_shared(random_logits(T, E, seed=T + bm, ties=True), K)
    note(f"align T={T} E={E} K={K} bm={bm}")
    check_align(ids, E + 1, bm)


def test_align_skewed_with_empty_experts():
    T, E, K = 20000, 160, 8
    lg = np.full((T, E), -3.0, np.float32)
    lg[:, :8] = np.arange(8, 0, -1, dtype=np.float32)   # every token: experts 0..7; 8..159 empty
    ids, _ = oracle.route_topk_plus_shared(lg, K)
    for bm in (16, 128):
        check_align(ids, E + 1, bm)


def test_align_gpu_route_chain_and_determinism():
    inp = generate(CONFIGS["prefill16k_zipf"], with_weights=False)
    ids, _ = gpu_route(inp.logits, 8)
    a = check_align(ids, 161, 128)
    b = gpu_align(ids, 161, 128)
    for k in a:
        assert np.array_equal(a[k], b[k])


def test_align_empty():
    g = gpu_align(np.zeros((0, 9), np.int32), 161, 16)
    s, b, c, o, n = oracle.align_by_expert(np.zeros((0, 9), np.int32), 161, 16)
    assert g["num_padded"][0] == 0 and np.array_equal(g["sorted"], s) and np.array_equal(g["block_expert"], b)
    assert np.array_equal(g["counts"], c) and np.array_equal(g["offsets"], o)
