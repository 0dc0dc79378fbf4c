"""moe_layer_forward (one C call) against the four calls: identical bits in every output."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, note, to_dev, bf16_dev, make_layer, small_cfg
from workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu


def _outputs(layer):
    T, H = layer.T, layer.H
    return {
        "topk_ids": layer.topk_ids.cpu().numpy().copy(),
        "topk_w": layer.topk_w.cpu().numpy().view(np.int32).copy(),
        "sorted": layer.sorted_slot_ids.cpu().numpy().copy(),
        "block_expert": layer.block_expert.cpu().numpy().copy(),
        "counts": layer.expert_counts.cpu().numpy().copy(),
        "offsets": layer.expert_offsets.cpu().numpy().copy(),
        "num_padded": layer.num_padded.cpu().numpy().copy(),
        "xq": layer.ws_view("xq", torch.uint8, (T, H)).cpu().numpy().copy(),
        "out": layer.out.view(torch.int16).cpu().numpy().copy(),
    }


@pytest.mark.parametrize("cfg,bm", [
    (CONFIGS["tiny"], 16),
    (small_cfg("ragged", T=77, H=384, I=96, E=12, K=3, seed=11), 32),
    (small_cfg("block", T=50, H=384, I=256, E=6, K=2, mode="block128", seed=15), 16),
    (small_cfg("edge_e255", T=30, H=256, I=64, E=255, K=15, seed=21), 16),
    (small_cfg("single_wg_align", T=455, H=256, I=64, E=40, K=8, seed=22), 64),  # 4095 entries: one-workgroup align
    (small_cfg("three_pass_align", T=600, H=256, I=64, E=40, K=8, seed=23), 64),  # 5400 entries: count/scan/scatter
    (CONFIGS["decode"], 16),
    (CONFIGS["prefill"], 128),   # the bench's prefill launch configuration
    (CONFIGS["prefill16k_zipf"], 128),   # 16,384 tokens, one expert with 13,856 of them
    # decode-shaped blocks: routed experts with more than 16 entries (several row
    # blocks per expert), and I = 256
    (small_cfg("decode_multigroup", T=64, H=256, I=128, E=4, K=2, seed=24), 16),
    (small_cfg("decode_i256", T=40, H=512, I=256, E=10, K=4, seed=25), 16),
    # the in-kernel align of the one-kernel expert FFN: at its limit (4095 entries, 16-row
    # blocks, many blocks per expert) and just past it (4104: the separate align runs)
    (small_cfg("fold_align_max", T=455, H=256, I=64, E=40, K=8, seed=27), 16),
    (small_cfg("fold_align_over", T=456, H=256, I=64, E=40, K=8, seed=28), 16),
    # degenerate routing: the shared expert alone, and one routed expert
    (small_cfg("shared_only", T=37, H=256, I=64, E=6, K=0, seed=31), 16),
    (small_cfg("shared_only_wide", T=37, H=256, I=96, E=6, K=0, seed=31), 64),
    (small_cfg("one_routed", T=29, H=256, I=64, E=1, K=1, seed=32), 16),
    # 128-row blocks: the shared expert's down GEMM and the combine in one launch. Ragged
    # last blocks, column groups past H, the shared expert alone (no routed slot to add),
    # 15 routed slots (two rounds of slot loads), block scales with one and two K steps
    (small_cfg("ragged", T=77, H=384, I=96, E=12, K=3, seed=11), 128),
    (small_cfg("three_blocks", T=300, H=640, I=192, E=20, K=8, seed=33), 128),
    (small_cfg("shared_only", T=37, H=256, I=64, E=6, K=0, seed=31), 128),
    (small_cfg("edge_e255", T=30, H=256, I=64, E=255, K=15, seed=21), 128),
    (small_cfg("block", T=50, H=384, I=256, E=6, K=2, mode="block128", seed=15), 128),
    (small_cfg("block_i128", T=140, H=256, I=128, E=5, K=2, mode="block128", seed=34), 128),
    # the smallest shapes: one token; H = 128 (one column group), I = 32 (a partial K step)
    (small_cfg("one_token", T=1, H=256, I=64, E=20, K=8, seed=35), 128),
    (small_cfg("h128_i32", T=200, H=128, I=32, E=8, K=2, seed=36), 128),
    # I > 256 at block_m 128: the K-looped down GEMM and the separate combine
    (small_cfg("wide_i384_block", T=150, H=256, I=384, E=6, K=2, mode="block128", seed=37), 128),
    (small_cfg("wide_i320", T=90, H=384, I=320, E=7, K=3, seed=38), 128),
])
def test_layer_forward_matches_four_calls(cfg, bm):
    inp = generate(cfg)
    note(f"layer_forward {cfg.name} bm={bm}")
    x, lg = bf16_dev(inp.x_bf16), to_dev(inp.logits)
    a, W = make_layer(inp, bm)
    a.forward(x, lg, W, 0.75)
    torch.cuda.synchronize()
    ref = _outputs(a)
    b, _ = make_layer(inp, bm)
    b.forward_fused(x, lg, W, 0.75)
    torch.cuda.synchronize()
    got = _outputs(b)
    for k in ref:
        assert np.array_equal(ref[k], got[k]), k


@pytest.mark.parametrize("name,bm,stages", [
    ("decode", 16, ["front", "experts", "combine"]),
    ("prefill", 128, ["front", "align", "gate_up", "quant_a", "down_routed", "down_shared_combine"]),
])
def test_layer_forward_staged_matches(name, bm, stages):
    """The measurement form records one event per stage and computes the same bits."""
    from shared_routed_expert_amd import _lib as L
    inp = generate(CONFIGS[name])
    note(f"layer_forward_staged {name} bm={bm}")
    x, lg = bf16_dev(inp.x_bf16), to_dev(inp.logits)
    a, W = make_layer(inp, bm)
    a.forward_fused(x, lg, W, 1.0)
    torch.cuda.synchronize()
    ref = _outputs(a)
    b, _ = make_layer(inp, bm)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for e in evs:
        e.record()   # creates the underlying events
    torch.cuda.synchronize()
    names = b.forward_staged(x, lg, W, 1.0, evs)
    torch.cuda.synchronize()
    assert names == stages
    got = _outputs(b)
    for k in ref:
        assert np.array_equal(ref[k], got[k]), k
    ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    assert all(m >= 0 for m in ms)


@pytest.mark.parametrize("cfg,bm", [(CONFIGS["decode"], 16), (CONFIGS["prefill"], 128),
                                    (small_cfg("ragged", T=77, H=384, I=96, E=12, K=3, seed=11), 32)])
def test_one_workspace_serves_align_and_ffn(cfg, bm):
    """One buffer of moe_workspace_bytes passed as both the align and the FFN workspace (the
    four calls and moe_layer_forward) gives the same bits as separate buffers; moe_combine
    gives the same bits with topk_w NULL or given."""
    from shared_routed_expert_amd import _lib as L
    inp = generate(cfg)
    c = inp.cfg
    note(f"one workspace {cfg.name} bm={bm}")
    x, lg = bf16_dev(inp.x_bf16), to_dev(inp.logits)
    a, W = make_layer(inp, bm)
    a.forward(x, lg, W, 1.0)
    torch.cuda.synchronize()
    ref = a.out.view(torch.int16).clone()
    n = L.moe_workspace_bytes(c.T, c.H, c.I, c.E1, c.K1, bm, W.scale_mode)
    assert n >= max(a.ws_bytes, a.align_ws_bytes)
    b, _ = make_layer(inp, bm)
    one = torch.empty(n, dtype=torch.uint8, device=DEV)
    b.ws, b.ws_bytes, b.align_ws, b.align_ws_bytes = one, n, one, n
    b.forward(x, lg, W, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(b.out.view(torch.int16), ref)
    b.out.zero_()
    b.forward_fused(x, lg, W, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(b.out.view(torch.int16), ref)
    # the combine alone, on the slot rows the four calls left: topk_w given or NULL
    b.forward(x, lg, W, 1.0)
    b.out.zero_()
    L.moe_combine(None, c.T, c.K1, c.H, b.ws, b.ws_bytes, b.out)
    torch.cuda.synchronize()
    assert torch.equal(b.out.view(torch.int16), ref)
