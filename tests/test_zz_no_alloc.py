"""moe_layer_forward_noalloc (the entry point whose intermediates live in the library's own
device array) against moe_layer_forward (caller workspaces): identical output bits, on two
calls in a row with the second one smaller, at 16-row and 128-row blocks; and the host-side
rejection of sizes beyond the array."""
import numpy as np
import pytest
import torch

from tests.gpu_util import DEV, note, to_dev, bf16_dev, make_layer, small_cfg
from workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu


def _reference(inp, W, T, bm):
    """moe_layer_forward on the first T tokens (its own caller-allocated buffers)."""
    from shared_routed_expert_amd import FusedMoE
    c = inp.cfg
    layer = FusedMoE(T, c.H, c.I, c.E, c.K, bm, W.scale_mode, device=DEV)
    layer.forward_fused(bf16_dev(inp.x_bf16[:T]), to_dev(inp.logits[:T]), W, 1.0)
    torch.cuda.synchronize()
    return layer.out.view(torch.int16).clone()


def _noalloc(inp, W, T, bm):
    from shared_routed_expert_amd import _lib as L
    c = inp.cfg
    out = torch.full((T, c.H), -1, dtype=torch.int16, device=DEV)
    L.moe_layer_forward_noalloc(bf16_dev(inp.x_bf16[:T]), to_dev(inp.logits[:T]), W.w13, W.s13, W.w2, W.s2,
                                W.scale_mode, T, c.H, c.I, c.E, c.K, 1.0, bm, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("cfg,bm,sizes", [
    (CONFIGS["decode"], 16, (64, 20)),
    (small_cfg("noalloc_bm128", T=300, H=1024, I=192, E=40, K=8, seed=41), 128, (300, 77)),
    (small_cfg("noalloc_block", T=90, H=512, I=256, E=12, K=4, mode="block128", seed=42), 64, (90, 33)),
])
def test_noalloc_matches_layer_forward(cfg, bm, sizes):
    inp = generate(cfg)
    _, W = make_layer(inp, bm)
    for T in sizes:   # two calls in a row, the second smaller
        note(f"noalloc {cfg.name} bm={bm} T={T}")
        got = _noalloc(inp, W, T, bm)
        ref = _reference(inp, W, T, bm)
        assert torch.equal(got, ref), f"T={T}: {int((got != ref).sum())} values differ"
