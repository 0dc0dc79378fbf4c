"""moe_layer_forward at the full workload sizes, in the launch configuration bench.py times,
against the oracle.

Coverage: every token at decode (64) and prefill (4,096); at the 16k Zipf chunk and the
unsharded block-scale layer, a token set that puts at least one real row in every row block
of the sorted layout (every workgroup's tile of rows meets the oracle), plus the hottest
expert's first and last token. A further case runs every token of a shape large enough for
the routed down launch's 1,280-column workgroups. Routing ids, the sorted layout, counts and
offsets are compared exactly; values per token at 2e-2 (inf-norm relative), with the FP8 tie
allowance.
The oracle is the unchanged plain definition (intelliparadigm, section 2.1; Optimizing
GLM4-MoE for production, section 1).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (note, to_dev, bf16_dev, bf16_to_np, make_layer, x_f32, check_rows_with_ties,
                            small_cfg, token_rel_err, generate_cached)
from workloads import CONFIGS, generate

pytestmark = pytest.mark.gpu

BENCH_BLOCK_M = {"decode": 16, "prefill": 128, "prefill16k_zipf": 128, "unsharded_block": 128}


def block_cover_tokens(ids, E1, block_m, seed):
    """Tokens such that every block_m-row block of the expert-sorted layout holds a row of one
    of them (a real row chosen at random per uncovered block), plus the first and last token
    routed to the hottest routed expert."""
    T, K1 = ids.shape
    sentinel = T * K1
    srt, _, counts, _, npad = oracle.align_by_expert(ids, E1, block_m)
    rows = srt[:npad]
    nb = npad // block_m
    slot_block = np.full(sentinel, -1, np.int64)
    real = np.nonzero(rows < sentinel)[0]
    slot_block[rows[real]] = real // block_m
    covered = np.zeros(nb, bool)
    rng = np.random.default_rng(seed)
    chosen = set()
    for b in range(nb):
        if covered[b]:
            continue
        blk = rows[b * block_m:(b + 1) * block_m]
        t = int(rng.choice(blk[blk < sentinel])) // K1
        chosen.add(t)
        covered[slot_block[t * K1:(t + 1) * K1]] = True
    assert covered.all()
    hot = int(np.argmax(counts[:E1 - 1]))
    hot_tok = np.nonzero((ids[:, :K1 - 1] == hot).any(axis=1))[0]
    chosen |= {int(hot_tok[0]), int(hot_tok[-1])}
    return np.array(sorted(chosen)), nb


# unsharded_block first: test_gpu_ffn's last full-size case leaves its inputs in the cache
@pytest.mark.parametrize("name", ["unsharded_block", "decode", "prefill", "prefill16k_zipf"])
def test_layer_forward_full_size(name):
    bm = BENCH_BLOCK_M[name]
    note(f"full parity {name}: generating inputs")
    inp = generate_cached(CONFIGS[name])
    c = inp.cfg
    layer, W = make_layer(inp, bm)
    note(f"full parity {name}: moe_layer_forward bm={bm}")
    layer.forward_fused(bf16_dev(inp.x_bf16), to_dev(inp.logits), W, 1.0)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.route_topk_plus_shared(inp.logits, c.K)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), ids_ref)
    s, b, cnt, off, npad = oracle.align_by_expert(ids_ref, c.E1, bm)
    assert np.array_equal(layer.sorted_slot_ids.cpu().numpy(), s)
    assert np.array_equal(layer.block_expert.cpu().numpy(), b)
    assert np.array_equal(layer.expert_counts.cpu().numpy(), cnt)
    assert np.array_equal(layer.expert_offsets.cpu().numpy(), off)
    assert int(layer.num_padded.item()) == npad
    if name in ("decode", "prefill"):
        tokens, what = np.arange(c.T), "every token"
    else:
        tokens, nb = block_cover_tokens(ids_ref, c.E1, bm, seed=c.seed)
        what = f"{len(tokens)} tokens covering all {nb} row blocks"
    t0 = time.time()
    note(f"full parity {name}: oracle on {what}")
    out_ref = oracle.moe_fused(x_f32(inp), inp.logits, c.K, inp.w13_q, inp.s13, inp.w2_q, inp.s2, tokens=tokens)
    out = bf16_to_np(layer.out)[tokens]
    e, n_tie = check_rows_with_ties(out, out_ref, inp, [[(int(t), k) for k in range(c.K1)] for t in tokens],
                                    ids_ref, w_ref)
    note(f"full parity {name}: {what}: max per-token rel err {e:.3e}, mean "
         f"{token_rel_err(out, out_ref).mean():.3e}, tokens on the tie allowance {n_tie} "
         f"(oracle {time.time() - t0:.1f} s)")
    full = layer.out.float()
    assert torch.isfinite(full).all()
    assert (full.abs().amax(dim=1) > 0).all()


def test_layer_forward_wide_routed_down_every_token():
    """The routed experts' down launch at 1,280 columns per workgroup, which moe_layer_forward
    takes once the routed row blocks give at least 2,048 workgroups at that width, against the
    oracle on every token. H = 128 keeps the oracle fast; T * K1 = 262,800 slot rows give 2,053
    row blocks of 128 in H's one column group. Values per token at 2e-2 with the FP8 tie
    allowance; routing ids exact."""
    cfg = small_cfg("wide_down", T=29200, H=128, I=64, E=16, K=8, seed=41)
    assert cfg.T * (cfg.K + 1) // 128 * ((cfg.H + 1279) // 1280) >= 2048
    inp = generate(cfg)
    c = inp.cfg
    layer, W = make_layer(inp, 128)
    note("wide routed down: moe_layer_forward bm=128, T=29200, H=128")
    layer.forward_fused(bf16_dev(inp.x_bf16), to_dev(inp.logits), W, 1.0)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.route_topk_plus_shared(inp.logits, c.K)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), ids_ref)
    t0 = time.time()
    out_ref = oracle.moe_fused(x_f32(inp), inp.logits, c.K, inp.w13_q, inp.s13, inp.w2_q, inp.s2)
    out = bf16_to_np(layer.out)
    e, n_tie = check_rows_with_ties(out, out_ref, inp, [[(t, k) for k in range(c.K1)] for t in range(c.T)],
                                    ids_ref, w_ref)
    note(f"wide routed down: every token: max per-token rel err {e:.3e}, tokens on the tie allowance "
         f"{n_tie} (oracle {time.time() - t0:.1f} s)")
