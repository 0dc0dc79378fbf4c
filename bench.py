#!/usr/bin/env python3
"""Benchmark of the fused shared + routed MoE layer on one MI355X.

One step = one pass of the whole layer (route + shared append, align/sort/pad,
the fused FP8 expert FFN over all 9 slots, weighted combine) over one batch of
synthetic input already resident in HBM, through moe_layer_forward. The line's
value is the TP8 decode shard: T=64 tokens, H=5120, 160 routed + 1 shared
experts, I=192, top-8 + shared. The default run adds a "prefill" record for the
4,096-token chunk of the same shard (the prefill half of the metric). Two
independent weight sets (2 x 475 MB) are cycled so the weights stream from HBM
rather than from the 256 MB last-level cache.

Each record carries tokens/s and time per step, per-stage times (HIP events that
the library records between its launches, moe_layer_forward_staged), the roofline
of the dominant kernel (its algorithmic flops or bytes over its measured launch
time; the bound follows its arithmetic intensity: the fp8 MFMA peak above the
ridge, 8 TB/s below), the layer's fp8 and HBM fractions, the four separate calls,
the fused-vs-unfused comparison and the CPU oracle's rate on a token sample. The
decode record also times the router gate, the layer from x and the QK-Norm + RoPE
step. `--gpus` above 1 is refused: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (no sparsity)

WORKLOAD_TEXT = {
    "decode": "GLM4-MoE TP8 shard, decode: T=64 tokens, H=5120, 160 routed + 1 shared SwiGLU experts, "
              "I=192, top-8 + shared = 9 slots, fp8 e4m3 weights with per-output-channel fp32 scales",
    "prefill": "GLM4-MoE TP8 shard, prefill chunk: T=4096 tokens, H=5120, 160 routed + 1 shared, I=192, "
               "top-8 + shared, per-channel fp8 e4m3 weights",
    "prefill16k_zipf": "GLM4-MoE TP8 shard, 16384-token chunked-prefill batch with Zipf(1.1)-skewed routing",
    "unsharded_block": "unsharded expert width: T=4096, H=5120, 160+1 experts, I=1536, top-8 + shared, "
                       "fp8 e4m3 weights with 128x128 block scales",
}
DEFAULT_BLOCK_M = {"decode": 16, "prefill": 128, "prefill16k_zipf": 128, "unsharded_block": 128, "tiny": 16}

# HBM traffic of the dominant kernel per launch (the one-kernel expert FFN for decode, the
# gate/up GEMM for prefill), from the committed rocprofv3 counter summary of the workload:
# FETCH_SIZE and WRITE_SIZE passes, each scaled by what the counter reads for a plain copy
# of known size. The summary records a hash of the kernel's source files; when the sources
# have changed since, the figure is null.
TRAFFIC_PROFILES = {
    ("decode", "experts"): ("profiles/expert_ffn_decode_T64_hbm_traffic.txt",
                            ["shared_routed_expert_amd/csrc/ffn_expert_decode.hip",
                             "shared_routed_expert_amd/csrc/common.hpp"]),
    ("prefill", "gate_up"): ("profiles/gate_up_tile_prefill_T4096_hbm_traffic.txt",
                             ["shared_routed_expert_amd/csrc/ffn_tile.hip", "shared_routed_expert_amd/csrc/common.hpp"]),
    ("prefill16k_zipf", "gate_up"): ("profiles/gate_up_tile_prefill16k_zipf_hbm_traffic.txt",
                                     ["shared_routed_expert_amd/csrc/ffn_tile.hip",
                                      "shared_routed_expert_amd/csrc/common.hpp"]),
    ("prefill16k_zipf", "down_routed"): ("profiles/down_routed_prefill16k_zipf_hbm_traffic.txt",
                                         ["shared_routed_expert_amd/csrc/ffn_tile.hip",
                                          "shared_routed_expert_amd/csrc/common.hpp"]),
    ("unsharded_block", "gate_up"): ("profiles/gate_up_tile_unsharded_block_T4096_hbm_traffic.txt",
                                     ["shared_routed_expert_amd/csrc/ffn_tile.hip",
                                      "shared_routed_expert_amd/csrc/common.hpp"]),
}


def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, kernel):
    entry = TRAFFIC_PROFILES.get((workload, kernel))
    if entry is None:
        return None
    path, files = entry
    try:
        fields = dict(line.split(":", 1) for line in open(os.path.join(ROOT, path)) if ":" in line)
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != source_hash(files):
        return None
    return int(fields["traffic_bytes_per_launch"])


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def copy_calibration(mib: int, reps: int):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "reps": reps}), flush=True)


CPU_SAMPLE_TOKENS = {"decode": 64, "prefill": 128, "prefill16k_zipf": 128, "unsharded_block": 16, "tiny": 16}


def host_cpu():
    """The host's logical CPU count, the process's affinity and the CPU model."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        aff = None
    return {"cpu_count": os.cpu_count(), "affinity": aff, "cpu_model": model}


def cpu_baseline(inp, budget_s: float, n_tokens: int):
    """The CPU oracle (fused form, as it stands) on a bounded token sample."""
    import numpy as np
    import oracle
    from workloads import f32_from_bf16_bits
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    c = inp.cfg
    x = f32_from_bf16_bits(inp.x_bf16)
    n = min(c.T, n_tokens)
    times = []
    t_all = time.perf_counter()
    # at least 3 runs and about 10 s of work, within the budget
    while len(times) < 3 or (sum(times) < 10.0 and len(times) < 15 and
                             (time.perf_counter() - t_all) < budget_s):
        tok = np.arange(n)
        t0 = time.perf_counter()
        oracle.moe_fused(x, inp.logits, c.K, inp.w13_q, inp.s13, inp.w2_q, inp.s2, tokens=tok)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    rec = {"value": n / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"first {n} tokens of the {c.name} batch (routing over all {c.T}), float64 numpy "
                     f"oracle, median of {len(times)} runs ({med:.2f} s each)"}
    rec.update(host_cpu())
    return rec


def router_timing(inp, x, steps):
    """The router gate upstream of the layer (moe_router_logits), timed on graph replays:
    duration, float32-equivalent TFLOP/s and the bytes of x and the router weight."""
    import torch
    from shared_routed_expert_amd import _lib as L
    c = inp.cfg
    w = torch.from_numpy(inp.router_w).cuda()
    bias = torch.from_numpy(inp.bias).cuda()
    out = torch.empty((c.T, c.E), dtype=torch.float32, device="cuda")
    wsb = L.moe_router_workspace_bytes(c.T, c.H, c.E)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    fn = lambda: L.moe_router_logits(x, w, bias, c.T, c.H, c.E, out, ws, wsb, side)
    us = graph_time([fn], side, steps)
    flops = 2.0 * c.T * c.H * c.E
    nbytes = c.T * c.H * 2 + c.E * c.H * 4 + c.T * c.E * 4
    return {"us": round(us, 2), "tflops_fp32_equiv": round(flops / us / 1e6, 2), "GBps": round(nbytes / us / 1e3, 1),
            "bytes": nbytes, "timing": "graph replay"}


def from_x_timing(inp, x, layer, weights, steps):
    """Routing and the whole layer from x (the router gate folded into the route call):
    moe_route_from_x, and moe_layer_forward_from_x against moe_router_logits +
    moe_layer_forward; timed on graph replays over the cycled weight sets."""
    import torch
    from shared_routed_expert_amd import _lib as L
    c = inp.cfg
    w = torch.from_numpy(inp.router_w).cuda()
    bias = torch.from_numpy(inp.bias).cuda() if inp.bias.any() else None
    side = torch.cuda.Stream()
    rwb = L.moe_route_from_x_workspace_bytes(c.T, c.H, c.E)
    rws = torch.empty(rwb, dtype=torch.uint8, device="cuda")
    ids = torch.empty((c.T, c.K1), dtype=torch.int32, device="cuda")
    tw = torch.empty((c.T, c.K1), dtype=torch.float32, device="cuda")
    route_us = graph_time([lambda: L.moe_route_from_x(x, w, bias, c.T, c.H, c.E, c.K, 1.0, ids, tw, rws, rwb,
                                                      side)], side, steps)
    lg = torch.empty((c.T, c.E), dtype=torch.float32, device="cuda")
    wsb = L.moe_router_workspace_bytes(c.T, c.H, c.E)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")

    def two_calls(Wt):
        def f():
            L.moe_router_logits(x, w, bias, c.T, c.H, c.E, lg, ws, wsb, side)
            layer.forward_fused(x, lg, Wt, 1.0, side)
        return f
    sep_us = graph_time([two_calls(Wt) for Wt in weights], side, steps)
    fold_us = graph_time([(lambda Wt=Wt: layer.forward_from_x(x, w, bias, Wt, 1.0, side)) for Wt in weights], side,
                         steps)
    return {"route_from_x_us": round(route_us, 2), "layer_from_x_us": round(fold_us, 2),
            "gate_then_layer_us": round(sep_us, 2), "timing": "graph replay"}


def qk_norm_rope_timing(steps):
    """The attention-side QK-Norm + RoPE step (moe_qk_norm_rope) on one GPU's share of GLM4-MoE
    attention (12 q + 1 kv heads of 128, half of each rotated), fused and as two passes, at
    the decode and prefill token counts; timed on graph replays of the call in place."""
    import numpy as np
    import torch
    from shared_routed_expert_amd import _lib as L
    from workloads import QK_CONFIGS, generate_qk
    side = torch.cuda.Stream()
    res = {}
    for name in ("decode", "prefill"):
        inp = generate_qk(QK_CONFIGS[name])
        c = inp.cfg
        qkv = torch.from_numpy(inp.qkv_bf16.view(np.int16)).cuda()
        pos = torch.from_numpy(inp.positions).cuda()
        qw, kw = torch.from_numpy(inp.q_norm_w).cuda(), torch.from_numpy(inp.k_norm_w).cuda()
        cs = torch.empty((c.max_pos, c.rotary_dim), dtype=torch.float32, device="cuda")
        L.moe_rope_cos_sin_table(cs, c.max_pos, c.rotary_dim, c.theta, side)
        torch.cuda.synchronize()

        def call(fused):
            return lambda: L.moe_qk_norm_rope(qkv, c.T, c.num_q_heads, c.num_kv_heads, c.head_dim, c.rotary_dim,
                                              c.neox, qw, kw, c.eps, pos, cs, c.max_pos, fused, side)
        fused_us = graph_time([call(True)], side, steps)
        unfused_us = graph_time([call(False)], side, steps)
        # q and k heads read and written once, positions, the table rows, the two weight vectors
        nbytes = 2 * c.T * (c.num_q_heads + c.num_kv_heads) * c.head_dim * 2 + c.T * 4 + c.T * c.rotary_dim * 4 \
            + 2 * c.head_dim * 4
        res[name] = {"T": c.T, "fused_us": round(fused_us, 2), "unfused_us": round(unfused_us, 2),
                     "unfused_over_fused": round(unfused_us / fused_us, 3), "alg_bytes": nbytes,
                     "fused_GBps": round(nbytes / fused_us / 1e3, 1),
                     "fused_hbm_frac": round(nbytes / fused_us / 1e3 / HBM_PEAK_GBS, 4)}
    res["timing"] = "graph replay"
    return res


GRAPH_ROUNDS = 8   # captured rounds per graph, so that the host's launch of a replay is amortised


def graph_time(fns, stream, steps):
    """Average GPU duration (us) of one call of the step functions in `fns` (called in turn,
    e.g. one per weight set): GRAPH_ROUNDS rounds of them are captured as one HIP graph,
    which is replayed until about `steps` calls have run."""
    import torch
    with torch.cuda.stream(stream):
        for fn in fns:
            fn()   # warm-up and one-time setup outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(GRAPH_ROUNDS):
            for fn in fns:
                fn()
    per_replay = GRAPH_ROUNDS * len(fns)
    replays = max(1, steps // per_replay)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / (replays * per_replay)


def fusion_ab(cfg, bm, x, logits, weights, fused, steps):
    """The pages' comparison: the layer with the shared-experts fusion (one top-(K+1) pass) and
    without it (a top-K routed pass plus a separate shared pass, added in the combine), same
    kernels. Each flow is captured as a HIP graph of several steps over the weight sets in
    turn and replayed, so host launch overhead is out of the timing."""
    import torch
    from shared_routed_expert_amd import UnfusedMoE
    unf = UnfusedMoE(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, bm, weights[0].scale_mode, device="cuda")
    flows = {
        "fused_one_call": lambda W, s: fused.forward_fused(x, logits, W, 1.0, s),
        "fused_four_calls": lambda W, s: fused.forward(x, logits, W, 1.0, s),
        "unfused": lambda W, s: unf.forward(x, logits, W, 1.0, s),
        "unfused_split_shared": lambda W, s: unf.forward(x, logits, W, 1.0, s, shared_split=True),
    }
    side = torch.cuda.Stream()
    res = {}
    timing = f"graph replay ({GRAPH_ROUNDS} rounds of the weight sets per graph)"
    for name, fn in flows.items():
        steps_fns = [lambda W=W, fn=fn: fn(W, side) for W in weights]
        try:
            us = graph_time(steps_fns, side, steps)
        except Exception as exc:  # pragma: no cover - capture not available
            log(f"bench: graph capture failed for {name} ({exc}); timing eager launches")
            timing = "eager launches (graph capture failed)"
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(side)
            for i in range(steps):
                steps_fns[i % len(steps_fns)]()
            e1.record(side)
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / steps
        res[name + "_us"] = round(us, 2)
    # the unfused baseline at its best: the shared pass on whichever kernels run it faster
    res["unfused_best_us"] = min(res["unfused_us"], res["unfused_split_shared_us"])
    res["unfused_over_fused"] = round(res["unfused_best_us"] / res["fused_one_call_us"], 4)
    res["timing"] = timing
    return res


RIDGE = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # flop/B where the fp8 MFMA and HBM bounds meet


def stage_work(stage, cfg, active, active_routed, P):
    """Algorithmic (flops, bytes) of one launch of a stage of moe_layer_forward: the weights and
    scales of the experts it serves read once, the activations it needs read once and the results
    it hands on written once (in their smallest form: FP8 codes plus one scale per row). Not
    counted: padding rows, re-reads, and the slot rows of the routed experts (the slot buffer's
    round trip is an overhead of the design, not work of the method)."""
    T, H, I, E, K, K1 = cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.K1
    blk = cfg.scale_mode == "block128"
    s13 = (2 * I // 128) * (H // 128) * 4 if blk else 2 * I * 4
    s2 = (H // 128) * (I // 128) * 4 if blk else H * 4
    gx = H // 128 if blk else 1
    ga = I // 128 if blk else 1
    rows = T * K1
    if stage == "front":        # logits in, routing tables out; x in, x codes + scales out
        return 0.0, T * E * 4 + T * K1 * 8 + T * H * 2 + T * (H + 4 * gx)
    if stage == "align":
        return 0.0, rows * 4 + P * 4
    if stage == "experts":      # the whole expert FFN of a decode batch, slot rows out
        return rows * 6.0 * H * I, active * (3 * I * H + s13 + s2) + T * (H + 4 * gx) + rows * H * 2
    if stage == "gate_up":      # w13 + x codes in, the SwiGLU rows out (as FP8 codes + scales)
        return rows * 4.0 * H * I, active * (2 * I * H + s13) + T * (H + 4 * gx) + rows * (I + 4 * ga)
    if stage == "quant_a":
        return 0.0, rows * (I * 4 + I + 4 * ga + 4)
    if stage == "down_routed":  # w2 of the routed experts + the routed SwiGLU rows in
        return T * K * 2.0 * H * I, active_routed * (I * H + s2) + T * K * (I + 4 * ga)
    if stage == "down_shared_combine":   # the shared expert's down GEMM and the combine: out written
        return T * 2.0 * H * I, (I * H + s2) + T * (I + 4 * ga) + T * H * 2
    if stage == "combine":
        return 0.0, rows * H * 2 + T * H * 2
    return None


def roofline_of(flops, nbytes, us):
    """Bound from the arithmetic intensity: the fp8 MFMA peak above the ridge, HBM below."""
    if flops / max(nbytes, 1) > RIDGE:
        ach = flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / FP8_PEAK_TFLOPS, 4)}
    ach = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4)}


def measure(name, args, with_extras):
    """One workload: the layer through moe_layer_forward, timed over args.steps steps after
    args.warmup, its stages timed with events recorded by the library between its launches,
    the dominant kernel's roofline, the four separate calls, and the CPU oracle."""
    import numpy as np
    import torch
    from workloads import CONFIGS, generate
    from shared_routed_expert_amd import FusedMoE, DeviceWeights

    cfg = CONFIGS[name]
    bm = args.block_m or DEFAULT_BLOCK_M[name]
    dev = "cuda:0"
    log(f"bench: generating {name} inputs ({args.weight_sets} weight sets)")
    sets = [generate(cfg, weight_set=j) for j in range(args.weight_sets)]
    inp = sets[0]
    weights = [DeviceWeights.from_numpy(s.w13_q, s.s13, s.w2_q, s.s2, device=dev) for s in sets]
    for s in sets[1:]:
        s.w13_q = s.w2_q = None
    x = torch.from_numpy(inp.x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(inp.logits).to(dev)
    layer = FusedMoE(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, bm, weights[0].scale_mode, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):   # the whole layer through one C call (moe_layer_forward)
        layer.forward_fused(x, logits, weights[i % len(weights)], 1.0, stream)

    def step_four_calls(i):   # the same layer as the four separate C calls
        layer.forward(x, logits, weights[i % len(weights)], 1.0, stream)

    log(f"bench: {name}: warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: the whole layer, K steps, bracketed by synchronisations.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    log(f"bench: {name}: {ms_per_step * 1e3:.1f} us/step on the GPU, {wall * 1e6 / args.steps:.1f} us/step "
        f"wall-clock")

    # Per-step durations of the same call (events around each step): median and 10th / 90th percentiles.
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    sev[0].record(stream)
    for i in range(args.steps):
        step(i)
        sev[i + 1].record(stream)
    torch.cuda.synchronize()
    step_us = sorted(1e3 * sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps))
    pct = lambda q: step_us[min(len(step_us) - 1, int(q * (len(step_us) - 1) + 0.5))]

    # The same layer call with events recorded by the library between its launches (same
    # stream, same kernels): each stage's average duration, the dominant kernel's included.
    nev = 12
    sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for evl in sevs:
        for e in evl:
            e.record(stream)   # creates the underlying HIP events
    torch.cuda.synchronize()
    names = None
    for i in range(args.steps):
        names = layer.forward_staged(x, logits, weights[i % len(weights)], 1.0, sevs[i], stream)
    torch.cuda.synchronize()
    stage_us = {n: 1e3 * statistics.mean(sevs[i][j].elapsed_time(sevs[i][j + 1]) for i in range(args.steps))
                for j, n in enumerate(names)}

    # The four separate calls, warmed up first.
    for i in range(args.warmup):
        step_four_calls(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step_four_calls(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    four_ms = ev0.elapsed_time(ev1) / args.steps

    counts = layer.expert_counts.cpu().numpy()
    active = int((counts > 0).sum())
    active_routed = int((counts[:cfg.E] > 0).sum())
    P = int(layer.num_padded.item())
    T, H, I, E1, K1 = cfg.T, cfg.H, cfg.I, cfg.E1, cfg.K1
    blk = cfg.scale_mode == "block128"
    s13_bytes = (2 * I // 128) * (H // 128) * 4 if blk else 2 * I * 4
    s2_bytes = (H // 128) * (I // 128) * 4 if blk else H * 4
    dom = max(stage_us, key=stage_us.get)
    work = stage_work(dom, cfg, active, active_routed, P)
    if work is None:   # a stage made of several kernels (the split FFN path)
        dom = max((n for n in stage_us if stage_work(n, cfg, active, active_routed, P)), key=stage_us.get)
        work = stage_work(dom, cfg, active, active_routed, P)
    flops_k, bytes_k = work
    roof = roofline_of(flops_k, bytes_k, stage_us[dom])
    roof.update({"kernel": dom, "traffic": traffic_from_profile(name, dom), "alg_bytes_per_launch": int(bytes_k),
                 "alg_flops_per_launch": int(flops_k), "avg_launch_us": round(stage_us[dom], 2),
                 "timing": "HIP events recorded by moe_layer_forward_staged around the launch"})
    layer_bytes = active * (3 * I * H + s13_bytes + s2_bytes) + T * H * 2 * 2 + T * cfg.E * 4 + T * K1 * 8
    flops = T * K1 * 6 * H * I
    step_s = ms_per_step * 1e-3
    rec = {
        "workload": WORKLOAD_TEXT[name], "T": T, "H": H, "I": I, "routed_experts": cfg.E, "shared_experts": 1,
        "top_k": cfg.K, "slots": K1, "block_m": bm, "weight_sets_cycled": len(weights), "active_experts": active,
        "tokens_per_s": round(T / step_s, 1), "ms_per_step": round(ms_per_step, 5),
        "roofline": roof,
        "layer": {"alg_bytes": layer_bytes, "alg_GBps": round(layer_bytes / step_s / 1e9, 1),
                  "hbm_frac": round(layer_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
                  "alg_TFLOPs": round(flops / step_s / 1e12, 2),
                  "fp8_frac": round(flops / step_s / 1e12 / FP8_PEAK_TFLOPS, 4),
                  "roofline_frac": round(max(flops / (FP8_PEAK_TFLOPS * 1e12), layer_bytes / (HBM_PEAK_GBS * 1e9))
                                         / (pct(0.5) * 1e-6), 4),
                  "step_us_p10_p50_p90": [round(pct(0.1), 2), round(pct(0.5), 2), round(pct(0.9), 2)],
                  "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
                  "stage_roofline": {k: roofline_of(*stage_work(k, cfg, active, active_routed, P), v)["frac"]
                                     for k, v in stage_us.items() if stage_work(k, cfg, active, active_routed, P)},
                  "entry_point": "moe_layer_forward",
                  "four_call_ms_per_step": round(four_ms, 5)},
    }
    if with_extras:
        log("bench: router gate (graph replays)")
        rec["router_gate"] = router_timing(inp, x, args.steps)
        log("bench: routing and the layer from x (graph replays)")
        rec["from_x"] = from_x_timing(inp, x, layer, weights, args.steps)
        log("bench: QK-Norm + RoPE, fused and unfused (graph replays)")
        rec["qk_norm_rope"] = qk_norm_rope_timing(args.steps)
    if not args.no_fusion_ab:
        log(f"bench: {name}: fused vs unfused layer (graph replays)")
        rec["fusion_ab"] = fusion_ab(cfg, bm, x, logits, weights, layer, args.steps)
    del weights, layer
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log(f"bench: {name}: timing the CPU oracle")
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, CPU_SAMPLE_TOKENS.get(name, 64))
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="default", choices=["default"] + sorted(WORKLOAD_TEXT),
                    help="default: the decode workload (the line's value) plus the prefill record")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--weight-sets", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=30.0)
    ap.add_argument("--no-fusion-ab", action="store_true", help="skip the fused-vs-unfused comparison")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (under TP8 each GPU "
              "runs this layer on its 192-wide slice of every expert and an all-reduce sums the "
              "partial outputs; that exchange is not built).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calib_mib:
        copy_calibration(args.copy_calib_mib, max(args.steps, 1))
        return

    head = "decode" if args.workload == "default" else args.workload
    rec = measure(head, args, with_extras=True)
    result = {
        "metric": "fused MoE layer tokens/s + % fp8 MFMA peak (prefill) / % HBM BW (decode)",
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded; random-init fp8 expert weights of the GLM4-MoE TP8 shard shape)",
        "config": {k: rec[k] for k in ("workload", "T", "H", "I", "routed_experts", "shared_experts", "top_k",
                                       "slots", "block_m", "weight_sets_cycled", "active_experts")},
        "roofline": rec["roofline"],
    }
    result["config"]["parallelism"] = "single GPU"
    for k in ("layer", "router_gate", "from_x", "qk_norm_rope", "fusion_ab", "cpu_baseline"):
        if k in rec:
            result[k] = rec[k]
    if args.workload == "default":
        # the prefill half of the metric: the 4,096-token chunk (the pages' input length)
        pre = measure("prefill", args, with_extras=False)
        result["prefill"] = pre
    # which library ran: its path and the source stamp it was built with (the binding
    # refuses a library whose stamp differs from the sources in the tree)
    from shared_routed_expert_amd import _lib
    result["library"] = {"path": os.path.relpath(_lib.LIB_PATH, ROOT),
                         "source_hash": _lib.lib.srmoe_source_hash().decode()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
