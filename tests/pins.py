"""Pins for the CPU oracle: each check compares an oracle function with something
other than itself (brute force, a library routine, a closed form, a printed
value, an invariant the pages fix). Every check takes the function under test
as an argument, so the mutation tests can hand it a deliberately broken oracle
and confirm that some pin fails.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


class PinFailure(AssertionError):
    pass


def _require(cond, msg):
    if not cond:
        raise PinFailure(msg)


# ----------------------------------------------------------------------------- FP8 codec
def golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def check_e4m3_decode(decode):
    codes = np.arange(256, dtype=np.uint8)
    got = decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    _require(np.array_equal(np.isnan(got), nan), "decode: NaN codes differ from torch float8_e4m3fn")
    _require(np.array_equal(got[~nan], ref[~nan]), "decode: values differ from torch float8_e4m3fn")
    _require(np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "decode: sign of zero")
    for c, v in golden_e4m3():
        g = decode(np.array([c], np.uint8))[0]
        if math.isnan(v):
            _require(math.isnan(g), f"decode golden {c:#x}")
        else:
            _require(g == v and math.copysign(1, g) == math.copysign(1, v), f"decode golden {c:#x}: {g} != {v}")


def check_e4m3_encode(encode, decode):
    codes = np.arange(256, dtype=np.uint8)
    vals = decode(codes)
    finite = ~np.isnan(vals)
    _require(np.array_equal(encode(vals[finite]), codes[finite]), "encode(decode(c)) != c")
    # midpoints between consecutive magnitudes: ties go to the even code
    mags = vals[:127]
    mids = (mags[:-1] + mags[1:]) / 2
    got = encode(mids)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    _require(np.array_equal(got, want), "encode: ties not to even")
    _require(np.array_equal(encode(-mids), want | 0x80), "encode: negative ties")
    # saturation
    big = np.array([448.0, 449.0, 464.0, 465.0, 480.0, 1e6, 1e30], np.float64)
    _require(np.all(encode(big) == 0x7E), "encode: positive saturation")
    _require(np.all(encode(-big) == 0xFE), "encode: negative saturation")
    _require(encode(np.array([np.nan]))[0] & 0x7F == 0x7F, "encode: NaN")
    # random float32 values across the whole range vs torch's RNE cast (in range)
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(200_000) * np.exp(rng.uniform(-14, 6.1, 200_000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    _require(np.array_equal(encode(v), ref), "encode: differs from torch float8_e4m3fn on random values")
    for c, val in golden_e4m3():
        if not math.isnan(val):
            _require(encode(np.array([val]))[0] == c, f"encode golden {val}")


# ----------------------------------------------------------------------------- routing
def golden_routes():
    rows, cur = [], {}
    with open(os.path.join(GOLDEN, "route_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            cur[key] = [float(v) for v in vals]
            if key == "weights":
                rows.append(cur)
                cur = {}
    return rows


def _before(l, i, j):
    """Expert i ranks before expert j: higher logit, ties to the lower id."""
    return l[i] > l[j] or (l[i] == l[j] and i < j)


def check_route_bruteforce(route_plus_shared, logits, K):
    """For every token, exactly one K-subset has every member ranked before every
    non-member, and the oracle picks it, in rank order; the shared slot follows."""
    T, E = logits.shape
    ids, w = route_plus_shared(logits, K, 1.0)
    _require(ids.shape == (T, K + 1) and w.shape == (T, K + 1), "route shape")
    for t in range(T):
        l = [float(v) for v in logits[t]]
        good = [S for S in itertools.combinations(range(E), K)
                if all(_before(l, i, j) for i in S for j in range(E) if j not in S)]
        _require(len(good) == 1, "brute force found no unique top-K set")
        _require(sorted(ids[t, :K].tolist()) == list(good[0]), f"token {t}: wrong top-K set")
        for a, b in zip(ids[t, :K - 1], ids[t, 1:K]):
            _require(_before(l, int(a), int(b)), f"token {t}: routed slots out of order")
        _require(ids[t, K] == E and w[t, K] == 1.0, f"token {t}: shared slot")


def check_route_lexsort(route_plus_shared, logits, K):
    """Independent ordering by numpy lexsort and weights by scipy's softmax."""
    T, E = logits.shape
    ids, w = route_plus_shared(logits, K, 1.0)
    order = np.lexsort((np.broadcast_to(np.arange(E), logits.shape), -logits.astype(np.float64)), axis=1)
    _require(np.array_equal(ids[:, :K], order[:, :K]), "ids differ from lexsort")
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    pk = np.take_along_axis(p, order[:, :K], axis=1)
    want = pk / pk.sum(axis=1, keepdims=True)
    _require(np.allclose(w[:, :K], want, rtol=1e-12, atol=0), "weights differ from scipy softmax renormalised")
    _require(np.all(ids[:, K] == E) and np.all(w[:, K] == 1.0), "shared slot")
    _require(np.allclose(w[:, :K].sum(axis=1), 1.0, rtol=1e-12), "routed weights do not sum to 1")


def check_route_golden(route_plus_shared):
    for row in golden_routes():
        lg = np.array([row["logits"]], np.float32)
        K = len(row["ids"]) - 1
        ids, w = route_plus_shared(lg, K, 1.0)
        _require(ids[0].tolist() == [int(v) for v in row["ids"]], f"golden ids {row['ids']} vs {ids[0]}")
        _require(np.allclose(w[0], row["weights"], rtol=1e-6, atol=0), f"golden weights {w[0]}")


def check_route_k_equals_e(route_plus_shared, logits):
    """K = E: every routed expert is taken and the weights are the plain softmax."""
    T, E = logits.shape
    ids, w = route_plus_shared(logits, E, 1.0)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    got = np.zeros_like(p)
    np.put_along_axis(got, ids[:, :E].astype(np.int64), w[:, :E], axis=1)
    _require(np.allclose(got, p, rtol=1e-12, atol=1e-300), "K=E weights are not the softmax")


# ----------------------------------------------------------------------------- align
def check_align_bruteforce(align, ids, E1, bm):
    T, K1 = ids.shape
    sentinel = T * K1
    sorted_ids, block_expert, counts, offsets, num_padded = align(ids, E1, bm)
    pairs = sorted((int(ids[s // K1, s % K1]), s) for s in range(T * K1))
    want_rows = []
    want_counts = [0] * E1
    for e in range(E1):
        mem = [s for (ee, s) in pairs if ee == e]
        want_counts[e] = len(mem)
        pad = -len(mem) % bm
        want_rows += mem + [sentinel] * pad
    _require(int(num_padded) == len(want_rows), "num_padded")
    cap = len(sorted_ids)
    _require(cap >= len(want_rows) and cap % bm == 0, "capacity")
    _require(sorted_ids[:num_padded].tolist() == want_rows, "sorted slot ids differ from brute-force sort")
    _require(np.all(sorted_ids[num_padded:] == sentinel), "tail not sentinel")
    _require(counts.tolist() == want_counts, "expert counts")
    want_off = np.concatenate([[0], np.cumsum([-(-c // bm) * bm for c in want_counts])])
    _require(offsets.tolist() == want_off.tolist(), "expert offsets")
    for b in range(cap // bm):
        rows = sorted_ids[b * bm:(b + 1) * bm]
        real = [int(r) for r in rows if r != sentinel]
        if b * bm < num_padded:
            e = int(block_expert[b])
            _require(0 <= e < E1 and offsets[e] <= b * bm < offsets[e + 1], f"block {b} expert")
            _require(all(int(ids[r // K1, r % K1]) == e for r in real), f"block {b} mixes experts")
        else:
            _require(block_expert[b] == -1 and not real, f"block {b} beyond the end")
    _require(counts[E1 - 1] == T or np.any(ids[:, -1] != E1 - 1), "shared expert count")


# ----------------------------------------------------------------------------- activations
def check_quantize_act(quantize_act, v, group):
    """Against torch: per-row (or per-group) absmax scale in float32, then torch's float8 cast."""
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    n, c = t.shape
    g = c if group is None else group
    tb = t.reshape(n, c // g, g)
    amax = tb.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / torch.tensor(448.0), torch.ones_like(amax))
    want_q = (tb / s[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, c)
    q, sc = quantize_act(v, group)
    want_s = s[:, 0].numpy() if group is None else s.numpy()
    _require(np.array_equal(sc, want_s), "activation scales")
    _require(np.array_equal(q, want_q.numpy()), "activation codes")


# ----------------------------------------------------------------------------- FFN
def ffn_triple_loop(xd_rows, w13, w2, quant_a):
    """Pure-Python float64 loops over one SwiGLU expert (tiny sizes only)."""
    I = len(w13) // 2
    H = len(w2)
    out = []
    for x in xd_rows:
        g = [sum(x[h] * w13[i][h] for h in range(len(x))) for i in range(I)]
        u = [sum(x[h] * w13[I + i][h] for h in range(len(x))) for i in range(I)]
        a = [g[i] / (1.0 + math.exp(-g[i])) * u[i] for i in range(I)]
        a = quant_a(a)
        out.append([sum(w2[h][i] * a[i] for i in range(I)) for h in range(H)])
    return np.array(out)


def check_expert_ffn(expert_ffn, rng, n=3, H=128, I=32, group=None, quant_a=None):
    """expert_ffn vs plain loops on random dequantised operands."""
    xd = rng.standard_normal((n, H))
    w13 = rng.standard_normal((2 * I, H)) / math.sqrt(H)
    w2 = rng.standard_normal((H, I)) / math.sqrt(I)
    got = expert_ffn(xd, w13, w2, group)
    want = ffn_triple_loop(xd.tolist(), w13.tolist(), w2.tolist(), quant_a)
    err = np.max(np.abs(got - want)) / np.max(np.abs(want))
    _require(err < 1e-12, f"expert FFN differs from triple loop: {err}")


def check_ffn_closed_form(expert_ffn, decode, encode):
    """A one-hot input through an expert whose gate/up columns are the only non-zeros:
    g_i = v*Wg[i,h0], u_i = v*Wu[i,h0], a_i = silu(g_i)*u_i, y = W2 q(a) in closed form."""
    H, I, h0, v = 128, 32, 5, 1.5
    xd = np.zeros((1, H))
    xd[0, h0] = v
    w13 = np.zeros((2 * I, H))
    gi = np.linspace(-3, 3, I)
    ui = np.linspace(0.5, -1.0, I)
    w13[:I, h0] = gi
    w13[I:, h0] = ui
    w2 = np.outer(np.linspace(-1, 1, H), np.ones(I)) + np.eye(H, I)
    got = expert_ffn(xd, w13, w2, None)[0]
    a = (v * gi) / (1 + np.exp(-v * gi)) * (v * ui)
    a32 = a.astype(np.float32)
    s = np.float32(np.abs(a32).max()) / np.float32(448.0)
    aq = decode(encode((a32 / s).astype(np.float32))) * np.float64(s)
    want = w2 @ aq
    _require(np.allclose(got, want, rtol=1e-13, atol=1e-13), "closed-form expert output")


def check_fused_equals_unfused(moe_fused, moe_unfused, inp, tokens=None):
    """The pages' own check of the fusion (intelliparadigm, section 5, item 3):
    fused and original outputs agree within atol 1e-5. Returns the max abs diff."""
    from workloads import f32_from_bf16_bits
    x = f32_from_bf16_bits(inp.x_bf16)
    a = moe_fused(x, inp.logits, inp.cfg.K, inp.w13_q, inp.s13, inp.w2_q, inp.s2, tokens=tokens)
    b = moe_unfused(x, inp.logits, inp.cfg.K, inp.w13_q, inp.s13, inp.w2_q, inp.s2, tokens=tokens)
    d = float(np.max(np.abs(a - b)))
    _require(np.allclose(a, b, atol=1e-5, rtol=0), f"fused != unfused (max diff {d})")
    return d


def check_zero_routed_is_dense_shared(moe_fused_slots, combine, dense_shared, inp):
    """With every routed weight set to zero the layer reduces to the dense shared FFN."""
    from workloads import f32_from_bf16_bits
    x = f32_from_bf16_bits(inp.x_bf16)
    out, y, ids, w = moe_fused_slots(x, inp.logits, inp.cfg.K, inp.w13_q, inp.s13, inp.w2_q,
                                     inp.s2, return_slots=True)
    w0 = w.copy()
    w0[:, :-1] = 0.0
    got = combine(y, w0)
    want = dense_shared(x, inp.w13_q, inp.s13, inp.w2_q, inp.s2)
    _require(np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max()),
             "zero routed weights do not give the dense shared FFN")


def check_k_equals_e_mixture(moe_fused, expert_ffn_all, inp):
    """K = E: output = shared FFN + softmax-weighted mixture of every routed expert."""
    from workloads import f32_from_bf16_bits
    x = f32_from_bf16_bits(inp.x_bf16)
    E = inp.cfg.E
    got = moe_fused(x, inp.logits, E, inp.w13_q, inp.s13, inp.w2_q, inp.s2)
    p = scipy.special.softmax(inp.logits.astype(np.float64), axis=1)
    ys = expert_ffn_all(x)  # [E1, T, H]
    want = ys[E] + np.einsum("te,eth->th", p, ys[:E])
    _require(np.allclose(got, want, rtol=0, atol=1e-10 * np.abs(want).max()), "K=E mixture")


def check_permutation_equivariance(moe_fused, inp, perm):
    from workloads import f32_from_bf16_bits
    x = f32_from_bf16_bits(inp.x_bf16)
    K = inp.cfg.K
    a = moe_fused(x, inp.logits, K, inp.w13_q, inp.s13, inp.w2_q, inp.s2)
    b = moe_fused(x[perm], inp.logits[perm], K, inp.w13_q, inp.s13, inp.w2_q, inp.s2)
    _require(np.allclose(a[perm], b, rtol=0, atol=1e-12 * np.abs(a).max()), "token permutation")


# ----------------------------------------------------------------------------- router gate
def check_router_bruteforce(router_logits):
    """Pure-Python triple loop on tiny inputs (no numpy matmul), bias included."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 7)).astype(np.float32)
    w = rng.standard_normal((4, 7)).astype(np.float32)
    b = rng.standard_normal(4).astype(np.float32)
    got = router_logits(x, w, b)
    for t in range(3):
        for e in range(4):
            acc = float(b[e])
            for h in range(7):
                acc += float(x[t, h]) * float(w[e, h])
            _require(abs(got[t, e] - acc) <= 1e-12 * (1 + abs(acc)), f"router logit ({t},{e})")


def check_router_one_hot(router_logits):
    """x = unit vectors: the logits are the router weight's columns (plus the bias), exactly."""
    rng = np.random.default_rng(6)
    w = rng.standard_normal((5, 8)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    got = router_logits(np.eye(8, dtype=np.float32), w, b)
    _require(np.array_equal(got, w.T.astype(np.float64) + b.astype(np.float64)[None, :]), "one-hot rows + bias")
    _require(np.array_equal(router_logits(np.eye(8, dtype=np.float32), w), w.T.astype(np.float64)),
             "one-hot rows")


# ----------------------------------------------------------------------------- QK-Norm + RoPE
def check_head_rms_norm(head_rms_norm):
    # a constant head c: every entry becomes sign(c) / sqrt(1 + eps / c^2) * w
    w = np.linspace(0.5, 1.5, 8)
    got = head_rms_norm(np.full((1, 8), -3.0), w, 1e-6)
    _require(np.allclose(got, -w / np.sqrt(1 + 1e-6 / 9.0), rtol=0, atol=1e-15), "constant head")
    # unit weight, eps 0: mean square exactly 1 (up to rounding); scale invariance
    x = np.random.default_rng(1).standard_normal((5, 3, 16))
    y = head_rms_norm(x, np.ones(16), 0.0)
    _require(np.allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-14), "unit mean square")
    _require(np.allclose(head_rms_norm(7.5 * x, np.ones(16), 0.0), y, atol=1e-14), "scale invariance")


def check_rope_angles(rope_angles):
    # hand values: theta = 100, rotary_dim = 4 -> frequencies 100^0 = 1 and 100^(-1/2) = 1/10
    got = rope_angles(np.array([0, 10, 30]), 4, 100.0)
    _require(np.allclose(got, [[0.0, 0.0], [10.0, 1.0], [30.0, 3.0]], rtol=0, atol=1e-12), "angles")


def check_rope_half(rope_half, rope_angles):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 2, 16))
    rd, h = 8, 4
    _require(np.array_equal(rope_half(x, rope_angles(np.zeros(4), rd, 10000.0), rd), x), "position 0")
    pos = np.array([1, 5, 17, 1000])
    y = rope_half(x, rope_angles(pos, rd, 10000.0), rd)
    _require(np.array_equal(y[..., rd:], x[..., rd:]), "dims past rotary_dim pass through")
    _require(np.allclose(y[..., :h] ** 2 + y[..., h:rd] ** 2, x[..., :h] ** 2 + x[..., h:rd] ** 2, atol=1e-12),
             "pair lengths")
    q = np.array([3, 4, 5, 6])
    _require(np.allclose(rope_half(y, rope_angles(q, rd, 10000.0), rd),
                         rope_half(x, rope_angles(pos + q, rd, 10000.0), rd), atol=1e-10), "composition")
    # pair 0 (dims 0 and h) at position p is (x0 + i x_h) e^{i p}
    z = (x[:, :, 0] + 1j * x[:, :, h]) * np.exp(1j * pos.astype(np.float64))[:, None]
    _require(np.allclose(y[:, :, 0], z.real, atol=1e-12) and np.allclose(y[:, :, h], z.imag, atol=1e-12),
             "pair 0")
    # pair 1 (dims 1 and h + 1) with theta = 100, rd = 8 turns by p * 100^(-1/4) = p / sqrt(10)
    y2 = rope_half(x[:1], rope_angles(np.array([10]), rd, 100.0), rd)
    z1 = (x[0, :, 1] + 1j * x[0, :, h + 1]) * np.exp(1j * 10.0 / math.sqrt(10.0))
    _require(np.allclose(y2[0, :, 1], z1.real, atol=1e-12) and np.allclose(y2[0, :, h + 1], z1.imag, atol=1e-12),
             "pair 1")


def check_rope_interleaved(rope_interleaved, rope_half, rope_angles):
    """Interleaved pairs (2i, 2i+1) are rotate-half pairs (i, i + rd/2) once the even dims
    are moved to the front; position 0 leaves x as it is; pair 0 is a complex product."""
    rng = np.random.default_rng(4)
    D, rd = 16, 8
    x = rng.standard_normal((3, 2, D))
    pos = np.array([0.0, 7.0, 123.0])
    ang = rope_angles(pos, rd, 500.0)
    perm = np.concatenate([np.arange(0, rd, 2), np.arange(1, rd, 2), np.arange(rd, D)])
    via_half = rope_half(x[..., perm], ang, rd)[..., np.argsort(perm)]
    y = rope_interleaved(x, ang, rd)
    _require(np.allclose(y, via_half, atol=1e-13), "permuted rotate-half")
    _require(np.array_equal(rope_interleaved(x[:1], ang[:1], rd), x[:1]), "position 0")
    z = (x[:, :, 0] + 1j * x[:, :, 1]) * np.exp(1j * pos)[:, None]
    _require(np.allclose(y[:, :, 0], z.real, atol=1e-12) and np.allclose(y[:, :, 1], z.imag, atol=1e-12), "pair 0")
    _require(np.array_equal(y[..., rd:], x[..., rd:]), "dims past rotary_dim pass through")


def check_qk_layout(qk_norm_rope, head_rms_norm):
    """q and k heads are normalised with their own weights and rotated; v passes through."""
    rng = np.random.default_rng(3)
    T, Hq, Hkv, D, rd = 3, 2, 1, 8, 4
    qkv = rng.standard_normal((T, (Hq + 2 * Hkv) * D))
    qw, kw = rng.uniform(0.5, 1.5, D), rng.uniform(0.5, 1.5, D)
    out = qk_norm_rope(qkv, Hq, Hkv, D, rd, qw, kw, 1e-6, np.array([0, 2, 9]), 10000.0)
    heads_in = qkv.reshape(T, Hq + 2 * Hkv, D)
    heads = out.reshape(T, Hq + 2 * Hkv, D)
    _require(np.array_equal(heads[:, Hq + Hkv:], heads_in[:, Hq + Hkv:]), "v heads untouched")
    _require(np.allclose(heads[0, :Hq], head_rms_norm(heads_in[0, :Hq], qw, 1e-6)), "q at position 0")
    _require(np.allclose(heads[0, Hq], head_rms_norm(heads_in[0, Hq], kw, 1e-6)), "k at position 0")
    _require(np.allclose(heads[:, :Hq, rd:], head_rms_norm(heads_in[:, :Hq], qw, 1e-6)[..., rd:]),
             "dims past rotary_dim are the normalised values")
