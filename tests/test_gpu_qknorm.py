"""GPU QK-Norm + RoPE (moe_qk_norm_rope, moe_rope_cos_sin_table) against the oracle.

Bar, per output value, with ref the float64 oracle on the same bf16 inputs and m the
length of the rotated pair the value belongs to (|ref| for unrotated dims):
  fused:   |gpu - ref| <= 2^-8 |ref| + 2^-15 m   (one bf16 rounding of a float32 result --
           bf16 keeps 8 significant bits, unit roundoff 2^-8; float32 error of the 128-term
           sum of squares, rsqrt and rotation < 2^-15 m)
  unfused: |gpu - ref| <= 2^-8 |ref| + (1.5 * 2^-8 + 2^-15) m   (the normalised pair is also
           stored as bf16 before the rotation: 2^-8 (|a c| + |b s|) <= 2^-8 sqrt(2) m more)
v heads and every byte outside the q and k heads are unchanged bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from shared_routed_expert_amd import _lib as L
from tests.gpu_util import note, DEV
from workloads import QK_CONFIGS, QKConfig, generate_qk, f32_from_bf16_bits

pytestmark = pytest.mark.gpu

GUARD = 4096   # bf16 values of guard before and after the qkv rows


def table(max_pos, rd, theta):
    cs = torch.empty((max_pos, rd), dtype=torch.float32, device=DEV)
    L.moe_rope_cos_sin_table(cs, max_pos, rd, theta)
    return cs


def run(inp, fused=True, cfg=None, positions=None):
    cfg = cfg or inp.cfg
    T, row = inp.qkv_bf16.shape
    buf = np.full(T * row + 2 * GUARD, 0x7FC1, dtype=np.uint16)   # guard: a NaN pattern
    buf[GUARD:GUARD + T * row] = inp.qkv_bf16.reshape(-1)
    dbuf = torch.from_numpy(buf.view(np.int16)).to(DEV)
    qkv_ptr = dbuf.data_ptr() + 2 * GUARD
    cs = table(cfg.max_pos, cfg.rotary_dim, cfg.theta)
    pos = torch.from_numpy(inp.positions if positions is None else positions).to(DEV)
    qw = torch.from_numpy(inp.q_norm_w).to(DEV)
    kw = torch.from_numpy(inp.k_norm_w).to(DEV)
    note(f"qk_norm_rope {cfg.name} T={T} Hq={cfg.num_q_heads} Hkv={cfg.num_kv_heads} D={cfg.head_dim} "
         f"rd={cfg.rotary_dim} neox={cfg.neox} fused={fused}")
    L.moe_qk_norm_rope(qkv_ptr, T, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rotary_dim, cfg.neox,
                       qw, kw, cfg.eps, pos, cs, cfg.max_pos, fused)
    torch.cuda.synchronize()
    out = dbuf.cpu().numpy().view(np.uint16)
    assert np.array_equal(out[:GUARD], buf[:GUARD]) and np.array_equal(out[-GUARD:], buf[-GUARD:])
    return out[GUARD:GUARD + T * row].reshape(T, row)


def reference(inp, cfg=None, positions=None):
    cfg = cfg or inp.cfg
    x = f32_from_bf16_bits(inp.qkv_bf16)
    pos = inp.positions if positions is None else positions
    return oracle.qk_norm_rope(x, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rotary_dim,
                               inp.q_norm_w, inp.k_norm_w, cfg.eps, pos, cfg.theta, neox=cfg.neox)


def pair_len(ref, cfg):
    T = ref.shape[0]
    D, rd = cfg.head_dim, cfg.rotary_dim
    h = ref.reshape(T, -1, D)
    d = np.arange(D)
    if cfg.neox:
        partner = np.where(d < rd // 2, d + rd // 2, d - rd // 2)
    else:
        partner = d ^ 1
    partner = np.where(d < rd, partner, d)
    m = np.sqrt(h * h + np.where(d < rd, h[..., partner] ** 2, 0.0))
    return m.reshape(T, -1)


def check(got_bits, ref, inp, cfg, fused):
    nq = (cfg.num_q_heads + cfg.num_kv_heads) * cfg.head_dim
    # v heads: untouched
    assert np.array_equal(got_bits[:, nq:], inp.qkv_bf16[:, nq:])
    got = f32_from_bf16_bits(got_bits).astype(np.float64)[:, :nq]
    r = ref[:, :nq]
    m = pair_len(ref, cfg)[:, :nq]
    slack = 2.0 ** -15 if fused else 1.5 * 2.0 ** -8 + 2.0 ** -15
    err = np.abs(got - r)
    bound = 2.0 ** -8 * np.abs(r) + slack * m
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{len(bad)} values out of bound, first {bad[:3]}: got {got[tuple(bad[0])]} ref {r[tuple(bad[0])]}"
    return float(np.max(err / np.maximum(m, 1e-30)))


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", ["decode", "prefill", "prefill16k", "tiny"])
def test_workloads(name, fused):
    inp = generate_qk(QK_CONFIGS[name])
    got = run(inp, fused)
    e = check(got, reference(inp), inp, inp.cfg, fused)
    note(f"  max err / pair length {e:.3e}")


SHAPES = [
    # (T, Hq, Hkv, D, rd, neox)
    (1, 12, 1, 128, 64, True),
    (3, 12, 1, 128, 64, False),
    (77, 2, 1, 64, 16, True),      # heads per wavefront 8, a ragged last workgroup
    (77, 2, 1, 64, 64, False),
    (33, 3, 2, 256, 128, True),
    (33, 3, 2, 256, 256, True),    # everything rotated
    (9, 4, 0, 128, 32, True),      # q heads only
    (9, 0, 3, 128, 128, False),    # k (and v) heads only
    (1000, 12, 1, 128, 64, True),
    (64, 96, 8, 128, 64, True),    # the unsharded attention (all 96 q and 8 kv heads on one GPU)
    (3, 500, 262, 64, 32, True),   # 1024 heads per token, the limit
]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("T,Hq,Hkv,D,rd,neox", SHAPES)
def test_shapes(T, Hq, Hkv, D, rd, neox, fused):
    cfg = QKConfig(f"shape_{T}_{Hq}_{Hkv}_{D}_{rd}", T=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                   rotary_dim=rd, neox=neox, max_pos=4096, theta=10000.0, eps=1e-6, seed=T * 7 + D + rd)
    inp = generate_qk(cfg)
    got = run(inp, fused)
    check(got, reference(inp), inp, cfg, fused)


def test_positions_are_clamped_to_the_table():
    cfg = QK_CONFIGS["tiny"]
    inp = generate_qk(cfg)
    wild = np.array([-5, 0, cfg.max_pos - 1, cfg.max_pos, 10 ** 6], np.int32)
    got = run(inp, True, positions=wild)
    clamped = np.clip(wild, 0, cfg.max_pos - 1)
    check(got, reference(inp, positions=clamped), inp, cfg, True)


def test_zero_head_is_finite_and_eps_matters():
    """An all-zero head normalises to zero (eps keeps the divisor positive)."""
    cfg = QK_CONFIGS["tiny"]
    inp = generate_qk(cfg)
    inp.qkv_bf16[2, :cfg.head_dim] = 0
    got = run(inp, True)
    assert np.all(got[2, :cfg.head_dim] & 0x7FFF == 0)
    check(got, reference(inp), inp, cfg, True)


@pytest.mark.parametrize("max_pos,rd,theta", [(131072, 64, 1e6), (4096, 16, 10000.0), (1, 128, 500.0)])
def test_cos_sin_table(max_pos, rd, theta):
    got = table(max_pos, rd, theta).cpu().numpy().astype(np.float64)
    ang = oracle.rope_angles(np.arange(max_pos), rd, theta)
    ref = np.concatenate([np.cos(ang), np.sin(ang)], axis=1)
    # float64 values rounded once to float32 (one float32 ulp), plus the float64 angle's
    # own rounding (a few double ulps of the angle, which moves cos / sin by as much)
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref) + 2.0 ** -48 * np.abs(np.concatenate([ang, ang], 1)))


def test_graph_replays_match_eager():
    """The fused call captured in a graph and replayed several times on fresh inputs."""
    cfg = QK_CONFIGS["decode"]
    inp = generate_qk(cfg)
    T = cfg.T
    cs = table(cfg.max_pos, cfg.rotary_dim, cfg.theta)
    qkv = torch.empty((T, cfg.row), dtype=torch.int16, device=DEV)
    pos = torch.from_numpy(inp.positions).to(DEV)
    qw, kw = torch.from_numpy(inp.q_norm_w).to(DEV), torch.from_numpy(inp.k_norm_w).to(DEV)
    src = torch.from_numpy(inp.qkv_bf16.view(np.int16)).to(DEV)

    def call(stream):
        L.moe_qk_norm_rope(qkv, T, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rotary_dim, cfg.neox,
                           qw, kw, cfg.eps, pos, cs, cfg.max_pos, True, stream)

    qkv.copy_(src)
    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = qkv.cpu().numpy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        qkv.copy_(src)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call(s)
    for rep in range(3):
        qkv.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(qkv.cpu().numpy(), eager), rep
        qkv.copy_(src)                         # eager work between replays
        call(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert np.array_equal(qkv.cpu().numpy(), eager), rep
