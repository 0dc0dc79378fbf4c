"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/srmoe.h declares, and rejects bad arguments before any launch.

Only invalid calls are made here: each returns from the host-side checks, so no
HIP call is issued (the pointers are fake, 16-byte aligned integers).
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "srmoe.h")


@pytest.fixture(scope="module")
def L():
    from shared_routed_expert_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    from shared_routed_expert_amd import _lib
    return _lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("moe_route_topk_plus_shared", "moe_align_by_expert", "moe_fused_ffn", "moe_combine"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(L.lib, n)  # resolvable through ctypes
    assert set(L.EXPORTED) == set(names)


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4):
        assert L.lib.srmoe_status_string(st)
    assert L.lib.srmoe_last_hip_error() == 0


def test_capacity_and_workspace_sizes(L):
    from oracle import sorted_capacity
    for T, K1, E1, bm in [(64, 9, 161, 16), (4096, 9, 161, 64), (16384, 9, 161, 128), (0, 3, 9, 16), (16, 3, 9, 32)]:
        assert L.moe_sorted_capacity(T, K1, E1, bm) == sorted_capacity(T, K1, E1, bm)
    assert L.moe_sorted_capacity(16, 3, 9, 48) == 0
    off = L.moe_ffn_workspace_offsets(64, 5120, 192, 161, 9, 16, 0)
    assert off["slot_out"] == 0
    assert off["total"] == L.moe_ffn_workspace_bytes(64, 5120, 192, 161, 9, 16, 0)
    keys = ["slot_out", "xq", "sx", "a", "aq", "sa", "rs", "total"]
    vals = [off[k] for k in keys]
    assert vals == sorted(vals) and all(v % 256 == 0 for v in vals)
    assert off["xq"] >= 64 * 9 * 5120 * 2
    assert L.moe_ffn_workspace_bytes(64, 5000, 192, 161, 9, 16, 0) == 0     # H % 128
    assert L.moe_ffn_workspace_bytes(64, 5120, 192, 161, 9, 16, 1) == 0     # block mode, I % 128
    assert L.moe_ffn_workspace_bytes(64, 5120, 1536, 161, 9, 16, 1) > 0
    assert L.moe_align_workspace_bytes(16384, 9, 161) >= 144 * 161 * 4


FAKE = 0x10000          # aligned fake device pointers: never dereferenced on these paths
MIS = 0x10004           # misaligned


def test_route_rejects(L):
    f = lambda *a: L.moe_route_topk_plus_shared(*a, stream=0, check=False)
    assert f(FAKE, -1, 160, 8, 1.0, FAKE, FAKE) == -1
    assert f(FAKE, 4, 0, 0, 1.0, FAKE, FAKE) == -1
    assert f(FAKE, 4, 160, -1, 1.0, FAKE, FAKE) == -1
    assert f(FAKE, 4, 256, 8, 1.0, FAKE, FAKE) == -2
    assert f(FAKE, 4, 8, 9, 1.0, FAKE, FAKE) == -2
    assert f(FAKE, 4, 160, 16, 1.0, FAKE, FAKE) == -2
    assert f(None, 4, 160, 8, 1.0, FAKE, FAKE) == -1
    assert f(FAKE, 4, 160, 8, 1.0, None, FAKE) == -1
    assert f(MIS, 4, 160, 8, 1.0, FAKE, FAKE) == -1
    assert f(FAKE, 0, 160, 8, 1.0, None, None) == 0     # T == 0: nothing to do, nothing launched


def test_align_rejects(L):
    def f(T=64, K1=9, E1=161, bm=16, ptrs=None, ws=FAKE, ws_bytes=1 << 20):
        p = ptrs or [FAKE] * 6
        return L.moe_align_by_expert(p[0], T, K1, E1, bm, p[1], p[2], p[3], p[4], p[5], ws, ws_bytes,
                                     stream=0, check=False)
    assert f(T=-1) == -1
    assert f(K1=0) == -1
    assert f(K1=17) == -2
    assert f(E1=257) == -2
    for bm in (0, 8, 48, 256):
        assert f(bm=bm) == -2
    for i in range(6):
        p = [FAKE] * 6
        p[i] = None
        assert f(ptrs=p) == -1
        p[i] = MIS
        assert f(ptrs=p) == -1
    assert f(ws=None) == -1
    assert f(T=16384, ws_bytes=1024) == -3


def _ffn_args(**kw):
    a = dict(x=FAKE, w13=FAKE, s13=FAKE, w2=FAKE, s2=FAKE, scale_mode=0, T=64, H=5120, I=192, E1=161,
             K1=9, block_m=16, sorted_slot_ids=FAKE, block_expert=FAKE, num_padded=FAKE, topk_w=FAKE,
             workspace=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return a


def test_ffn_rejects(L):
    f = lambda **kw: L.moe_fused_ffn(**_ffn_args(**kw), stream=0, check=False)
    assert f(T=-1) == -1
    assert f(H=0) == -1
    assert f(I=-32) == -1
    assert f(scale_mode=2) == -1
    assert f(H=5000) == -2
    assert f(I=200) == -2
    assert f(scale_mode=1, I=192) == -2
    assert f(E1=300) == -2
    assert f(K1=17) == -2
    assert f(block_m=24) == -2
    assert f(T=1 << 21) == -1
    for name in ("x", "w13", "s13", "w2", "s2", "sorted_slot_ids", "block_expert", "num_padded",
                 "topk_w", "workspace"):
        assert f(**{name: None}) == -1, name
        assert f(**{name: MIS}) == -1, name
    need = L.moe_ffn_workspace_bytes(64, 5120, 192, 161, 9, 16, 0)
    assert f(ws_bytes=need - 1) == -3
    assert f(T=0, x=None) == 0


def test_ffn_stage_rejects(L):
    a = _ffn_args()
    assert L.moe_ffn_quant_x(FAKE, 0, 64, 5120, 192, 161, 9, 16, None, 1 << 40, stream=0, check=False) == -1
    assert L.moe_ffn_quant_x(FAKE, 0, 64, 5120, 192, 161, 9, 16, FAKE, 10, stream=0, check=False) == -3
    assert L.moe_ffn_gate_up(FAKE, None, 0, 64, 5120, 192, 161, 9, 16, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                             stream=0, check=False) == -1
    assert L.moe_ffn_down(FAKE, FAKE, 0, 64, 5120, 192, 161, 9, 16, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                          stream=0, check=False) == -1
    assert L.moe_ffn_down(FAKE, FAKE, 0, 64, 5120, 192, 161, 9, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 100,
                          stream=0, check=False) == -3
    del a


def test_ffn_experts_rejects(L):
    def f(**kw):
        args = dict(w13=FAKE, s13=FAKE, w2=FAKE, s2=FAKE, scale_mode=0, T=64, H=5120, I=192, E1=161, K1=9,
                    block_m=16, sorted_slot_ids=FAKE, block_expert=FAKE, num_padded=FAKE, topk_w=FAKE,
                    workspace=FAKE, ws_bytes=1 << 40)
        args.update(kw)
        return L.moe_ffn_experts(**args, stream=0, check=False)
    for name in ("w13", "s13", "w2", "s2", "sorted_slot_ids", "block_expert", "num_padded", "topk_w",
                 "workspace"):
        assert f(**{name: None}) == -1, name
        assert f(**{name: MIS}) == -1, name
    assert f(I=100) == -2 and f(block_m=8) == -2 and f(scale_mode=1, I=192) == -2
    assert f(ws_bytes=L.moe_ffn_workspace_bytes(64, 5120, 192, 161, 9, 16, 0) - 1) == -3
    assert f(T=0, w13=None) == 0


def test_ffn_experts_one_kernel_shapes(L):
    one = L.moe_ffn_experts_one_kernel
    # 16-row blocks, I a multiple of 64 in 64..256, H <= 5120 (the x rows of a block live in LDS)
    assert one(5120, 192, 16) and one(5120, 64, 16) and one(256, 256, 16) and one(384, 128, 16)
    assert not one(5120, 192, 32) and not one(5120, 96, 16) and not one(5120, 320, 16)
    assert not one(5248, 192, 16) and not one(5120, 32, 16)


def test_router_logits_rejects(L):
    f = lambda **kw: L.moe_router_logits(**{**dict(x=FAKE, w_router=FAKE, bias=None, T=64, H=5120, E=160,
                                                    logits=FAKE, workspace=FAKE, ws_bytes=1 << 30), **kw},
                                         stream=0, check=False)
    assert f(T=-1) == -1 and f(H=0) == -1 and f(E=0) == -1
    assert f(H=5000) == -2 and f(E=257) == -2
    for name in ("x", "w_router", "logits", "workspace"):
        assert f(**{name: None}) == -1, name
        assert f(**{name: MIS}) == -1, name
    assert f(bias=MIS) == -1
    assert f(ws_bytes=L.moe_router_workspace_bytes(64, 5120, 160) - 1) == -3
    assert f(T=0, x=None) == 0
    # batches too small to fill the GPU with tiles split K (partials in the workspace)
    assert L.moe_router_workspace_bytes(64, 5120, 160) > 64 * 160 * 4
    assert L.moe_router_workspace_bytes(4096, 5120, 160) >= 256


def test_route_topk_rejects(L):
    f = lambda *a: L.moe_route_topk(*a, stream=0, check=False)
    assert f(FAKE, -1, 160, 8, FAKE, FAKE) == -1
    assert f(FAKE, 64, 160, 0, FAKE, FAKE) == -1
    assert f(FAKE, 64, 160, 16, FAKE, FAKE) == -2 and f(FAKE, 64, 4, 5, FAKE, FAKE) == -2
    assert f(FAKE, 64, 257, 8, FAKE, FAKE) == -2
    assert f(None, 64, 160, 8, FAKE, FAKE) == -1 and f(FAKE, 64, 160, 8, MIS, FAKE) == -1
    assert f(None, 0, 160, 8, None, None) == 0


def test_combine_unfused_rejects(L):
    f = lambda *a: L.moe_combine_unfused(*a, stream=0, check=False)
    need_r, need_s = 64 * 8 * 5120 * 2, 64 * 5120 * 2
    assert f(-1, 8, 5120, FAKE, need_r, FAKE, need_s, FAKE) == -1
    assert f(64, 0, 5120, FAKE, need_r, FAKE, need_s, FAKE) == -1
    assert f(64, 17, 5120, FAKE, need_r, FAKE, need_s, FAKE) == -2
    assert f(64, 8, 5000, FAKE, need_r, FAKE, need_s, FAKE) == -2
    assert f(64, 8, 5120, None, need_r, FAKE, need_s, FAKE) == -1
    assert f(64, 8, 5120, FAKE, need_r, MIS, need_s, FAKE) == -1
    assert f(64, 8, 5120, FAKE, need_r - 1, FAKE, need_s, FAKE) == -3
    assert f(64, 8, 5120, FAKE, need_r, FAKE, need_s - 1, FAKE) == -3
    assert f(0, 8, 5120, None, 0, None, 0, None) == 0


def test_combine_rejects(L):
    f = lambda *a: L.moe_combine(*a, stream=0, check=False)
    assert f(FAKE, -1, 9, 5120, FAKE, 1 << 30, FAKE) == -1
    assert f(FAKE, 64, 0, 5120, FAKE, 1 << 30, FAKE) == -1
    assert f(FAKE, 64, 9, 5000, FAKE, 1 << 30, FAKE) == -2
    assert f(FAKE, 64, 9, 5120, None, 1 << 30, FAKE) == -1
    assert f(FAKE, 64, 9, 5120, FAKE, 1 << 30, MIS) == -1
    assert f(MIS, 64, 9, 5120, FAKE, 1 << 30, FAKE) == -1        # topk_w misaligned
    assert f(FAKE, 64, 9, 5120, FAKE, 64 * 9 * 5120 * 2 - 1, FAKE) == -3
    assert f(None, 64, 9, 5120, FAKE, 64 * 9 * 5120 * 2 - 1, FAKE) == -3   # topk_w may be NULL
    assert f(None, 0, 9, 5120, None, 0, None) == 0


def test_combine_signature_takes_topk_w(L):
    """moe_combine(topk_w, T, K1, H, workspace, ws_bytes, out, stream): the routing weights
    come first, as the boundary's contract lists them."""
    import ctypes
    hdr = open(HEADER).read()
    assert re.search(r"int moe_combine\(const float\* topk_w, int T, int K1, int H, const void\* workspace,"
                     r"\s+size_t ws_bytes,\s+uint16_t\* out, void\* stream\);", hdr)
    assert L.lib.moe_combine.argtypes[0] is ctypes.c_void_p and len(L.lib.moe_combine.argtypes) == 8


def test_one_workspace_size_for_align_ffn_and_combine(L):
    """moe_workspace_bytes covers both the align and the FFN workspace for every shape, and is
    0 exactly where the FFN shape is unsupported."""
    shapes = [(64, 5120, 192, 161, 9, 16, 0), (4096, 5120, 192, 161, 9, 128, 0), (16384, 5120, 192, 161, 9, 128, 0),
              (4096, 5120, 1536, 161, 9, 128, 1), (16, 128, 32, 9, 3, 16, 0), (0, 256, 64, 9, 3, 32, 0),
              (20000, 256, 64, 256, 16, 64, 0)]
    for T, H, I, E1, K1, bm, mode in shapes:
        n = L.moe_workspace_bytes(T, H, I, E1, K1, bm, mode)
        assert n >= L.moe_ffn_workspace_bytes(T, H, I, E1, K1, bm, mode) > 0
        assert n >= L.moe_align_workspace_bytes(T, K1, E1)
        assert n == max(L.moe_ffn_workspace_bytes(T, H, I, E1, K1, bm, mode), L.moe_align_workspace_bytes(T, K1, E1))
    assert L.moe_workspace_bytes(64, 5000, 192, 161, 9, 16, 0) == 0     # H % 128
    assert L.moe_workspace_bytes(64, 5120, 192, 161, 9, 16, 1) == 0     # block mode needs I % 128 == 0
    assert L.moe_workspace_bytes(64, 5120, 192, 161, 9, 48, 0) == 0     # block_m


def test_moe_status_string_matches(L):
    for st in (0, -1, -2, -3, -4, 7):
        assert L.moe_status_string(st) == L.lib.srmoe_status_string(st).decode()
    assert L.moe_status_string(-3) == "workspace too small"


def test_layer_forward_staged_rejects(L):
    """The measurement form runs the layer's checks (nothing is launched) and checks its event list."""
    import ctypes
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 5120, 192, 160, 8, 1.0, 16] + [FAKE] * 7 + \
           [FAKE, 1 << 30, FAKE, 1 << 40, FAKE, 0]
    ev = (ctypes.c_void_p * 2)(FAKE, FAKE)
    nul = (ctypes.c_void_p * 2)(FAKE, None)
    f = lambda args, events, n: L.lib.moe_layer_forward_staged(*args, events, n, None, None)
    assert f(base, ev, -1) == -1
    assert f(base, None, 2) == -1
    assert f(base, nul, 2) == -1
    bad = list(base); bad[7] = -1
    assert f(bad, ev, 2) == -1
    bad = list(base); bad[8] = 1000
    assert f(bad, ev, 2) == -2


def test_no_cpu_fallback_in_product(L):
    """The product path never imports the oracle."""
    pkg = os.path.join(ROOT, "shared_routed_expert_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn


def test_layer_forward_rejects(L):
    def f(**kw):
        a = dict(x=FAKE, logits=FAKE, w13=FAKE, s13=FAKE, w2=FAKE, s2=FAKE, scale_mode=0, T=64, H=5120, I=192,
                 E=160, K=8, shared_weight=1.0, block_m=16, topk_ids=FAKE, topk_w=FAKE, sorted_slot_ids=FAKE,
                 block_expert=FAKE, expert_counts=FAKE, expert_offsets=FAKE, num_padded=FAKE, align_ws=FAKE,
                 align_ws_bytes=1 << 30, ffn_ws=FAKE, ffn_ws_bytes=1 << 40, out=FAKE)
        a.update(kw)
        return L.moe_layer_forward(**a, stream=0, check=False)
    assert f(T=-1) == -1
    assert f(E=0) == -1
    assert f(K=9, E=8) == -2
    assert f(E=256) == -2
    assert f(H=1000) == -2
    assert f(block_m=8) == -2
    assert f(scale_mode=1) == -2          # I=192 is not a multiple of 128
    for name in ("x", "logits", "w13", "s13", "w2", "s2", "topk_ids", "topk_w", "sorted_slot_ids",
                 "block_expert", "expert_counts", "expert_offsets", "num_padded", "align_ws", "ffn_ws",
                 "out"):
        assert f(**{name: None}) == -1, name
        assert f(**{name: MIS}) == -1, name
    assert f(align_ws_bytes=16) == -3
    assert f(ffn_ws_bytes=1024) == -3
    assert f(T=0, x=None, out=None) == 0


def test_qk_norm_rope_rejects(L):
    def f(**kw):
        a = dict(qkv=FAKE, T=64, num_q_heads=12, num_kv_heads=1, head_dim=128, rotary_dim=64, neox=1,
                 q_norm_w=FAKE, k_norm_w=FAKE, eps=1e-5, positions=FAKE, cos_sin=FAKE, max_pos=131072, fused=1)
        a.update(kw)
        return L.moe_qk_norm_rope(**a, stream=0, check=False)
    assert f(T=-1) == -1 and f(num_q_heads=-1) == -1 and f(num_q_heads=0, num_kv_heads=0) == -1
    assert f(max_pos=0) == -1 and f(eps=-1.0) == -1 and f(eps=float("nan")) == -1
    assert f(head_dim=96) == -2 and f(rotary_dim=8) == -2 and f(rotary_dim=48) == -2
    assert f(rotary_dim=256) == -2 and f(num_q_heads=1000, num_kv_heads=20) == -2
    for name in ("qkv", "positions", "cos_sin", "q_norm_w", "k_norm_w"):
        assert f(**{name: None}) == -1, name
        assert f(**{name: MIS}) == -1, name
    assert f(T=0, qkv=None, positions=None) == 0


def test_rope_table_rejects(L):
    f = lambda *a: L.moe_rope_cos_sin_table(*a, stream=0, check=False)
    assert f(FAKE, 0, 64, 1e6) == -1 and f(FAKE, 16, 63, 1e6) == -1 and f(FAKE, 16, 64, 1.0) == -1
    assert f(None, 16, 64, 1e6) == -1 and f(MIS, 16, 64, 1e6) == -1
    assert f(FAKE, 1 << 26, 64, 1e6) == -2


def test_route_from_x_rejects(L):
    wsb = L.moe_route_from_x_workspace_bytes(64, 5120, 160)
    assert wsb >= 64 * 160 * 4 and L.moe_route_from_x_workspace_bytes(0, 5120, 160) == 0
    f = lambda **kw: L.moe_route_from_x(**{**dict(x=FAKE, w_router=FAKE, bias=None, T=64, H=5120, E=160, K=8,
                                                   shared_weight=1.0, topk_ids=FAKE, topk_w=FAKE, workspace=FAKE,
                                                   ws_bytes=wsb), **kw}, stream=0, check=False)
    assert f(T=-1) == -1 and f(E=0) == -1 and f(K=-1) == -1 and f(H=0) == -1
    assert f(E=256) == -2 and f(K=16) == -2 and f(H=5000) == -2
    for name in ("x", "w_router", "topk_ids", "topk_w", "workspace"):
        assert f(**{name: None}) == -1, name
        assert f(**{name: MIS}) == -1, name
    assert f(bias=MIS) == -1
    assert f(ws_bytes=wsb - 1) == -3
    assert f(T=0, x=None, topk_ids=None) == 0


def test_layer_forward_from_x_rejects(L):
    T, H, I, E, K, bm = 64, 5120, 192, 160, 8, 16
    rwb = L.moe_route_from_x_workspace_bytes(T, H, E)
    awb = L.moe_align_workspace_bytes(T, K + 1, E + 1)
    fwb = L.moe_ffn_workspace_bytes(T, H, I, E + 1, K + 1, bm, 0)

    def f(**kw):
        a = dict(x=FAKE, w_router=FAKE, bias=None, w13=FAKE, s13=FAKE, w2=FAKE, s2=FAKE, scale_mode=0, T=T, H=H,
                 I=I, E=E, K=K, shared_weight=1.0, block_m=bm, topk_ids=FAKE, topk_w=FAKE, sorted_slot_ids=FAKE,
                 block_expert=FAKE, expert_counts=FAKE, expert_offsets=FAKE, num_padded=FAKE, router_ws=FAKE,
                 router_ws_bytes=rwb, align_ws=FAKE, align_ws_bytes=awb, ffn_ws=FAKE, ffn_ws_bytes=fwb, out=FAKE)
        a.update(kw)
        return L.moe_layer_forward_from_x(**a, stream=0, check=False)
    assert f(T=-1) == -1 and f(E=0) == -1 and f(H=0) == -1
    assert f(E=256) == -2 and f(I=100) == -2 and f(block_m=48) == -2
    for name in ("x", "w_router", "w13", "out", "router_ws", "ffn_ws", "topk_ids"):
        assert f(**{name: None}) == -1, name
    assert f(router_ws_bytes=rwb - 1) == -3 and f(ffn_ws_bytes=fwb - 1) == -3 and f(align_ws_bytes=awb - 1) == -3
    assert f(T=0, x=None, out=None) == 0


def test_noalloc_rejects_sizes_beyond_the_array(L):
    """Host-side checks of moe_layer_forward_noalloc: nothing is launched and the array is
    never looked up for these."""
    args = [FAKE] * 6
    # 4,096 prefill tokens need ~450 MB of intermediates: refused before any launch
    assert L.lib.moe_layer_forward_noalloc(*args, 0, 4096, 5120, 192, 160, 8, 1.0, 128, FAKE, None) == -3
    assert L.lib.moe_layer_forward_noalloc(*args, 0, 64, 5120, 192, 160, 8, 1.0, 48, FAKE, None) == -2
    assert L.lib.moe_layer_forward_noalloc(*args, 0, 64, 5120, 192, 160, 8, 1.0, 16, 0x10004, None) == -1
    assert L.lib.moe_layer_forward_noalloc(*args, 0, 0, 5120, 192, 160, 8, 1.0, 16, None, None) == 0


def test_library_stamp_matches_the_sources(L):
    """The library reports the hash of the sources it was built from, and that is the hash
    of the sources in the tree (the binding refuses to load it otherwise)."""
    from shared_routed_expert_amd.build import source_hash
    assert L.lib.srmoe_source_hash().decode() == source_hash()


def test_a_library_from_other_sources_is_refused(L, monkeypatch):
    """A stale build fails loudly at load instead of running old kernels."""
    from shared_routed_expert_amd import build as b
    monkeypatch.setattr(b, "source_hash", lambda: "0000000000000000")
    with pytest.raises(ImportError, match="other sources"):
        L._load()
