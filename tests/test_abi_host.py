"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/moe.h declares, validates configurations, sizes workspaces and
rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

import expert_layer_amd as m
from expert_layer_amd import _ffi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            src = open(os.path.join(inc, f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    decl = _declared()
    assert decl >= set(_ffi.EXPORTS) and decl == set(_ffi.EXPORTS)
    L = ctypes.CDLL(_ffi.LIB_PATH)
    for n in sorted(decl):
        assert hasattr(L, n), n


def _dsv3(**kw):
    base = dict(T=8192, H=7168, E=256, k=8, I=2048, n_groups=8, topk_groups=4, score_fn=m.MOE_SCORE_SIGMOID,
                routed_scale=2.5, has_shared=True, I_shared=2048)
    base.update(kw)
    return m.make_cfg(**base)


def test_validate_accepts_workload_shapes():
    assert m.moe_validate(_dsv3()) == m.MOE_OK
    assert m.moe_validate(m.make_cfg(T=256, H=512, E=8, k=2, I=1024, act_dtype=m.MOE_F32)) == m.MOE_OK
    assert m.moe_validate(m.make_cfg(T=16384, H=4096, E=128, k=8, I=1536)) == m.MOE_OK
    assert m.moe_validate(m.make_cfg(T=0, H=64, E=4, k=1, I=64)) == m.MOE_OK


@pytest.mark.parametrize("kw,code", [
    (dict(k=9, E=8), m.MOE_ERR_INVALID_ARG),
    (dict(k=0), m.MOE_ERR_INVALID_ARG),
    (dict(k=33, E=64), m.MOE_ERR_INVALID_ARG),
    (dict(E=1025, k=8, n_groups=5), m.MOE_ERR_INVALID_ARG),
    (dict(n_groups=3), m.MOE_ERR_INVALID_ARG),
    (dict(topk_groups=9), m.MOE_ERR_INVALID_ARG),
    (dict(topk_groups=0), m.MOE_ERR_INVALID_ARG),
    (dict(k=8, topk_groups=1, n_groups=64), m.MOE_ERR_INVALID_ARG),
    (dict(H=7170), m.MOE_ERR_INVALID_ARG),
    (dict(I=0), m.MOE_ERR_INVALID_ARG),
    (dict(T=-1), m.MOE_ERR_INVALID_ARG),
    (dict(score_fn=2), m.MOE_ERR_INVALID_ARG),
    (dict(group_score=5), m.MOE_ERR_INVALID_ARG),
    (dict(I_shared=0), m.MOE_ERR_INVALID_ARG),
    (dict(y_dtype=m.MOE_FP8_E4M3), m.MOE_ERR_INVALID_ARG),
    (dict(out_dtype=7), m.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=m.MOE_BF16, w_dtype=m.MOE_F32), m.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=m.MOE_FP8_E4M3), m.MOE_ERR_UNSUPPORTED),  # fp8 + shared expert
    (dict(m_tile=-1), m.MOE_ERR_INVALID_ARG),
    (dict(routed_scale=float("inf")), m.MOE_ERR_INVALID_ARG),
    (dict(x_layout=3), m.MOE_ERR_INVALID_ARG),
    (dict(x_layout=m.MOE_LAYOUT_INDEXED, act_dtype=m.MOE_F32), m.MOE_ERR_UNSUPPORTED),
    (dict(x_layout=m.MOE_LAYOUT_TILED, m_tile=8), m.MOE_ERR_INVALID_ARG),
    (dict(x_layout=m.MOE_LAYOUT_TILED, m_tile=0), m.MOE_ERR_INVALID_ARG),
    (dict(x_layout=m.MOE_LAYOUT_TILED, m_tile=16, act_dtype=m.MOE_F32), m.MOE_ERR_UNSUPPORTED),
])
def test_validate_rejects(kw, code):
    c = _dsv3(**kw)
    assert m.moe_validate(c) == code
    assert m.moe_last_error() != ""
    assert m.moe_max_rows(c) == -1
    assert m.moe_workspace_bytes(c, m.MOE_STAGE_LAYER) == ctypes.c_size_t(-1).value


def test_fp8_needs_128_multiples():
    c = m.make_cfg(T=64, H=7168, E=8, k=1, I=2048, act_dtype=m.MOE_FP8_E4M3, y_dtype=m.MOE_BF16)
    assert m.moe_validate(c) == m.MOE_OK
    c = m.make_cfg(T=64, H=7168 + 64, E=8, k=1, I=2048, act_dtype=m.MOE_FP8_E4M3)
    assert m.moe_validate(c) == m.MOE_ERR_INVALID_ARG


def test_fp8_experts_cfg():
    """bf16 activations with e4m3 experts: accepted by moe_validate and sized
    for the layer; needs 128-multiples (I_shared too); moe_grouped_ffn refuses
    the pair (it takes the quantised rows); moe_quantize_fp8 checks its
    arguments before any launch."""
    kw = dict(T=64, H=7168, E=256, k=8, I=2048, n_groups=8, topk_groups=4, has_shared=True, I_shared=2048,
              act_dtype=m.MOE_BF16, w_dtype=m.MOE_FP8_E4M3, y_dtype=m.MOE_BF16)
    c = m.make_cfg(**kw)
    assert m.moe_validate(c) == m.MOE_OK
    bf = m.make_cfg(**dict(kw, w_dtype=m.MOE_BF16))
    # the layer holds the quantised tokens and their scales besides the bf16 layer's buffers
    assert m.moe_workspace_bytes(c, m.MOE_STAGE_LAYER) > 64 * 7168
    assert m.moe_validate(m.make_cfg(**dict(kw, I_shared=2048 + 64))) == m.MOE_ERR_UNSUPPORTED
    assert m.moe_validate(m.make_cfg(**dict(kw, I=2048 + 64))) == m.MOE_ERR_INVALID_ARG
    assert m.moe_validate(m.make_cfg(**dict(kw, act_dtype=m.MOE_F32))) == m.MOE_ERR_UNSUPPORTED
    assert m.moe_validate(bf) == m.MOE_OK
    lib = m._ffi.lib()
    fake = ctypes.c_void_p(0x100000)
    w = m.moe_weights(w_gate=0x100000, w_up=0x100000, w_down=0x100000, s_gate=0x100000, s_up=0x100000,
                      s_down=0x100000)
    st = lib.moe_grouped_ffn(ctypes.byref(c), 64, fake, fake, fake, None, ctypes.byref(w), fake, fake, fake,
                             fake, 1 << 40, None)
    assert st == m.MOE_ERR_UNSUPPORTED and "moe_quantize_fp8" in m.moe_last_error()
    # the shared expert's block scales are required
    st = lib.moe_layer(ctypes.byref(c), fake, None, ctypes.byref(w), fake, fake, fake, 1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG and "sh_gate" in m.moe_last_error()
    w.sh_gate = w.sh_up = w.sh_down = 0x100000
    st = lib.moe_layer(ctypes.byref(c), fake, None, ctypes.byref(w), fake, fake, fake, 1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG and "sh_s_gate" in m.moe_last_error()
    w.sh_s_gate = w.sh_s_up = w.sh_s_down = 0x100000
    st = lib.moe_layer(ctypes.byref(c), fake, None, ctypes.byref(w), ctypes.c_void_p(0x100008), fake, fake,
                       1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG and "aligned" in m.moe_last_error()
    # moe_quantize_fp8
    st = lib.moe_quantize_fp8(ctypes.byref(c), ctypes.c_void_p(0x100008), fake, fake, None)
    assert st == m.MOE_ERR_INVALID_ARG and "aligned" in m.moe_last_error()
    st = lib.moe_quantize_fp8(ctypes.byref(c), fake, None, fake, None)
    assert st == m.MOE_ERR_INVALID_ARG and "x_q" in m.moe_last_error()
    f8 = m.make_cfg(T=64, H=128, E=8, k=1, I=128, act_dtype=m.MOE_FP8_E4M3, y_dtype=m.MOE_BF16)
    assert lib.moe_quantize_fp8(ctypes.byref(f8), fake, fake, fake, None) == m.MOE_ERR_UNSUPPORTED
    st = lib.moe_quantize_fp8(ctypes.byref(c), fake, fake, ctypes.c_void_p(0x100002), None)
    assert st == m.MOE_ERR_INVALID_ARG and "x_scale" in m.moe_last_error()
    z = m.make_cfg(**dict(kw, T=0))
    assert lib.moe_quantize_fp8(ctypes.byref(z), None, None, None, None) == m.MOE_OK


def test_route_quantize_checks_arguments():
    """moe_route_quantize: bf16 x and H a multiple of 128, every pointer given
    and aligned, a workspace of the route's size; all refused before a launch."""
    lib = m._ffi.lib()
    fake = ctypes.c_void_p(0x100000)
    c = m.make_cfg(T=64, H=7168, E=256, k=8, I=2048, n_groups=8, topk_groups=4)
    need = m.moe_workspace_bytes(c, m.MOE_STAGE_ROUTE)

    def call(cfg, x=fake, w_r=fake, ids=fake, w=fake, xq=fake, xs=fake, ws=fake, n=need):
        return lib.moe_route_quantize(ctypes.byref(cfg), x, w_r, None, None, ids, w, xq, xs, ws, n, None)

    assert call(m.make_cfg(T=64, H=128, E=8, k=1, I=128, act_dtype=m.MOE_FP8_E4M3)) == m.MOE_ERR_UNSUPPORTED
    assert call(m.make_cfg(T=64, H=128, E=8, k=1, I=128, act_dtype=m.MOE_F32)) == m.MOE_ERR_UNSUPPORTED
    h = m.make_cfg(T=64, H=192, E=8, k=2, I=128)
    assert m.moe_validate(h) == m.MOE_OK
    assert call(h) == m.MOE_ERR_INVALID_ARG and "multiple of 128" in m.moe_last_error()
    for kw, name in ((dict(x=None), "x"), (dict(w_r=None), "w_router"), (dict(ids=None), "topk_ids"),
                     (dict(w=None), "topk_w"), (dict(xq=None), "x_q"), (dict(xs=None), "x_scale")):
        assert call(c, **kw) == m.MOE_ERR_INVALID_ARG and name in m.moe_last_error()
    odd8, odd4, odd2 = ctypes.c_void_p(0x100008), ctypes.c_void_p(0x100004), ctypes.c_void_p(0x100002)
    for kw, name in ((dict(x=odd8), "x"), (dict(w_r=odd8), "w_router"), (dict(xq=odd4), "x_q"),
                     (dict(xs=odd2), "x_scale")):
        assert call(c, **kw) == m.MOE_ERR_INVALID_ARG and "aligned" in m.moe_last_error()
        assert name in m.moe_last_error()
    assert call(c, ws=None) == m.MOE_ERR_WORKSPACE
    assert call(c, n=need - 1) == m.MOE_ERR_WORKSPACE
    assert call(m.make_cfg(T=0, H=7168, E=256, k=8, I=2048), ws=None, n=0) == m.MOE_OK


def test_status_strings():
    names = ["MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP"]
    for i, n in enumerate(names):
        assert m.moe_status_string(i) == n
    assert m.moe_status_string(99) == "MOE_ERR_UNKNOWN"


def test_max_rows_and_workspace_sizes():
    for mt in (0, 1, 16, 128):
        c = _dsv3(m_tile=mt)
        assert m.moe_max_rows(c) == 8192 * 8 + 256 * (max(mt, 1) - 1)
    c = _dsv3()
    ws = [m.moe_workspace_bytes(c, s) for s in range(4)]
    # the router's K-split partial logits: whole [T][E] fp32 copies
    assert ws[m.MOE_STAGE_ROUTE] % (8192 * 256 * 4) == 0 and 8192 * 256 * 4 <= ws[m.MOE_STAGE_ROUTE] <= 8 * 8192 * 256 * 4
    assert all(w % 256 == 0 for w in ws)
    # the layer workspace holds y_rows (fp32) and y_shared at least, plus the
    # h tile slots (one per possible M tile: up to rows / 288 + E + shared tiles);
    # a bf16 layer materialises no x_perm (its GEMM reads x through row_src)
    rows = 8192 * 8
    rows16 = rows + 256 * 15  # the layer pads expert segments to 16 rows
    slots = (rows16 + 287) // 288 + 256 + (8192 + 287) // 288 + 1
    y_bytes = rows16 * 7168 * 4 + 8192 * 7168 * 4
    assert y_bytes <= ws[m.MOE_STAGE_LAYER] < y_bytes + slots * 288 * 2048 * 2 + (64 << 20)
    assert ws[m.MOE_STAGE_FFN] >= rows * 2048 * 2  # h in bf16
    assert m.moe_workspace_bytes(c, 7) == ctypes.c_size_t(-1).value
    assert m.moe_ffn_workspace_bytes(c, rows) == ws[m.MOE_STAGE_FFN]
    assert m.moe_ffn_workspace_bytes(c, 10) < ws[m.MOE_STAGE_FFN]
    assert m.moe_ffn_workspace_bytes(c, -1) == ctypes.c_size_t(-1).value


def test_x_perm_sizes():
    c = _dsv3(m_tile=16)
    assert m.moe_x_perm_bytes(c) == m.moe_max_rows(c) * 7168 * 2
    t = _dsv3(m_tile=16, x_layout=m.MOE_LAYOUT_TILED)
    r16 = (m.moe_max_rows(t) + 15) // 16 * 16
    assert m.moe_x_perm_bytes(t) == (r16 // 16 + 8192 // 16) * (7168 // 32) * 1024
    # H not a multiple of 32: every 16-row band spans ceil(H / 32) KiB
    t = m.make_cfg(T=77, H=520, E=6, k=2, I=264, m_tile=32, x_layout=m.MOE_LAYOUT_TILED)
    r16 = (m.moe_max_rows(t) + 15) // 16 * 16
    assert m.moe_x_perm_bytes(t) == r16 // 16 * 17 * 1024
    assert m.moe_x_perm_bytes(_dsv3(x_layout=m.MOE_LAYOUT_INDEXED)) == 0
    assert m.moe_x_perm_bytes(_dsv3(x_layout=3)) == ctypes.c_size_t(-1).value


def test_entry_points_reject_bad_arguments_before_any_launch():
    c = m.make_cfg(T=16, H=64, E=8, k=2, I=64)
    lib = _ffi.lib()
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails its checks
    st = lib.moe_route(ctypes.byref(c), fake, fake, None, None, None, None, fake, fake, 1 << 20, None)
    assert st == m.MOE_ERR_INVALID_ARG and "topk_ids" in m.moe_last_error()
    st = lib.moe_route(ctypes.byref(c), fake, fake, None, None, None, fake, fake, None, 0, None)
    assert st == m.MOE_ERR_WORKSPACE
    st = lib.moe_route(ctypes.byref(c), fake, fake, None, None, None, fake, fake, ctypes.c_void_p(0x100010),
                       1 << 20, None)
    assert st == m.MOE_ERR_WORKSPACE and "aligned" in m.moe_last_error()
    st = lib.moe_route(ctypes.byref(c), fake, fake, None, None, None, fake, fake, fake, 16, None)
    assert st == m.MOE_ERR_WORKSPACE
    w = m.moe_weights(w_gate=0x100000, w_up=0x100000, w_down=None)
    st = lib.moe_grouped_ffn(ctypes.byref(c), 32, fake, None, fake, None, ctypes.byref(w), None, fake, None, fake,
                             1 << 30, None)
    assert st == m.MOE_ERR_INVALID_ARG and "w_down" in m.moe_last_error()
    w = m.moe_weights(w_gate=0x100000, w_up=0x100000, w_down=0x100000)
    st = lib.moe_grouped_ffn(ctypes.byref(c), 1 << 31, fake, None, fake, None, ctypes.byref(w), None, fake, None, fake,
                             1 << 30, None)
    assert st == m.MOE_ERR_INVALID_ARG and "n_rows_cap" in m.moe_last_error()
    st = lib.moe_grouped_ffn(ctypes.byref(c), 10**6, fake, None, fake, None, ctypes.byref(w), None, fake, None, fake,
                             1 << 20, None)
    assert st == m.MOE_ERR_WORKSPACE
    st = lib.moe_grouped_ffn(ctypes.byref(c), 32, fake, None, fake, None, ctypes.byref(w), None,
                             ctypes.c_void_p(0x100008), None, fake, 1 << 30, None)
    assert st == m.MOE_ERR_INVALID_ARG and "y_rows" in m.moe_last_error() and "aligned" in m.moe_last_error()
    ct = m.make_cfg(T=16, H=64, E=8, k=2, I=64, m_tile=16, x_layout=m.MOE_LAYOUT_TILED)
    st = lib.moe_grouped_ffn(ctypes.byref(ct), 32, fake, None, fake, None, ctypes.byref(w), None, fake, None, fake,
                             1 << 30, None)
    assert st == m.MOE_ERR_INVALID_ARG and "n_rows_cap" in m.moe_last_error()
    ci = m.make_cfg(T=16, H=64, E=8, k=2, I=64, m_tile=16, x_layout=m.MOE_LAYOUT_INDEXED)
    st = lib.moe_grouped_ffn(ctypes.byref(ci), 32, fake, None, fake, None, ctypes.byref(w), None, fake, None, fake,
                             1 << 30, None)
    assert st == m.MOE_ERR_INVALID_ARG and "row_src" in m.moe_last_error()
    st = lib.moe_combine(ctypes.byref(c), fake, None, fake, None, fake, None)
    assert st == m.MOE_ERR_INVALID_ARG
    st = lib.moe_layer(ctypes.byref(c), fake, None, ctypes.byref(w), fake, None, fake, 1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG and "out" in m.moe_last_error()
    cs = m.make_cfg(T=16, H=64, E=8, k=2, I=64, has_shared=True, I_shared=64)
    st = lib.moe_layer(ctypes.byref(cs), fake, None, ctypes.byref(w), fake, fake, fake, 1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG and "sh_gate" in m.moe_last_error()
    fp8 = m.make_cfg(T=16, H=128, E=8, k=2, I=128, act_dtype=m.MOE_FP8_E4M3, y_dtype=m.MOE_BF16)
    st = lib.moe_route(ctypes.byref(fp8), fake, fake, None, None, fake, fake, fake, fake, 1 << 20, None)
    assert st == m.MOE_ERR_UNSUPPORTED


def test_zero_tokens_enqueue_nothing():
    """T == 0 returns MOE_OK without a launch (fake pointers, no GPU here)."""
    c = m.make_cfg(T=0, H=64, E=8, k=2, I=64)
    lib = _ffi.lib()
    fake = ctypes.c_void_p(0x100000)
    w = m.moe_weights(w_gate=0x100000, w_up=0x100000, w_down=0x100000)
    ws = ctypes.c_void_p(0x100000)
    assert lib.moe_route(ctypes.byref(c), fake, fake, None, None, fake, fake, fake, None, 0, None) == m.MOE_OK
    assert lib.moe_permute(ctypes.byref(c), fake, None, fake, fake, fake, fake, fake, fake, None, ws, 1 << 20,
                           None) == m.MOE_OK
    assert lib.moe_combine(ctypes.byref(c), fake, fake, fake, None, fake, None) == m.MOE_OK
    assert lib.moe_layer(ctypes.byref(c), fake, None, ctypes.byref(w), fake, fake, ws, 1 << 20, None) == m.MOE_OK


def test_binding_refuses_host_tensors():
    import torch
    c = m.make_cfg(T=4, H=64, E=8, k=2, I=64)
    with pytest.raises(ValueError):
        m.moe_combine(c, torch.zeros(8, 64), torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2), None,
                      torch.zeros(4, 64))


def test_weight_table_host_addresses():
    """moe_weight_table writes, per layer and expert, the addresses of that
    expert's matrices in contiguous weights (fake addresses: nothing is
    dereferenced), the shared expert as entry E, scales for fp8 only; and the
    entry points check a table's own fields before any launch."""
    lib = _ffi.lib()
    E, H, I, Ish = 4, 256, 384, 128
    c = m.make_cfg(T=8, H=H, E=E, k=1, I=I, has_shared=True, I_shared=Ish)
    base = [0x10000000 * (i + 1) for i in range(12)]
    lay0 = m.moe_weights(w_gate=base[0], w_up=base[1], w_down=base[2], sh_gate=base[3], sh_up=base[4],
                         sh_down=base[5])
    lay1 = m.moe_weights(w_gate=base[6], w_up=base[7], w_down=base[8], sh_gate=base[9], sh_up=base[10],
                         sh_down=base[11])
    t = m.moe_weight_table(c, [lay0, lay1])
    G = E + 1
    assert len(t) == 2 * G * 6
    mat = I * H * 2
    for L, b in ((0, base[:6]), (1, base[6:])):
        for e in range(E):
            assert t[(L * G + e) * 6:(L * G + e + 1) * 6] == [b[0] + e * mat, b[1] + e * mat, b[2] + e * mat, 0, 0, 0]
        assert t[(L * G + E) * 6:(L * G + E + 1) * 6] == [b[3], b[4], b[5], 0, 0, 0]
    # tiled bf16: one expert's gate+up matrix is 2 * roundup(I, 128) rows in
    # groups of 64, each group ceil(H / 32) stages of 4 KiB; down: ceil(H / 64)
    # groups of ceil(I / 32) stages
    tl = m.moe_weights(w_gate=base[0], w_down=base[2], sh_gate=base[3], sh_down=base[5],
                       layout=m.MOE_LAYOUT_TILED)
    tt = m.moe_weight_table(c, [tl])
    m13 = (2 * ((I + 127) // 128 * 128) // 64) * ((H + 31) // 32) * 4096
    m2 = ((H + 63) // 64) * ((I + 31) // 32) * 4096
    assert E * (m13 + m2) + ((2 * Ish // 64) * (H // 32) + (H // 64) * (Ish // 32)) * 4096 == \
        m.moe_tiled_weights_bytes(c)
    for e in range(E):
        assert tt[e * 6:(e + 1) * 6] == [base[0] + e * m13, 0, base[2] + e * m2, 0, 0, 0]
    assert tt[E * 6:(E + 1) * 6] == [base[3], 0, base[5], 0, 0, 0]
    # fp8 experts: codes are bytes, one fp32 scale per 128 x 128 block
    f8 = m.make_cfg(T=8, H=H, E=E, k=1, I=I, w_dtype=m.MOE_FP8_E4M3)
    w8 = m.moe_weights(w_gate=base[0], w_up=base[1], w_down=base[2], s_gate=base[3], s_up=base[4],
                       s_down=base[5])
    t8 = m.moe_weight_table(f8, [w8])
    nsc = (I // 128) * (H // 128) * 4
    for e in range(E):
        assert t8[e * 6:(e + 1) * 6] == [base[0] + e * I * H, base[1] + e * I * H, base[2] + e * I * H,
                                         base[3] + e * nsc, base[4] + e * nsc, base[5] + e * nsc]
    # tiled e4m3: the merged gate+up matrix (2 I rows) and the down matrix keep
    # the row-major byte counts; the scale entries are the caller's arrays
    assert m.moe_tiled_weights_bytes(f8) == E * 3 * I * H
    f8s = m.make_cfg(T=8, H=H, E=E, k=1, I=I, w_dtype=m.MOE_FP8_E4M3, has_shared=True, I_shared=Ish)
    # each of the four matrices starts on a 256-byte boundary
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert m.moe_tiled_weights_bytes(f8s) == al(E * 2 * I * H) + al(E * I * H) + al(2 * Ish * H) + al(Ish * H)
    t8t = m.moe_weight_table(f8, [m.moe_weights(w_gate=base[0], w_down=base[2], s_gate=base[3], s_up=base[4],
                                                s_down=base[5], layout=m.MOE_LAYOUT_TILED)])
    for e in range(E):
        assert t8t[e * 6:(e + 1) * 6] == [base[0] + e * 2 * I * H, 0, base[2] + e * I * H,
                                          base[3] + e * nsc, base[4] + e * nsc, base[5] + e * nsc]
    # MXFP4 weights have no tiled layout
    f4 = m.make_cfg(T=8, H=H, E=E, k=1, I=I, w_dtype=m.MOE_FP4_E2M1)
    assert m.moe_tiled_weights_bytes(f4) == ctypes.c_size_t(-1).value
    assert "bf16 or e4m3" in m.moe_last_error()
    # refusals
    f32 = m.make_cfg(T=8, H=H, E=E, k=1, I=I, act_dtype=m.MOE_F32)
    with pytest.raises(m.MoeError) as ex:
        m.moe_weight_table(f32, [lay0])
    assert ex.value.status == m.MOE_ERR_UNSUPPORTED
    bad = m.moe_weights(w_gate=base[0], w_up=base[1], w_down=base[2], table=0x2000, layer=0x3000, n_layers=1)
    with pytest.raises(m.MoeError) as ex:
        m.moe_weight_table(c, [bad])
    assert ex.value.status == m.MOE_ERR_INVALID_ARG
    out = (ctypes.c_void_p * 12)()
    assert lib.moe_weight_table(ctypes.byref(c), (m.moe_weights * 1)(lay0), 0, out) == m.MOE_ERR_INVALID_ARG
    # a table call is checked on its own fields, the contiguous pointers ignored
    fake = ctypes.c_void_p(0x100000)
    cf = m.make_cfg(T=8, H=H, E=E, k=1, I=I)
    for w, code, msg in ((m.moe_weights(table=0x100000, n_layers=1), m.MOE_ERR_INVALID_ARG, "layer"),
                         (m.moe_weights(table=0x100000, layer=0x100000, n_layers=0), m.MOE_ERR_INVALID_ARG,
                          "n_layers"),
                         (m.moe_weights(table=0x100004, layer=0x100000, n_layers=1), m.MOE_ERR_INVALID_ARG,
                          "table")):
        st = lib.moe_grouped_ffn(ctypes.byref(cf), 32, fake, None, fake, None, ctypes.byref(w), None, fake, None,
                                 fake, 1 << 30, None)
        assert st == code and msg in m.moe_last_error(), m.moe_last_error()
    w = m.moe_weights(table=0x100000, layer=0x100000, n_layers=1)
    cf32 = m.make_cfg(T=8, H=H, E=E, k=1, I=I, act_dtype=m.MOE_F32)
    st = lib.moe_grouped_ffn(ctypes.byref(cf32), 32, fake, None, fake, None, ctypes.byref(w), None, fake, None,
                             fake, 1 << 30, None)
    assert st == m.MOE_ERR_UNSUPPORTED
    st = lib.moe_tile_weights(ctypes.byref(cf), ctypes.byref(m.moe_weights(w_gate=0x100000, w_up=0x100000,
                                                                              w_down=0x100000, table=0x100000,
                                                                              layer=0x100000, n_layers=1)),
                              fake, 1 << 40, ctypes.byref(m.moe_weights()), None)
    assert st == m.MOE_ERR_INVALID_ARG


def test_mxfp4_cfg_and_table():
    """MXFP4 expert weights: accepted with e4m3 rows (grouped FFN) or bf16
    activations (layer), with H, I multiple of 128; refused with fp32 or bf16
    rows in the grouped FFN sense (act == w required otherwise); the table
    helper steps half a byte per element and one scale byte per 32."""
    kw = dict(T=64, H=7168, E=8, k=2, I=2048)
    c = m.make_cfg(**kw, act_dtype=m.MOE_FP8_E4M3, w_dtype=m.MOE_FP4_E2M1, y_dtype=m.MOE_BF16)
    assert m.moe_validate(c) == m.MOE_OK
    lay = m.make_cfg(**kw, act_dtype=m.MOE_BF16, w_dtype=m.MOE_FP4_E2M1, has_shared=True, I_shared=1024)
    assert m.moe_validate(lay) == m.MOE_OK
    assert m.moe_validate(m.make_cfg(**kw, act_dtype=m.MOE_F32, w_dtype=m.MOE_FP4_E2M1)) == m.MOE_ERR_UNSUPPORTED
    assert m.moe_validate(m.make_cfg(**dict(kw, I=2048 + 64), act_dtype=m.MOE_FP8_E4M3,
                                     w_dtype=m.MOE_FP4_E2M1)) == m.MOE_ERR_INVALID_ARG
    assert m.moe_validate(m.make_cfg(**kw, act_dtype=m.MOE_FP4_E2M1)) == m.MOE_ERR_INVALID_ARG
    assert m.moe_validate(m.make_cfg(**kw, w_dtype=7)) == m.MOE_ERR_INVALID_ARG
    # the scales are required
    lib = _ffi.lib()
    fake = ctypes.c_void_p(0x100000)
    w = m.moe_weights(w_gate=0x100000, w_up=0x100000, w_down=0x100000)
    st = lib.moe_grouped_ffn(ctypes.byref(c), 64, fake, fake, fake, None, ctypes.byref(w), None, fake, None, fake,
                             1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG and "s_gate" in m.moe_last_error()
    E, H, I = 3, 256, 384
    f4 = m.make_cfg(T=8, H=H, E=E, k=1, I=I, act_dtype=m.MOE_FP8_E4M3, w_dtype=m.MOE_FP4_E2M1)
    base = [0x10000000 * (i + 1) for i in range(6)]
    t = m.moe_weight_table(f4, [m.moe_weights(w_gate=base[0], w_up=base[1], w_down=base[2], s_gate=base[3],
                                              s_up=base[4], s_down=base[5])])
    for e in range(E):
        assert t[e * 6:(e + 1) * 6] == [base[0] + e * I * H // 2, base[1] + e * I * H // 2, base[2] + e * I * H // 2,
                                        base[3] + e * I * H // 32, base[4] + e * I * H // 32,
                                        base[5] + e * I * H // 32]


def test_combine_route_permute_layer_check_pointers():
    """The shared expert's rows are required when has_shared; the vector
    loads and stores of combine, route, permute and the layer need 16-byte
    aligned rows (checked before any launch)."""
    lib = _ffi.lib()
    fake = ctypes.c_void_p(0x100000)
    odd = ctypes.c_void_p(0x100008)
    cs = m.make_cfg(T=16, H=64, E=8, k=2, I=64, has_shared=True, I_shared=64)
    st = lib.moe_combine(ctypes.byref(cs), fake, fake, fake, None, fake, None)
    assert st == m.MOE_ERR_INVALID_ARG and "y_shared" in m.moe_last_error()
    c = m.make_cfg(T=16, H=64, E=8, k=2, I=64)
    for args, name in (((odd, fake, fake, None, fake), "y_rows"), ((fake, fake, fake, odd, fake), "y_shared"),
                       ((fake, fake, fake, None, odd), "out")):
        st = lib.moe_combine(ctypes.byref(c), *args, None)
        assert st == m.MOE_ERR_INVALID_ARG and name in m.moe_last_error() and "aligned" in m.moe_last_error()
    st = lib.moe_route(ctypes.byref(c), odd, fake, None, None, None, fake, fake, fake, 1 << 20, None)
    assert st == m.MOE_ERR_INVALID_ARG and "x" in m.moe_last_error() and "aligned" in m.moe_last_error()
    st = lib.moe_route(ctypes.byref(c), fake, odd, None, None, None, fake, fake, fake, 1 << 20, None)
    assert st == m.MOE_ERR_INVALID_ARG and "w_router" in m.moe_last_error()
    st = lib.moe_permute(ctypes.byref(c), odd, None, fake, fake, fake, fake, fake, fake, None, fake, 1 << 20, None)
    assert st == m.MOE_ERR_INVALID_ARG and "aligned" in m.moe_last_error()
    st = lib.moe_permute(ctypes.byref(c), fake, None, fake, fake, fake, fake, fake, odd, None, fake, 1 << 20, None)
    assert st == m.MOE_ERR_INVALID_ARG and "x_perm" in m.moe_last_error()
    w = m.moe_weights(w_gate=0x100000, w_up=0x100000, w_down=0x100000)
    st = lib.moe_layer(ctypes.byref(c), fake, None, ctypes.byref(w), odd, fake, fake, 1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG and "aligned" in m.moe_last_error()
    st = lib.moe_layer(ctypes.byref(c), fake, None, ctypes.byref(w), fake, odd, fake, 1 << 40, None)
    assert st == m.MOE_ERR_INVALID_ARG and "out" in m.moe_last_error()


def test_layer_dispatches_a_large_x_into_x_perm():
    """The layer's GEMM1 reads x through one buffer descriptor (32-bit byte
    offsets): from 2 GiB of x on, the layer dispatches the rows into a tiled
    x_perm instead (bf16), or a row-major one with its scales (e4m3 tokens of
    low-precision experts), and its workspace grows by that much."""
    def ws(T, **kw):
        return m.moe_workspace_bytes(_dsv3(T=T, **kw), m.MOE_STAGE_LAYER)

    below, above = (2 ** 31 - 1) // (7168 * 2), (2 ** 31) // (7168 * 2) + 1
    tiled = m.moe_x_perm_bytes(_dsv3(T=above, m_tile=16, x_layout=m.MOE_LAYOUT_TILED))
    assert tiled > above * 8 * 7168 * 2
    per_token = ws(below) / below
    assert ws(below) < below * per_token * 1.01
    assert ws(above) >= tiled + above * per_token * 0.99
    fp8 = dict(w_dtype=m.MOE_FP8_E4M3, y_dtype=m.MOE_BF16)
    below8, above8 = (2 ** 31 - 1) // 7168, (2 ** 31) // 7168 + 1
    rows = m.moe_max_rows(_dsv3(T=above8, m_tile=16))
    assert ws(above8, **fp8) - ws(below8, **fp8) * above8 / below8 >= rows * 7168 * 0.99


def test_permute_noalloc_checks_before_any_launch():
    """The allocation-free permute refuses a batch whose per-block counts
    exceed its static scratch (2 * ceil(T / 256) * E <= 2^20) and bad pointers
    before it touches the HIP runtime; T = 0 enqueues nothing."""
    lib = _ffi.lib()
    fake = ctypes.c_void_p(0x100000)
    big = m.make_cfg(T=524288 + 256, H=64, E=256, k=8, I=64)
    st = lib.moe_permute_noalloc(ctypes.byref(big), fake, None, fake, fake, fake, fake, fake, fake, None, None)
    assert st == m.MOE_ERR_UNSUPPORTED and "moe_permute_noalloc" in m.moe_last_error()
    c = m.make_cfg(T=16, H=64, E=8, k=2, I=64)
    st = lib.moe_permute_noalloc(ctypes.byref(c), fake, None, None, fake, fake, fake, fake, fake, None, None)
    assert st == m.MOE_ERR_INVALID_ARG and "topk_ids" in m.moe_last_error()
    st = lib.moe_permute_noalloc(ctypes.byref(c), ctypes.c_void_p(0x100008), None, fake, fake, fake, fake, fake,
                                 fake, None, None)
    assert st == m.MOE_ERR_INVALID_ARG and "aligned" in m.moe_last_error()
    z = m.make_cfg(T=0, H=64, E=8, k=2, I=64)
    assert lib.moe_permute_noalloc(ctypes.byref(z), fake, None, fake, fake, fake, fake, fake, fake, None,
                                   None) == m.MOE_OK
    # the largest batch it holds at E = 256
    ok = m.make_cfg(T=524288, H=64, E=256, k=8, I=64)
    assert 2 * ((524288 + 255) // 256) * 256 == 1 << 20 and m.moe_validate(ok) == m.MOE_OK
