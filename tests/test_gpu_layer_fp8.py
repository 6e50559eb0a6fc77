"""GPU parity of fp8 experts: moe_quantize_fp8, the fused route and
quantisation (moe_route_quantize) and moe_layer with bf16 activations and e4m3
expert weights, against the oracle.

The per-token quantisation is decided in fp32 on both sides from the same bf16
values, so its codes and scales are compared bit for bit.  The layer is
compared with the oracle composed step by step: routing on the same margin
cases as the bf16 layer tests (ids bit-exact), the oracle's quantisation of x,
each chosen expert's fp8 block-scaled SwiGLU FFN on its token rows (the shared
expert on every token), then the weighted combine.  Bound: max|err| / rms(ref)
<= 4e-2, the fp8 tolerance; the rms of the error is also held under 1e-2."""
import math

import numpy as np
import pytest
import torch

import expert_layer_amd as moe
import oracle
import synth
from tests._cases import cover_tokens, dev, lib_cfg, rel_err, route_kw, router_case
from tests._np import e4m3_f64, f64, to_np

pytestmark = pytest.mark.gpu


def test_quantize_fp8_is_bit_exact():
    T, H = 131, 7168
    g = torch.Generator(device="cpu").manual_seed(11)
    x = torch.randn((T, H), generator=g) * torch.exp(2.0 * torch.randn((T, H // 128, 1), generator=g)).repeat(
        1, 1, 128).view(T, H)
    x[3, :128] = 0.0                       # an all-zero block: scale 1, zero codes
    x[5, 128:256] *= 1e-30                 # a block of tiny (normal fp32) values: a tiny scale
    # exact round-to-nearest-even ties: e4m3 midpoints times 2^3, with 448 * 2^3 the block maximum
    mids = np.array([(a + b) / 2 for a, b in zip(e4m3_f64(np.arange(0, 0x7E)), e4m3_f64(np.arange(1, 0x7F)))])
    blk = np.resize(mids, 128) * 8.0
    blk[0] = 448.0 * 8.0
    x[9, 512:640] = torch.from_numpy(blk)
    x[9, 640:768] = -torch.from_numpy(blk)
    x[11, 768:896] = 1e30                  # a constant block of large values: every code 448
    xb = x.to(torch.bfloat16).to(dev())
    c = moe.make_cfg(T=T, H=H, E=8, k=1, I=128)
    xq = torch.full((T, H), 0xFF, dtype=torch.uint8, device=dev())
    xs = torch.full((T, H // 128), float("nan"), device=dev())
    moe.moe_quantize_fp8(c, xb, xq, xs)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows_e4m3(to_np(xb))
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)


def _route_quantize(c, x, w_r, bias):
    T, H, E, k = c.T, c.H, c.E, c.k
    ids = torch.full((T, k), -7, dtype=torch.int32, device=dev())
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev())
    lg = torch.full((T, E), float("nan"), dtype=torch.float32, device=dev())
    xq = torch.full((T, H), 0xFF, dtype=torch.uint8, device=dev())
    xs = torch.full((T, H // 128), float("nan"), device=dev())
    moe.moe_route_quantize(c, x, w_r, bias, lg, ids, w, xq, xs, moe.workspace(c, moe.MOE_STAGE_ROUTE, dev()))
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy(), xq.cpu().numpy(), xs.cpu().numpy()


def _route_on(c, x, w_r, bias, logits_in=None):
    T, E, k = c.T, c.E, c.k
    ids = torch.full((T, k), -7, dtype=torch.int32, device=dev())
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev())
    lg = torch.full((T, E), float("nan"), dtype=torch.float32, device=dev())
    ws = None if logits_in is not None else moe.workspace(c, moe.MOE_STAGE_ROUTE, dev())
    moe.moe_route(c, x, w_r, bias, logits_in, lg, ids, w, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


@pytest.mark.parametrize("name,T", [
    ("c3_dsv3_bf16", 1000),
    ("c4_qwen3_skew_bf16", 777),
    ("c3_dsv3_bf16", None),          # full size, T = 8192
])
def test_route_quantize_matches_oracle(name, T):
    """The fused route: ids bit-exact and weights as moe_route against the
    oracle (margin cases), codes and scales bit-exact against the oracle's
    quantiser, and -- the K splits being whole 128-column blocks here too --
    the same logits, ids and weights as moe_route bit for bit."""
    s = synth.config(name)
    rc = router_case(s, T)
    T = rc["x"].shape[0]
    c = lib_cfg(s, T=T)
    ids, w, lg, xq, xs = _route_quantize(c, rc["x"], rc["w_r"], rc["bias"])
    ref_ids, ref_w = oracle.route_select(rc["logits"], s.k, renormalize=s.renormalize,
                                         routed_scale=s.routed_scale, bias=rc["bh"], **route_kw(s))
    scale = np.sqrt(np.mean(rc["logits"].astype(np.float64) ** 2))
    assert np.max(np.abs(lg - rc["logits"])) <= 2e-5 * scale
    assert np.array_equal(ids, ref_ids)
    assert np.max(np.abs(w - ref_w)) <= 1e-5 * s.routed_scale
    q_ref, s_ref = oracle.quantize_rows_e4m3(rc["xh"])
    assert np.array_equal(xs, s_ref)
    assert np.array_equal(xq, q_ref)
    ids2, w2, lg2 = _route_on(c, rc["x"], rc["w_r"], rc["bias"])
    assert np.array_equal(lg2, lg) and np.array_equal(ids2, ids) and np.array_equal(w2, w)


@pytest.mark.parametrize("T,H,E,k,groups", [
    (131, 7168, 64, 4, 1),      # the quantiser's edge blocks; 2 token blocks, 8 K splits
    (200, 1024, 512, 8, 8),     # two expert blocks: only the first quantises
    (77, 640, 96, 6, 1),        # 3 K splits of whole blocks (256, 256, 128 columns): other boundaries
    (1, 128, 8, 2, 1),          # one token, one block
])
def test_route_quantize_edge_shapes(T, H, E, k, groups):
    """Shapes the workloads do not reach: codes and scales bit-exact against the
    oracle's quantiser (with all-zero, tiny, tie and saturating blocks), logits
    within fp32 accumulation of the oracle's, and the ids and weights exactly
    those of moe_route's selection on the fused call's own logits."""
    g = torch.Generator(device="cpu").manual_seed(1000 + T)
    x = torch.randn((T, H), generator=g) * torch.exp(2.0 * torch.randn((T, H // 128, 1), generator=g)).repeat(
        1, 1, 128).view(T, H)
    if T > 11 and H >= 896:
        x[3, :128] = 0.0
        x[5, 128:256] *= 1e-30
        mids = np.array([(a + b) / 2 for a, b in zip(e4m3_f64(np.arange(0, 0x7E)), e4m3_f64(np.arange(1, 0x7F)))])
        blk = np.resize(mids, 128) * 8.0
        blk[0] = 448.0 * 8.0
        x[9, 512:640] = torch.from_numpy(blk)
        x[9, 640:768] = -torch.from_numpy(blk)
        x[11, 768:896] = 1e30
    xb = x.to(torch.bfloat16)
    w_r = (torch.randn((E, H), generator=g) * H ** -0.5).to(torch.bfloat16)
    c = moe.make_cfg(T=T, H=H, E=E, k=k, I=128, n_groups=groups, topk_groups=min(groups, 4))
    ids, w, lg, xq, xs = _route_quantize(c, xb.to(dev()), w_r.to(dev()), None)
    xh = to_np(xb)
    q_ref, s_ref = oracle.quantize_rows_e4m3(xh)
    assert np.array_equal(xs, s_ref)
    assert np.array_equal(xq, q_ref)
    ref = oracle.router_logits(xh, to_np(w_r))
    fin = np.isfinite(ref)
    # fp32 sums of exact bf16 products: far inside 1e-4 of sum |x w|, while a
    # 128-column block lost or counted twice moves a logit by about 128 / H of it
    mag = np.abs(f64(xb)) @ np.abs(f64(w_r)).T
    assert np.all((np.abs(lg.astype(np.float64) - ref) <= 1e-4 * mag)[fin])
    ids2, w2, _ = _route_on(c, None, None, None, torch.from_numpy(lg).to(dev()))
    assert np.array_equal(ids2, ids) and np.array_equal(w2, w)


_W8 = {}
_W8 = {}


def _fp8_weights(s):
    """Routed fp8 experts stacked on the device ([E][I][H] codes, [E][I/128][H/128]
    scales, ...) and the shared expert's, drawn by synth (block scales with the
    survey's jitter)."""
    key = (s.name, s.E, s.I, s.H, s.I_shared, s.seed)
    if key not in _W8:
        _W8.clear()
        torch.cuda.empty_cache()
        d = dev()
        wg = torch.empty((s.E, s.I, s.H), dtype=torch.uint8, device=d)
        wu, wd = torch.empty_like(wg), torch.empty((s.E, s.H, s.I), dtype=torch.uint8, device=d)
        sg = torch.empty((s.E, s.I // 128, s.H // 128), device=d)
        su, sd = torch.empty_like(sg), torch.empty((s.E, s.H // 128, s.I // 128), device=d)
        for e in range(s.E):
            g, gs, u, us, dn, ds = synth.fp8_expert_weights(s, e, d)
            wg[e], sg[e], wu[e], su[e], wd[e], sd[e] = g, gs, u, us, dn, ds
        sh = None
        if s.shared:
            sh = synth.fp8_expert_weights(s.with_(I=s.I_shared), s.E, d)
        _W8[key] = ((wg, sg, wu, su, wd, sd), sh)
    return _W8[key]


def _oracle_fp8_layer(s, rc, w8):
    (wg, sg, wu, su, wd, sd), sh = w8
    T, k = rc["xh"].shape[0], s.k
    ids, w = oracle.route_select(rc["logits"], k, renormalize=s.renormalize, routed_scale=s.routed_scale,
                                 bias=rc["bh"], **route_kw(s))
    xq, xs = oracle.quantize_rows_e4m3(rc["xh"])
    y_rows = np.zeros((T * k, s.H))
    for e in np.unique(ids):
        ti, j = np.nonzero(ids == e)
        y_rows[ti * k + j] = oracle.expert_ffn_fp8(xq[ti], xs[ti], to_np(wg[e]), to_np(sg[e]), to_np(wu[e]),
                                                   to_np(su[e]), to_np(wd[e]), to_np(sd[e]))
    y_sh = None
    if sh is not None:
        y_sh = oracle.expert_ffn_fp8(xq, xs, *(to_np(t) for t in sh))
    tok_row = np.arange(T * k, dtype=np.int32).reshape(T, k)
    return oracle.combine(y_rows, tok_row, w, y_sh)


def _small_shape():
    return synth.config("c3_dsv3_bf16").with_(H=512, I=256, E=16, k=4, n_groups=4, topk_groups=2, I_shared=384)


@pytest.mark.parametrize("shape,T,ydt,tiled", [
    ("small", 77, moe.MOE_F32, False),
    ("small", 77, moe.MOE_BF16, False),
    ("small", 77, moe.MOE_BF16, True),   # weights in the tiled e4m3 layout (routed and shared)
    ("c3", 24, moe.MOE_BF16, False),     # DeepSeek-V3 dimensions: 256 fp8 experts and the shared one
    ("c3", 24, moe.MOE_BF16, True),
    ("c4", 48, moe.MOE_BF16, False),     # softmax routing skewed by a Zipf logit bias, 128 experts, no shared
])
def test_layer_fp8_experts_matches_oracle(shape, T, ydt, tiled):
    s = {"small": _small_shape, "c3": lambda: synth.config("c3_dsv3_bf16"),
         "c4": lambda: synth.config("c4_qwen3_skew_bf16")}[shape]()
    rc = router_case(s, T)
    w8 = _fp8_weights(s)
    ref = _oracle_fp8_layer(s, rc, w8)
    (wg, sg, wu, su, wd, sd), sh = w8
    c = lib_cfg(s, T=T, y_dtype=ydt, out_dtype=moe.MOE_F32)
    c.w_dtype = moe.MOE_FP8_E4M3
    sh = sh if sh is not None else (None,) * 6
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd,
                    sh_gate=sh[0], sh_up=sh[2], sh_down=sh[4], sh_s_gate=sh[1], sh_s_up=sh[3], sh_s_down=sh[5])
    keep = None
    if tiled:
        w, keep = moe.tile_weights(c, w, dev())
    out = torch.full((T, s.H), float("nan"), device=dev())
    ws = moe.workspace(c, moe.MOE_STAGE_LAYER, dev())
    moe.moe_layer(c, rc["w_r"], rc["bias"], w, rc["x"], out, ws)
    torch.cuda.synchronize()
    del keep
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= 4e-2
    rms = math.sqrt(float(np.mean(ref ** 2)))
    assert math.sqrt(float(np.mean((got - ref) ** 2))) / rms <= 1e-2


def _u8(t):
    return t.detach().contiguous().cpu().numpy().astype(np.uint8)


@pytest.mark.parametrize("wfmt", ["e4m3-tiled", "e4m3", "mxfp4"])
def test_layer_lowp_experts_full_size_sampled(wfmt):
    """The benchmarked configuration: the c3 layer (T = 8192, 256 routed
    experts and the shared one) with e4m3 experts (tiled, as timed, or
    row-major) or MXFP4 experts, bf16 expert outputs.  Routing is checked for every token; the output on at least 512
    seeded tokens covering every expert with routed rows (with the first, the
    last, and tokens of the hottest and coldest experts) against the oracle
    composed step by step, to the bounds above."""
    s = synth.config("c3_dsv3_bf16")
    d = dev()
    _W8.clear()
    torch.cuda.empty_cache()
    rc = router_case(s)
    T = s.T
    gen = synth.mxfp4_expert_weights if wfmt == "mxfp4" else synth.fp8_expert_weights
    wq = [gen(s, e, d) for e in range(s.E)]
    stack = [torch.stack([w[i] for w in wq]) for i in range(6)]
    sh = gen(s.with_(I=s.I_shared), s.E, d)
    c = lib_cfg(s, T=T, y_dtype=moe.MOE_BF16, out_dtype=moe.MOE_F32)
    c.w_dtype = moe.MOE_FP4_E2M1 if wfmt == "mxfp4" else moe.MOE_FP8_E4M3
    wg, sg, wu, su, wd, sd = stack
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd, sh_gate=sh[0], sh_up=sh[2], sh_down=sh[4],
                    sh_s_gate=sh[1], sh_s_up=sh[3], sh_s_down=sh[5])
    keep = None
    if wfmt == "e4m3-tiled":
        w, keep = moe.tile_weights(c, w, d)
    out = torch.full((T, s.H), float("nan"), device=d)
    ws = moe.workspace(c, moe.MOE_STAGE_LAYER, d)
    moe.moe_layer(c, rc["w_r"], rc["bias"], w, rc["x"], out, ws)
    torch.cuda.synchronize()
    del ws, keep
    ids, tw = oracle.route_select(rc["logits"], s.k, renormalize=s.renormalize, routed_scale=s.routed_scale,
                                  bias=rc["bh"], **route_kw(s))
    toks = cover_tokens(ids, T, s.E, 512, s.seed + 3)
    xq, xs = oracle.quantize_rows_e4m3(rc["xh"][toks])
    ffn = oracle.expert_ffn_mxfp4 if wfmt == "mxfp4" else oracle.expert_ffn_fp8
    conv = _u8 if wfmt == "mxfp4" else (lambda t: to_np(t))
    y = np.zeros((len(toks), s.k, s.H))
    sub = ids[toks]
    for e in np.unique(sub):
        r, j = np.nonzero(sub == e)
        y[r, j] = ffn(xq[r], xs[r], *(conv(t) for t in wq[e]))
    y_sh = ffn(xq, xs, *(conv(t) for t in sh))
    ref = np.einsum("tj,tjh->th", tw[toks].astype(np.float64), y) + y_sh
    got = out[torch.as_tensor(toks, device=d)].cpu().numpy()
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    err_rms = math.sqrt(float(np.mean((got - ref) ** 2))) / math.sqrt(float(np.mean(ref ** 2)))
    print(f"{wfmt} experts: {len(toks)} tokens, max|err|/rms {err:.3e}, rms(err)/rms {err_rms:.3e}")
    assert err <= 4e-2 and err_rms <= 1e-2, (err, err_rms)
