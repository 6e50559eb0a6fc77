"""Pins of the oracle to results fixed independently of it.

Each test checks one oracle function against something other than the oracle:
a library routine (numpy fp64 matmul, numpy's stable sort, torch's bf16 and
float8_e4m3fn casts), a closed form, an invariant of the definition, brute
force over all subsets on tiny inputs, or a printed value of a published
format specification (tests/golden/).  A plausible slip in the oracle -- a
dropped term, a wrong sign or index, a transposed operand, a wrong tie rule --
fails at least one of them.  No GPU is needed.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._np import e4m3_f64, f64, to_np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ formats

def test_e4m3_decode_matches_spec_values():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_ocp.json")))
    for code, val in g["values"].items():
        got = float(oracle.e4m3_to_f64([int(code, 16)])[0])
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)
    for code in g["nan"]:
        assert math.isnan(float(oracle.e4m3_to_f64([int(code, 16)])[0]))


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f64(codes)
    ref = e4m3_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 100, 2000), rng.uniform(-2**-6, 2**-6, 2000),
        # every midpoint between neighbouring positive codes, both signs
        0.5 * (e4m3_f64(np.arange(0, 126)) + e4m3_f64(np.arange(1, 127))),
        -0.5 * (e4m3_f64(np.arange(0, 126)) + e4m3_f64(np.arange(1, 127))),
        np.array([448.0, 449.0, 463.9, 464.0, 1e6, -1e6, 0.0]),
    ]).astype(np.float32).astype(np.float64)
    got = oracle.e4m3_rne_sat(v)
    ref = to_np(torch.tensor(np.clip(v, -448, 448), dtype=torch.float32).to(torch.float8_e4m3fn))
    # torch keeps the sign of a negative value that rounds to zero (0x80); the
    # oracle returns +0 there: both decode to zero.
    same = (got == ref) | ((e4m3_f64(got) == 0) & (e4m3_f64(ref) == 0))
    assert same.all(), v[~same][:10]


def test_bf16_rounding_golden_and_torch():
    g = json.load(open(os.path.join(GOLDEN, "bf16_rne.json")))
    for src, dst, _ in g["cases"]:
        f = np.array([int(src, 16)], dtype=np.uint32).view(np.float32)[0]
        assert int(oracle.bf16_rne([float(f)])[0]) == int(dst, 16), (src, dst)
    rng = np.random.default_rng(1)
    v = rng.normal(0, 3, 5000).astype(np.float32)
    got = oracle.bf16_rne(v.astype(np.float64))
    ref = to_np(torch.tensor(v).to(torch.bfloat16))
    assert np.array_equal(got, ref)
    bits = rng.integers(0, 2**16, 3000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    ref = f64(torch.tensor(bits.view(np.int16)).view(torch.bfloat16))
    assert np.array_equal(oracle.bf16_to_f64(bits), ref)


def test_bf16_round_array_matches_torch_casts():
    """bf16_round (the stored value of a bf16 activation) against torch's own
    fp64 -> fp32 -> bf16 casts, on values of every magnitude and on the golden
    halfway cases."""
    rng = np.random.default_rng(3)
    v = rng.normal(0, 1, 20000) * np.exp(rng.normal(0, 8, 20000))
    g = json.load(open(os.path.join(GOLDEN, "bf16_rne.json")))
    half = np.array([np.array([int(src, 16)], dtype=np.uint32).view(np.float32)[0] for src, _, _ in g["cases"]],
                    dtype=np.float64)
    v = np.concatenate([v, half, -half, [0.0, -0.0]])
    ref = torch.tensor(v, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(v.reshape(2, -1)).reshape(-1)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ router

def _bf16(rng, shape, std=1.0):
    return to_np(torch.tensor(rng.normal(0, std, shape), dtype=torch.float32).to(torch.bfloat16))


def test_router_logits_match_numpy_matmul():
    rng = np.random.default_rng(2)
    x = _bf16(rng, (37, 96))
    w = _bf16(rng, (11, 96), 1 / math.sqrt(96))
    got = oracle.router_logits(x, w)
    ref = (oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(w).T).astype(np.float32)
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(got - ref) <= ulp)
    xf = rng.normal(0, 1, (5, 33)).astype(np.float32)
    wf = rng.normal(0, 1, (4, 33)).astype(np.float32)
    ref = (xf.astype(np.float64) @ wf.astype(np.float64).T).astype(np.float32)
    assert np.all(np.abs(oracle.router_logits(xf, wf) - ref) <= np.spacing(np.abs(ref)))


def _keys_py(l, score, bias):
    """Selection keys written from the definition with Python floats."""
    E = len(l)
    b = [0.0] * E if bias is None else [float(v) for v in bias]
    if score == oracle.SOFTMAX:
        return [float(np.float32(float(l[e]) + b[e])) for e in range(E)]
    return [float(np.float32(1.0 / (1.0 + math.exp(-float(l[e]))) + b[e])) for e in range(E)]


def _raw_py(l, score, bias):
    E = len(l)
    if score == oracle.SOFTMAX:
        z = [float(np.float32(float(l[e]) + (0.0 if bias is None else float(bias[e])))) for e in range(E)]
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        s = sum(ex)
        return [v / s for v in ex]
    return [1.0 / (1.0 + math.exp(-float(l[e]))) for e in range(E)]


def _beats(key, i, j):
    """i precedes j: larger key, or equal key and lower index."""
    return key[i] > key[j] or (key[i] == key[j] and i < j)


def _brute_route(l, k, score, G, KG, gscore_kind, renorm, scale, bias):
    """Enumerate every group subset and every expert subset; keep the unique
    subset whose members all precede every non-member."""
    E = len(l)
    key = _keys_py(l, score, bias)
    gs = E // G
    gsc = []
    for g in range(G):
        ks = sorted((key[e] for e in range(g * gs, (g + 1) * gs)), reverse=True)
        if gscore_kind == oracle.MAX or gs == 1:
            gsc.append(ks[0])
        else:
            gsc.append(float(np.float32(ks[0] + ks[1])))
    kept = [S for S in itertools.combinations(range(G), KG)
            if all(_beats(gsc, i, j) for i in S for j in range(G) if j not in S)]
    assert len(kept) == 1
    allowed = [e for e in range(E) if e // gs in kept[0]]
    chosen = [S for S in itertools.combinations(allowed, k)
              if all(_beats(key, i, j) for i in S for j in allowed if j not in S)]
    assert len(chosen) == 1
    order = sorted(chosen[0], key=lambda e: (-key[e], e))
    raw = _raw_py(l, score, bias)
    tot = sum(raw[e] for e in order)
    w = [(raw[e] / tot if renorm else raw[e]) * scale for e in order]
    return order, w


@pytest.mark.parametrize("case", range(40))
def test_route_select_matches_brute_force(case):
    rng = np.random.default_rng(100 + case)
    G = [1, 2, 3, 4][case % 4]
    gs = [1, 2, 3][case % 3]
    E = G * gs
    if E < 2:
        G, gs, E = 2, 3, 6
    KG = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, min(4, KG * gs) + 1))
    score = case % 2
    gkind = (case // 2) % 2
    renorm = bool((case // 4) % 2)
    scale = [1.0, 2.5][case % 2]
    T = 8
    # coarse values make exact ties common
    logits = (rng.integers(-3, 4, (T, E)) * 0.5).astype(np.float32)
    if case % 3 == 0:
        logits += rng.normal(0, 1, (T, E)).astype(np.float32)
    bias = None if case % 5 else rng.normal(0, 0.3, E).astype(np.float32)
    ids, w = oracle.route_select(logits, k, score, G, KG, gkind, renorm, scale, bias)
    for t in range(T):
        order, wref = _brute_route(logits[t], k, score, G, KG, gkind, renorm, scale, bias)
        assert list(ids[t]) == order, (t, logits[t], ids[t], order)
        np.testing.assert_allclose(w[t], np.array(wref, dtype=np.float32), rtol=1e-6)


def test_route_weights_closed_forms():
    rng = np.random.default_rng(3)
    logits = rng.normal(0, 1, (200, 16)).astype(np.float32)
    ids, w = oracle.route_select(logits, 4, oracle.SOFTMAX, renormalize=True)
    # renormalised softmax over the selected = softmax of the selected logits
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), 1)
    ref = np.exp(sel - sel.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=2e-7, atol=1e-8)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-6)
    ids, w = oracle.route_select(logits, 4, oracle.SIGMOID, 4, 2, oracle.TOP2_SUM, True, 2.5)
    np.testing.assert_allclose(w.sum(1), 2.5, rtol=1e-6)
    ids, w = oracle.route_select(logits, 4, oracle.SIGMOID, renormalize=False)
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, 1 / (1 + np.exp(-sel)), rtol=2e-7)


def test_group_limit_reduces_to_plain_topk():
    rng = np.random.default_rng(4)
    logits = rng.normal(0, 1, (64, 24)).astype(np.float32)
    plain = oracle.route_select(logits, 5, oracle.SIGMOID, 1, 1)
    allg = oracle.route_select(logits, 5, oracle.SIGMOID, 6, 6, oracle.TOP2_SUM)
    assert np.array_equal(plain[0], allg[0]) and np.array_equal(plain[1], allg[1])
    ref = np.argsort(-(1 / (1 + np.exp(-logits.astype(np.float64)))), axis=1, kind="stable")[:, :5]
    assert np.array_equal(plain[0], ref)


def test_ties_go_to_lower_index():
    z = np.zeros((3, 8), dtype=np.float32)
    for score in (oracle.SOFTMAX, oracle.SIGMOID):
        ids, w = oracle.route_select(z, 3, score)
        assert np.array_equal(ids, np.tile([0, 1, 2], (3, 1)))
        np.testing.assert_allclose(w, 1 / 3, rtol=1e-7)
    ids, _ = oracle.route_select(z, 3, oracle.SIGMOID, 4, 2, oracle.TOP2_SUM)
    assert np.array_equal(ids, np.tile([0, 1, 2], (3, 1)))
    l = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.0]], dtype=np.float32)
    ids, _ = oracle.route_select(l, 3, oracle.SOFTMAX)
    assert list(ids[0]) == [1, 2, 4]


def test_route_margin_matches_definition():
    rng = np.random.default_rng(5)
    logits = rng.normal(0, 1, (50, 12)).astype(np.float32)
    m = oracle.route_margin(logits, 3, oracle.SIGMOID, 4, 2, oracle.TOP2_SUM)
    for t in range(50):
        s = 1 / (1 + np.exp(-logits[t].astype(np.float64)))
        g = np.array([np.sort(s[3 * i:3 * i + 3])[::-1][:2].sum() for i in range(4)])
        gsort = np.sort(g)[::-1]
        kept = np.argsort(-g, kind="stable")[:2]
        allowed = np.sort(np.concatenate([s[3 * i:3 * i + 3] for i in kept]))[::-1]
        ref = min(gsort[1] - gsort[2], allowed[2] - allowed[3])
        assert abs(m[t] - ref) < 1e-12
    m = oracle.route_margin(logits, 12, oracle.SOFTMAX)
    assert np.all(np.isinf(m))


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("m_tile", [1, 4, 16])
def test_dispatch_is_a_stable_counting_sort(m_tile):
    rng = np.random.default_rng(6)
    T, k, E = 97, 3, 10
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[:5] = [0, 1, 2]  # load expert 0..2 a bit more
    d = oracle.dispatch(ids, E, m_tile)
    assert d["counts"].sum() == T * k
    assert np.array_equal(d["counts"], np.bincount(ids.ravel(), minlength=E))
    assert np.array_equal(d["offsets"], np.concatenate([[0], np.cumsum(d["counts"])]))
    padded = -(-d["counts"] // m_tile) * m_tile
    assert np.array_equal(d["padded_offsets"], np.concatenate([[0], np.cumsum(padded)]))
    # library routine: numpy's stable sort of the flat (t, j) pairs by expert
    order = np.argsort(ids.ravel(), kind="stable")
    rs = d["row_src"]
    valid = rs[rs >= 0]
    assert np.array_equal(valid, order)
    # padding rows hold -1 and sit only at the end of each expert segment
    for e in range(E):
        seg = rs[d["padded_offsets"][e]:d["padded_offsets"][e + 1]]
        n = d["counts"][e]
        assert np.all(seg[:n] >= 0) and np.all(seg[n:] == -1)
        assert np.all(ids.ravel()[seg[:n]] == e)
    # tok_row and row_src are inverse maps
    flat = d["tok_row"].ravel()
    assert np.array_equal(rs[flat], np.arange(T * k))


def test_permute_then_combine_is_identity():
    rng = np.random.default_rng(7)
    T, k, E, H = 40, 2, 5, 12
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch(ids, E, 1)
    x = rng.normal(0, 1, (T, H))
    x_perm = x[d["row_src"] // k]
    for j in range(k):
        onehot = np.zeros((T, k), dtype=np.float32)
        onehot[:, j] = 1.0
        out = oracle.combine(x_perm, d["tok_row"], onehot)
        assert np.array_equal(out, x)


def test_combine_matches_numpy():
    rng = np.random.default_rng(8)
    T, k, H, R = 30, 3, 20, 100
    y = rng.normal(0, 1, (R, H))
    tok_row = rng.integers(0, R, (T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    ys = rng.normal(0, 1, (T, H))
    ref = (w.astype(np.float64)[:, :, None] * y[tok_row]).sum(1) + ys
    np.testing.assert_allclose(oracle.combine(y, tok_row, w, ys), ref, rtol=1e-14, atol=1e-14)
    ref0 = (w.astype(np.float64)[:, :, None] * y[tok_row]).sum(1)
    np.testing.assert_allclose(oracle.combine(y, tok_row, w), ref0, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------ experts

def _np_ffn(x, wg, wu, wd, round_h=None):
    g = x @ wg.T
    u = x @ wu.T
    a = g / (1.0 + np.exp(-g)) * u
    if round_h is not None:
        a = round_h(a)
    return a @ wd.T


def test_expert_ffn_matches_numpy_chain():
    rng = np.random.default_rng(9)
    n, H, I = 7, 64, 48          # H != I: a transposed operand cannot pass
    x = _bf16(rng, (n, H))
    wg = _bf16(rng, (I, H), 1 / 8)
    wu = _bf16(rng, (I, H), 1 / 8)
    wd = _bf16(rng, (H, I), 1 / 7)
    got = oracle.expert_ffn(x, wg, wu, wd)
    X, G, U, D = (oracle.bf16_to_f64(a) for a in (x, wg, wu, wd))
    np.testing.assert_allclose(got, _np_ffn(X, G, U, D), rtol=1e-12, atol=1e-12)
    rb = lambda a: f64(torch.tensor(a).to(torch.float32).to(torch.bfloat16))
    got = oracle.expert_ffn(x, wg, wu, wd, h_bf16=True)
    np.testing.assert_allclose(got, _np_ffn(X, G, U, D, rb), rtol=1e-12, atol=1e-12)
    xf = rng.normal(0, 1, (3, 16)).astype(np.float32)
    wgf, wuf = (rng.normal(0, 0.25, (8, 16)).astype(np.float32) for _ in range(2))
    wdf = rng.normal(0, 0.35, (16, 8)).astype(np.float32)
    ref = _np_ffn(*(a.astype(np.float64) for a in (xf, wgf, wuf, wdf)))
    np.testing.assert_allclose(oracle.expert_ffn(xf, wgf, wuf, wdf), ref, rtol=1e-12, atol=1e-12)


def test_expert_ffn_fp8_matches_numpy_and_torch():
    cfg = synth.config("c5_dsv3_ep_fp8", H=256, I=384)
    wg, sg, wu, su, wd, sd = fp8w = synth.fp8_expert_weights(cfg, 0)
    xq, xs = synth.fp8_rows(cfg, 5)
    got = oracle.expert_ffn_fp8(*(to_np(t) for t in (xq, xs, wg, sg, wu, su, wd, sd)))

    def deq(q, s, rb, cb):
        v = e4m3_f64(to_np(q))
        s = f64(s)
        return v * np.repeat(np.repeat(s, rb, 0), cb, 1)
    X = deq(xq, xs, 1, 128)
    G, U, D = deq(wg, sg, 128, 128), deq(wu, su, 128, 128), deq(wd, sd, 128, 128)
    g = X @ G.T
    u = X @ U.T
    a = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    ab = a.reshape(5, 3, 128)
    amax = np.abs(ab).max(2, keepdims=True)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = torch.tensor(np.clip(ab / s, -448, 448)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    a2 = (q * s.astype(np.float64)).reshape(5, 384)
    ref = a2 @ D.T
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())
    # the intermediate before requantisation
    got2, a_or = oracle.expert_ffn_fp8(*(to_np(t) for t in (xq, xs, wg, sg, wu, su, wd, sd)), return_h=True)
    np.testing.assert_array_equal(got2, got)
    a64 = g / (1 + np.exp(-g)) * u
    np.testing.assert_allclose(a_or, a64, rtol=1e-12, atol=1e-12 * np.abs(a64).max())


def test_fp8_h_alternatives_flags_midpoints():
    """Rows of 128 values with amax = 448, so the block scale is exactly 1 and
    v = a: e4m3 neighbours around 1 are 1 and 1.125 (midpoint 1.0625), around
    300 are 288 and 320 (midpoint 304), and 2^-9, 2^-8 below 2^-6 (midpoint
    1.5 * 2^-9).  The helper flags exactly the values near a midpoint and gives
    the step to the other neighbour (ties go to the even code)."""
    a = np.full((1, 128), 1.03, dtype=np.float64)
    a[0, 0] = 448.0
    a[0, 1] = 1.0625                     # exact tie -> 1.0 (even); other = 1.125
    a[0, 2] = 1.0625 * (1 + 2.0 ** -20)  # just above -> 1.125; other = 1.0
    a[0, 3] = -1.0625                    # tie -> -1.0; other = -1.125
    a[0, 4] = 304.0 * (1 - 2.0 ** -16)   # just below 304 -> 288; other = 320
    a[0, 5] = 1.5 * 2.0 ** -9            # subnormal tie -> 2^-8 (even); other = 2^-9
    a[0, 6] = 0.0
    a[0, 7] = 1.0625 * (1 + 2.0 ** -8)   # far from the midpoint
    def rel(x, eta):  # an error bound of eta relative to max(|a|, 2^-6)
        return eta * np.maximum(np.abs(x), 2.0 ** -6)
    alt = dict(oracle.fp8_h_alternatives(a, rel(a, 2.0 ** -12))[0])
    assert set(alt) == {1, 2, 3, 4, 5}
    assert alt[1] == 0.125 and alt[2] == -0.125 and alt[3] == -0.125
    assert alt[4] == 32.0 and alt[5] == -(2.0 ** -9)
    # a tighter bound drops the values that are not exact ties
    tight = dict(oracle.fp8_h_alternatives(a, rel(a, 2.0 ** -22))[0])
    assert set(tight) == {1, 3, 5}
    # no error at all leaves only the exact ties
    assert set(dict(oracle.fp8_h_alternatives(a, 0.0)[0])) == {1, 3, 5}
    # scale != 1: amax 224 gives s = 0.5, v = 2 a, dh in units of a
    b = np.full((1, 128), 1.03, dtype=np.float64)
    b[0, 0] = 224.0
    b[0, 1] = 1.0625 / 2
    alt_b = dict(oracle.fp8_h_alternatives(b, rel(b, 2.0 ** -12))[0])
    assert alt_b[1] == 0.125 * 0.5
    # a bound on the block maximum moves s, and with it every v of the block:
    # 1.03 is 0.0325 from the midpoint 1.0625, which a 4% move of s covers
    # (and 448 itself may land below the midpoint 432 of 416 and 448)
    c = np.full((1, 128), 1.03, dtype=np.float64)
    c[0, 0] = 448.0
    dc = np.zeros((1, 128))
    dc[0, 0] = 0.04 * 448.0
    assert set(dict(oracle.fp8_h_alternatives(c, dc)[0])) == set(range(128))
    dc[0, 0] = 0.01 * 448.0  # 1%: 1.03 stays, 448 stays above 432
    assert set(dict(oracle.fp8_h_alternatives(c, dc)[0])) == set()


def _fp32_block_scaled_swiglu(xc, xs, wc, ws, order, kb=128):
    """An fp32 evaluation of a = silu(x . wg^T) * (x . wu^T) the way the bound
    describes: per K block, the fp32 sum of code products (numpy's float32
    matmul), times the fp32 product of the two scales, accumulated in fp32 in
    the given block order; silu and the product in fp32."""
    n, K = xc.shape
    out = []
    for w, s in zip(wc, ws):
        acc = np.zeros((n, w.shape[0]), dtype=np.float32)
        for b in order:
            t = xc[:, b * kb:(b + 1) * kb].astype(np.float32) @ w[:, b * kb:(b + 1) * kb].astype(np.float32).T
            q = xs[:, b][:, None].astype(np.float32) * s[:, b][None, :].astype(np.float32)
            acc = (acc + (t * q).astype(np.float32)).astype(np.float32)
        out.append(acc)
    g, u = out
    sil = (g / (np.float32(1.0) + np.exp(-g))).astype(np.float32)
    return (sil * u).astype(np.float32)


def test_ffn_h_error_bound_covers_fp32_evaluations():
    """The bound on |a~ - a| holds for fp32 evaluations of the block-scaled
    SwiGLU intermediate in two block orders (fp64 is the exact value: products
    of e4m3 codes and scales are exact there), and it is informative: at
    K = 1024 its median is below 2^-9 of |a|."""
    rng = np.random.default_rng(5)
    n, K, I = 24, 1024, 256
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    codes = np.concatenate([codes, codes | 0x80])
    xq = rng.choice(codes, size=(n, K))
    wgq, wuq = rng.choice(codes, size=(I, K)), rng.choice(codes, size=(I, K))
    xs = (2.0 ** rng.uniform(-12, -6, size=(n, K // 128))).astype(np.float32)
    sg = (2.0 ** rng.uniform(-14, -8, size=(I // 128, K // 128))).astype(np.float32)
    su = (2.0 ** rng.uniform(-14, -8, size=(I // 128, K // 128))).astype(np.float32)
    xc, wgc, wuc = (oracle.e4m3_to_f64(q) for q in (xq, wgq, wuq))
    X = xc * np.repeat(xs.astype(np.float64), 128, axis=1)
    Wg = wgc * np.repeat(np.repeat(sg.astype(np.float64), 128, 0), 128, 1)
    Wu = wuc * np.repeat(np.repeat(su.astype(np.float64), 128, 0), 128, 1)
    g, u = X @ Wg.T, X @ Wu.T
    a = g / (1 + np.exp(-g)) * u
    bound = oracle.ffn_h_error_bound(X, Wg, Wu)
    # the weight scales of a row block, per row
    sgr, sur = np.repeat(sg, 128, axis=0), np.repeat(su, 128, axis=0)
    for order in (range(K // 128), reversed(range(K // 128))):
        a32 = _fp32_block_scaled_swiglu(xc, xs, (wgc, wuc), (sgr, sur), list(order))
        assert np.all(np.abs(a32.astype(np.float64) - a) <= bound)
    assert np.median(bound / np.maximum(np.abs(a), 1e-300)) < 2.0 ** -9


def test_quantize_rows_e4m3_closed_forms():
    """Blocks built from e4m3 values times 2^k with a +-448 * 2^k element come
    back as exactly those codes with s = 2^k; an all-zero block has s = 1 and
    zero codes; negating x flips the sign bit of every nonzero code; random
    rows dequantise within half an e4m3 step."""
    rng = np.random.default_rng(31)
    for k in (-7, 0, 5):
        mag = rng.integers(1, 0x7F, size=(3, 384)).astype(np.uint8)   # finite nonzero magnitudes
        mag[:, ::128] = 0x7E                                           # 448 in every block
        codes = mag | (rng.integers(0, 2, size=mag.shape).astype(np.uint8) << 7)
        x = (e4m3_f64(codes) * 2.0 ** k).astype(np.float32)
        q, sc = oracle.quantize_rows_e4m3(x)
        assert np.array_equal(q, codes)
        assert np.array_equal(sc, np.full((3, 3), 2.0 ** k, dtype=np.float32))
        qn, scn = oracle.quantize_rows_e4m3(-x)
        assert np.array_equal(qn, codes ^ 0x80) and np.array_equal(scn, sc)
    z = np.zeros((2, 256), dtype=np.float32)
    z[1, 128:] = rng.standard_normal(128).astype(np.float32)
    q, sc = oracle.quantize_rows_e4m3(z)
    assert sc[0, 0] == 1.0 and sc[0, 1] == 1.0 and sc[1, 0] == 1.0 and not (q[:, :128] & 0x7F).any()
    x = rng.standard_normal((8, 512)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # bf16 input (truncated): same rule on its values
    xb = (bits.astype(np.uint32) << 16).view(np.float32)
    q, sc = oracle.quantize_rows_e4m3(bits)
    deq = e4m3_f64(q).reshape(8, 4, 128) * sc[:, :, None].astype(np.float64)
    err = np.abs(deq.reshape(8, 512) - xb.astype(np.float64))
    # normal e4m3 values carry 3 fraction bits: half a step is 2^-4 of the value; below 2^-6 the step is 2^-9
    bound = np.maximum(2.0 ** -4 * np.abs(xb.astype(np.float64)), 2.0 ** -10 * np.repeat(sc, 128, axis=1))
    assert (err <= bound * (1 + 1e-12)).all()
    # the block maximum maps to 448: it comes back as 448 s, within the rounding of s = fp32(max / 448)
    dmax = np.abs(deq).reshape(8, 4, 128).max(axis=2)
    amax = np.abs(xb.astype(np.float64)).reshape(8, 4, 128).max(axis=2)
    assert (np.abs(dmax - amax) <= 2.0 ** -23 * amax).all()


def test_fp8_power_of_two_scales_are_exact():
    """With power-of-two scales the dequantised operands are exact, so the
    fp8 expert equals the bf16/fp64 expert on the decoded values up to the
    requantisation of a; check the GEMM-1 part through an identity down."""
    rng = np.random.default_rng(10)
    H = I = 128
    codes = lambda shape: rng.integers(0, 0x7E, shape).astype(np.uint8) | \
        (rng.integers(0, 2, shape).astype(np.uint8) << 7)
    xq, wg, wu = codes((2, H)), codes((I, H)), codes((I, H))
    wd = np.zeros((H, I), dtype=np.uint8)
    xs = np.full((2, 1), 0.25, np.float32)
    sg = np.full((1, 1), 2.0**-10, np.float32)
    su = np.full((1, 1), 2.0**-9, np.float32)
    sd = np.ones((1, 1), np.float32)
    y = oracle.expert_ffn_fp8(xq, xs, wg, sg, wu, su, wd, sd)
    assert np.all(y == 0.0)  # zero down projection (code 0) gives exact zeros


# -------------------------------------------------------------------- layer

def _layer_inputs(rng, T, H, E, I, dtype="bf16"):
    if dtype == "bf16":
        mk = lambda shape, std: _bf16(rng, shape, std)
    else:
        mk = lambda shape, std: rng.normal(0, std, shape).astype(np.float32)
    x = mk((T, H), 1.0)
    wr = mk((E, H), 1 / math.sqrt(H))
    wg = mk((E, I, H), 1 / math.sqrt(H))
    wu = mk((E, I, H), 1 / math.sqrt(H))
    wd = mk((E, H, I), 1 / math.sqrt(I))
    return x, wr, wg, wu, wd


def _val(a):
    return oracle.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layer_single_expert_is_dense_ffn(dtype):
    rng = np.random.default_rng(11)
    T, H, I = 9, 32, 24
    x, wr, wg, wu, wd = _layer_inputs(rng, T, H, 1, I, dtype)
    for scale in (1.0, 2.5):
        r = oracle.layer(x, wr, wg, wu, wd, k=1, routed_scale=scale)
        ref = scale * _np_ffn(_val(x), _val(wg[0]), _val(wu[0]), _val(wd[0]))
        np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
        assert np.all(r["topk_ids"] == 0)
    sh = tuple(a[0] for a in _layer_inputs(rng, 1, H, 1, 20, dtype)[2:])
    r = oracle.layer(x, wr, wg, wu, wd, k=1, routed_scale=2.5, shared=sh)
    ref = 2.5 * _np_ffn(_val(x), _val(wg[0]), _val(wu[0]), _val(wd[0])) + \
        _np_ffn(_val(x), *(_val(a) for a in sh))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def test_layer_all_experts_is_soft_mixture():
    rng = np.random.default_rng(12)
    T, H, E, I = 6, 16, 4, 8
    x, wr, wg, wu, wd = _layer_inputs(rng, T, H, E, I)
    r = oracle.layer(x, wr, wg, wu, wd, k=E, renormalize=True)
    lg = _val(x) @ _val(wr).T
    lg = lg.astype(np.float32).astype(np.float64)
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = sum(p[:, e:e + 1] * _np_ffn(_val(x), _val(wg[e]), _val(wu[e]), _val(wd[e]))
              for e in range(E))
    np.testing.assert_allclose(r["out"], ref, rtol=1e-6, atol=1e-7)


def test_layer_linearity_and_zero_input():
    rng = np.random.default_rng(13)
    T, H, E, I = 10, 16, 6, 12
    x, wr, wg, wu, wd = _layer_inputs(rng, T, H, E, I)
    kw = dict(k=2, score=oracle.SIGMOID, n_groups=3, topk_groups=2, routed_scale=2.5)
    r1 = oracle.layer(x, wr, wg, wu, wd, **kw)
    wd2 = to_np(torch.tensor(2.0 * oracle.bf16_to_f64(wd), dtype=torch.float32).to(torch.bfloat16))
    r2 = oracle.layer(x, wr, wg, wu, wd2, **kw)
    assert np.array_equal(r1["topk_ids"], r2["topk_ids"])
    assert np.array_equal(2.0 * r1["out"], r2["out"])
    z = np.zeros_like(x)
    r0 = oracle.layer(z, wr, wg, wu, wd, **kw)
    assert np.all(r0["out"] == 0.0)
    assert np.array_equal(r0["topk_ids"], np.tile([0, 1], (T, 1)))


def test_layer_duplicated_router_rows_pick_lower_index():
    rng = np.random.default_rng(14)
    T, H, E, I = 12, 16, 5, 8
    x, wr, wg, wu, wd = _layer_inputs(rng, T, H, E, I)
    wr[3] = wr[1]
    r = oracle.layer(x, wr, wg, wu, wd, k=2)
    assert not np.any(r["topk_ids"] == 3) or np.all(
        np.any(r["topk_ids"] == 1, axis=1)[np.any(r["topk_ids"] == 3, axis=1)])
    assert np.all(r["logits"][:, 1] == r["logits"][:, 3])


def test_layer_composes_steps():
    """The layer equals its steps chained by hand (catches a wrong row map or
    a dropped shared term in the composition)."""
    rng = np.random.default_rng(15)
    T, H, E, I, k = 23, 16, 6, 12, 2
    x, wr, wg, wu, wd = _layer_inputs(rng, T, H, E, I)
    bias = rng.normal(0, 0.5, E).astype(np.float32)
    r = oracle.layer(x, wr, wg, wu, wd, k=k, bias=bias)
    lg = oracle.router_logits(x, wr)
    ids, w = oracle.route_select(lg, k, bias=bias)
    assert np.array_equal(ids, r["topk_ids"]) and np.array_equal(w, r["topk_w"])
    ref = np.zeros((T, H))
    X = _val(x)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            ref[t] += w[t, j] * _np_ffn(X[t:t + 1], _val(wg[e]), _val(wu[e]), _val(wd[e]))[0]
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ MXFP4

def test_e2m1_and_e8m0_decode_closed_forms():
    """E2M1 (OCP MX v1.0): sign, 2 exponent bits with bias 1, 1 mantissa bit;
    the eight magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  E8M0: 2^(c - 127),
    255 is NaN."""
    got = oracle.e2m1_to_f64(np.arange(16))
    assert list(got[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(got[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert math.copysign(1.0, got[8]) == -1.0
    sc = oracle.e8m0_to_f64(np.arange(256))
    assert all(sc[c] == math.ldexp(1.0, c - 127) for c in range(255))
    assert math.isnan(sc[255])


def test_mxfp4_dequant_brute_force():
    """Packed codes: element k of a row in byte k // 2, the low nibble for even
    k; scale block k // 32.  Checked element by element with Python loops."""
    rng = np.random.default_rng(3)
    rows, K = 3, 96
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(110, 140, size=(rows, K // 32), dtype=np.uint8)
    got = oracle.mxfp4_to_f64(codes, scales)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for r in range(rows):
        for k in range(K):
            b = int(codes[r, k // 2])
            c = (b >> 4) if k % 2 else (b & 0xF)
            v = (-1.0 if c & 8 else 1.0) * mags[c & 7] * 2.0 ** (int(scales[r, k // 32]) - 127)
            assert got[r, k] == v, (r, k)


def test_quantize_mxfp4_rule():
    """synth.quantize_mxfp4 follows the OCP conversion: the shared exponent is
    floor(log2(amax)) - 2, so the block maximum maps into [4, 8) and every
    element lies within half an E2M1 step of its code;
    an all-zero block gets scale 127 and zero codes; past 6 units the code
    saturates."""
    w = torch.randn(4, 128, generator=torch.Generator().manual_seed(2)) * 0.05
    w[1, 32:64] = 0.0
    w[2, :32] = torch.tensor([1.25, 0.75, 2.5, 3.5, 5.0, 0.25, -1.75, -6.5] * 4) * 0.5   # ties at scale 2^-1
    q, s = synth.quantize_mxfp4(w)
    deq = oracle.mxfp4_to_f64(q.numpy(), s.numpy())
    wf = w.double().numpy()
    assert s[1, 1] == 127 and not q[1, 16:32].any()
    blk = wf.reshape(4, 4, 32)
    amax = np.abs(blk).max(2)
    x = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2
    assert np.array_equal(s.numpy().astype(np.int64), np.where(amax > 0, x + 127, 127).astype(np.int64))
    unit = np.repeat(2.0 ** x, 32, axis=1)
    v = wf / unit
    sat = np.abs(v) > 6.0
    assert np.array_equal(deq[sat], np.sign(v[sat]) * 6.0 * unit[sat])  # saturated at +-6
    half = np.where(np.abs(v) < 2, 0.25, np.where(np.abs(v) < 4, 0.5, 1.0)) * unit  # half the E2M1 spacing
    assert np.all(np.abs(deq - wf)[~sat] <= half[~sat])
    # ties to even: 1.25 -> 1, 0.75 -> 1, 2.5 -> 2, 3.5 -> 4, 5 -> 4, 0.25 -> 0, -1.75 -> -2; -6.5 saturates
    assert list(deq[2, :8]) == [0.5, 0.5, 1.0, 2.0, 2.0, 0.0, -1.0, -3.0]


def test_expert_ffn_mxfp4_reduces_to_fp8_with_block_constant_scales():
    """MXFP4 weights whose E8M0 scales are constant over every 128 x 128 block
    are exactly e4m3 weights (each E2M1 value is an e4m3 value) with the fp32
    block scale 2^(c - 127): the two oracle functions must then agree bit for
    bit.  Scales varying inside a block are covered by the dequantisation pin."""
    rng = np.random.default_rng(7)
    cfg = synth.config("c5_dsv3_ep_fp8", H=256, I=384)
    H, I = cfg.H, cfg.I
    xq, xs = (to_np(t) for t in synth.fp8_rows(cfg, 4))

    def mat(R, C):
        codes = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
        sb = rng.integers(120, 132, size=(R // 128, C // 128), dtype=np.uint8)
        scales = np.repeat(np.repeat(sb, 128, 0), 4, 1)
        vals = oracle.mxfp4_to_f64(codes, np.full_like(scales, 127))
        e4 = oracle.e4m3_rne_sat(vals.ravel()).reshape(R, C)
        assert np.array_equal(e4m3_f64(e4), vals)
        return codes, scales, e4, np.ldexp(1.0, sb.astype(np.int64) - 127).astype(np.float32)
    g, u, d = mat(I, H), mat(I, H), mat(H, I)
    y4 = oracle.expert_ffn_mxfp4(xq, xs, g[0], g[1], u[0], u[1], d[0], d[1])
    y8 = oracle.expert_ffn_fp8(xq, xs, g[2], g[3], u[2], u[3], d[2], d[3])
    assert np.array_equal(y4, y8)
