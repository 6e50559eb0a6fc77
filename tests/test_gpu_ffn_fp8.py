"""GPU parity of the fp8 (OCP e4m3) grouped SwiGLU FFN against the oracle.

The operands are e4m3 codes with fp32 block scales (1 x 128 per row for the
dispatched rows, 128 x 128 for the weights); the oracle dequantises them
exactly in fp64 and requantises the SwiGLU intermediate per row and 128
columns, as the layer does.

That requantisation turns floating point into integer codes.  Both sides take
each decision in fp32, but from values of the intermediate that differ by
fp32 rounding (accumulation order, exponential), so where a value sits within
that rounding of an e4m3 midpoint either neighbour is a correct code.  The
oracle bounds that rounding per element from the fp32 arithmetic of the
block-scale promotion (ffn_h_error_bound: the recursive-summation bound over
the 128 + H/128 + 2 roundings a term of g or u passes through, carried
through silu and the product), lists the decisions whose midpoint lies within
it (fp8_h_alternatives), and a row matches when its output equals the
oracle's for some choice of at most two of them.  One flip moves a whole output row by up to ~7% of
rms(ref), which is what the plain comparison of a large layer would otherwise
report.  Bounds on the resolved difference: max|err| / rms(ref) <= 4e-2 and
rms(err) / rms(ref) <= 1e-3 (a regression detector: a wrong scale or a dropped
K block moves every row), 2.5e-3 for bf16 outputs, whose round-to-nearest
storage alone contributes 2^-9 / sqrt(3) ~ 1.1e-3."""
import numpy as np
import pytest
import torch

import expert_layer_amd as moe
import oracle
import synth
from tests._cases import dev

pytestmark = pytest.mark.gpu

TOL = 4e-2
TOL_RMS = 1e-3
TOL_RMS_BF16 = 2.5e-3


def _u8(t):
    return t.detach().contiguous().cpu().numpy().astype(np.uint8)


def _f32(t):
    return t.detach().contiguous().cpu().numpy().astype(np.float32)


def _inputs(E, H, I, n_rows, seed, device):
    s = synth.MoeShape("fp8t", T=max(n_rows, 1), H=H, E=E, k=1, I=I, dtype="fp8", seed=seed)
    wq = [synth.fp8_expert_weights(s, e, device) for e in range(E)]
    stack = [torch.stack([w[i] for w in wq]) for i in range(6)]  # wg, sg, wu, su, wd, sd
    xq, xs = synth.fp8_rows(s, max(n_rows, 1), device)
    return s, wq, stack, xq, xs


def _run(E, H, I, counts, ydt, extra_rows, seed, wlayout=moe.MOE_LAYOUT_ROWMAJOR):
    d = dev()
    n = int(sum(counts))
    cap = n + extra_rows
    s, wq, (wg, sg, wu, su, wd, sd), xq, xs = _inputs(E, H, I, cap, seed, d)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=d)
    c = moe.make_cfg(T=max(cap, 1), H=H, E=E, k=1, I=I, act_dtype=moe.MOE_FP8_E4M3, y_dtype=ydt)
    assert moe.moe_validate(c) == moe.MOE_OK, moe.moe_last_error()
    ytd = torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16
    sentinel = -12345.0
    y = torch.full((max(cap, 1), H), sentinel, dtype=ytd, device=d)
    ws = moe.workspace(c, moe.MOE_STAGE_FFN, d, n_rows_cap=cap)
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd)
    keep = None
    if wlayout == moe.MOE_LAYOUT_TILED:
        w, keep = moe.tile_weights(c, w, d)
    moe.moe_grouped_ffn(c, cap, xq, xs, offs, w, None, y, None, ws)
    torch.cuda.synchronize()
    del keep
    return wq, xq, xs, y, sentinel


_E4M3 = None


def _deq(codes, scales, rows_only=False):
    """e4m3 codes times their fp32 scales (1 x 128 per row, or 128 x 128), fp64;
    the codes go through a table of the oracle's value of each of the 256."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    sc = scales.astype(np.float64)
    full = np.repeat(sc, 128, axis=1) if rows_only else np.repeat(np.repeat(sc, 128, 0), 128, 1)
    return _E4M3[np.asarray(codes, dtype=np.uint8)] * full


def _resolve(resid, alts, WD, n_cand=64):
    """The smallest max|resid - sum of flips| over the row's ambiguous
    decisions, choosing none, one or two of the n_cand nearest their midpoints
    (fp8_h_alternatives lists those first)."""
    best, bm = resid, np.abs(resid).max()
    cands = alts[:n_cand]
    if not cands:
        return best
    C = np.stack([dh * WD[:, i] for i, dh in cands])  # the output change of each flip
    R1 = resid[None, :] - C
    m1 = np.abs(R1).max(axis=1)
    k = int(np.argmin(m1))
    if m1[k] < bm:
        best, bm = R1[k], m1[k]
    for i in range(len(cands) - 1):
        R2 = R1[i][None, :] - C[i + 1:]
        m2 = np.abs(R2).max(axis=1)
        k = int(np.argmin(m2))
        if m2[k] < bm:
            best, bm = R2[k], m2[k]
    return best


def _check_rows(wq, xq, xs, y, rows_by_expert):
    """Oracle on the listed rows of each expert, flips of ambiguous h codes
    resolved; returns (max err, rms err) / rms(ref) and the number of rows
    that needed a flip."""
    refs, res = [], []
    flipped = 0
    for e, rows in rows_by_expert.items():
        if len(rows) == 0:
            continue
        rows = np.asarray(rows)
        wg, sg, wu, su, wd, sd = (_u8(t) if i % 2 == 0 else _f32(t) for i, t in enumerate(wq[e]))
        xr, xsr = _u8(xq[rows]), _f32(xs[rows])
        ref, a = oracle.expert_ffn_fp8(xr, xsr, wg, sg, wu, su, wd, sd, return_h=True)
        alts = oracle.fp8_h_alternatives(a, oracle.ffn_h_error_bound(
            _deq(xr, xsr, rows_only=True), _deq(wg, sg), _deq(wu, su)))
        WD = _deq(wd, sd)
        got = y[torch.as_tensor(rows, device=y.device)].float().cpu().numpy().astype(np.float64)
        for r in range(len(rows)):
            resid = got[r] - ref[r]
            if alts[r]:
                rr = _resolve(resid, alts[r], WD)
                flipped += int(np.abs(rr).max() < np.abs(resid).max())
                resid = rr
            res.append(resid)
        refs.append(ref)
    ref = np.concatenate(refs)
    res = np.stack(res)
    scale = np.sqrt(np.mean(ref ** 2))
    return float(np.abs(res).max() / scale), float(np.sqrt(np.mean(res ** 2)) / scale), flipped


@pytest.mark.parametrize("H,I,counts,ydt,extra", [
    (512, 256, [37, 0, 5, 300, 64, 1, 0, 257], moe.MOE_F32, 0),   # unaligned offsets, empty experts, 2 tiles
    (384, 384, [129, 3, 260], moe.MOE_BF16, 11),                  # odd K blocks, a partial GEMM2 N tile
    (1024, 512, [600], moe.MOE_BF16, 0),                          # one expert over 3 M tiles
    (256, 128, [1, 1, 1, 1], moe.MOE_F32, 5),                     # single rows
    (256, 256, [20, 50, 90, 120, 150, 180, 220, 256, 300], moe.MOE_BF16, 0),  # every tile height, 1 .. 8 units
])
@pytest.mark.parametrize("wlayout", [moe.MOE_LAYOUT_ROWMAJOR, moe.MOE_LAYOUT_TILED])
def test_grouped_ffn_fp8_matches_oracle(H, I, counts, ydt, extra, wlayout):
    E = len(counts)
    wq, xq, xs, y, sentinel = _run(E, H, I, counts, ydt, extra, seed=H + 7 * I, wlayout=wlayout)
    oc = np.concatenate([[0], np.cumsum(counts)]).astype(int)
    rows = {e: list(range(oc[e], oc[e + 1])) for e in range(E)}
    err, rms, flipped = _check_rows(wq, xq, xs, y, rows)
    assert err <= TOL and rms <= (TOL_RMS if ydt == moe.MOE_F32 else TOL_RMS_BF16), (err, rms, flipped)
    # rows past expert_offsets[E] are not written
    if extra:
        assert torch.all(y[oc[-1]:] == torch.tensor(sentinel, dtype=y.dtype, device=y.device))


@pytest.mark.parametrize("wlayout", [moe.MOE_LAYOUT_TILED, moe.MOE_LAYOUT_ROWMAJOR])
def test_grouped_ffn_fp8_full_size_sampled(wlayout):
    """The c5 workload: 65536 dispatched rows over 8 experts (Zipf(1.0) counts),
    H = 7168, I = 2048, bf16 output, weights tiled (as timed) or row-major; the
    oracle checks at least 512 seeded rows spread over every expert, including
    each expert's first and last row."""
    s = synth.config("c5_dsv3_ep_fp8")
    counts = synth.fp8_counts(s)
    assert sum(counts) == s.T
    d = dev()
    wq = [synth.fp8_expert_weights(s, e, d) for e in range(s.E)]
    wg, sg, wu, su, wd, sd = (torch.stack([w[i] for w in wq]) for i in range(6))
    xq, xs = synth.fp8_rows(s, s.T, d)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=d)
    c = moe.make_cfg(T=s.T, H=s.H, E=s.E, k=1, I=s.I, act_dtype=moe.MOE_FP8_E4M3, y_dtype=moe.MOE_BF16)
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=d)
    ws = moe.workspace(c, moe.MOE_STAGE_FFN, d, n_rows_cap=s.T)
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd)
    keep = None
    if wlayout == moe.MOE_LAYOUT_TILED:
        w, keep = moe.tile_weights(c, w, d)
    moe.moe_grouped_ffn(c, s.T, xq, xs, offs, w, None, y, None, ws)
    torch.cuda.synchronize()
    del keep
    rng = np.random.default_rng(s.seed)
    oc = np.concatenate([[0], np.cumsum(counts)]).astype(int)
    # at least 512 rows: every expert's first and last row, the rest seeded
    # across the experts in proportion to their rows (at least 16 each)
    rows = {}
    for e in range(s.E):
        want = max(16, int(np.ceil(512 * counts[e] / s.T)))
        pick = rng.choice(np.arange(oc[e], oc[e + 1]), size=min(want, counts[e]), replace=False)
        rows[e] = sorted(set(pick.tolist()) | {oc[e], oc[e + 1] - 1})
    assert sum(len(r) for r in rows.values()) >= 512
    err, rms, flipped = _check_rows(wq, xq, xs, y, rows)
    print(f"c5: {sum(len(r) for r in rows.values())} rows, max {err:.3e}, rms {rms:.3e}, {flipped} resolved")
    assert err <= TOL and rms <= TOL_RMS_BF16, (err, rms, flipped)


def test_tiled_e4m3_weights_equal_rowmajor():
    """moe_tile_weights only moves the e4m3 codes into the order in which a
    wave loads its MFMA fragments; the kernel sums the same products in the
    same order either way, so y is bit-identical (fp32 and bf16 outputs, a
    partial GEMM2 N tile, tiles of 1 .. 8 row units)."""
    d = dev()
    for H, I, counts in ((640, 384, [300, 17, 0, 260, 33]), (1152, 256, [512, 1])):
        for ydt in (moe.MOE_F32, moe.MOE_BF16):
            ys = [_run(len(counts), H, I, counts, ydt, 0, seed=H + I, wlayout=wl)[3]
                  for wl in (moe.MOE_LAYOUT_ROWMAJOR, moe.MOE_LAYOUT_TILED)]
            assert torch.equal(ys[0].view(torch.int16 if ydt == moe.MOE_BF16 else torch.int32),
                               ys[1].view(torch.int16 if ydt == moe.MOE_BF16 else torch.int32)), (H, I, ydt)


@pytest.mark.parametrize("wfmt", ["e4m3", "mxfp4"])
def test_indexed_e4m3_rows_equal_materialised_rows(wfmt):
    """The layer's dispatch for low-precision experts: moe_permute writes the
    maps only (MOE_LAYOUT_INDEXED) and GEMM1 reads each dispatched row and its
    scale from the quantised tokens through row_src.  Same kernels, same
    operand values in LDS: y must equal, bit for bit, the call on the
    materialised e4m3 x_perm (with m_tile padding rows in both)."""
    d = dev()
    T, H, E, k, I = 333, 512, 6, 3, 384
    s = synth.MoeShape("idx8", T=T, H=H, E=E, k=k, I=I, dtype="fp8", seed=17)
    g = torch.Generator(device="cpu").manual_seed(4)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32).to(d)
    xb = synth.normal(synth.stream_key(17, "x"), (T, H), 1.0, d, torch.bfloat16)
    gen = synth.mxfp4_expert_weights if wfmt == "mxfp4" else synth.fp8_expert_weights
    wq = [gen(s, e, d) for e in range(E)]
    wg, sg, wu, su, wd, sd = (torch.stack([w[i] for w in wq]) for i in range(6))
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd)
    wdt = moe.MOE_FP4_E2M1 if wfmt == "mxfp4" else moe.MOE_FP8_E4M3
    ys = []
    for layout in (moe.MOE_LAYOUT_ROWMAJOR, moe.MOE_LAYOUT_INDEXED):
        c = moe.make_cfg(T=T, H=H, E=E, k=k, I=I, act_dtype=moe.MOE_FP8_E4M3, w_dtype=wdt, y_dtype=moe.MOE_F32,
                         m_tile=16, x_layout=layout)
        assert moe.moe_validate(c) == moe.MOE_OK, moe.moe_last_error()
        xq = torch.empty((T, H), dtype=torch.uint8, device=d)
        xs = torch.empty((T, H // 128), device=d)
        moe.moe_quantize_fp8(moe.make_cfg(T=T, H=H, E=E, k=k, I=I), xb, xq, xs)
        rows = moe.moe_max_rows(c)
        i32 = dict(dtype=torch.int32, device=d)
        counts, offs = torch.empty(E, **i32), torch.empty(E + 1, **i32)
        row_src, tok_row = torch.empty(rows, **i32), torch.empty((T, k), **i32)
        indexed = layout == moe.MOE_LAYOUT_INDEXED
        x_perm = None if indexed else torch.empty((rows, H), dtype=torch.uint8, device=d)
        xps = None if indexed else torch.empty((rows, H // 128), device=d)
        moe.moe_permute(c, xq, xs, ids, counts, offs, row_src, tok_row, x_perm, xps,
                        moe.workspace(c, moe.MOE_STAGE_PERMUTE, d))
        y = torch.full((rows, H), -12345.0, device=d)
        moe.moe_grouped_ffn(c, rows, xq if indexed else x_perm, xs if indexed else xps, offs, w, None, y, None,
                            moe.workspace(c, moe.MOE_STAGE_FFN, d, n_rows_cap=rows), row_src=row_src)
        torch.cuda.synchronize()
        ys.append((y, offs.cpu().numpy(), row_src.cpu().numpy()))
    (y0, o0, r0), (y1, o1, r1) = ys
    assert np.array_equal(o0, o1) and np.array_equal(r0, r1)
    n = int(o0[-1])
    assert torch.equal(y0[:n], y1[:n])
    assert bool(torch.isfinite(y0[:n]).all())
