"""GPU parity of MXFP4 expert weights against the oracle: the grouped SwiGLU
FFN on e4m3 rows (1 x 128 fp32 scales) with OCP MX FP4 weights (E2M1 codes,
one E8M0 scale per 32 elements of a row, applied by the scaled MFMA), and the
layer with such experts on bf16 activations.

The intermediate h is requantised to e4m3 per row and 128 columns as on the
fp8 path, so the same reading of ambiguous codes applies (decisions whose
e4m3 midpoint lies within the fp32 rounding bound of the intermediate may go
either way; a row matches if its output equals the oracle's for some choice
of at most two of them), with the fp8 bounds: max|err| / rms(ref) <= 4e-2, rms(err) / rms(ref) <= 1e-3 (fp32 y) or
2.5e-3 (bf16 y)."""
import math

import numpy as np
import pytest
import torch

import expert_layer_amd as moe
import oracle
import synth
from tests._cases import dev, lib_cfg, rel_err, route_kw, router_case
from tests._np import to_np
from tests.test_gpu_ffn_fp8 import TOL, TOL_RMS, TOL_RMS_BF16, _deq, _resolve

pytestmark = pytest.mark.gpu


def _u8(t):
    return t.detach().contiguous().cpu().numpy().astype(np.uint8)


def _f32(t):
    return t.detach().contiguous().cpu().numpy().astype(np.float32)


def _check_rows(wq, xq, xs, y, rows_by_expert):
    refs, res = [], []
    flipped = 0
    for e, rows in rows_by_expert.items():
        if len(rows) == 0:
            continue
        rows = np.asarray(rows)
        wg, sg, wu, su, wd, sd = (_u8(t) for t in wq[e])
        xr, xsr = _u8(xq[rows]), _f32(xs[rows])
        ref, a = oracle.expert_ffn_mxfp4(xr, xsr, wg, sg, wu, su, wd, sd, return_h=True)
        alts = oracle.fp8_h_alternatives(a, oracle.ffn_h_error_bound(
            _deq(xr, xsr, rows_only=True), oracle.mxfp4_to_f64(wg, sg), oracle.mxfp4_to_f64(wu, su)))
        WD = oracle.mxfp4_to_f64(wd, sd)
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


def _stack(wq):
    return [torch.stack([w[i] for w in wq]) for i in range(6)]  # wg, sg, wu, su, wd, sd


def _run(s, counts, ydt, extra):
    d = dev()
    n = int(sum(counts))
    cap = n + extra
    wq = [synth.mxfp4_expert_weights(s, e, d) for e in range(len(counts))]
    wg, sg, wu, su, wd, sd = _stack(wq)
    xq, xs = synth.fp8_rows(s, max(cap, 1), d)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=d)
    c = moe.make_cfg(T=max(cap, 1), H=s.H, E=len(counts), k=1, I=s.I, act_dtype=moe.MOE_FP8_E4M3,
                     w_dtype=moe.MOE_FP4_E2M1, y_dtype=ydt)
    assert moe.moe_validate(c) == moe.MOE_OK, moe.moe_last_error()
    sentinel = -12345.0
    y = torch.full((max(cap, 1), s.H), sentinel, dtype=torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16,
                   device=d)
    ws = moe.workspace(c, moe.MOE_STAGE_FFN, d, n_rows_cap=cap)
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd)
    moe.moe_grouped_ffn(c, cap, xq, xs, offs, w, None, y, None, ws)
    torch.cuda.synchronize()
    return wq, xq, xs, y, sentinel


@pytest.mark.parametrize("H,I,counts,ydt,extra", [
    (512, 256, [37, 0, 5, 300, 64, 1, 0, 257], moe.MOE_F32, 0),   # unaligned offsets, empty experts, 128-row tiles
    (384, 384, [129, 3, 260], moe.MOE_BF16, 11),                  # odd K blocks, a partial GEMM2 N tile
    (1024, 512, [600], moe.MOE_BF16, 0),                          # 256-row tiles
    (512, 384, [300, 5, 270, 0, 129], moe.MOE_F32, 3),            # 256-row tiles, ragged groups
    (256, 128, [1, 1, 1, 1], moe.MOE_F32, 5),                     # single rows
    # every count of 32-row units holding rows in each half of a tile (the waves
    # of a half issue MFMAs for those only): 256-row tiles, then 128-row tiles
    (256, 256, [20, 50, 100, 140, 170, 200, 230, 256, 300], moe.MOE_BF16, 0),
    (256, 256, [10, 40, 70, 100, 128], moe.MOE_F32, 0),
])
def test_grouped_ffn_mxfp4_matches_oracle(H, I, counts, ydt, extra):
    s = synth.MoeShape("mx", T=1, H=H, E=len(counts), k=1, I=I, dtype="fp8", seed=H + 5 * I)
    wq, xq, xs, y, sentinel = _run(s, counts, ydt, extra)
    oc = np.concatenate([[0], np.cumsum(counts)]).astype(int)
    rows = {e: list(range(oc[e], oc[e + 1])) for e in range(len(counts))}
    err, rms, flipped = _check_rows(wq, xq, xs, y, rows)
    assert err <= TOL and rms <= (TOL_RMS if ydt == moe.MOE_F32 else TOL_RMS_BF16), (err, rms, flipped)
    if extra:
        assert torch.all(y[oc[-1]:] == torch.tensor(sentinel, dtype=y.dtype, device=y.device))


def test_grouped_ffn_mxfp4_full_size_sampled():
    """The c5 workload shape (65536 rows over 8 experts, Zipf(1.0) counts, H =
    7168, I = 2048) with MXFP4 weights: at least 512 seeded rows spread over
    every expert, including each expert's first and last row."""
    s = synth.config("c5_dsv3_ep_fp8")
    counts = synth.fp8_counts(s)
    wq, xq, xs, y, _ = _run(s, counts, moe.MOE_BF16, 0)
    rng = np.random.default_rng(s.seed + 1)
    oc = np.concatenate([[0], np.cumsum(counts)]).astype(int)
    rows = {}
    for e in range(s.E):
        want = max(16, int(np.ceil(512 * counts[e] / s.T)))
        pick = rng.choice(np.arange(oc[e], oc[e + 1]), size=min(want, counts[e]), replace=False)
        rows[e] = sorted(set(pick.tolist()) | {oc[e], oc[e + 1] - 1})
    assert sum(len(r) for r in rows.values()) >= 512
    err, rms, flipped = _check_rows(wq, xq, xs, y, rows)
    print(f"c5 MXFP4: {sum(len(r) for r in rows.values())} rows, max {err:.3e}, rms {rms:.3e}, {flipped} resolved")
    assert err <= TOL and rms <= TOL_RMS_BF16, (err, rms, flipped)


def _small_shape():
    return synth.config("c3_dsv3_bf16").with_(H=512, I=256, E=16, k=4, n_groups=4, topk_groups=2, I_shared=384)


@pytest.mark.parametrize("shape,T", [("small", 77), ("c3", 24)])
def test_layer_mxfp4_experts_matches_oracle(shape, T):
    """moe_layer with bf16 x and MXFP4 experts (routed and shared): routing,
    the oracle's per-token e4m3 quantisation of x, each chosen expert's MXFP4
    FFN, the weighted combine; max|err| / rms(ref) <= 4e-2 and rms(err) /
    rms(ref) <= 1e-2, as for fp8 experts."""
    s = _small_shape() if shape == "small" else synth.config("c3_dsv3_bf16")
    d = dev()
    rc = router_case(s, T)
    wq = [synth.mxfp4_expert_weights(s, e, d) for e in range(s.E)]
    wg, sg, wu, su, wd, sd = _stack(wq)
    sh = synth.mxfp4_expert_weights(s.with_(I=s.I_shared), s.E, d)
    c = lib_cfg(s, T=T, y_dtype=moe.MOE_BF16, out_dtype=moe.MOE_F32)
    c.w_dtype = moe.MOE_FP4_E2M1
    w = moe.weights(wg, wu, wd, s_gate=sg, s_up=su, s_down=sd, sh_gate=sh[0], sh_up=sh[2], sh_down=sh[4],
                    sh_s_gate=sh[1], sh_s_up=sh[3], sh_s_down=sh[5])
    out = torch.full((T, s.H), float("nan"), device=d)
    ws = moe.workspace(c, moe.MOE_STAGE_LAYER, d)
    moe.moe_layer(c, rc["w_r"], rc["bias"], w, rc["x"], out, ws)
    torch.cuda.synchronize()
    # the oracle composed step by step
    ids, tw = oracle.route_select(rc["logits"], s.k, renormalize=s.renormalize, routed_scale=s.routed_scale,
                                  bias=rc["bh"], **route_kw(s))
    xq, xs = oracle.quantize_rows_e4m3(rc["xh"])
    y_rows = np.zeros((T * s.k, s.H))
    for e in np.unique(ids):
        ti, j = np.nonzero(ids == e)
        y_rows[ti * s.k + j] = oracle.expert_ffn_mxfp4(xq[ti], xs[ti], *(_u8(t) for t in wq[e]))
    y_sh = oracle.expert_ffn_mxfp4(xq, xs, *(_u8(t) for t in sh))
    ref = oracle.combine(y_rows, np.arange(T * s.k, dtype=np.int32).reshape(T, s.k), tw, y_sh)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= 4e-2
    assert math.sqrt(float(np.mean((got - ref) ** 2))) / math.sqrt(float(np.mean(ref ** 2))) <= 1e-2
