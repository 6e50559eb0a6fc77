"""Builds seeded parity cases: inputs from synth, expected values from the
oracle, device tensors for the HIP path.  Only tests import this module."""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

import expert_layer_amd as moe
import oracle
import synth
from tests._np import f64, to_np

MARGIN = 1e-4  # decision margin of generated routing inputs (selection keys and group scores)

SCORE = {"softmax": oracle.SOFTMAX, "sigmoid": oracle.SIGMOID}
GSCORE = {"top2_sum": oracle.TOP2_SUM, "max": oracle.MAX}
LIB_DT = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "fp8": moe.MOE_FP8_E4M3}


def dev():
    return torch.device("cuda:0")


def lib_cfg(s: synth.MoeShape, T: Optional[int] = None, y_dtype=moe.MOE_F32, out_dtype=moe.MOE_F32,
            m_tile: int = 0, x_layout: int = moe.MOE_LAYOUT_ROWMAJOR):
    return moe.make_cfg(T=s.T if T is None else T, H=s.H, E=s.E, k=s.k, I=s.I, n_groups=s.n_groups,
                        topk_groups=s.topk_groups, score_fn=SCORE[s.score] if s.score in SCORE else 0,
                        group_score=GSCORE[s.group_score], renormalize=s.renormalize,
                        routed_scale=s.routed_scale, has_shared=s.shared, I_shared=s.I_shared,
                        act_dtype=LIB_DT[s.dtype], y_dtype=y_dtype, out_dtype=out_dtype, m_tile=m_tile,
                        x_layout=x_layout)


def route_kw(s: synth.MoeShape):
    return dict(score=SCORE[s.score], n_groups=s.n_groups, topk_groups=s.topk_groups,
                group_score=GSCORE[s.group_score])


def router_case(s: synth.MoeShape, T: Optional[int] = None, device=None, margin: float = MARGIN,
                bias: Optional[np.ndarray] = None):
    """x, w_router, bias on `device` (drawn there), host copies, and the oracle
    logits; activation rows whose routing decision is closer than `margin`
    are redrawn until every token clears it.  `bias` overrides the workload's
    logit bias."""
    device = device or dev()
    T = s.T if T is None else T
    x, w_r, bias_w = synth.router_inputs(s, device, T)
    bias = bias_w if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(device)
    xh, wh = to_np(x), to_np(w_r)
    bh = None if bias is None else bias.cpu().numpy()
    logits = oracle.router_logits(xh, wh)
    rk = route_kw(s)
    for attempt in range(1, 40):
        mg = oracle.route_margin(logits, s.k, bias=bh, **rk)
        bad = np.nonzero(mg < margin)[0]
        if len(bad) == 0:
            break
        synth.resample_rows(s, x, bad.tolist(), attempt)
        xb = to_np(x[torch.as_tensor(bad, device=x.device)])
        logits[bad] = oracle.router_logits(xb, wh)
        xh[bad] = xb
    else:
        raise RuntimeError("could not meet the routing margin")
    return dict(x=x, w_r=w_r, bias=bias, xh=xh, wh=wh, bh=bh, logits=logits)


def expert_stack(s: synth.MoeShape, device=None):
    """Routed expert weights stacked [E][I][H], [E][I][H], [E][H][I] on device."""
    device = device or dev()
    dt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    wg = torch.empty((s.E, s.I, s.H), dtype=dt, device=device)
    wu = torch.empty_like(wg)
    wd = torch.empty((s.E, s.H, s.I), dtype=dt, device=device)
    for e in range(s.E):
        g, u, d = synth.expert_weights(s, e, device)
        wg[e], wu[e], wd[e] = g, u, d
    return wg, wu, wd


def shared_stack(s: synth.MoeShape, device=None):
    if not s.shared:
        return None
    return tuple(synth.shared_weights(s, device or dev()))


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / rms(ref)."""
    rms = math.sqrt(float(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(got.astype(np.float64) - ref))) / max(rms, 1e-300)


def rel_err_bf16_out(got: np.ndarray, ref: np.ndarray) -> float:
    """Error of a bf16-rounded output beyond its own rounding: the bf16 store
    may move a value by up to 2^-8 |ref| (one half-ulp plus the fp32 error
    below it), which is removed before the max|err| / rms(ref) measure."""
    rms = math.sqrt(float(np.mean(ref.astype(np.float64) ** 2)))
    e = np.maximum(np.abs(got.astype(np.float64) - ref) - 2.0 ** -8 * np.abs(ref), 0.0)
    return float(np.max(e)) / max(rms, 1e-300)


def rel_err_allow(got: np.ndarray, ref: np.ndarray, allow: np.ndarray) -> float:
    """max(|got - ref| - allow, 0) / rms(ref): the error beyond a per-element
    allowance for roundings that the definition leaves to storage (bf16
    stores of an output or of the expert outputs)."""
    rms = math.sqrt(float(np.mean(ref.astype(np.float64) ** 2)))
    e = np.maximum(np.abs(got.astype(np.float64) - ref) - allow, 0.0)
    return float(np.max(e)) / max(rms, 1e-300)


def cover_tokens(ids, T, E, n, seed):
    """At least n seeded tokens, then one more for every expert with routed
    rows that none of them reaches (the survey's token-subset rule), plus the
    first and last token and tokens of the hottest and the coldest expert."""
    rng = np.random.default_rng(seed)
    toks = set(rng.choice(T, min(n, T), replace=False).tolist()) | {0, T - 1}
    cnt = np.bincount(ids.ravel(), minlength=E)
    seen = np.zeros(E, bool)
    seen[np.unique(ids[sorted(toks)])] = True
    for e in np.nonzero((cnt > 0) & ~seen)[0]:
        if seen[e]:
            continue
        cand = np.nonzero((ids == e).any(1))[0]
        t = int(cand[rng.integers(len(cand))])
        toks.add(t)
        seen[ids[t]] = True
    hot, cold = int(np.argmax(cnt)), int(np.argmin(np.where(cnt > 0, cnt, 1 << 30)))
    toks |= {int(np.nonzero((ids == hot).any(1))[0][0]), int(np.nonzero((ids == cold).any(1))[0][-1])}
    toks = np.array(sorted(toks))
    assert set(np.unique(ids[toks]).tolist()) == set(np.nonzero(cnt)[0].tolist())
    return toks


def host(t: torch.Tensor) -> np.ndarray:
    return to_np(t)


def values(t: torch.Tensor) -> np.ndarray:
    return f64(t)
