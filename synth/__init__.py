"""Seeded synthetic inputs for the MoE layer of a prefill step.

This module draws the layer's inputs (activations, router weights, expert
weights, biases, fp8 codes and scales, dispatched row counts).  It holds none of
the layer's own arithmetic: no routing, no dispatch, no GEMM, no combine.  Both
the oracle and the HIP path consume exactly the arrays produced here.

Random numbers come from one counter-based generator, SplitMix64 (Steele, Lea
and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): the
n-th 64-bit output of stream `key` is mix(key + (n + 1) * 0x9E3779B97F4A7C15).
Two outputs give one standard normal by the Box-Muller transform in fp64.  The
same torch integer code runs on the CPU and on the GPU, so a tensor drawn on
either device holds the same values (up to the last bit of fp64 log/cos, which
the fp32/bf16 rounding that follows hides in all but ~1e-13 of the elements).

Workload shapes follow the configurations the layer is measured on:
  c1_tiny_fp32      T=256   H=512  E=8   k=2 I=1024  softmax, renormalised, fp32
  c2_mixtral_bf16   T=4096  H=4096 E=8   k=2 I=14336 softmax, renormalised
  c3_dsv3_bf16      T=8192  H=7168 E=256 k=8 I=2048  sigmoid, 8 groups keep 4,
                    renormalised then x2.5, one shared expert (I=2048)
  c4_qwen3_skew_bf16 T=16384 (12 sequences, CV 0.2) H=4096 E=128 k=8 I=1536
                    softmax, renormalised, Zipf(1.1) logit bias (hottest expert
                    about 10x the mean load)
  c5_dsv3_ep_fp8    65536 dispatched rows, 8 local experts, H=7168 I=2048,
                    counts ~ Multinomial(65536, p_e ~ 1/(e+1)), e4m3 operands
                    with 128x128 weight block scales and 1x128 row scales
Distributions: activations ~ N(0, 1); weights ~ N(0, 1/fan_in) (fan_in = H for
the router, gate and up matrices, I for the down matrix).  Matrices are stored
[out][in] row-major.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os
from typing import Dict, Optional, Sequence

import torch

__all__ = [
    "MoeShape", "CONFIGS", "config", "normal", "uniform", "router_inputs",
    "resample_rows", "expert_weights", "shared_weights", "zipf_logit_bias",
    "sequence_lengths", "fp8_counts", "quantize_rows_fp8", "quantize_blocks_fp8",
    "fp8_expert_weights", "fp8_rows", "stream_key",
]

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_CHUNK = 1 << 24


def _s64(c: int) -> int:
    """Python int in [0, 2^64) -> the int64 with the same bit pattern."""
    c &= (1 << 64) - 1
    return c - (1 << 64) if c >= (1 << 63) else c


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _s64(_M1)
    z = (z ^ _srl(z, 27)) * _s64(_M2)
    return z ^ _srl(z, 31)


def _mix_int(z: int) -> int:
    m = (1 << 64) - 1
    z &= m
    z = ((z ^ (z >> 30)) * _M1) & m
    z = ((z ^ (z >> 27)) * _M2) & m
    return z ^ (z >> 31)


def stream_key(seed: int, *names) -> int:
    """A 64-bit stream key derived from a seed and a tuple of names/ints."""
    k = _mix_int(seed * _GOLDEN + 0x1234567)
    for n in names:
        if isinstance(n, str):
            for ch in n.encode():
                k = _mix_int(k ^ (ch + 0x100))
        else:
            k = _mix_int(k ^ ((int(n) + 0x10000) * _GOLDEN))
    return k


def _bits(key: int, start: int, n: int, device) -> torch.Tensor:
    """Outputs start .. start+n-1 of stream `key` as int64 bit patterns."""
    idx = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix(idx * _s64(_GOLDEN) + _s64(key))


def _unit(bits: torch.Tensor) -> torch.Tensor:
    """53 random bits -> fp64 uniform in (0, 1)."""
    return (_srl(bits, 11).to(torch.float64) + 0.5) * (2.0 ** -53)


def uniform(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """n fp64 uniforms in (0, 1): elements start .. start+n-1 of stream key."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        out[c0:c1] = _unit(_bits(key, start + c0, c1 - c0, device))
    return out


def normal(key: int, shape: Sequence[int], std: float = 1.0, device="cpu",
           dtype=torch.float32, start: int = 0) -> torch.Tensor:
    """Standard normals scaled by std, element i drawn from outputs 2i, 2i+1
    of stream key (Box-Muller), computed in fp64 and rounded to dtype."""
    n = int(math.prod(shape))
    out = torch.empty(n, dtype=dtype, device=device)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        b = _bits(key, 2 * (start + c0), 2 * (c1 - c0), device).view(-1, 2)
        u1 = _unit(b[:, 0])
        u2 = _unit(b[:, 1])
        z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
        out[c0:c1] = (z * std).to(torch.float32).to(dtype)
    return out.view(*shape)


# ------------------------------------------------------------------ configs

@dataclasses.dataclass(frozen=True)
class MoeShape:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    score: str = "softmax"          # "softmax" | "sigmoid"
    n_groups: int = 1
    topk_groups: int = 1
    group_score: str = "top2_sum"   # "top2_sum" | "max"
    renormalize: bool = True
    routed_scale: float = 1.0
    shared: bool = False
    I_shared: int = 0
    dtype: str = "bf16"             # "f32" | "bf16" | "fp8"
    seed: int = 0
    zipf_s: float = 0.0             # softmax logit bias exponent (0 = none)
    n_seqs: int = 1
    seq_cv: float = 0.0

    def with_(self, **kw) -> "MoeShape":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, MoeShape] = {
    "c1_tiny_fp32": MoeShape("c1_tiny_fp32", T=256, H=512, E=8, k=2, I=1024,
                             dtype="f32", seed=1),
    "c2_mixtral_bf16": MoeShape("c2_mixtral_bf16", T=4096, H=4096, E=8, k=2, I=14336,
                                seed=2),
    "c3_dsv3_bf16": MoeShape("c3_dsv3_bf16", T=8192, H=7168, E=256, k=8, I=2048,
                             score="sigmoid", n_groups=8, topk_groups=4,
                             routed_scale=2.5, shared=True, I_shared=2048, seed=3),
    "c4_qwen3_skew_bf16": MoeShape("c4_qwen3_skew_bf16", T=16384, H=4096, E=128, k=8,
                                   I=1536, seed=4, zipf_s=1.1, n_seqs=12, seq_cv=0.2),
    "c5_dsv3_ep_fp8": MoeShape("c5_dsv3_ep_fp8", T=65536, H=7168, E=8, k=1, I=2048,
                               dtype="fp8", seed=5, zipf_s=1.0),
}


def config(name: str, **overrides) -> MoeShape:
    return CONFIGS[name].with_(**overrides) if overrides else CONFIGS[name]


def _tdtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


# ------------------------------------------------------------ routed layers

def router_inputs(cfg: MoeShape, device="cpu", T: Optional[int] = None, with_bias: bool = True):
    """x [T][H] and w_router [E][H] in the layer dtype (fp32 or bf16), and the
    softmax logit bias [E] (fp32) or None."""
    T = cfg.T if T is None else T
    dt = _tdtype(cfg.dtype)
    x = normal(stream_key(cfg.seed, "x", 0), (T, cfg.H), 1.0, device, dt)
    w_r = normal(stream_key(cfg.seed, "w_router"), (cfg.E, cfg.H),
                 1.0 / math.sqrt(cfg.H), device, dt)
    bias = None
    if with_bias and cfg.zipf_s > 0 and cfg.score == "softmax":
        bias = zipf_logit_bias(cfg, device)
    return x, w_r, bias


def resample_rows(cfg: MoeShape, x: torch.Tensor, rows: Sequence[int], attempt: int) -> None:
    """Redraw the listed activation rows in place from the stream of the given
    attempt (attempt >= 1); row t of attempt a is a fixed function of
    (seed, a, t), so any row can be regenerated on any device."""
    key = stream_key(cfg.seed, "x", attempt)
    for t in rows:
        x[t] = normal(key, (cfg.H,), 1.0, x.device, x.dtype, start=int(t) * cfg.H)


def expert_weights(cfg: MoeShape, e: int, device="cpu", I: Optional[int] = None,
                   tag: str = "expert"):
    """(w_gate [I][H], w_up [I][H], w_down [H][I]) of expert e in the layer dtype."""
    I = cfg.I if I is None else I
    dt = _tdtype(cfg.dtype)
    g = normal(stream_key(cfg.seed, tag, e, "gate"), (I, cfg.H), 1.0 / math.sqrt(cfg.H), device, dt)
    u = normal(stream_key(cfg.seed, tag, e, "up"), (I, cfg.H), 1.0 / math.sqrt(cfg.H), device, dt)
    d = normal(stream_key(cfg.seed, tag, e, "down"), (cfg.H, I), 1.0 / math.sqrt(I), device, dt)
    return g, u, d


def shared_weights(cfg: MoeShape, device="cpu"):
    return expert_weights(cfg, 0, device, I=cfg.I_shared, tag="shared")


_ALPHA_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_alpha.json")


def zipf_alpha(cfg: MoeShape) -> float:
    """Scale of the Zipf logit bias, calibrated offline (calibrate_zipf.py) so
    that the hottest expert receives about 10x the mean load."""
    with open(_ALPHA_FILE) as f:
        table = json.load(f)
    if cfg.name not in table:
        raise KeyError(f"no calibrated Zipf scale for {cfg.name}; run synth/calibrate_zipf.py")
    return float(table[cfg.name]["alpha"])


def zipf_logit_bias(cfg: MoeShape, device="cpu", alpha: Optional[float] = None) -> torch.Tensor:
    """b_e = -alpha * s * ln(e + 1): a Zipf(s) preference over experts, as a
    logit offset (fp32)."""
    a = zipf_alpha(cfg) if alpha is None else alpha
    e = torch.arange(cfg.E, dtype=torch.float64)
    return (-a * cfg.zipf_s * torch.log(e + 1.0)).to(torch.float32).to(device)


def sequence_lengths(cfg: MoeShape):
    """Per-sequence lengths ~ N(mu, (cv*mu)^2), mu = T / n_seqs, rounded,
    clamped to >= 1, the last one adjusted so that they sum to T.  They are
    batch metadata only: the layer is token-wise."""
    n = cfg.n_seqs
    if n <= 1:
        return [cfg.T]
    mu = cfg.T / n
    z = normal(stream_key(cfg.seed, "seq_lens"), (n,), 1.0, "cpu", torch.float64)
    lens = [max(1, int(round(mu + cfg.seq_cv * mu * float(v)))) for v in z[:-1]]
    lens.append(cfg.T - sum(lens))
    if lens[-1] < 1:
        raise ValueError("sequence length draw left no tokens for the last sequence")
    return lens


# ------------------------------------------------------------------- fp8 EP

def fp8_counts(cfg: MoeShape):
    """Per-expert row counts ~ Multinomial(T, p_e ~ 1/(e+1)^s): each row draws
    one uniform and takes the expert whose cumulative probability first exceeds
    it."""
    s = cfg.zipf_s if cfg.zipf_s > 0 else 1.0
    p = [1.0 / (e + 1.0) ** s for e in range(cfg.E)]
    tot = sum(p)
    cum, acc = [], 0.0
    for v in p:
        acc += v / tot
        cum.append(acc)
    cum[-1] = 1.0
    u = uniform(stream_key(cfg.seed, "counts"), cfg.T)
    idx = torch.searchsorted(torch.tensor(cum, dtype=torch.float64), u, right=True)
    idx = torch.clamp(idx, max=cfg.E - 1)
    return torch.bincount(idx, minlength=cfg.E).tolist()


def _e4m3(v: torch.Tensor) -> torch.Tensor:
    """fp32 -> OCP e4m3 codes (uint8), nearest-even, saturated to +-448."""
    return torch.clamp(v, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_rows_fp8(cfg: MoeShape, x: torch.Tensor, key: int, row_start: int = 0):
    """Per-row 1x128 block quantisation of fp32 rows [n][C]:
    s = u * absmax / 448 with u ~ U(0.5, 2) per block (fp32), q = e4m3(x / s).
    Returns (codes uint8 [n][C], scales fp32 [n][C/128])."""
    n, C = x.shape
    xb = x.view(n, C // 128, 128)
    amax = xb.abs().amax(dim=2)
    u = 0.5 + 1.5 * uniform(key, n * (C // 128), x.device,
                            start=row_start * (C // 128)).view(n, C // 128)
    s = (u.to(torch.float32) * amax / 448.0).to(torch.float32)
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = _e4m3(xb / s.unsqueeze(2)).view(n, C)
    return q, s


def quantize_blocks_fp8(cfg: MoeShape, w: torch.Tensor, key: int):
    """128x128 block quantisation of an fp32 matrix [R][C] (R, C multiples of
    128): s = u * absmax / 448 per block, u ~ U(0.5, 2).  Returns (codes uint8
    [R][C], scales fp32 [R/128][C/128])."""
    R, C = w.shape
    wb = w.view(R // 128, 128, C // 128, 128)
    amax = wb.abs().amax(dim=(1, 3))
    u = 0.5 + 1.5 * uniform(key, (R // 128) * (C // 128), w.device).view(R // 128, C // 128)
    s = (u.to(torch.float32) * amax / 448.0).to(torch.float32)
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = _e4m3(wb / s.view(R // 128, 1, C // 128, 1)).view(R, C)
    return q, s


def fp8_expert_weights(cfg: MoeShape, e: int, device="cpu"):
    """e4m3 codes and 128x128 scales of expert e:
    (wg, sg, wu, su, wd, sd), wg/wu [I][H], wd [H][I], scales [out/128][in/128]."""
    out = []
    for name, shape, fan in (("gate", (cfg.I, cfg.H), cfg.H), ("up", (cfg.I, cfg.H), cfg.H),
                             ("down", (cfg.H, cfg.I), cfg.I)):
        w = normal(stream_key(cfg.seed, "expert", e, name), shape, 1.0 / math.sqrt(fan),
                   device, torch.float32)
        q, s = quantize_blocks_fp8(cfg, w, stream_key(cfg.seed, "wscale", e, name))
        out += [q, s]
    return tuple(out)


def quantize_mxfp4(w: torch.Tensor):
    """OCP MX v1.0 conversion of an fp32 matrix [R][C] (C a multiple of 32) to
    MXFP4: per 32 consecutive elements of a row, the shared exponent
    x = floor(log2(max|w|)) - 2 (2: the largest E2M1 exponent) as an E8M0 code
    x + 127 (127 for an all-zero block), and each element w / 2^x rounded to
    the nearest E2M1 value (ties to even, saturating at +-6).  Returns (packed
    codes uint8 [R][C/2], the even element in the low nibble; scales uint8
    [R][C/32])."""
    R, C = w.shape
    wb = w.view(R, C // 32, 32).to(torch.float32)
    amax = wb.abs().amax(dim=2)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2,
                    torch.zeros_like(amax))
    v = wb / torch.exp2(e)[:, :, None]
    a = v.abs()
    # E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); a tie goes to the even code
    idx = ((a > 0.25).to(torch.int32) + (a >= 0.75).to(torch.int32) + (a > 1.25).to(torch.int32)
           + (a >= 1.75).to(torch.int32) + (a > 2.5).to(torch.int32) + (a >= 3.5).to(torch.int32)
           + (a > 5.0).to(torch.int32))
    code = (idx | torch.where(v < 0, 8, 0).to(torch.int32)).view(R, C)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).to(torch.uint8)
    return packed, (e + 127).to(torch.uint8)


def mxfp4_expert_weights(cfg: MoeShape, e: int, device="cpu"):
    """MXFP4 codes and E8M0 scales of expert e, from the same fp32 draws as
    fp8_expert_weights: (wg, sg, wu, su, wd, sd), wg/wu [I][H/2], wd [H][I/2],
    scales [out][in/32]."""
    out = []
    for name, shape, fan in (("gate", (cfg.I, cfg.H), cfg.H), ("up", (cfg.I, cfg.H), cfg.H),
                             ("down", (cfg.H, cfg.I), cfg.I)):
        w = normal(stream_key(cfg.seed, "expert", e, name), shape, 1.0 / math.sqrt(fan),
                   device, torch.float32)
        out += list(quantize_mxfp4(w))
    return tuple(out)


def fp8_rows(cfg: MoeShape, n: int, device="cpu", start: int = 0):
    """Dispatched activation rows start .. start+n-1: N(0, 1) quantised with
    1x128 row scales.  Returns (codes uint8 [n][H], scales fp32 [n][H/128])."""
    x = normal(stream_key(cfg.seed, "rows"), (n, cfg.H), 1.0, device, torch.float32,
               start=start * cfg.H)
    return quantize_rows_fp8(cfg, x, stream_key(cfg.seed, "rowscale"), row_start=start)
