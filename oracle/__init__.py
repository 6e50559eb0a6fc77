"""Oracle of the MoE layer of a prefill step: numpy bindings of oracle.c.

TEST INFRASTRUCTURE ONLY.  The oracle is the independent, plain, fp64 CPU
definition the HIP path is checked against.  Only the tests, the smoke check of
the entry module and the CPU-baseline leg of the benchmark may import it.  It
shares no code with expert_layer_amd/ and never imports it.

Parity pins: every function here is pinned by the CPU test suite
(tests/test_oracle_pins.py) to results fixed independently of the oracle -- a
library routine, a closed form, an invariant, brute force or a printed value.
The only part with no such pin is a random full-size layer as a whole, whose
numerical values are fixed by nothing but the oracle itself ("parity unpinned"
beyond the invariants; the pins cover each step separately).

Array conventions: fp32 arrays are float32; bf16 arrays are uint16 bit
patterns; e4m3 arrays are uint8 codes; MXFP4 matrices are packed E2M1 codes
(uint8, two per byte, the even element in the low nibble) with uint8 E8M0
scales per 32 elements of a row.  Matrices are [out][in] row-major.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, E4M3 = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1
TOP2_SUM, MAX = 0, 1


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.orc_threads.argtypes = []
        L.orc_threads.restype = i32
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = dbl
        L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f64.restype = dbl
        L.orc_e4m3_rne_sat.argtypes = [dbl]
        L.orc_e4m3_rne_sat.restype = ctypes.c_uint8
        L.orc_bf16_rne.argtypes = [dbl]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_router_logits.argtypes = [i64, i64, i64, i32, P, i32, P, P]
        L.orc_router_logits.restype = None
        L.orc_route_select.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, dbl, P, P, P, P]
        L.orc_route_select.restype = i32
        L.orc_route_margin.argtypes = [i64, i32, i32, i32, i32, i32, i32, P, P, P]
        L.orc_route_margin.restype = i32
        L.orc_dispatch.argtypes = [i64, i32, i32, i32, P, i64, P, P, P, P, P]
        L.orc_dispatch.restype = i32
        L.orc_expert_ffn.argtypes = [i64, i64, i64, i32, P, i32, P, P, P, i32, P]
        L.orc_expert_ffn.restype = None
        L.orc_expert_ffn_fp8.argtypes = [i64, i64, i64, P, P, P, P, P, P, P, P, P, P]
        L.orc_expert_ffn_fp8.restype = None
        L.orc_e2m1_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_to_f64.restype = dbl
        L.orc_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_f64.restype = dbl
        L.orc_mxfp4_dequant.argtypes = [i64, i64, P, P, P]
        L.orc_mxfp4_dequant.restype = None
        L.orc_expert_ffn_mxfp4.argtypes = [i64, i64, i64, P, P, P, P, P, P, P, P, P, P]
        L.orc_expert_ffn_mxfp4.restype = None
        L.orc_combine.argtypes = [i64, i32, i64, P, P, P, P, P]
        L.orc_combine.restype = None
        L.orc_bf16_round_array.argtypes = [i64, P, P]
        L.orc_bf16_round_array.restype = None
        L.orc_layer.argtypes = [i64, i64, i32, i32, i64, i32, i32, i32, i32, i32, dbl,
                                i32, P, P, P, i32, P, P, P, i64, P, P, P, i32, P, P, P, P]
        L.orc_layer.restype = i32
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError(f"unsupported oracle operand dtype {a.dtype}")


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_threads())


# ---------------------------------------------------------------- formats

def bf16_to_f64(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([L.orc_bf16_to_f64(int(v)) for v in b.ravel()]).reshape(b.shape)


def e4m3_to_f64(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.orc_e4m3_to_f64(int(v)) for v in c.ravel()]).reshape(c.shape)


def e4m3_rne_sat(values) -> np.ndarray:
    L = lib()
    v = np.asarray(values, dtype=np.float64)
    return np.array([L.orc_e4m3_rne_sat(float(x)) for x in v.ravel()],
                    dtype=np.uint8).reshape(v.shape)


def quantize_rows_e4m3(x):
    """Per-token 1 x 128 quantisation of activations for fp8 experts.  For each
    row and block of 128 columns: s = fp32(max|x|) / 448 in fp32 (1 for an
    all-zero block), code = e4m3_rne_sat(fp32(x / s)).  The AFD page runs its
    MoE GEMMs in fp8 (section 1, the MoE MFU figure's caption: "fp8 DeepGEMM";
    section 7: W8A8) without printing a quantiser; the fp8 expert-parallel
    workload states per-token 1 x 128 activation scales.  The rule is read as
    the one this oracle applies to the SwiGLU intermediate (S9).
    x: bf16 bit patterns (uint16) or fp32, [n][H] with H a multiple of 128.
    Returns (codes uint8 [n][H], scales float32 [n][H/128])."""
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bf16: the top half of an fp32
        x = (x.astype(np.uint32) << 16).view(np.float32)
    x = x.astype(np.float32)
    n, H = x.shape
    assert H % 128 == 0
    blk = x.reshape(n, H // 128, 128)
    amax = np.abs(blk).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    v = (blk / s[:, :, None]).astype(np.float32)
    q = e4m3_rne_sat(v.reshape(-1)).reshape(n, H)
    return q, s


def bf16_rne(values) -> np.ndarray:
    L = lib()
    v = np.asarray(values, dtype=np.float64)
    return np.array([L.orc_bf16_rne(float(x)) for x in v.ravel()],
                    dtype=np.uint16).reshape(v.shape)


def bf16_round(values) -> np.ndarray:
    """Each value rounded to bf16 as bf16_rne does (nearest-even, decided on
    its fp32 value) and widened back to fp64: what a bf16 store keeps."""
    v = _c(np.asarray(values, dtype=np.float64))
    out = np.empty_like(v)
    lib().orc_bf16_round_array(v.size, _p(v), _p(out))
    return out


# ----------------------------------------------------------------- layer

def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """fp32 logits [T][E] = fp32(x @ w_router^T) summed in fp64."""
    x, w_router = _c(x), _c(w_router)
    T, H = x.shape
    E = w_router.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(T, H, E, _dtype_code(x), _p(x), _dtype_code(w_router),
                            _p(w_router), _p(out))
    return out


def route_select(logits: np.ndarray, k: int, score: int = SOFTMAX, n_groups: int = 1,
                 topk_groups: int = 1, group_score: int = TOP2_SUM, renormalize: bool = True,
                 routed_scale: float = 1.0, bias: Optional[np.ndarray] = None):
    """(topk_ids int32 [T][k], topk_w float32 [T][k]) from fp32 logits."""
    logits = _c(np.asarray(logits, dtype=np.float32))
    bias = None if bias is None else _c(np.asarray(bias, dtype=np.float32))
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = lib().orc_route_select(T, E, k, score, n_groups, topk_groups, group_score,
                                int(renormalize), float(routed_scale), _p(logits),
                                _p(bias), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("orc_route_select: invalid routing arguments")
    return ids, w


def route_margin(logits: np.ndarray, k: int, score: int = SOFTMAX, n_groups: int = 1,
                 topk_groups: int = 1, group_score: int = TOP2_SUM,
                 bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-token gap (fp64) at the k-th expert key and at the last kept group."""
    logits = _c(np.asarray(logits, dtype=np.float32))
    bias = None if bias is None else _c(np.asarray(bias, dtype=np.float32))
    T, E = logits.shape
    m = np.empty(T, dtype=np.float64)
    rc = lib().orc_route_margin(T, E, k, score, n_groups, topk_groups, group_score,
                                _p(logits), _p(bias), _p(m))
    if rc != 0:
        raise ValueError("orc_route_margin: invalid routing arguments")
    return m


def dispatch(ids: np.ndarray, E: int, m_tile: int = 1, rows_cap: Optional[int] = None):
    """Counting sort of (token, choice) pairs by expert; see orc_dispatch."""
    ids = _c(np.asarray(ids, dtype=np.int32))
    T, k = ids.shape
    if rows_cap is None:
        rows_cap = T * k + E * (m_tile - 1)
    counts = np.empty(E, dtype=np.int32)
    offs = np.empty(E + 1, dtype=np.int32)
    poffs = np.empty(E + 1, dtype=np.int32)
    row_src = np.empty(max(rows_cap, 1), dtype=np.int32)
    tok_row = np.empty((T, k), dtype=np.int32)
    rc = lib().orc_dispatch(T, k, E, m_tile, _p(ids), rows_cap, _p(counts), _p(offs),
                            _p(poffs), _p(row_src), _p(tok_row))
    if rc != 0:
        raise ValueError("orc_dispatch: id out of range or rows_cap too small")
    return dict(counts=counts, offsets=offs, padded_offsets=poffs,
                row_src=row_src[:rows_cap], tok_row=tok_row)


def expert_ffn(x_rows: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
               h_bf16: bool = False) -> np.ndarray:
    """y [n][H] (fp64) of one SwiGLU expert on n rows; h_bf16 stores the
    intermediate activation in bf16 (the activation format of a bf16 layer)."""
    x_rows, w_gate, w_up, w_down = _c(x_rows), _c(w_gate), _c(w_up), _c(w_down)
    n, H = x_rows.shape
    I = w_gate.shape[0]
    assert w_gate.shape == (I, H) and w_up.shape == (I, H) and w_down.shape == (H, I)
    assert w_gate.dtype == w_up.dtype == w_down.dtype
    y = np.empty((n, H), dtype=np.float64)
    lib().orc_expert_ffn(n, H, I, _dtype_code(x_rows), _p(x_rows), _dtype_code(w_gate),
                         _p(w_gate), _p(w_up), _p(w_down), int(h_bf16), _p(y))
    return y


def expert_ffn_fp8(xq, xs, wg, sg, wu, su, wd, sd, return_h: bool = False):
    """y [n][H] (fp64) of one fp8 block-scaled SwiGLU expert; see orc_expert_ffn_fp8.
    With return_h, also the SwiGLU intermediate a [n][I] before its requantisation."""
    xq, xs, wg, sg, wu, su, wd, sd = (_c(a) for a in (xq, xs, wg, sg, wu, su, wd, sd))
    n, H = xq.shape
    I = wg.shape[0]
    assert H % 128 == 0 and I % 128 == 0
    assert xs.shape == (n, H // 128) and sg.shape == (I // 128, H // 128)
    assert sd.shape == (H // 128, I // 128) and wd.shape == (H, I)
    y = np.empty((n, H), dtype=np.float64)
    a = np.empty((n, I), dtype=np.float64) if return_h else None
    lib().orc_expert_ffn_fp8(n, H, I, _p(xq), _p(xs), _p(wg), _p(sg), _p(wu), _p(su),
                             _p(wd), _p(sd), _p(y), _p(a))
    return (y, a) if return_h else y


def e2m1_to_f64(codes) -> np.ndarray:
    """OCP MX FP4 E2M1 code (low 4 bits) -> value."""
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.orc_e2m1_to_f64(int(v) & 0xF) for v in c.ravel()]).reshape(c.shape)


def e8m0_to_f64(codes) -> np.ndarray:
    """OCP MX E8M0 scale code -> 2^(code - 127) (255: NaN)."""
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.orc_e8m0_to_f64(int(v)) for v in c.ravel()]).reshape(c.shape)


def mxfp4_to_f64(codes, scales) -> np.ndarray:
    """Dequantised MXFP4 matrix [rows][K] from packed codes [rows][K/2] (the
    low nibble holds the even element) and E8M0 scales [rows][K/32]."""
    codes, scales = _c(np.asarray(codes, np.uint8)), _c(np.asarray(scales, np.uint8))
    rows, K = codes.shape[0], codes.shape[1] * 2
    assert K % 32 == 0 and scales.shape == (rows, K // 32)
    out = np.empty((rows, K), dtype=np.float64)
    lib().orc_mxfp4_dequant(rows, K, _p(codes), _p(scales), _p(out))
    return out


def expert_ffn_mxfp4(xq, xs, wg, sg, wu, su, wd, sd, return_h: bool = False):
    """y [n][H] (fp64) of one SwiGLU expert on e4m3 rows with MXFP4 weights
    (packed codes wg, wu [I][H/2], wd [H][I/2]; E8M0 scales sg, su [I][H/32],
    sd [H][I/32]); see orc_expert_ffn_mxfp4."""
    xq, xs, wg, sg, wu, su, wd, sd = (_c(a) for a in (xq, xs, wg, sg, wu, su, wd, sd))
    n, H = xq.shape
    I = wg.shape[0]
    assert H % 128 == 0 and I % 128 == 0 and xs.shape == (n, H // 128)
    assert wg.shape == (I, H // 2) and sg.shape == (I, H // 32) and wd.shape == (H, I // 2) and sd.shape == (H, I // 32)
    y = np.empty((n, H), dtype=np.float64)
    a = np.empty((n, I), dtype=np.float64) if return_h else None
    lib().orc_expert_ffn_mxfp4(n, H, I, _p(xq), _p(xs), _p(wg), _p(sg), _p(wu), _p(su), _p(wd), _p(sd),
                               _p(y), _p(a))
    return (y, a) if return_h else y


U32 = 2.0 ** -24  # unit roundoff of fp32


def ffn_h_error_bound(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, kblock: int = 128) -> np.ndarray:
    """A bound on |a~ - a| for the SwiGLU intermediate a = silu(g) * u of one
    block-scaled expert, g = x . w_gate^T and u = x . w_up^T; x [n][K] and the
    weights [I][K] are the exact dequantised operands (code * scale, fp64).
    a~ is what any fp32 evaluation of the block-scale promotion may give that
      (i)   sums each kblock-wide K block of code products in fp32, in any order,
      (ii)  multiplies each block sum by the fp32 product of its scales and
            accumulates the K / kblock results in fp32, in any order,
      (iii) evaluates silu(g) in fp32 with a relative error of at most
            (8 + |g|) u (an exponential of a rounded fp32 argument: the
            argument's rounding moves the result by |g| u), and
      (iv)  rounds silu * u to fp32.
    Each term of g then passes through at most m = kblock + K / kblock + 2
    roundings, so |g~ - g| <= gamma_m * sum_k |x_k w_k| with gamma_m =
    m u / (1 - m u) (the recursive-summation bound for any order, Higham,
    "Accuracy and Stability of Numerical Algorithms", section 3.1), likewise
    for u; |silu'| <= 1.1 carries dg into silu."""
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    wu = np.asarray(w_up, dtype=np.float64)
    K = x.shape[1]
    assert wg.shape[1] == K and wu.shape == wg.shape and K % kblock == 0
    m = kblock + K // kblock + 2
    gam = m * U32 / (1.0 - m * U32)
    g, u = x @ wg.T, x @ wu.T
    ax = np.abs(x)
    dg = gam * (ax @ np.abs(wg).T)
    du = gam * (ax @ np.abs(wu).T)
    with np.errstate(over="ignore"):
        sil = g / (1.0 + np.exp(-g))
    dsil = 1.1 * dg + (8.0 + np.abs(g)) * U32 * np.abs(sil)
    return dsil * (np.abs(u) + du) + np.abs(sil) * du + U32 * np.abs(sil * u)


def fp8_h_alternatives(a: np.ndarray, da):
    """The requantisation decisions of the fp8 intermediate that an evaluation
    within da of a (da: a bound on |a~ - a| per element, as ffn_h_error_bound
    gives, or one number for all) may take the other way.  For each row and
    128-column block of a (fp64, [n][I]) the decision is the one
    orc_expert_ffn_fp8 takes: s = fp32(max|fp32(a)|) / 448, v = fp32(fp32(a) / s),
    code = e4m3_rne_sat(v).  An evaluation a~ may move v by up to
      dv = da / s + |v| (max_block(da) / max|a| + 4 u)
    (its own block maximum moves s; two roundings on each side), so a decision
    is ambiguous when v lies within dv of the midpoint between its two
    neighbouring e4m3 values.  Returns, per row, a list of (column i, dh), the
    decisions nearest their midpoint (relative to dv) first: dh is the change of
    the dequantised intermediate a'_i when the other neighbour is taken."""
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    n, I = a32.shape
    assert I % 128 == 0
    da = np.broadcast_to(np.asarray(da, dtype=np.float64), (n, I))
    vals = e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8))  # the finite non-negative values, ascending
    blk = a32.reshape(n, I // 128, 128)
    dab = da.reshape(n, I // 128, 128)
    amax = np.abs(blk).max(axis=2)
    s = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
    v = (blk / s[:, :, None]).astype(np.float32).astype(np.float64)
    av = np.minimum(np.abs(v), 448.0)
    rel_s = np.where(amax > 0, dab.max(axis=2) / np.maximum(amax.astype(np.float64), 1e-300), 0.0)
    dv = dab / s[:, :, None].astype(np.float64) + np.abs(v) * (rel_s[:, :, None] + 4.0 * U32)
    hi_i = np.clip(np.searchsorted(vals, av, side="left"), 1, len(vals) - 1)
    lo, hi = vals[hi_i - 1], vals[hi_i]
    mid = 0.5 * (lo + hi)
    amb = np.abs(av - mid) <= dv
    chosen = e4m3_to_f64(e4m3_rne_sat(v.reshape(-1))).reshape(v.shape)
    other = np.where(np.abs(chosen) == lo, hi, lo) * np.sign(v)
    dh = (other - chosen) * s[:, :, None].astype(np.float64)
    closeness = np.abs(av - mid) / np.maximum(dv, 1e-300)
    out = [[] for _ in range(n)]
    for r, b, j in zip(*np.nonzero(amb)):
        out[r].append((float(closeness[r, b, j]), int(b * 128 + j), float(dh[r, b, j])))
    return [[(i, d) for _, i, d in sorted(row)] for row in out]


def combine(y_rows: np.ndarray, tok_row: np.ndarray, topk_w: np.ndarray,
            y_shared: Optional[np.ndarray] = None) -> np.ndarray:
    """out [T][H] (fp64) = sum_j w[t][j] * y_rows[tok_row[t][j]] (+ y_shared[t])."""
    y_rows = _c(np.asarray(y_rows, dtype=np.float64))
    tok_row = _c(np.asarray(tok_row, dtype=np.int32))
    topk_w = _c(np.asarray(topk_w, dtype=np.float32))
    y_shared = None if y_shared is None else _c(np.asarray(y_shared, dtype=np.float64))
    T, k = tok_row.shape
    H = y_rows.shape[1]
    assert tok_row.min(initial=0) >= 0 and tok_row.max(initial=-1) < y_rows.shape[0]
    out = np.empty((T, H), dtype=np.float64)
    lib().orc_combine(T, k, H, _p(y_rows), _p(tok_row), _p(topk_w), _p(y_shared), _p(out))
    return out


def layer(x, w_router, w_gate, w_up, w_down, k: int, score: int = SOFTMAX, n_groups: int = 1,
          topk_groups: int = 1, group_score: int = TOP2_SUM, renormalize: bool = True,
          routed_scale: float = 1.0, bias=None, shared=None, h_bf16: bool = False):
    """The whole layer.  w_gate/w_up [E][I][H], w_down [E][H][I]; shared is
    None or (sh_gate [Is][H], sh_up [Is][H], sh_down [H][Is]).
    Returns dict(out fp64 [T][H], logits, topk_ids, topk_w)."""
    x, w_router = _c(x), _c(w_router)
    w_gate, w_up, w_down = _c(w_gate), _c(w_up), _c(w_down)
    T, H = x.shape
    E, I, _ = w_gate.shape
    assert w_router.shape == (E, H) and w_down.shape == (E, H, I)
    assert x.dtype == w_router.dtype
    bias = None if bias is None else _c(np.asarray(bias, dtype=np.float32))
    if shared is not None:
        sg, su, sd = (_c(a) for a in shared)
        Is = sg.shape[0]
    else:
        sg = su = sd = None
        Is = 0
    out = np.empty((T, H), dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = lib().orc_layer(T, H, E, k, I, score, n_groups, topk_groups, group_score,
                         int(renormalize), float(routed_scale), _dtype_code(x), _p(x),
                         _p(w_router), _p(bias), _dtype_code(w_gate), _p(w_gate), _p(w_up),
                         _p(w_down), Is, _p(sg), _p(su), _p(sd), int(h_bf16), _p(out),
                         _p(logits), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("orc_layer: invalid arguments")
    return dict(out=out, logits=logits, topk_ids=ids, topk_w=w)
