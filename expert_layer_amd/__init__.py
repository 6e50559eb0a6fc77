"""MI355X-native Mixture-of-Experts layer of a prefill step.

Thin Python binding of the C ABI in include/moe.h: each function has the name
of the C entry point and only marshals arguments (torch tensors -> device
pointers, the current torch stream -> hipStream_t).  Every step of the layer
runs in the HIP kernels of libexpert_layer_amd.so; if the library is missing
the first call raises ImportError -- there is no other path.

    cfg = make_cfg(T=8192, H=7168, E=256, k=8, I=2048, ...)
    ws = workspace(cfg, MOE_STAGE_LAYER, device)
    moe_layer(cfg, w_router, bias, weights(w_gate, w_up, w_down), x, out, ws)
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _ffi
from ._ffi import (MOE_BF16, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
                   MOE_F32, MOE_FP8_E4M3, MOE_FP4_E2M1, MOE_GROUP_MAX, MOE_GROUP_TOP2_SUM, MOE_OK, MOE_SCORE_SIGMOID,
                   MOE_SCORE_SOFTMAX, MOE_STAGE_FFN, MOE_STAGE_LAYER, MOE_STAGE_PERMUTE, MOE_STAGE_ROUTE,
                   MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_TILED, MOE_LAYOUT_INDEXED, moe_cfg, moe_weights)

__all__ = [
    "MoeError", "make_cfg", "weights", "workspace", "moe_validate", "moe_max_rows", "moe_workspace_bytes",
    "moe_ffn_workspace_bytes", "moe_route", "moe_route_quantize", "moe_permute", "moe_grouped_ffn",
    "moe_combine", "moe_quantize_fp8", "moe_layer", "moe_weight_table", "weight_table", "moe_status_string",
    "moe_last_error", "moe_cfg", "moe_weights", "lib_path", "MOE_OK", "MOE_ERR_INVALID_ARG",
    "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP", "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3",
    "MOE_FP4_E2M1", "MOE_SCORE_SOFTMAX", "MOE_SCORE_SIGMOID", "MOE_GROUP_TOP2_SUM", "MOE_GROUP_MAX",
    "MOE_STAGE_ROUTE", "MOE_STAGE_PERMUTE", "MOE_STAGE_FFN", "MOE_STAGE_LAYER", "MOE_LAYOUT_ROWMAJOR",
    "MOE_LAYOUT_TILED", "MOE_LAYOUT_INDEXED", "moe_tiled_weights_bytes", "moe_tile_weights", "tile_weights",
    "moe_x_perm_bytes", "x_perm_buffer", "moe_permute_noalloc",
]

lib_path = _ffi.LIB_PATH


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{moe_status_string(status)}: {message}")
        self.status = status


def make_cfg(T: int, H: int, E: int, k: int, I: int, n_groups: int = 1, topk_groups: int = 1,
             score_fn: int = MOE_SCORE_SOFTMAX, group_score: int = MOE_GROUP_TOP2_SUM,
             renormalize: bool = True, routed_scale: float = 1.0, has_shared: bool = False,
             I_shared: int = 0, act_dtype: int = MOE_BF16, w_dtype: Optional[int] = None,
             y_dtype: int = MOE_F32, out_dtype: int = MOE_BF16, m_tile: int = 0,
             x_layout: int = MOE_LAYOUT_ROWMAJOR) -> moe_cfg:
    return moe_cfg(T=T, H=H, E=E, k=k, I=I, n_groups=n_groups, topk_groups=topk_groups,
                   score_fn=score_fn, group_score=group_score, renormalize=int(bool(renormalize)),
                   routed_scale=routed_scale, has_shared=int(bool(has_shared)), I_shared=I_shared,
                   act_dtype=act_dtype, w_dtype=act_dtype if w_dtype is None else w_dtype,
                   y_dtype=y_dtype, out_dtype=out_dtype, m_tile=m_tile, x_layout=x_layout)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, torch.Tensor):
        if not t.is_cuda:
            raise ValueError("device tensors only: the C ABI takes device pointers")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        return t.data_ptr()
    raise TypeError(f"cannot pass {type(t)} as a device pointer")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, moe_last_error())


def weights(w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None, sh_gate=None, sh_up=None,
            sh_down=None, layout: int = MOE_LAYOUT_ROWMAJOR, sh_s_gate=None, sh_s_up=None,
            sh_s_down=None, table=None, layer=None, n_layers: int = 0) -> moe_weights:
    """table / layer / n_layers: pointer-table weights (moe_weights.table);
    the other matrices are then ignored and may be None."""
    return moe_weights(*(_ptr(t) for t in (w_gate, w_up, w_down, s_gate, s_up, s_down, sh_gate,
                                             sh_up, sh_down)), layout,
                       *(_ptr(t) for t in (sh_s_gate, sh_s_up, sh_s_down, table, layer)), n_layers)


def moe_weight_table(cfg: moe_cfg, layers) -> list:
    """Host table of moe_weight_table for contiguous per-layer moe_weights:
    n_layers * (E + has_shared) * 6 device addresses (0 for NULL)."""
    n = len(layers)
    arr = (moe_weights * n)(*layers)
    G = cfg.E + (1 if cfg.has_shared else 0)
    out = (ctypes.c_void_p * (n * G * 6))()
    _check(_ffi.lib().moe_weight_table(ctypes.byref(cfg), arr, n, out))
    return [v or 0 for v in out]


def weight_table(cfg: moe_cfg, layers, device) -> torch.Tensor:
    """The table of moe_weight_table copied to a device int64 tensor (torch
    allocates it; keep it alive while calls use it)."""
    return torch.tensor(moe_weight_table(cfg, layers), dtype=torch.int64).to(device)


def moe_x_perm_bytes(cfg: moe_cfg) -> int:
    return _ffi.lib().moe_x_perm_bytes(ctypes.byref(cfg))


def x_perm_buffer(cfg: moe_cfg, device) -> torch.Tensor:
    """An x_perm buffer for cfg.x_layout: [moe_max_rows, H] in the activation
    dtype when row-major, a flat byte buffer when tiled (one byte, unused, when
    indexed)."""
    if cfg.x_layout in (MOE_LAYOUT_TILED, MOE_LAYOUT_INDEXED):
        return torch.empty(max(moe_x_perm_bytes(cfg), 1), dtype=torch.uint8, device=device)
    dt = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_FP8_E4M3: torch.uint8}[cfg.act_dtype]
    return torch.empty((moe_max_rows(cfg), cfg.H), dtype=dt, device=device)


def moe_tiled_weights_bytes(cfg: moe_cfg) -> int:
    return _ffi.lib().moe_tiled_weights_bytes(ctypes.byref(cfg))


def moe_tile_weights(cfg: moe_cfg, src: moe_weights, dst, stream=None) -> moe_weights:
    """Writes the tiled copy of row-major bf16 weights into the device buffer dst
    and returns the moe_weights that point into it (keep dst alive)."""
    out = moe_weights()
    _check(_ffi.lib().moe_tile_weights(ctypes.byref(cfg), ctypes.byref(src), _ptr(dst),
                                       dst.numel() * dst.element_size(), ctypes.byref(out), _stream(stream)))
    return out


def tile_weights(cfg: moe_cfg, src: moe_weights, device):
    """(tiled moe_weights, owning byte buffer): allocates the buffer (torch) and
    calls moe_tile_weights on the current stream."""
    buf = torch.empty(max(moe_tiled_weights_bytes(cfg), 1), dtype=torch.uint8, device=device)
    return moe_tile_weights(cfg, src, buf), buf


def moe_validate(cfg: moe_cfg) -> int:
    return _ffi.lib().moe_validate(ctypes.byref(cfg))


def moe_max_rows(cfg: moe_cfg) -> int:
    return _ffi.lib().moe_max_rows(ctypes.byref(cfg))


def moe_workspace_bytes(cfg: moe_cfg, stage: int) -> int:
    return _ffi.lib().moe_workspace_bytes(ctypes.byref(cfg), stage)


def moe_ffn_workspace_bytes(cfg: moe_cfg, n_rows_cap: int) -> int:
    return _ffi.lib().moe_ffn_workspace_bytes(ctypes.byref(cfg), int(n_rows_cap))


def workspace(cfg: moe_cfg, stage: int, device, n_rows_cap: Optional[int] = None) -> torch.Tensor:
    """A device byte buffer of moe_workspace_bytes(cfg, stage), or of
    moe_ffn_workspace_bytes(cfg, n_rows_cap) when n_rows_cap is given
    (torch allocates it)."""
    n = moe_workspace_bytes(cfg, stage) if n_rows_cap is None else moe_ffn_workspace_bytes(cfg, n_rows_cap)
    if n == ctypes.c_size_t(-1).value:
        _check(moe_validate(cfg))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def moe_route(cfg, x, w_router, bias, logits_in, logits_out, topk_ids, topk_w, ws=None, stream=None):
    p, n = _ws(ws)
    _check(_ffi.lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits_in),
                                _ptr(logits_out), _ptr(topk_ids), _ptr(topk_w), p, n, _stream(stream)))


def moe_route_quantize(cfg, x, w_router, bias, logits_out, topk_ids, topk_w, x_q, x_scale, ws=None, stream=None):
    """moe_route on bf16 x that also writes moe_quantize_fp8's x_q and x_scale."""
    p, n = _ws(ws)
    _check(_ffi.lib().moe_route_quantize(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits_out),
                                         _ptr(topk_ids), _ptr(topk_w), _ptr(x_q), _ptr(x_scale), p, n,
                                         _stream(stream)))


def moe_permute(cfg, x, x_scale, topk_ids, expert_counts, expert_offsets, row_src, tok_row, x_perm,
                x_perm_scale, ws, stream=None):
    p, n = _ws(ws)
    _check(_ffi.lib().moe_permute(ctypes.byref(cfg), _ptr(x), _ptr(x_scale), _ptr(topk_ids),
                                  _ptr(expert_counts), _ptr(expert_offsets), _ptr(row_src), _ptr(tok_row),
                                  _ptr(x_perm), _ptr(x_perm_scale), p, n, _stream(stream)))


def moe_permute_noalloc(cfg, x, x_scale, topk_ids, expert_counts, expert_offsets, row_src, tok_row, x_perm,
                        x_perm_scale, stream=None):
    """moe_permute with the library's static scratch instead of a workspace."""
    _check(_ffi.lib().moe_permute_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(x_scale), _ptr(topk_ids),
                                          _ptr(expert_counts), _ptr(expert_offsets), _ptr(row_src), _ptr(tok_row),
                                          _ptr(x_perm), _ptr(x_perm_scale), _stream(stream)))


def moe_grouped_ffn(cfg, n_rows_cap, x_rows, x_scale, expert_offsets, w: moe_weights, x_tokens, y_rows,
                    y_shared, ws, stream=None, row_src=None):
    """row_src: the dispatch map of moe_permute, read with cfg.x_layout ==
    MOE_LAYOUT_INDEXED (x_rows is then x itself)."""
    p, n = _ws(ws)
    _check(_ffi.lib().moe_grouped_ffn(ctypes.byref(cfg), int(n_rows_cap), _ptr(x_rows), _ptr(x_scale),
                                      _ptr(expert_offsets), _ptr(row_src), ctypes.byref(w), _ptr(x_tokens),
                                      _ptr(y_rows), _ptr(y_shared), p, n, _stream(stream)))


def moe_combine(cfg, y_rows, tok_row, topk_w, y_shared, out, stream=None):
    _check(_ffi.lib().moe_combine(ctypes.byref(cfg), _ptr(y_rows), _ptr(tok_row), _ptr(topk_w),
                                  _ptr(y_shared), _ptr(out), _stream(stream)))


def moe_quantize_fp8(cfg, x, x_q, x_scale, stream=None):
    """x [T][H] bf16 -> x_q [T][H] e4m3 codes (uint8) and x_scale [T][H/128] fp32."""
    _check(_ffi.lib().moe_quantize_fp8(ctypes.byref(cfg), _ptr(x), _ptr(x_q), _ptr(x_scale), _stream(stream)))


def moe_layer(cfg, w_router, bias, w: moe_weights, x, out, ws, stream=None):
    p, n = _ws(ws)
    _check(_ffi.lib().moe_layer(ctypes.byref(cfg), _ptr(w_router), _ptr(bias), ctypes.byref(w), _ptr(x),
                                _ptr(out), p, n, _stream(stream)))


def moe_status_string(status: int) -> str:
    return _ffi.lib().moe_status_string(status).decode()


def moe_last_error() -> str:
    return _ffi.lib().moe_last_error().decode()
