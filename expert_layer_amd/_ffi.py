"""ctypes declarations of the C ABI in include/moe.h (libexpert_layer_amd.so).

Loading fails loudly if the library has not been built: there is no fallback
path of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libexpert_layer_amd.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP4_E2M1 = 0, 1, 2, 3
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_GROUP_TOP2_SUM, MOE_GROUP_MAX = 0, 1
MOE_STAGE_ROUTE, MOE_STAGE_PERMUTE, MOE_STAGE_FFN, MOE_STAGE_LAYER = 0, 1, 2, 3
MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_TILED, MOE_LAYOUT_INDEXED = 0, 1, 2

EXPORTS = ("moe_validate", "moe_max_rows", "moe_workspace_bytes", "moe_ffn_workspace_bytes",
           "moe_x_perm_bytes", "moe_tiled_weights_bytes", "moe_tile_weights", "moe_route", "moe_permute", "moe_grouped_ffn",
           "moe_combine", "moe_quantize_fp8", "moe_layer", "moe_weight_table", "moe_permute_noalloc",
           "moe_route_quantize", "moe_status_string",
           "moe_last_error")


class moe_cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "E", "k", "I", "n_groups", "topk_groups",
                                              "score_fn", "group_score", "renormalize")] + \
               [("routed_scale", ctypes.c_float)] + \
               [(n, ctypes.c_int32) for n in ("has_shared", "I_shared", "act_dtype", "w_dtype",
                                              "y_dtype", "out_dtype", "m_tile", "x_layout")]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                                               "sh_gate", "sh_up", "sh_down")] + [("layout", ctypes.c_int32)] + \
               [(n, ctypes.c_void_p) for n in ("sh_s_gate", "sh_s_up", "sh_s_down", "table", "layer")] + \
               [("n_layers", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m expert_layer_amd.build` "
                              "(there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        C = ctypes.POINTER(moe_cfg)
        W = ctypes.POINTER(moe_weights)
        L.moe_validate.argtypes = [C]
        L.moe_validate.restype = i32
        L.moe_max_rows.argtypes = [C]
        L.moe_max_rows.restype = i64
        L.moe_workspace_bytes.argtypes = [C, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_ffn_workspace_bytes.argtypes = [C, i64]
        L.moe_ffn_workspace_bytes.restype = sz
        L.moe_x_perm_bytes.argtypes = [C]
        L.moe_x_perm_bytes.restype = sz
        L.moe_tiled_weights_bytes.argtypes = [C]
        L.moe_tiled_weights_bytes.restype = sz
        L.moe_tile_weights.argtypes = [C, W, P, sz, W, P]
        L.moe_tile_weights.restype = i32
        L.moe_route.argtypes = [C, P, P, P, P, P, P, P, P, sz, P]
        L.moe_route.restype = i32
        L.moe_route_quantize.argtypes = [C, P, P, P, P, P, P, P, P, P, sz, P]
        L.moe_route_quantize.restype = i32
        L.moe_permute.argtypes = [C, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.moe_permute.restype = i32
        L.moe_permute_noalloc.argtypes = [C, P, P, P, P, P, P, P, P, P, P]
        L.moe_permute_noalloc.restype = i32
        L.moe_grouped_ffn.argtypes = [C, i64, P, P, P, P, W, P, P, P, P, sz, P]
        L.moe_grouped_ffn.restype = i32
        L.moe_combine.argtypes = [C, P, P, P, P, P, P]
        L.moe_combine.restype = i32
        L.moe_quantize_fp8.argtypes = [C, P, P, P, P]
        L.moe_quantize_fp8.restype = i32
        L.moe_layer.argtypes = [C, P, P, W, P, P, P, sz, P]
        L.moe_layer.restype = i32
        L.moe_weight_table.argtypes = [C, W, i32, P]
        L.moe_weight_table.restype = i32
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib
