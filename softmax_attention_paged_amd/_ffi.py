"""ctypes mirror of include/attn.h and the loader of the in-tree HIP library.

Argument marshalling only: no step of the attention is computed here. If the
library has not been built, loading raises immediately; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libattn_mi355x.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE_TOO_SMALL = 3
ATTN_ERR_HIP = 4

ATTN_BF16 = 0
ATTN_FP8_E4M3 = 1
ATTN_FP32 = 2

_c = ctypes
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class PrefillParams(ctypes.Structure):
    _fields_ = [
        ("q", _p), ("q_stride_tok", _i64), ("q_stride_head", _i64),
        ("k", _p), ("v", _p),
        ("k_stride_page", _i64), ("k_stride_tok", _i64), ("k_stride_head", _i64),
        ("v_stride_page", _i64), ("v_stride_tok", _i64), ("v_stride_head", _i64),
        ("cu_seqlens_q", _p), ("cu_seqlens_kv", _p), ("seq_lens_kv", _p),
        ("block_table", _p), ("block_table_stride", _i32), ("page_size", _i32), ("num_pages", _i32),
        ("batch", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
        ("head_dim_qk", _i32), ("head_dim_v", _i32),
        ("max_seqlen_q", _i32), ("max_seqlen_kv", _i32),
        ("softmax_scale", ctypes.c_float), ("causal", _i32),
        ("o", _p), ("o_stride_tok", _i64), ("o_stride_head", _i64),
        ("lse", _p), ("window_enabled", _i32), ("window_left", _i32),
        ("qkv_dtype", ctypes.c_int), ("q_scale", ctypes.c_float), ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float), ("total_q", _i32), ("kv_splits", _i32),
        ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
    ]


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("q", _p), ("k_cache", _p), ("v_cache", _p),
        ("k_stride_page", _i64), ("k_stride_tok", _i64), ("k_stride_head", _i64),
        ("v_stride_page", _i64), ("v_stride_tok", _i64), ("v_stride_head", _i64),
        ("kv_dtype", ctypes.c_int), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("seq_lens", _p), ("block_table", _p), ("block_table_stride", _i32),
        ("batch", _i32), ("q_len", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
        ("head_dim_qk", _i32), ("head_dim_v", _i32),
        ("page_size", _i32), ("num_pages", _i32), ("max_seq_len", _i32),
        ("softmax_scale", ctypes.c_float), ("causal", _i32), ("num_splits", _i32),
        ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
        ("o", _p), ("lse", _p),
        ("window_enabled", _i32), ("window_left", _i32), ("packed_q", _i32),
        ("total_kv_tokens", _i64), ("q_dtype", ctypes.c_int), ("q_scale", ctypes.c_float),
    ]


class DecodePlanInfo(ctypes.Structure):
    _fields_ = [
        ("group", _i32), ("fold", _i32), ("q_groups", _i32), ("rows_per_unit", _i32),
        ("num_splits", _i32), ("split_tokens", _i32), ("num_units", _i64),
        ("workspace_bytes", ctypes.c_size_t), ("key_ranges", _i32),
    ]


class CacheAppendParams(ctypes.Structure):
    _fields_ = [
        ("k_new", _p), ("k_new_stride_tok", _i64), ("k_new_stride_head", _i64),
        ("v_new", _p), ("v_new_stride_tok", _i64), ("v_new_stride_head", _i64),
        ("k_cache", _p), ("k_stride_page", _i64), ("k_stride_tok", _i64), ("k_stride_head", _i64),
        ("v_cache", _p), ("v_stride_page", _i64), ("v_stride_tok", _i64), ("v_stride_head", _i64),
        ("cache_dtype", ctypes.c_int), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("slot_mapping", _p), ("layer_base_rows", _i64), ("num_cache_rows", _i64),
        ("num_tokens", _i32), ("num_kv_heads", _i32), ("head_dim_k", _i32), ("head_dim_v", _i32),
        ("page_size", _i32),
    ]


class MlaKvPackParams(ctypes.Structure):
    _fields_ = [
        ("k_nope", _p), ("k_nope_stride_tok", _i64), ("k_nope_stride_head", _i64),
        ("k_rope", _p), ("k_rope_stride_tok", _i64),
        ("v", _p), ("v_stride_tok", _i64), ("v_stride_head", _i64),
        ("k_out", _p), ("k_out_stride_tok", _i64), ("k_out_stride_head", _i64),
        ("v_out", _p), ("v_out_stride_tok", _i64), ("v_out_stride_head", _i64),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("num_tokens", _i32), ("num_heads", _i32), ("d_nope", _i32), ("d_rope", _i32), ("d_v", _i32),
    ]


EXPORTS = {
    "attn_prefill": (ctypes.c_int, [ctypes.POINTER(PrefillParams), _p]),
    "attn_prefill_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(PrefillParams)]),
    "attn_decode_plan": (ctypes.c_int, [ctypes.POINTER(DecodeParams), ctypes.POINTER(DecodePlanInfo)]),
    "attn_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(DecodeParams)]),
    "attn_decode_paged": (ctypes.c_int, [ctypes.POINTER(DecodeParams), _p]),
    "attn_decode_paged_noalloc": (ctypes.c_int, [ctypes.POINTER(DecodeParams), _p]),
    "attn_decode_paged_split": (ctypes.c_int, [ctypes.POINTER(DecodeParams), _p]),
    "attn_decode_paged_merge": (ctypes.c_int, [ctypes.POINTER(DecodeParams), _p]),
    "attn_merge_lse": (ctypes.c_int, [_p, _p, _i32, _i64, _i32, _p, ctypes.c_int, _p, _p]),
    "attn_cache_append": (ctypes.c_int, [ctypes.POINTER(CacheAppendParams), _p]),
    "attn_mla_kv_pack_fp8": (ctypes.c_int, [ctypes.POINTER(MlaKvPackParams), _p]),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (once). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not built: {LIB_PATH} is missing. "
                "Build it with `python -m softmax_attention_paged_amd.build` "
                "(or __graft_entry__.build()).")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        self.status = status
        name = lib.attn_status_string(status).decode()
        msg = lib.attn_last_error().decode()
        super().__init__(f"{where}: {name}: {msg}")


def check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, where)
