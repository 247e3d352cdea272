"""Torch-facing binding of the C ABI (include/attn.h).

Argument marshalling only: every function here checks tensor metadata, takes
data_ptr()s and strides, allocates outputs/workspace with torch (plumbing) and
calls the HIP library on torch's current stream. Nothing is computed here,
and there is no fallback path: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import math

import torch

from . import _ffi

_BF16 = torch.bfloat16


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _rows_contiguous(t: torch.Tensor) -> bool:
    """Channels (the last dimension) adjacent in memory; an empty tensor has
    no rows to read."""
    return t.numel() == 0 or t.stride(-1) == 1


def _check_out(t: torch.Tensor, shape: tuple, dtypes: tuple, dev: torch.device, name: str) -> None:
    """A caller-provided output: the kernels write exactly `shape` elements
    of one of `dtypes`, rows contiguous, on q's device."""
    _need(t.device == dev, f"{name} must be on {dev}")
    _need(t.dtype in dtypes, f"{name} must be {' or '.join(str(d) for d in dtypes)}")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_decode_inputs(q, k_cache, v_cache, block_table, seq_lens, dv) -> None:
    """Tensor metadata the C ABI cannot see: devices, ranks and the sizes the
    kernels index with."""
    k4 = _as_4d_cache(k_cache)
    _need(k4.dim() == 4, "k_cache must be [pages, page_size, Hkv, D] or a latent [pages, page_size, D]")
    for t, name in ((k_cache, "k_cache"), (block_table, "block_table"), (seq_lens, "seq_lens")):
        _need(t.device == q.device, f"{name} must be on {q.device}")
    _need(k4.shape[3] == q.shape[3] and _rows_contiguous(k4), "k_cache rows must hold the query's head_dim, contiguous")
    if v_cache is not None:
        v4 = _as_4d_cache(v_cache)
        _need(v_cache.device == q.device, f"v_cache must be on {q.device}")
        _need(v4.dim() == 4 and tuple(v4.shape[:3]) == tuple(k4.shape[:3]), "v_cache must match k_cache's pages, rows and heads")
        _need(v4.shape[3] >= dv and _rows_contiguous(v4), "v_cache rows must hold head_dim_v channels, contiguous")
    else:
        _need(dv <= k4.shape[3], "a latent cache's V (its first head_dim_v channels) cannot exceed its rows")
    b = q.shape[0]
    _need(block_table.dim() == 2 and block_table.shape[0] >= b, "block_table must be [B, max_pages]")
    _need(seq_lens.dim() == 1 and seq_lens.numel() >= b, "seq_lens must hold B lengths")


def _kv_code(cache: torch.Tensor, kv_dtype: str | None) -> int:
    if cache.dtype == _BF16:
        return _ffi.ATTN_BF16
    if cache.dtype in (torch.float8_e4m3fn, torch.uint8):
        _need(cache.dtype == torch.float8_e4m3fn or kv_dtype == "fp8_e4m3",
              "uint8 caches need kv_dtype='fp8_e4m3'")
        return _ffi.ATTN_FP8_E4M3
    raise ValueError(f"unsupported cache dtype {cache.dtype}")


def _as_4d_cache(cache: torch.Tensor) -> torch.Tensor:
    # A latent cache [pages, page_size, D] is the 4-D layout with one KV head.
    return cache.unsqueeze(2) if cache.dim() == 3 else cache


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------

def decode_params(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len, softmax_scale,
                  causal=False, head_dim_v=None, kv_dtype=None, k_scale=1.0, v_scale=1.0,
                  num_splits=0, workspace=None, out=None, lse=None, window_left=-1,
                  packed_q=False, total_kv_tokens=0, q_scale=None) -> _ffi.DecodeParams:
    """Fill the C parameter struct from tensors (no device access). A uint8
    (or float8_e4m3fn) q holds E4M3 codes with dequantisation scale q_scale."""
    k4 = _as_4d_cache(k_cache)
    v4 = _as_4d_cache(v_cache if v_cache is not None else k_cache)
    b, q_len, hq, dqk = q.shape
    dv = head_dim_v if head_dim_v is not None else v4.shape[3]
    p = _ffi.DecodeParams()
    p.q = _ptr(q)
    p.k_cache, p.v_cache = _ptr(k4), _ptr(v4)
    p.k_stride_page, p.k_stride_tok, p.k_stride_head = k4.stride(0), k4.stride(1), k4.stride(2)
    p.v_stride_page, p.v_stride_tok, p.v_stride_head = v4.stride(0), v4.stride(1), v4.stride(2)
    p.kv_dtype = _kv_code(k4, kv_dtype)
    p.k_scale, p.v_scale = float(k_scale), float(v_scale)
    p.seq_lens, p.block_table = _ptr(seq_lens), _ptr(block_table)
    p.block_table_stride = block_table.stride(0)
    p.batch, p.q_len, p.num_q_heads, p.num_kv_heads = b, q_len, hq, k4.shape[2]
    p.head_dim_qk, p.head_dim_v = dqk, dv
    p.page_size, p.num_pages, p.max_seq_len = k4.shape[1], k4.shape[0], int(max_seq_len)
    p.softmax_scale, p.causal, p.num_splits = float(softmax_scale), int(bool(causal)), int(num_splits)
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p.o, p.lse = _ptr(out), _ptr(lse)
    p.window_enabled, p.window_left = int(window_left >= 0), max(int(window_left), 0)
    p.packed_q = int(bool(packed_q))
    p.total_kv_tokens = int(total_kv_tokens)
    if _is_fp8_codes(q):
        _need(q_scale is not None, "fp8 q needs q_scale")
        p.q_dtype, p.q_scale = _ffi.ATTN_FP8_E4M3, float(q_scale)
    else:
        p.q_dtype, p.q_scale = _ffi.ATTN_BF16, 1.0
    return p


def _is_fp8_codes(t: torch.Tensor) -> bool:
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def decode_plan(params: _ffi.DecodeParams) -> dict:
    info = _ffi.DecodePlanInfo()
    _ffi.check(_ffi.load().attn_decode_plan(ctypes.byref(params), ctypes.byref(info)), "attn_decode_plan")
    return {name: getattr(info, name) for name, _ in _ffi.DecodePlanInfo._fields_}


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len, softmax_scale,
                 causal=False, head_dim_v=None, kv_dtype=None, k_scale=1.0, v_scale=1.0,
                 num_splits=0, workspace=None, out=None, return_lse=False, window_left=-1,
                 packed_q=False, total_kv_tokens=0, lse=None, phase="both", q_scale=None):
    """Paged decode (split-KV + LSE merge). Returns out, or (out, lse).

    phase "split" or "merge" enqueues only that kernel of the call
    (attn_decode_paged_split / attn_decode_paged_merge): pass the same out,
    lse and workspace to both.

    q [B, q_len, Hq, Dqk] bf16; caches [pages, page_size, Hkv, D] (or a 3-D
    latent cache, pass v_cache=None and head_dim_v=512); block_table
    [B, max_pages] int32; seq_lens [B] int32. window_left >= 0 limits each
    row to the q_len block plus window_left keys of context (-1: full
    history); packed_q packs rows as token * G + head. total_kv_tokens (the
    host's sum of seq_lens, 0 if unknown) lets the planner size the splits
    so every unit is resident at once.
    """
    _need(q.is_cuda and (q.dtype == _BF16 or _is_fp8_codes(q)) and q.is_contiguous(),
          "q must be a contiguous bf16 (or fp8 code) CUDA tensor")
    _need(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "block_table/seq_lens must be int32")
    _need(block_table.stride(1) == 1 and seq_lens.is_contiguous(), "block_table rows and seq_lens must be contiguous")
    b, q_len, hq, _ = q.shape
    k4 = _as_4d_cache(k_cache)
    dv = head_dim_v if head_dim_v is not None else _as_4d_cache(v_cache if v_cache is not None else k_cache).shape[3]
    _check_decode_inputs(q, k_cache, v_cache, block_table, seq_lens, dv)
    if out is None:
        out = torch.empty((b, q_len, hq, dv), dtype=_BF16, device=q.device)
    _check_out(out, (b, q_len, hq, dv), (_BF16,), q.device, "out")
    _need(out.is_contiguous(), "out must be contiguous bf16")
    if lse is not None:
        _check_out(lse, (b, q_len, hq), (torch.float32,), q.device, "lse")
    _need(lse is None or (lse.dtype == torch.float32 and lse.is_contiguous()), "lse must be contiguous float32")
    _need(workspace is None or (workspace.device == q.device and workspace.is_contiguous()),
          f"workspace must be a contiguous tensor on {q.device}")
    if lse is not None:
        return_lse = True
    elif return_lse:
        lse = torch.empty((b, q_len, hq), dtype=torch.float32, device=q.device)
    entry = {"both": "attn_decode_paged", "split": "attn_decode_paged_split",
             "merge": "attn_decode_paged_merge"}.get(phase)
    _need(entry is not None, "phase must be 'both', 'split' or 'merge'")
    p = decode_params(q, k_cache, v_cache, block_table, seq_lens, max_seq_len=max_seq_len,
                      softmax_scale=softmax_scale, causal=causal, head_dim_v=dv, kv_dtype=kv_dtype,
                      k_scale=k_scale, v_scale=v_scale, num_splits=num_splits, workspace=workspace,
                      out=out, lse=lse, window_left=window_left, packed_q=packed_q,
                      total_kv_tokens=total_kv_tokens, q_scale=q_scale)
    lib = _ffi.load()
    if workspace is None:
        need = lib.attn_decode_workspace_size(ctypes.byref(p))
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            p.workspace, p.workspace_bytes = workspace.data_ptr(), need
    _ffi.check(getattr(lib, entry)(ctypes.byref(p), _stream(q.device)), entry)
    del k4
    return (out, lse) if return_lse else out


def decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, *, max_seq_len, softmax_scale,
                         causal=False, head_dim_v=None, kv_dtype=None, k_scale=1.0, v_scale=1.0,
                         num_splits=0, out=None, lse=None, window_left=-1, packed_q=False,
                         total_kv_tokens=0, q_scale=None):
    """decode_paged through attn_decode_paged_noalloc: the split partials go
    to the library's static per-device scratch, so with `out` (and `lse`,
    if wanted) given the call allocates nothing. Returns out, or (out, lse)
    when lse is given."""
    _need(q.is_cuda and (q.dtype == _BF16 or _is_fp8_codes(q)) and q.is_contiguous(),
          "q must be a contiguous bf16 (or fp8 code) CUDA tensor")
    _need(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "block_table/seq_lens must be int32")
    _need(block_table.stride(1) == 1 and seq_lens.is_contiguous(), "block_table rows and seq_lens must be contiguous")
    b, q_len, hq, _ = q.shape
    dv = head_dim_v if head_dim_v is not None else _as_4d_cache(v_cache if v_cache is not None else k_cache).shape[3]
    _check_decode_inputs(q, k_cache, v_cache, block_table, seq_lens, dv)
    if out is None:
        out = torch.empty((b, q_len, hq, dv), dtype=_BF16, device=q.device)
    _check_out(out, (b, q_len, hq, dv), (_BF16,), q.device, "out")
    _need(out.is_contiguous(), "out must be contiguous bf16")
    if lse is not None:
        _check_out(lse, (b, q_len, hq), (torch.float32,), q.device, "lse")
    _need(lse is None or (lse.dtype == torch.float32 and lse.is_contiguous()), "lse must be contiguous float32")
    p = decode_params(q, k_cache, v_cache, block_table, seq_lens, max_seq_len=max_seq_len,
                      softmax_scale=softmax_scale, causal=causal, head_dim_v=dv, kv_dtype=kv_dtype,
                      k_scale=k_scale, v_scale=v_scale, num_splits=num_splits, workspace=None,
                      out=out, lse=lse, window_left=window_left, packed_q=packed_q,
                      total_kv_tokens=total_kv_tokens, q_scale=q_scale)
    _ffi.check(_ffi.load().attn_decode_paged_noalloc(ctypes.byref(p), _stream(q.device)), "attn_decode_paged_noalloc")
    return (out, lse) if lse is not None else out


# --------------------------------------------------------------------------
# Prefill
# --------------------------------------------------------------------------

def _prefill_params(q, k, v, cu_seqlens_q, out, lse, max_seqlen_q, max_seqlen_kv, softmax_scale, causal,
                    cu_seqlens_kv, seq_lens_kv, block_table, window_left, q_scale, k_scale, v_scale, kv_splits):
    fp8 = q.dtype == torch.float8_e4m3fn
    _need(q.is_cuda and q.dtype in (_BF16, torch.float8_e4m3fn) and (q.stride(2) == 1 or q.numel() == 0),
          "q must be bf16 or float8_e4m3fn CUDA with contiguous channels")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share one dtype")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.is_contiguous(), "cu_seqlens_q must be contiguous int32")
    paged = block_table is not None
    tq, hq, dqk = q.shape
    dv = v.shape[-1]
    _need(k.dim() == (4 if paged else 3) and v.dim() == k.dim(),
          "k and v must be [pages, page_size, Hkv, D] (paged) or [Tk, Hkv, D] (dense)")
    for t, name in ((k, "k"), (v, "v"), (cu_seqlens_q, "cu_seqlens_q")):
        _need(t.device == q.device, f"{name} must be on {q.device}")
    _need(tuple(v.shape[:-1]) == tuple(k.shape[:-1]), "k and v must match in all but their channels")
    _need(k.shape[-1] == dqk and _rows_contiguous(k) and _rows_contiguous(v),
          "k rows must hold the query's head_dim and k, v rows must be contiguous")
    hkv = k.shape[2] if paged else k.shape[1]
    p = _ffi.PrefillParams()
    p.q, p.q_stride_tok, p.q_stride_head = q.data_ptr(), q.stride(0), q.stride(1)
    p.k, p.v = k.data_ptr(), v.data_ptr()
    if paged:
        _need(block_table.dtype == torch.int32 and block_table.stride(1) == 1, "block_table must be int32 rows")
        _need(seq_lens_kv is not None and seq_lens_kv.dtype == torch.int32, "paged mode needs int32 seq_lens_kv")
        _need(block_table.device == q.device and seq_lens_kv.device == q.device, f"block_table, seq_lens_kv must be on {q.device}")
        _need(block_table.dim() == 2 and block_table.shape[0] >= cu_seqlens_q.numel() - 1,
              "block_table must be [B, max_pages]")
        _need(seq_lens_kv.numel() >= cu_seqlens_q.numel() - 1, "seq_lens_kv must hold B lengths")
        p.k_stride_page, p.k_stride_tok, p.k_stride_head = k.stride(0), k.stride(1), k.stride(2)
        p.v_stride_page, p.v_stride_tok, p.v_stride_head = v.stride(0), v.stride(1), v.stride(2)
        p.seq_lens_kv, p.block_table = seq_lens_kv.data_ptr(), block_table.data_ptr()
        p.block_table_stride, p.page_size, p.num_pages = block_table.stride(0), k.shape[1], k.shape[0]
    else:
        _need(cu_seqlens_kv is not None and cu_seqlens_kv.dtype == torch.int32, "dense mode needs int32 cu_seqlens_kv")
        _need(cu_seqlens_kv.device == q.device and cu_seqlens_kv.numel() == cu_seqlens_q.numel(),
              f"cu_seqlens_kv must be on {q.device} and hold B + 1 offsets")
        p.k_stride_tok, p.k_stride_head = k.stride(0), k.stride(1)
        p.v_stride_tok, p.v_stride_head = v.stride(0), v.stride(1)
        p.cu_seqlens_kv = cu_seqlens_kv.data_ptr()
    p.cu_seqlens_q = cu_seqlens_q.data_ptr()
    p.batch = cu_seqlens_q.numel() - 1
    p.num_q_heads, p.num_kv_heads, p.head_dim_qk, p.head_dim_v = hq, hkv, dqk, dv
    p.max_seqlen_q, p.max_seqlen_kv = int(max_seqlen_q), int(max_seqlen_kv)
    p.softmax_scale, p.causal = float(softmax_scale), int(bool(causal))
    if out is not None:
        _check_out(out, (tq, hq, dv), (_BF16,), q.device, "out")
        _need(_rows_contiguous(out), "out rows must be contiguous")
        p.o, p.o_stride_tok, p.o_stride_head = out.data_ptr(), out.stride(0), out.stride(1)
    else:                                   # sizing only: the layout a fresh output gets
        p.o, p.o_stride_tok, p.o_stride_head = 0, hq * dv, dv
    p.lse = _ptr(lse)
    p.window_enabled, p.window_left = int(window_left >= 0), max(int(window_left), 0)
    if fp8:
        p.qkv_dtype = _ffi.ATTN_FP8_E4M3
        p.q_scale, p.k_scale, p.v_scale = float(q_scale), float(k_scale), float(v_scale)
    p.total_q, p.kv_splits = tq, int(kv_splits)
    return p


def prefill_workspace_size(q, k, v, cu_seqlens_q, *, max_seqlen_q, max_seqlen_kv, causal=False, cu_seqlens_kv=None,
                           seq_lens_kv=None, block_table=None, window_left=-1, kv_splits=0):
    """Bytes of workspace prefill() with these arguments (and a fresh,
    contiguous output) would use for key splits; 0 when it runs unsplit."""
    p = _prefill_params(q, k, v, cu_seqlens_q, None, None, max_seqlen_q, max_seqlen_kv, 1.0, causal, cu_seqlens_kv,
                        seq_lens_kv, block_table, window_left, 1.0, 1.0, 1.0, kv_splits)
    return int(_ffi.load().attn_prefill_workspace_size(ctypes.byref(p)))


def prefill(q, k, v, cu_seqlens_q, *, max_seqlen_q, max_seqlen_kv, softmax_scale, causal=False,
            cu_seqlens_kv=None, seq_lens_kv=None, block_table=None, out=None, return_lse=False,
            window_left=-1, q_scale=1.0, k_scale=1.0, v_scale=1.0, kv_splits=0, workspace=None):
    """Ragged prefill over dense (cu_seqlens_kv) or paged (block_table +
    seq_lens_kv) KV. q [Tq, Hq, D] bf16; dense k/v [Tk, Hkv, D]; paged k/v
    [pages, page_size, Hkv, D]. FP8: q, k, v all float8_e4m3fn codes (dense,
    D = 192 for q/k and 128 for v) with per-tensor scales (value = code *
    scale); the output stays bf16. window_left >= 0: row i of a request sees
    no key before Lk - Lq - window_left + i (-1: full history). kv_splits
    (0: the planner's choice, 1: none) splits each query tile's keys over
    several workgroups merged by LSE; the workspace for it (a uint8 CUDA
    tensor) is allocated here unless passed. Returns out [Tq, Hq, Dv], or
    (out, lse)."""
    tq, hq, _ = q.shape
    if out is None:
        out = torch.empty((tq, hq, v.shape[-1]), dtype=_BF16, device=q.device)
    lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device) if return_lse else None
    p = _prefill_params(q, k, v, cu_seqlens_q, out, lse, max_seqlen_q, max_seqlen_kv, softmax_scale, causal,
                        cu_seqlens_kv, seq_lens_kv, block_table, window_left, q_scale, k_scale, v_scale, kv_splits)
    need = _ffi.load().attn_prefill_workspace_size(ctypes.byref(p))
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _need(workspace.device == q.device and workspace.is_contiguous(), f"workspace must be a contiguous tensor on {q.device}")
        p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _ffi.check(_ffi.load().attn_prefill(ctypes.byref(p), _stream(q.device)), "attn_prefill")
    return (out, lse) if return_lse else out


# --------------------------------------------------------------------------
# Merge
# --------------------------------------------------------------------------

def merge_lse(o_parts: torch.Tensor, lse_parts: torch.Tensor, *, out_dtype=_BF16, out=None,
              return_lse=True):
    """Merge split partials o_parts [S, R, Dv] fp32 / lse_parts [S, R] fp32
    (base 2). Returns (o [R, Dv], lse [R]) or o."""
    _need(o_parts.dtype == torch.float32 and lse_parts.dtype == torch.float32, "partials must be fp32")
    _need(o_parts.is_contiguous() and lse_parts.is_contiguous(), "partials must be contiguous")
    s, r, dv = o_parts.shape
    _need(tuple(lse_parts.shape) == (s, r), "lse_parts must be [S, R]")
    _need(o_parts.is_cuda and lse_parts.device == o_parts.device, "partials must be CUDA tensors on one device")
    if out is None:
        out = torch.empty((r, dv), dtype=out_dtype, device=o_parts.device)
    _check_out(out, (r, dv), (torch.bfloat16, torch.float32), o_parts.device, "out")
    _need(out.is_contiguous(), "out must be contiguous")
    code = {torch.bfloat16: _ffi.ATTN_BF16, torch.float32: _ffi.ATTN_FP32}[out.dtype]
    lse = torch.empty((r,), dtype=torch.float32, device=o_parts.device) if return_lse else None
    _ffi.check(_ffi.load().attn_merge_lse(o_parts.data_ptr(), lse_parts.data_ptr(), s, r, dv,
                                          out.data_ptr(), code, _ptr(lse), _stream(o_parts.device)),
               "attn_merge_lse")
    return (out, lse) if return_lse else out


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


# --------------------------------------------------------------------------
# The prologue: cache append and the MLA K/V pack
# --------------------------------------------------------------------------

def _cache_rows(cache: torch.Tensor) -> tuple[int, int, int, int]:
    """(page_size, stride_page, stride_tok, stride_head) of a paged cache
    [pages, page_size, Hkv, D] (a latent [pages, page_size, D] has one head)."""
    c = _as_4d_cache(cache)
    return c.shape[1], c.stride(0), c.stride(1), c.stride(2)


def cache_append(k_new, v_new, k_cache, v_cache, slot_mapping, *, layer_base_rows=0, k_scale=1.0,
                 v_scale=1.0, kv_dtype: str | None = None):
    """Write new tokens k_new / v_new [N, Hkv, D] (bf16) into the paged caches
    at token row layer_base_rows + max(slot_mapping[i], 0) (int64 [N]). FP8
    caches (float8_e4m3fn, or uint8 with kv_dtype='fp8_e4m3') store E4M3
    codes of value / scale. v_new / v_cache may be None (latent caches)."""
    _need(k_new.dtype == _BF16 and (v_new is None or v_new.dtype == _BF16), "new K/V must be bf16")
    _need(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
    _need((v_new is None) == (v_cache is None), "v_new and v_cache go together")
    kc = _as_4d_cache(k_cache)
    code = _kv_code(kc, kv_dtype)
    dev = k_new.device
    _need(k_new.dim() == 3 and kc.dim() == 4, "k_new must be [N, Hkv, D] and k_cache [pages, page_size, Hkv, D]")
    _need(kc.device == dev and slot_mapping.device == dev, f"k_cache and slot_mapping must be on {dev}")
    _need(tuple(k_new.shape[1:]) == tuple(kc.shape[2:]) and _rows_contiguous(k_new) and _rows_contiguous(kc),
          "k_new rows must match the cache's heads and channels, both contiguous")
    _need(slot_mapping.dim() == 1 and slot_mapping.numel() == k_new.shape[0] and slot_mapping.is_contiguous(),
          "slot_mapping must hold one contiguous int64 slot per new token")
    if v_new is not None:
        vc4 = _as_4d_cache(v_cache)
        _need(v_new.device == dev and v_cache.device == dev, f"v_new and v_cache must be on {dev}")
        _need(v_new.dim() == 3 and vc4.dim() == 4 and v_new.shape[0] == k_new.shape[0]
              and tuple(v_new.shape[1:]) == tuple(vc4.shape[2:]) and tuple(vc4.shape[:3]) == tuple(kc.shape[:3])
              and _rows_contiguous(v_new) and _rows_contiguous(vc4),
              "v_new and v_cache must match k_new and k_cache in tokens, rows and heads, rows contiguous")
        _need(vc4.dtype == kc.dtype, "k_cache and v_cache must share one dtype")
    ps, ksp, kst, ksh = _cache_rows(kc)
    p = _ffi.CacheAppendParams()
    p.k_new, p.k_new_stride_tok, p.k_new_stride_head = k_new.data_ptr(), k_new.stride(0), k_new.stride(1)
    p.k_cache, p.k_stride_page, p.k_stride_tok, p.k_stride_head = kc.data_ptr(), ksp, kst, ksh
    if v_new is not None:
        vc = _as_4d_cache(v_cache)
        _, vsp, vst, vsh = _cache_rows(vc)
        p.v_new, p.v_new_stride_tok, p.v_new_stride_head = v_new.data_ptr(), v_new.stride(0), v_new.stride(1)
        p.v_cache, p.v_stride_page, p.v_stride_tok, p.v_stride_head = vc.data_ptr(), vsp, vst, vsh
        p.head_dim_v = v_new.shape[2]
    p.cache_dtype = code
    p.k_scale, p.v_scale = float(k_scale), float(v_scale)
    p.slot_mapping = slot_mapping.data_ptr()
    p.layer_base_rows = int(layer_base_rows)
    p.num_cache_rows = kc.shape[0] * kc.shape[1]
    p.num_tokens, p.num_kv_heads, p.head_dim_k = k_new.shape[0], k_new.shape[1], k_new.shape[2]
    p.page_size = ps
    _ffi.check(_ffi.load().attn_cache_append(ctypes.byref(p), _stream(k_new.device)), "attn_cache_append")


def mla_kv_pack_fp8(k_nope, k_rope, v, *, k_scale=1.0, v_scale=1.0, k_out=None, v_out=None):
    """K = concat(k_nope [T, H, dn], k_rope [T, dr] shared by all heads) and V
    [T, H, dv] as E4M3 codes of value / scale (float8_e4m3fn tensors
    [T, H, dn + dr] and [T, H, dv]; pre-allocated outputs may be passed)."""
    _need(k_nope.dtype == _BF16 and k_rope.dtype == _BF16 and v.dtype == _BF16, "inputs must be bf16")
    if k_rope.dim() == 3:
        _need(k_rope.shape[1] == 1, "k_rope must be [T, dr] or [T, 1, dr]")
        k_rope = k_rope[:, 0, :]
    t, h, dn = k_nope.shape
    dr, dv = k_rope.shape[1], v.shape[2]
    dev = k_nope.device
    _need(k_rope.device == dev and v.device == dev, f"k_rope and v must be on {dev}")
    _need(k_rope.dim() == 2 and k_rope.shape[0] == t and v.dim() == 3 and tuple(v.shape[:2]) == (t, h),
          "k_rope must be [T, dr] and v [T, H, dv]")
    _need(_rows_contiguous(k_nope) and _rows_contiguous(k_rope) and _rows_contiguous(v), "input rows must be contiguous")
    if k_out is None:
        k_out = torch.empty((t, h, dn + dr), dtype=torch.float8_e4m3fn, device=dev)
    if v_out is None:
        v_out = torch.empty((t, h, dv), dtype=torch.float8_e4m3fn, device=dev)
    _check_out(k_out, (t, h, dn + dr), (torch.float8_e4m3fn, torch.uint8), dev, "k_out")
    _check_out(v_out, (t, h, dv), (torch.float8_e4m3fn, torch.uint8), dev, "v_out")
    _need(_rows_contiguous(k_out) and _rows_contiguous(v_out), "output rows must be contiguous")
    p = _ffi.MlaKvPackParams()
    p.k_nope, p.k_nope_stride_tok, p.k_nope_stride_head = k_nope.data_ptr(), k_nope.stride(0), k_nope.stride(1)
    p.k_rope, p.k_rope_stride_tok = k_rope.data_ptr(), k_rope.stride(0)
    p.v, p.v_stride_tok, p.v_stride_head = v.data_ptr(), v.stride(0), v.stride(1)
    p.k_out, p.k_out_stride_tok, p.k_out_stride_head = k_out.data_ptr(), k_out.stride(0), k_out.stride(1)
    p.v_out, p.v_out_stride_tok, p.v_out_stride_head = v_out.data_ptr(), v_out.stride(0), v_out.stride(1)
    p.k_scale, p.v_scale = float(k_scale), float(v_scale)
    p.num_tokens, p.num_heads, p.d_nope, p.d_rope, p.d_v = t, h, dn, dr, dv
    _ffi.check(_ffi.load().attn_mla_kv_pack_fp8(ctypes.byref(p), _stream(k_nope.device)), "attn_mla_kv_pack_fp8")
    return k_out, v_out
