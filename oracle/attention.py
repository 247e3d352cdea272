"""Softmax attention written as its plain definition, in numpy float64.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What every function here computes, for one query row of one head
("Flywheel Attention: Attention Kernels Built for the TPU", section 1,
softmax attention; "Writing Page Attention with PyPTO", section 1.1,
mathematical objective):

    s_j  = scale * <q, k_j>               for each key j the row may see
    p_j  = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j)
    o    = sum_j p_j v_j
    lse2 = log2(sum_j exp(s_j))            (base-2 log-sum-exp)

The whole score matrix is materialised; nothing is blocked, fused or
reordered. Query rows are independent in this definition, so long inputs
are evaluated a group of rows at a time, each row still in full.

Readings of the pages used here (each one is listed in the design notes):
  * LSE is returned in base 2 and as the log of the natural softmax
    denominator: lse2 = log2(sum_j exp(s_j)) ("TokenSpeed-MLA", the
    packed-query paragraph: base-2 LSE semantics).
  * A causal row is aligned bottom-right: with Lq query rows and Lk keys,
    query row i sees keys j < Lk - Lq + i + 1 ("TokenSpeed-MLA", prefill
    command's bottom-right alignment, and the window_left bound in the
    kernel capability summary).
  * A row that sees no key returns o = 0 and lse2 = -inf ("TokenSpeed-MLA",
    section "SM107 decode": rows with no visible keys).
  * A sliding window (window_left >= 0) also bounds each row from below:
    query row i of a block of Lq rows over Lk keys sees keys
    j >= max(0, Lk - Lq - window_left + i), i.e. the whole block plus
    window_left keys of context ("TokenSpeed-MLA", kernel capability
    summary, window_left); -1 means the full history. The same bound is
    applied to prefill rows, with Lq the request's query count.
  * Query head h reads KV head h // G with G = Hq / Hkv, i.e. consecutive
    query heads share a KV head ("Writing Page Attention with PyPTO",
    sections 1.2 and 1.3).
  * A paged cache is read through the block table: token j of request b
    lives in physical page block_table[b, j // page_size], slot
    j % page_size ("Writing Page Attention with PyPTO", sections 1.2 and
    5.2). Entries past the request's last page are never read (section 9).
  * For a latent (MLA-shaped) cache, K is the whole row and V its first Dv
    entries ("TokenSpeed-MLA", kernel capability summary: query width is
    kv_lora_rank + qk_rope_head_dim).
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf
_LN2 = math.log(2.0)


# ---------------------------------------------------------------------------
# Storage formats, widened exactly to float64.
# ---------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper half of an IEEE-754 binary32 value, so
    shifting its 16 bits into the top of a 32-bit word gives that binary32
    value, which float64 holds exactly.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def widen_e4m3fn(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64 value times a per-tensor scale.

    Format (OCP 8-bit Floating Point Specification, E4M3): 1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
    subnormals m * 2**-9; there is no infinity; S.1111.111 is NaN. The
    per-tensor dequantisation scale multiplies the decoded value
    ("TokenSpeed-MLA": FP8 e4m3 KV inputs; one scale per tensor).
    """
    return _E4M3FN_VALUES[np.asarray(codes, dtype=np.uint8)] * float(scale)


def _e4m3fn_value_table() -> np.ndarray:
    """The value of each of the 256 E4M3 codes, from the format's definition."""
    c = np.arange(256, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = man * 2.0 ** -9
    val = sign * np.where(exp == 0, subnormal, normal)
    return np.where((exp == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


_E4M3FN_VALUES = _e4m3fn_value_table()


def widen(x: np.ndarray, kv_format: str = "f64", kv_scale: float = 1.0) -> np.ndarray:
    """Values of stored data: "f64" (already values), "bf16" (uint16 bit
    patterns) or "e4m3fn" (uint8 codes times kv_scale)."""
    if kv_format == "f64":
        return np.asarray(x, dtype=np.float64)
    if kv_format == "bf16":
        return widen_bf16(x)
    if kv_format == "e4m3fn":
        return widen_e4m3fn(x, kv_scale)
    raise ValueError(kv_format)


# ---------------------------------------------------------------------------
# The definition.
# ---------------------------------------------------------------------------

def causal_key_bound(i: np.ndarray | int, lq: int, lk: int) -> np.ndarray:
    """Number of leading keys query row i sees under the bottom-right causal
    alignment: keys j < lk - lq + i + 1, clipped to [0, lk]."""
    return np.clip(np.asarray(i, dtype=np.int64) + (lk - lq) + 1, 0, lk)


def window_key_start(i: np.ndarray | int, lq: int, lk: int, window_left: int) -> np.ndarray:
    """First key query row i may see under a sliding window of window_left
    keys of context: max(0, lk - lq - window_left + i); 0 when window_left
    is -1 (full history)."""
    i = np.asarray(i, dtype=np.int64)
    if window_left < 0:
        return np.zeros_like(i)
    return np.maximum(0, i + (lk - lq - window_left))


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   key_bound: np.ndarray | None = None, key_start: np.ndarray | None = None,
                   row_group: int = 1024) -> tuple[np.ndarray, np.ndarray]:
    """Attention of R query rows over one key/value sequence.

    q: [R, Dqk], k: [Lk, Dqk], v: [Lk, Dv], all float64.
    key_bound: [R] ints; row r sees keys key_start[r] .. key_bound[r]-1
    (defaults: 0 and Lk).
    Returns o [R, Dv] and lse2 [R].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    r_total, lk, dv = q.shape[0], k.shape[0], v.shape[1]
    if key_bound is None:
        key_bound = np.full(r_total, lk, dtype=np.int64)
    key_bound = np.asarray(key_bound, dtype=np.int64)
    if key_start is None:
        key_start = np.zeros(r_total, dtype=np.int64)
    key_start = np.asarray(key_start, dtype=np.int64)
    o = np.zeros((r_total, dv), dtype=np.float64)
    lse2 = np.full(r_total, NEG_INF, dtype=np.float64)
    if lk == 0 or r_total == 0:
        return o, lse2
    cols = np.arange(lk, dtype=np.int64)
    for r0 in range(0, r_total, row_group):
        r1 = min(r_total, r0 + row_group)
        s = scale * (q[r0:r1] @ k.T)                       # [rows, Lk]
        visible = (cols[None, :] < key_bound[r0:r1, None]) & (cols[None, :] >= key_start[r0:r1, None])
        s = np.where(visible, s, NEG_INF)
        seen = visible.any(axis=1)
        if not seen.any():
            continue
        s = s[seen]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        idx = np.nonzero(seen)[0] + r0
        o[idx] = (e @ v) / l
        lse2[idx] = (m[:, 0] + np.log(l[:, 0])) / _LN2
    return o, lse2


def gather_paged_rows(cache: np.ndarray, block_table_row: np.ndarray, seq_len: int,
                      page_size: int, head: int, width: int | None = None) -> np.ndarray:
    """Contiguous [seq_len, width] copy of one request's keys (or values) for
    one KV head, read through the block table.

    cache: [num_pages, page_size, num_kv_heads, D] (any dtype; rows are
    returned as stored). Only the first ceil(seq_len / page_size) table
    entries are read.
    """
    n_pages = -(-seq_len // page_size)
    rows = []
    for logical in range(n_pages):
        physical = int(block_table_row[logical])
        take = min(page_size, seq_len - logical * page_size)
        rows.append(cache[physical, :take, head, :width])
    if not rows:
        d = cache.shape[-1] if width is None else width
        return np.zeros((0, d), dtype=cache.dtype)
    return np.concatenate(rows, axis=0)


# ---------------------------------------------------------------------------
# Decode over a paged cache.
# ---------------------------------------------------------------------------

def decode_paged_rows(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                      block_table: np.ndarray, seq_lens: np.ndarray, page_size: int,
                      scale: float, causal: bool, head_dim_v: int,
                      rows: list[tuple[int, int, int]], kv_format: str = "f64",
                      kv_scale: float = 1.0, q_format: str = "f64",
                      window_left: int = -1, q_scale: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Decode attention for selected (batch, query token, query head) rows.

    q: [B, q_len, Hq, Dqk] float64; k_cache: [P, ps, Hkv, Dqk];
    v_cache: [P, ps, Hkv, >=Dv] (V is its first head_dim_v entries); caches
    hold values (kv_format "f64") or raw storage ("bf16", "e4m3fn" with
    kv_scale), widened after gathering; q likewise ("f64", "bf16" bits, or
    "e4m3fn" codes times q_scale: the FP8 decode path of "TokenSpeed-MLA",
    whose FP8 inputs are the query and the latent cache);
    block_table: [B, max_pages] ints; seq_lens: [B] ints.
    Returns o [len(rows), Dv] and lse2 [len(rows)].
    """
    _, q_len, hq, _ = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    o = np.zeros((len(rows), head_dim_v), dtype=np.float64)
    lse2 = np.full(len(rows), NEG_INF, dtype=np.float64)
    by_req_head: dict[tuple[int, int], list[int]] = {}
    for n, (b, _, h) in enumerate(rows):
        by_req_head.setdefault((b, h // group), []).append(n)
    for (b, g), members in by_req_head.items():
        lk = int(seq_lens[b])
        k = widen(gather_paged_rows(k_cache, block_table[b], lk, page_size, g), kv_format, kv_scale)
        v = widen(gather_paged_rows(v_cache, block_table[b], lk, page_size, g, head_dim_v),
                  kv_format, kv_scale)
        qr = widen(np.stack([q[rows[n][0], rows[n][1], rows[n][2]] for n in members]), q_format, q_scale)
        t = np.array([rows[n][1] for n in members], dtype=np.int64)
        bound = causal_key_bound(t, q_len, lk) if causal else np.full(len(members), lk)
        start = window_key_start(t, q_len, lk, window_left)
        o_m, l_m = attention_rows(qr, k, v, scale, bound, start)
        o[members] = o_m
        lse2[members] = l_m
    return o, lse2


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, page_size, scale,
                 causal, head_dim_v, kv_format="f64", kv_scale=1.0, q_format="f64", window_left=-1,
                 q_scale=1.0):
    """Decode attention for every row: returns o [B, q_len, Hq, Dv] and
    lse2 [B, q_len, Hq]."""
    b_n, q_len, hq, _ = q.shape
    rows = [(b, t, h) for b in range(b_n) for t in range(q_len) for h in range(hq)]
    o, lse2 = decode_paged_rows(q, k_cache, v_cache, block_table, seq_lens, page_size,
                                scale, causal, head_dim_v, rows, kv_format, kv_scale, q_format,
                                window_left, q_scale)
    return o.reshape(b_n, q_len, hq, head_dim_v), lse2.reshape(b_n, q_len, hq)


# ---------------------------------------------------------------------------
# Prefill over ragged dense or paged KV.
# ---------------------------------------------------------------------------

def prefill_dense(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, causal, window_left=-1):
    """Ragged prefill over packed dense K/V ("TokenSpeed-MLA", kernel capability
    summary: Q [sum q_lens, h_q, d_qk], K [sum kv_lens, h_k, d_qk],
    V [sum kv_lens, h_k, d_v]; the two packings may differ).

    Returns o [Tq, Hq, Dv] and lse2 [Tq, Hq].
    """
    tq, hq, _ = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    group = hq // hkv
    o = np.zeros((tq, hq, dv), dtype=np.float64)
    lse2 = np.full((tq, hq), NEG_INF, dtype=np.float64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_kv[b]), int(cu_seqlens_kv[b + 1])
        lq, lk = q1 - q0, k1 - k0
        bound = causal_key_bound(np.arange(lq), lq, lk) if causal else np.full(lq, lk)
        start = window_key_start(np.arange(lq), lq, lk, window_left)
        for h in range(hq):
            g = h // group
            o[q0:q1, h], lse2[q0:q1, h] = attention_rows(
                q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], scale, bound, start)
    return o, lse2


def prefill_dense_fp8(q_codes, k_codes, v_codes, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_kv,
                      scale, causal, window_left=-1):
    """FP8 prefill ("TokenSpeed-MLA": the prefill command's FP8 E4M3 inputs,
    q and k 192 wide, v 128 wide; kernel capability summary: BF16 output and
    FP32 LSE): q, k, v are E4M3 codes (uint8) with per-tensor dequantisation
    scales, value = code * scale; the attention is prefill_dense on those
    values. Returns o [Tq, Hq, Dv] and lse2 [Tq, Hq]."""
    return prefill_dense(widen_e4m3fn(q_codes, q_scale), widen_e4m3fn(k_codes, k_scale),
                         widen_e4m3fn(v_codes, v_scale), cu_seqlens_q, cu_seqlens_kv, scale, causal, window_left)


def prefill_dense_fp8_rows(q_codes, k_codes, v_codes, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_kv,
                           scale, causal, rows, window_left=-1):
    """prefill_dense_fp8 for the listed (token, head) rows only: ([n, Dv], [n])."""
    hq, hkv = q_codes.shape[1], k_codes.shape[1]
    group = hq // hkv
    cu_q = np.asarray(cu_seqlens_q)
    cu_k = np.asarray(cu_seqlens_kv)
    o = np.zeros((len(rows), v_codes.shape[2]), dtype=np.float64)
    lse2 = np.full(len(rows), NEG_INF, dtype=np.float64)
    for n, (tok, h) in enumerate(rows):
        b = int(np.searchsorted(cu_q, tok, side="right") - 1)
        lq, k0, k1 = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b]), int(cu_k[b + 1])
        lk, i = k1 - k0, tok - int(cu_q[b])
        bound = causal_key_bound(np.array([i]), lq, lk) if causal else np.array([lk])
        start = window_key_start(np.array([i]), lq, lk, window_left)
        g = h // group
        oo, ll = attention_rows(widen_e4m3fn(q_codes[tok:tok + 1, h], q_scale),
                                widen_e4m3fn(k_codes[k0:k1, g], k_scale), widen_e4m3fn(v_codes[k0:k1, g], v_scale),
                                scale, bound, np.atleast_1d(start))
        o[n], lse2[n] = oo[0], ll[0]
    return o, lse2


def prefill_paged_rows(q, k_cache, v_cache, cu_seqlens_q, seq_lens_kv, block_table,
                       page_size, scale, causal, head_dim_v, rows, kv_format="f64", q_format="f64",
                       window_left=-1):
    """Ragged prefill over a paged cache for selected (query token, head) rows,
    where the query token index is global in the packed Q. Caches hold values
    or raw bf16 bits (kv_format "bf16"), widened after gathering."""
    hq = q.shape[1]
    hkv = k_cache.shape[2]
    group = hq // hkv
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    o = np.zeros((len(rows), head_dim_v), dtype=np.float64)
    lse2 = np.full(len(rows), NEG_INF, dtype=np.float64)
    by_req_head: dict[tuple[int, int], list[int]] = {}
    for n, (tok, h) in enumerate(rows):
        b = int(np.searchsorted(cu, tok, side="right") - 1)
        by_req_head.setdefault((b, h // group), []).append(n)
    for (b, g), members in by_req_head.items():
        lq = int(cu[b + 1] - cu[b])
        lk = int(seq_lens_kv[b])
        k = widen(gather_paged_rows(k_cache, block_table[b], lk, page_size, g), kv_format)
        v = widen(gather_paged_rows(v_cache, block_table[b], lk, page_size, g, head_dim_v), kv_format)
        qr = widen(np.stack([q[rows[n][0], rows[n][1]] for n in members]), q_format)
        i = np.array([rows[n][0] - cu[b] for n in members], dtype=np.int64)
        bound = causal_key_bound(i, lq, lk) if causal else np.full(len(members), lk)
        start = window_key_start(i, lq, lk, window_left)
        o_m, l_m = attention_rows(qr, k, v, scale, bound, start)
        o[members] = o_m
        lse2[members] = l_m
    return o, lse2


def prefill_paged(q, k_cache, v_cache, cu_seqlens_q, seq_lens_kv, block_table,
                  page_size, scale, causal, head_dim_v, kv_format="f64", q_format="f64", window_left=-1):
    """Ragged prefill over a paged cache for every row: o [Tq, Hq, Dv],
    lse2 [Tq, Hq]."""
    tq, hq, _ = q.shape
    rows = [(t, h) for t in range(tq) for h in range(hq)]
    o, lse2 = prefill_paged_rows(q, k_cache, v_cache, cu_seqlens_q, seq_lens_kv,
                                 block_table, page_size, scale, causal, head_dim_v, rows, kv_format,
                                 q_format, window_left)
    return o.reshape(tq, hq, head_dim_v), lse2.reshape(tq, hq)


# ---------------------------------------------------------------------------
# Combining partial results over disjoint key sets.
# ---------------------------------------------------------------------------

def merge_lse(o_parts: np.ndarray, lse_parts: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Combine S partial results computed over disjoint key subsets.

    Split-KV decode writes, per split i, the output o_i normalised over its
    own keys and lse2_i = log2 sum_{j in split i} exp(s_j); a second step
    reduces them ("TokenSpeed-MLA", section "Decode performance": one kernel
    computes split-KV partials, a second reduces them; partials and
    log-sum-exp stay FP32, section "FP8 split-KV partial storage").

    From the definition, with w_i = 2**lse2_i:
        o    = sum_i w_i o_i / sum_i w_i
        lse2 = log2 sum_i w_i
    evaluated with the largest lse2_i factored out. Splits with lse2 = -inf
    hold no key and get weight 0; a row where every split is empty returns
    o = 0, lse2 = -inf.

    o_parts: [S, R, Dv]; lse_parts: [S, R]. Returns o [R, Dv], lse2 [R].
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    s_n, r_n, dv = o_parts.shape
    o = np.zeros((r_n, dv), dtype=np.float64)
    lse2 = np.full(r_n, NEG_INF, dtype=np.float64)
    finite = np.isfinite(lse_parts)
    any_finite = finite.any(axis=0)
    if not any_finite.any():
        return o, lse2
    top = np.where(finite, lse_parts, NEG_INF).max(axis=0)           # [R]
    top_safe = np.where(any_finite, top, 0.0)
    w = np.where(finite, np.exp2(lse_parts - top_safe[None, :]), 0.0)  # [S, R]
    total = w.sum(axis=0)
    contrib = np.where(finite[:, :, None], o_parts, 0.0) * w[:, :, None]
    o[any_finite] = contrib.sum(axis=0)[any_finite] / total[any_finite, None]
    lse2[any_finite] = top[any_finite] + np.log2(total[any_finite])
    return o, lse2


# ---------------------------------------------------------------------------
# The pages' online recurrence (used to pin the definition, not by it).
# ---------------------------------------------------------------------------

def online_softmax_blocks(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                          block_edges: list[int]) -> tuple[np.ndarray, np.ndarray]:
    """The running-state recurrence over consecutive key blocks.

    With running max m, running sum l and running output o per row, a block
    of scores s updates them as
        m' = max(m, rowmax(s)),  p = exp(s - m'),
        l  = exp(m - m') l + rowsum(p),
        o  = exp(m - m') o + p V
    and the result is o / l ("Flywheel Attention: Attention Kernels Built for
    the TPU", section 1; "Writing Page Attention with PyPTO", section 6.3,
    which also stresses that p is divided by the final l only at the end).

    q: [R, D]; k: [Lk, D]; v: [Lk, Dv]; block_edges: increasing cut points
    0 = e_0 < e_1 < ... < e_n = Lk. Returns o [R, Dv], lse2 [R].
    """
    q = np.asarray(q, dtype=np.float64)
    r_n, dv = q.shape[0], v.shape[1]
    m = np.full(r_n, NEG_INF)
    l = np.zeros(r_n)
    o = np.zeros((r_n, dv))
    for a, b in zip(block_edges[:-1], block_edges[1:]):
        s = scale * (q @ np.asarray(k[a:b], dtype=np.float64).T)
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        p = np.exp(s - m_new[:, None])
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ np.asarray(v[a:b], dtype=np.float64)
        m = m_new
    return o / l[:, None], (m + np.log(l)) / _LN2
