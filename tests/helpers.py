"""Shared test helpers: run the oracle on generated cases and compare.

Tolerances (the bar every parity test applies):
  * bf16 KV: max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3 on O;
  * fp8 KV: max <= 6e-2 (mean <= 2e-3 still);
  * LSE (base 2): |gpu - oracle| <= 1e-3 where finite; -inf exactly where
    the oracle has -inf (rows without keys).
"""

from __future__ import annotations

import hashlib

import numpy as np
import torch

import oracle

TOL_BF16 = dict(max_abs=2e-2, mean_abs=2e-3)
TOL_FP8 = dict(max_abs=6e-2, mean_abs=2e-3)
TOL_LSE = 1e-3


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def widen_cache(t: torch.Tensor, kv_dtype: str, scale: float) -> np.ndarray:
    if kv_dtype == "bf16":
        return oracle.widen_bf16(bits(t))
    return oracle.widen_e4m3fn(bits(t), scale)


def f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return oracle.widen_bf16(bits(t))
    return t.to(torch.float64).numpy()


def oracle_decode(case, rows=None):
    """Oracle output for a DecodeCase: full ([B,q,H,Dv], [B,q,H]) or, with
    rows=[(b,t,h)...], ([n,Dv], [n])."""
    q = bits(case.q)
    fmt = "bf16" if case.kv_dtype == "bf16" else "e4m3fn"
    kc = bits(case.k_cache)
    vc = kc if case.v_cache is None else bits(case.v_cache)
    bt = case.block_table.numpy()
    sl = case.seq_lens.numpy()
    w = getattr(case, "window_left", -1)
    qfmt = "bf16" if getattr(case, "q_dtype", "bf16") == "bf16" else "e4m3fn"
    qs = getattr(case, "q_scale", 1.0)
    if rows is None:
        return oracle.decode_paged(q, kc, vc, bt, sl, case.page_size, case.scale, case.causal, case.head_dim_v,
                                   fmt, case.kv_scale, qfmt, w, qs)
    return oracle.decode_paged_rows(q, kc, vc, bt, sl, case.page_size, case.scale, case.causal,
                                    case.head_dim_v, rows, fmt, case.kv_scale, qfmt, w, qs)


def oracle_prefill(case, rows=None):
    """Oracle output for a PrefillCase: full ([Tq,H,Dv], [Tq,H]) or, with
    rows=[(token, head)...], ([n,Dv], [n])."""
    q = bits(case.q)
    w = getattr(case, "window_left", -1)
    if case.paged:
        k, v = bits(case.k), bits(case.v)
        bt = case.block_table.numpy()
        sl = case.seq_lens_kv.numpy()
        cu = case.cu_seqlens_q.numpy()
        if rows is None:
            return oracle.prefill_paged(q, k, v, cu, sl, bt, case.page_size, case.scale, case.causal,
                                        v.shape[-1], "bf16", "bf16", w)
        return oracle.prefill_paged_rows(q, k, v, cu, sl, bt, case.page_size, case.scale, case.causal,
                                         v.shape[-1], rows, "bf16", "bf16", w)
    cu_q = case.cu_seqlens_q.numpy()
    cu_k = case.cu_seqlens_kv.numpy()
    if rows is None:
        return oracle.prefill_dense(oracle.widen_bf16(q), f64(case.k), f64(case.v), cu_q, cu_k, case.scale,
                                    case.causal, w)
    # sampled rows of a dense case: widen only the (request, KV head) slices used
    kb, vb = bits(case.k), bits(case.v)
    hq, hkv = q.shape[1], kb.shape[1]
    group = hq // hkv
    o = np.zeros((len(rows), vb.shape[-1]))
    lse = np.full(len(rows), -np.inf)
    by = {}
    for n, (tok, h) in enumerate(rows):
        b = int(np.searchsorted(cu_q, tok, side="right") - 1)
        by.setdefault((b, h // group), []).append(n)
    for (b, g), members in by.items():
        lq, lk = int(cu_q[b + 1] - cu_q[b]), int(cu_k[b + 1] - cu_k[b])
        k0 = int(cu_k[b])
        k = oracle.widen_bf16(kb[k0:k0 + lk, g])
        v = oracle.widen_bf16(vb[k0:k0 + lk, g])
        qr = oracle.widen_bf16(np.stack([q[rows[n][0], rows[n][1]] for n in members]))
        i = np.array([rows[n][0] - cu_q[b] for n in members])
        bound = oracle.attention.causal_key_bound(i, lq, lk) if case.causal else np.full(len(members), lk)
        start = oracle.window_key_start(i, lq, lk, w)
        on, ln = oracle.attention_rows(qr, k, v, case.scale, bound, start)
        o[members], lse[members] = on, ln
    return o, lse


def compare(out: np.ndarray, ref: np.ndarray, lse: np.ndarray | None = None, lse_ref: np.ndarray | None = None,
            tol=TOL_BF16, lse_tol: float = TOL_LSE) -> dict:
    """Assert the parity bar; return the measured errors."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), "non-finite output"
    err = np.abs(out - ref)
    res = {"max_abs": float(err.max()) if err.size else 0.0, "mean_abs": float(err.mean()) if err.size else 0.0}
    assert res["max_abs"] <= tol["max_abs"], res
    assert res["mean_abs"] <= tol["mean_abs"], res
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isneginf(lse), ~fin), "LSE -inf rows differ"
        d = np.abs(lse[fin] - lse_ref[fin])
        res["lse_max"] = float(d.max()) if d.size else 0.0
        assert res["lse_max"] <= lse_tol, res
        # rows without keys are exactly zero
        assert np.all(out[~fin] == 0)
    return res


def block_edge_rows(cu_seqlens_q, num_heads: int, block: int = 32) -> list[tuple[int, int]]:
    """(token, head) rows at the first and the last query token of every
    block of 32 tokens of each request, counted from the request's end (the
    prefill's query tiles and the 32-row blocks of its waves are aligned to
    the end of the request), for every head: the first and last row of every
    wave, hence of every workgroup, of an unsplit or key-split launch."""
    cu = [int(x) for x in cu_seqlens_q]
    toks = set()
    for b in range(len(cu) - 1):
        lq = cu[b + 1] - cu[b]
        for k in range(-(-lq // block)):
            toks.add(cu[b] + lq - 1 - block * k)
            toks.add(cu[b] + max(0, lq - block * (k + 1)))
    return [(t, h) for t in sorted(toks) for h in range(num_heads)]


_ORACLE_CACHE: dict = {}


def oracle_prefill_cached(case, rows):
    """oracle_prefill(case, rows), remembered for the process by the case's
    name and the rows (full-size workloads checked by several tests)."""
    key = (case.name, hashlib.sha1(np.asarray(rows, dtype=np.int64).tobytes()).hexdigest())
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE.clear()
        _ORACLE_CACHE[key] = oracle_prefill(case, rows)
    return _ORACLE_CACHE[key]
