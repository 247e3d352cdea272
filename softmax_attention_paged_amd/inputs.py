"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no attention arithmetic: it draws random numbers, lays
tokens out in pages under a chosen block-table layout, and poisons every
cache slot no request owns with NaN. Both the HIP path (tests, bench) and
the oracle read what it returns; neither imports the other.

Recipe (same for every workload):
  * numpy.random.SeedSequence(seed) spawns four children: 0 draws the
    sequence lengths (when random) and the page layout, 1 draws Q, 2 draws
    K, 3 draws V; each of Q, K, V is split along its first axis into 64
    equal slabs, slab i drawn by PCG64 seeded with child.spawn(64)[i] (so
    the values do not depend on how many threads draw them).
  * Values are float32 N(0, 1) (Q optionally multiplied by q_mult), rounded
    to bf16 by torch (round to nearest even).
  * FP8 caches: per-tensor scale = amax / 448 over the float32 values; codes
    = torch float8_e4m3fn of clamp(x / scale, -448, 448).
  * Logical tokens of each request are scattered into physical pages through
    the block table; table entries past a request's last page are -1; every
    slot not written (unused pages, tails of last pages) holds NaN (bf16
    0x7FC0, fp8 0x7F).
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
import os

import numpy as np
import torch

BF16_NAN = 0x7FC0
FP8_NAN = 0x7F
FP8_MAX = 448.0
LAYOUTS = ("random", "identity", "reverse", "shared_prefix", "noncontiguous")


_SLABS = 64


def _streams(seed: int) -> list[np.random.SeedSequence]:
    """[layout, Q, K, V] seed sequences of a workload."""
    return np.random.SeedSequence(seed).spawn(4)


def _normal_f32(ss: np.random.SeedSequence, shape, mult: float = 1.0) -> np.ndarray:
    """float32 N(0, 1) * mult of the given shape, drawn in _SLABS slabs along
    axis 0 (slab i from PCG64(ss.spawn(_SLABS)[i])), in parallel threads."""
    import concurrent.futures
    shape = tuple(int(x) for x in shape)
    out = np.empty(shape, dtype=np.float32)
    n0 = shape[0]
    edges = [n0 * i // _SLABS for i in range(_SLABS + 1)]
    children = ss.spawn(_SLABS)

    def fill(i):
        a, b = edges[i], edges[i + 1]
        if b > a:
            g = np.random.Generator(np.random.PCG64(children[i]))
            g.standard_normal(size=(b - a,) + shape[1:], dtype=np.float32, out=out[a:b])
            if mult != 1.0:
                out[a:b] *= np.float32(mult)

    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(_SLABS)))
    return out


def _normal_bf16(ss: np.random.SeedSequence, shape, mult: float = 1.0) -> torch.Tensor:
    return torch.from_numpy(_normal_f32(ss, shape, mult)).to(torch.bfloat16)


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclasses.dataclass
class PagedLayout:
    block_table: torch.Tensor      # int32 [B, max_pages], -1 past each request
    num_pages: int
    slot_of_token: torch.Tensor    # int64 [sum(lens)]: page * page_size + slot of each logical token


def make_layout(rng: np.random.Generator, seq_lens: list[int], page_size: int, layout: str,
                pool_pages: int | None = None, max_pages: int | None = None,
                shared_prefix_pages: int = 0) -> PagedLayout:
    """Assign physical pages to every request's logical pages."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout {layout!r} not in {LAYOUTS}")
    b = len(seq_lens)
    n_pages = [_cdiv(n, page_size) for n in seq_lens]
    shared = shared_prefix_pages if layout == "shared_prefix" else 0
    if shared:
        if any(n < shared for n in n_pages):
            raise ValueError("every request must own at least shared_prefix_pages pages")
    need = sum(n_pages) - shared * max(0, b - 1)
    if pool_pages is None:
        pool_pages = 2 * need if layout == "noncontiguous" else need
    if pool_pages < need:
        raise ValueError(f"pool of {pool_pages} pages < {need} needed")
    if layout == "identity":
        order = np.arange(pool_pages)
    elif layout == "reverse":
        order = np.arange(pool_pages)[::-1].copy()
    else:
        order = rng.permutation(pool_pages)
    width = max_pages if max_pages is not None else max(1, max(n_pages, default=1))
    table = np.full((b, width), -1, dtype=np.int32)
    nxt = 0
    prefix = None
    for i, n in enumerate(n_pages):
        start = 0
        if shared and prefix is not None:
            table[i, :shared] = prefix
            start = shared
        for logical in range(start, n):
            table[i, logical] = order[nxt]
            nxt += 1
        if shared and prefix is None:
            prefix = table[i, :shared].copy()
    slots = []
    for i, n in enumerate(seq_lens):
        j = np.arange(n, dtype=np.int64)
        slots.append(table[i, j // page_size].astype(np.int64) * page_size + j % page_size)
    slot_of_token = torch.from_numpy(np.concatenate(slots) if slots else np.zeros(0, np.int64))
    return PagedLayout(torch.from_numpy(table), pool_pages, slot_of_token)


def _scatter_pages(tokens: torch.Tensor, layout: PagedLayout, page_size: int, fill_bits: int) -> torch.Tensor:
    """tokens [sum(lens), ...] -> pool [num_pages, page_size, ...] with NaN elsewhere."""
    tail = tuple(tokens.shape[1:])
    if tokens.dtype == torch.bfloat16:
        pool = torch.full((layout.num_pages * page_size,) + tail, fill_bits, dtype=torch.int16).view(torch.bfloat16)
    else:
        pool = torch.full((layout.num_pages * page_size,) + tail, fill_bits, dtype=torch.uint8)
    if tokens.shape[0]:
        pool.index_copy_(0, layout.slot_of_token, tokens)
    return pool.view((layout.num_pages, page_size) + tail)


def _fp8_codes(x: np.ndarray) -> tuple[torch.Tensor, float]:
    """Codes of x / scale with scale = amax / 448 (x is consumed)."""
    t = torch.from_numpy(x)
    amax = float(torch.linalg.vector_norm(t, ord=float("inf"))) if x.size else 1.0
    scale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    t.div_(scale).clamp_(-FP8_MAX, FP8_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8), scale


def _share_prefix(x: np.ndarray, seq_lens: list[int], tokens: int) -> None:
    """Make every request's first `tokens` logical tokens equal request 0's."""
    if tokens <= 0 or not seq_lens:
        return
    starts = np.concatenate([[0], np.cumsum(seq_lens)[:-1]])
    for s in starts[1:]:
        x[s:s + tokens] = x[:tokens]


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeCase:
    name: str
    q: torch.Tensor                 # bf16 [B, q_len, Hq, Dqk]
    k_cache: torch.Tensor           # bf16 or uint8 fp8 codes [pages, page_size, Hkv, Dqk]
    v_cache: torch.Tensor | None    # same layout; None for a latent cache (V = first Dv of K rows)
    block_table: torch.Tensor       # int32 [B, max_pages]
    seq_lens: torch.Tensor          # int32 [B]
    page_size: int
    head_dim_v: int
    scale: float
    causal: bool
    kv_dtype: str                   # "bf16" or "fp8_e4m3"
    kv_scale: float                 # dequantisation scale (1.0 for bf16)
    max_seq_len: int
    seed: int
    window_left: int = -1           # sliding window of context keys; -1: full history
    packed_q: bool = False          # continuous (token * H + head) row packing
    q_dtype: str = "bf16"           # "bf16", or "fp8_e4m3": q holds uint8 codes
    q_scale: float = 1.0            # dequantisation scale of fp8 q

    @property
    def latent(self) -> bool:
        return self.v_cache is None

    def kv_read_bytes(self) -> int:
        """Bytes of K and V the valid tokens occupy (each KV head read once;
        a latent row counted once for K and V)."""
        tokens = int(self.seq_lens.sum())
        row = self.k_cache.shape[2] * self.k_cache.shape[3] * self.k_cache.element_size()
        if self.v_cache is not None:
            row += self.v_cache.shape[2] * self.v_cache.shape[3] * self.v_cache.element_size()
        return tokens * row

    def to(self, device) -> "DecodeCase":
        f = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(self, q=f(self.q), k_cache=f(self.k_cache), v_cache=f(self.v_cache),
                                   block_table=f(self.block_table), seq_lens=f(self.seq_lens))


def decode_case(*, batch: int, q_len: int, hq: int, hkv: int, d: int, dv: int, page_size: int,
                seq_lens=None, seq_len_range=None, seed: int, layout: str = "random",
                pool_pages: int | None = None, max_pages: int | None = None, kv_dtype: str = "bf16",
                latent: bool = False, scale: float | None = None, causal: bool = False,
                q_mult: float = 1.0, shared_prefix_pages: int = 0, name: str = "",
                window_left: int = -1, packed_q: bool = False, q_dtype: str = "bf16") -> DecodeCase:
    s_layout, s_q, s_k, s_v = _streams(seed)
    rng = np.random.Generator(np.random.PCG64(s_layout))
    if seq_lens is None:
        lo, hi = seq_len_range
        seq_lens = rng.integers(lo, hi + 1, size=batch).tolist()
    seq_lens = [int(n) for n in seq_lens]
    assert len(seq_lens) == batch
    lay = make_layout(rng, seq_lens, page_size, layout, pool_pages, max_pages, shared_prefix_pages)
    if q_dtype == "bf16":
        q, q_scale = _normal_bf16(s_q, (batch, q_len, hq, d), q_mult), 1.0
    elif q_dtype == "fp8_e4m3":
        if kv_dtype != "fp8_e4m3":
            raise ValueError("fp8 q is generated with an fp8 latent cache only")
        q, q_scale = _fp8_codes(_normal_f32(s_q, (batch, q_len, hq, d), q_mult))
    else:
        raise ValueError(q_dtype)
    total = sum(seq_lens)
    shared_tokens = shared_prefix_pages * page_size

    def logical(ss, width):
        x = _normal_f32(ss, (total, hkv, width))
        _share_prefix(x, seq_lens, shared_tokens)
        return x

    kx = logical(s_k, d)
    vx = None if latent else logical(s_v, dv)
    if kv_dtype == "bf16":
        kc = _scatter_pages(torch.from_numpy(kx).to(torch.bfloat16), lay, page_size, BF16_NAN)
        vc = None if latent else _scatter_pages(torch.from_numpy(vx).to(torch.bfloat16), lay, page_size, BF16_NAN)
        kv_scale = 1.0
    elif kv_dtype == "fp8_e4m3":
        if not latent:
            raise ValueError("fp8 KV is generated for latent caches only")
        codes, kv_scale = _fp8_codes(kx)
        kc, vc = _scatter_pages(codes, lay, page_size, FP8_NAN), None
    else:
        raise ValueError(kv_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return DecodeCase(name=name, q=q, k_cache=kc, v_cache=vc, block_table=lay.block_table,
                      seq_lens=torch.tensor(seq_lens, dtype=torch.int32), page_size=page_size,
                      head_dim_v=dv, scale=float(scale), causal=causal, kv_dtype=kv_dtype,
                      kv_scale=kv_scale, max_seq_len=max(seq_lens, default=0), seed=seed,
                      window_left=window_left, packed_q=packed_q, q_dtype=q_dtype, q_scale=q_scale)


# --------------------------------------------------------------------------
# Prefill
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillCase:
    name: str
    q: torch.Tensor                  # bf16 [Tq, Hq, D]
    k: torch.Tensor                  # dense [Tk, Hkv, D] or paged [pages, ps, Hkv, D]
    v: torch.Tensor
    cu_seqlens_q: torch.Tensor       # int32 [B+1]
    cu_seqlens_kv: torch.Tensor | None   # dense
    seq_lens_kv: torch.Tensor        # int32 [B]
    block_table: torch.Tensor | None     # paged
    page_size: int
    scale: float
    causal: bool
    max_seqlen_q: int
    max_seqlen_kv: int
    seed: int
    window_left: int = -1            # sliding window of context keys; -1: full history

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    def to(self, device) -> "PrefillCase":
        f = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(self, q=f(self.q), k=f(self.k), v=f(self.v),
                                   cu_seqlens_q=f(self.cu_seqlens_q), cu_seqlens_kv=f(self.cu_seqlens_kv),
                                   seq_lens_kv=f(self.seq_lens_kv), block_table=f(self.block_table))


def prefill_case(*, q_lens: list[int], kv_lens: list[int], hq: int, hkv: int, d: int, seed: int,
                 causal: bool = True, paged: bool = False, page_size: int = 64, layout: str = "random",
                 pool_pages: int | None = None, scale: float | None = None, q_mult: float = 1.0,
                 name: str = "", window_left: int = -1) -> PrefillCase:
    s_layout, s_q, s_k, s_v = _streams(seed)
    rng = np.random.Generator(np.random.PCG64(s_layout))
    lay = make_layout(rng, kv_lens, page_size, layout, pool_pages) if paged else None
    tq, tk = sum(q_lens), sum(kv_lens)
    q = _normal_bf16(s_q, (tq, hq, d), q_mult)
    k = _normal_bf16(s_k, (tk, hkv, d))
    v = _normal_bf16(s_v, (tk, hkv, d))
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(kv_lens)]), dtype=torch.int32)
    bt = None
    if paged:
        k = _scatter_pages(k, lay, page_size, BF16_NAN)
        v = _scatter_pages(v, lay, page_size, BF16_NAN)
        bt = lay.block_table
    return PrefillCase(name=name, q=q, k=k, v=v, cu_seqlens_q=cu_q, cu_seqlens_kv=None if paged else cu_k,
                       seq_lens_kv=torch.tensor(kv_lens, dtype=torch.int32), block_table=bt,
                       page_size=page_size, scale=float(scale if scale is not None else 1.0 / math.sqrt(d)),
                       causal=causal, max_seqlen_q=max(q_lens, default=0), max_seqlen_kv=max(kv_lens, default=0),
                       seed=seed, window_left=window_left)


# --------------------------------------------------------------------------
# The pages' workloads
# --------------------------------------------------------------------------

def gqa_decode_tiny(seed: int = 1, layout: str = "random") -> DecodeCase:
    """Tiny paged GQA decode: batch 2, 1 query token, 8 query / 2 KV heads,
    head_dim 64, page_size 16, seq_lens {37, 100}, a 16-page pool (request 0
    takes 3 pages, request 1 takes 7; the other 6 are NaN), scale 1/8."""
    return decode_case(batch=2, q_len=1, hq=8, hkv=2, d=64, dv=64, page_size=16, seq_lens=[37, 100],
                       seed=seed, layout=layout, pool_pages=16, name="gqa_decode_tiny_b2_h8kv2_d64_ps16")


def qwen3_14b_decode(seed: int = 2) -> DecodeCase:
    """Qwen3-14B-shaped paged decode: batch 64, 1 query token, 40 query / 8 KV
    heads, head_dim 128, page_size 128, seq_lens uniform on [256, 8192], a
    pool of exactly the pages needed, randomly permuted, scale 1/sqrt(128)."""
    return decode_case(batch=64, q_len=1, hq=40, hkv=8, d=128, dv=128, page_size=128,
                       seq_len_range=(256, 8192), seed=seed, max_pages=64,
                       name="qwen3_14b_decode_b64_h40kv8_d128_ps128_len256to8192")


def dense_causal_prefill(d: int = 128, seed: int = 3, seq: int = 8192) -> PrefillCase:
    """Dense causal prefill: batch 1, 8192 tokens, 32 heads (MHA), head_dim
    128 or 256."""
    return prefill_case(q_lens=[seq], kv_lens=[seq], hq=32, hkv=32, d=d, seed=seed, causal=True,
                        name=f"dense_causal_prefill_t{seq}_h32_d{d}")


def ragged_paged_prefill(seed: int = 4) -> PrefillCase:
    """Ragged paged chunked prefill: 4 requests with q_len {512, 1024, 512,
    1024} appended to 80K-token contexts (kv_len 81920 each, bottom-right
    causal), 32 query / 8 KV heads, head_dim 128, page_size 64, random
    block table over a 5120-page pool."""
    return prefill_case(q_lens=[512, 1024, 512, 1024], kv_lens=[81920] * 4, hq=32, hkv=8, d=128,
                        seed=seed, causal=True, paged=True, page_size=64,
                        name="ragged_paged_prefill_q512-1024_kv80k_h32kv8_d128_ps64")


def single_chunk_prefill(seed: int = 6) -> PrefillCase:
    """One request's 512-token prefill chunk appended to an 80K-token context
    (kv_len 81920, bottom-right causal), otherwise as ragged_paged_prefill:
    too few query tiles to fill the CUs without key splits."""
    return prefill_case(q_lens=[512], kv_lens=[81920], hq=32, hkv=8, d=128, seed=seed, causal=True, paged=True,
                        page_size=64, name="single_chunk_prefill_q512_kv80k_h32kv8_d128_ps64")


def mla_decode(kv_dtype: str = "bf16", seed: int = 5, causal: bool = True, q_dtype: str = "bf16") -> DecodeCase:
    """MLA-shaped split-KV decode: batch 8, 4 query tokens, 64 heads folded
    with 2 tokens into 128 rows, one latent KV head of width 576 (K = all 576,
    V = the first 512), kv_len 81920, page_size 64, bf16 or fp8 e4m3 KV (and
    with fp8 KV optionally fp8 e4m3 q), scale 0.07216882."""
    qtag = "" if q_dtype == "bf16" else "_q" + q_dtype
    return decode_case(batch=8, q_len=4, hq=64, hkv=1, d=576, dv=512, page_size=64,
                       seq_lens=[81920] * 8, seed=seed, kv_dtype=kv_dtype, latent=True,
                       scale=0.07216882, causal=causal, q_dtype=q_dtype,
                       name=f"mla_decode_b8_q4_h64_kv80k_d576-512_ps64_{kv_dtype}{qtag}")


@dataclasses.dataclass
class Fp8PrefillCase:
    name: str
    q: torch.Tensor                  # E4M3 codes (uint8) [Tq, Hq, 192]
    k: torch.Tensor                  # [Tk, Hkv, 192]
    v: torch.Tensor                  # [Tk, Hkv, 128]
    q_scale: float
    k_scale: float
    v_scale: float
    cu_seqlens_q: torch.Tensor       # int32 [B+1]
    cu_seqlens_kv: torch.Tensor      # int32 [B+1]
    scale: float
    causal: bool
    max_seqlen_q: int
    max_seqlen_kv: int
    seed: int
    window_left: int = -1

    def to(self, device) -> "Fp8PrefillCase":
        return dataclasses.replace(self, q=self.q.to(device), k=self.k.to(device), v=self.v.to(device),
                                   cu_seqlens_q=self.cu_seqlens_q.to(device),
                                   cu_seqlens_kv=self.cu_seqlens_kv.to(device))


def fp8_prefill_case(*, q_lens: list[int], kv_lens: list[int], hq: int, hkv: int, seed: int, causal: bool = True,
                     dqk: int = 192, dv: int = 128, scale: float | None = None, q_mult: float = 1.0,
                     window_left: int = -1, name: str = "") -> Fp8PrefillCase:
    """FP8 MLA-shaped prefill inputs: float32 N(0, 1) Q, K, V (Q times
    q_mult) quantised to E4M3 codes with one scale per tensor (amax / 448).
    The softmax scale defaults to 1 / sqrt(dqk)."""
    _, s_q, s_k, s_v = _streams(seed)
    tq, tk = sum(q_lens), sum(kv_lens)
    q, qs = _fp8_codes(_normal_f32(s_q, (tq, hq, dqk), q_mult))
    k, ks = _fp8_codes(_normal_f32(s_k, (tk, hkv, dqk)))
    v, vs = _fp8_codes(_normal_f32(s_v, (tk, hkv, dv)))
    return Fp8PrefillCase(name=name, q=q, k=k, v=v, q_scale=qs, k_scale=ks, v_scale=vs,
                          cu_seqlens_q=torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32),
                          cu_seqlens_kv=torch.tensor(np.concatenate([[0], np.cumsum(kv_lens)]), dtype=torch.int32),
                          scale=float(scale if scale is not None else 1.0 / math.sqrt(dqk)), causal=causal,
                          max_seqlen_q=max(q_lens, default=0), max_seqlen_kv=max(kv_lens, default=0), seed=seed,
                          window_left=window_left)


def fp8_mla_prefill(seed: int = 6, seq: int = 8192, kv: int | None = None) -> Fp8PrefillCase:
    """The FP8 MLA prefill workload: batch 1, seq query tokens over kv keys
    (default seq), 128 heads, q/k 192 wide, v 128 wide, E4M3 inputs with
    per-tensor scales, causal bottom-right, softmax scale 1/sqrt(192)."""
    kv = seq if kv is None else kv
    return fp8_prefill_case(q_lens=[seq], kv_lens=[kv], hq=128, hkv=128, seed=seed, causal=True,
                            name=f"fp8_mla_prefill_q{seq}_kv{kv}_h128_d192-128")


def sha256_of(*tensors) -> str:
    h = hashlib.sha256()
    for t in tensors:
        if t is not None:
            h.update(t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.uint8
                     else t.contiguous().numpy().tobytes())
    return h.hexdigest()


# --------------------------------------------------------------------------
# The prologue: cache append and the MLA K/V pack
# --------------------------------------------------------------------------

@dataclasses.dataclass
class AppendCase:
    name: str
    k_new: torch.Tensor                 # bf16 [N, Hkv, Dk]
    v_new: torch.Tensor | None          # bf16 [N, Hkv, Dv] (None: latent cache)
    k_cache: torch.Tensor               # [pages, page_size, Hkv, Dk] bf16, or uint8 E4M3 codes
    v_cache: torch.Tensor | None
    slot_mapping: torch.Tensor          # int64 [N]: row within the layer, -1 for warm-up tokens
    layer_base_rows: int
    page_size: int
    kv_dtype: str                       # "bf16" or "fp8_e4m3"
    k_scale: float
    v_scale: float
    seed: int

    def to(self, device) -> "AppendCase":
        f = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(self, k_new=f(self.k_new), v_new=f(self.v_new), k_cache=f(self.k_cache),
                                   v_cache=f(self.v_cache), slot_mapping=f(self.slot_mapping))


def append_case(*, num_tokens: int, hkv: int, dk: int, dv: int | None, page_size: int, pages_per_layer: int,
                layers: int = 2, layer: int = 1, kv_dtype: str = "bf16", warmup_tokens: int = 0,
                seed: int, name: str = "") -> AppendCase:
    """New tokens for one layer of a packed multi-layer paged cache.

    The cache holds `layers` layers of pages_per_layer pages each, every byte
    drawn at random (a canary: any write shows). Slots are distinct random
    rows of the layer; the first warmup_tokens tokens get slot -1. FP8
    caches use one scale per tensor of amax / 400 (so the largest values of
    each tensor saturate at 448)."""
    s_layout, _, s_k, s_v = _streams(seed)
    rng = np.random.Generator(np.random.PCG64(s_layout))
    rows = pages_per_layer * page_size
    slots = rng.choice(rows, size=num_tokens, replace=False).astype(np.int64)
    slots[:warmup_tokens] = -1
    k = _normal_f32(s_k, (num_tokens, hkv, dk))
    v = None if dv is None else _normal_f32(s_v, (num_tokens, hkv, dv))
    cache_rng = np.random.Generator(np.random.PCG64(s_layout.spawn(1)[0]))
    total_pages = layers * pages_per_layer
    if kv_dtype == "bf16":
        draw = lambda d: torch.from_numpy(cache_rng.integers(0, 1 << 16, size=(total_pages, page_size, hkv, d),
                                                             dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
        k_scale = v_scale = 1.0
    elif kv_dtype == "fp8_e4m3":
        draw = lambda d: torch.from_numpy(cache_rng.integers(0, 256, size=(total_pages, page_size, hkv, d),
                                                             dtype=np.uint8))
        k_scale = float(np.abs(k).max()) / 400.0
        v_scale = 1.0 if v is None else float(np.abs(v).max()) / 400.0
    else:
        raise ValueError(kv_dtype)
    kc = draw(dk)
    vc = None if dv is None else draw(dv)
    return AppendCase(name=name, k_new=torch.from_numpy(k).to(torch.bfloat16),
                      v_new=None if v is None else torch.from_numpy(v).to(torch.bfloat16),
                      k_cache=kc, v_cache=vc, slot_mapping=torch.from_numpy(slots),
                      layer_base_rows=layer * rows, page_size=page_size, kv_dtype=kv_dtype,
                      k_scale=k_scale, v_scale=v_scale, seed=seed)


@dataclasses.dataclass
class PackCase:
    name: str
    k_nope: torch.Tensor     # bf16 [T, H, dn] (possibly a strided view)
    k_rope: torch.Tensor     # bf16 [T, dr] (possibly a strided view)
    v: torch.Tensor          # bf16 [T, H, dv] (possibly a strided view)
    k_scale: float
    v_scale: float
    seed: int

    def to(self, device) -> "PackCase":
        return dataclasses.replace(self, k_nope=self.k_nope.to(device), k_rope=self.k_rope.to(device),
                                   v=self.v.to(device))


def pack_case(*, num_tokens: int, heads: int, d_nope: int = 128, d_rope: int = 64, d_v: int = 128,
              seed: int, strided: bool = False, name: str = "") -> PackCase:
    """Chunked-prefill MLA inputs: k_nope, a per-token rope vector, V. With
    strided=True each is a view into a wider buffer (the layouts a fused
    kv_b projection leaves: k_nope and v side by side per head, rope with a
    padded row). Scales are amax / 448 per tensor (K over nope and rope)."""
    _, s_q, s_k, s_v = _streams(seed)
    if strided:
        kv = _normal_f32(s_k, (num_tokens, heads, d_nope + d_v))
        rope_buf = _normal_f32(s_q, (num_tokens, 1, d_rope + 16))
        k_nope_f, v_f, rope_f = kv[:, :, :d_nope], kv[:, :, d_nope:], rope_buf[:, 0, :d_rope]
        t_kv = torch.from_numpy(kv).to(torch.bfloat16)
        t_rope = torch.from_numpy(rope_buf).to(torch.bfloat16)
        k_nope_t, v_t, rope_t = t_kv[:, :, :d_nope], t_kv[:, :, d_nope:], t_rope[:, 0, :d_rope]
    else:
        k_nope_f = _normal_f32(s_k, (num_tokens, heads, d_nope))
        v_f = _normal_f32(s_v, (num_tokens, heads, d_v))
        rope_f = _normal_f32(s_q, (num_tokens, d_rope))
        k_nope_t = torch.from_numpy(k_nope_f).to(torch.bfloat16)
        v_t = torch.from_numpy(v_f).to(torch.bfloat16)
        rope_t = torch.from_numpy(rope_f).to(torch.bfloat16)
    k_amax = max(float(np.abs(k_nope_f).max()), float(np.abs(rope_f).max()) if d_rope else 0.0)
    return PackCase(name=name, k_nope=k_nope_t, k_rope=rope_t, v=v_t, k_scale=k_amax / FP8_MAX,
                    v_scale=float(np.abs(v_f).max()) / FP8_MAX, seed=seed)
