"""The prologue before attention: cache append and the MLA K/V pack, as plain
numpy definitions.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What is computed:

  * FP8 quantisation of a value x with a per-tensor scale: the OCP E4M3
    ("fn") code nearest to y = x / scale, with y formed as an IEEE binary32
    quotient, ties going to the code with an even mantissa, and |y| beyond
    the largest finite value (448) saturating to +-448. The pages ask for a
    cast to FP8 without naming a rounding or an overflow rule; this is the
    plainest reading (round-to-nearest-even, and saturation because E4M3
    has no infinity), listed among the design readings.
  * Cache append ("Writing Page Attention with PyPTO", section 4.3): the new
    token of batch row b goes to cache row layer_base + max(slot_mapping[b],
    0): the slot is clamped at zero BEFORE the layer base is added, so a
    warm-up slot of -1 writes the layer's own first row and never the last
    row of the previous layer. Section 9.2: the layer base selects one layer
    of a packed multi-layer cache; section 10.2: only the addressed row may
    change. A row of a paged cache [pages, page_size, Hkv, D] is token row
    page * page_size + slot.
  * MLA K/V pack + FP8 quantise ("TokenSpeed-MLA", kernel capability
    summary: one fused kernel replacing concatenate + cast + cast in chunked
    prefill): K = concat(k_nope[t, h], k_rope[t]) for every head h (the rope
    part is one vector per token, shared by all heads), then K and V are each
    quantised with their own per-tensor scale.
"""

from __future__ import annotations

import numpy as np

from .attention import widen_bf16

E4M3_MAX = 448.0


def _e4m3_grid() -> np.ndarray:
    """Non-negative finite E4M3 values, indexed by their code 0x00..0x7E.

    From the format: exponent field e (bias 7) and mantissa m (3 bits);
    e = 0 is subnormal, m * 2**-9; otherwise (1 + m/8) * 2**(e - 7); the
    code 0x7F (e = 15, m = 7) is NaN and is not a value.
    """
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


_GRID = _e4m3_grid()


def quantize_e4m3fn(x: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """float values -> uint8 E4M3 codes of x / scale (binary32 quotient),
    round-to-nearest-even, saturating at +-448, the sign kept (so -0 and a
    negative value that rounds to zero give 0x80). NaN gives 0x7F."""
    with np.errstate(over="ignore"):                        # a binary32 quotient may overflow to inf: it saturates
        y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    y = y.astype(np.float64)
    mag = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.searchsorted(_GRID, mag, side="left")          # first grid value >= mag
    hi = np.minimum(hi, len(_GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _GRID[lo]
    d_hi = _GRID[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(_GRID[hi] == mag, hi, np.where(take_hi, hi, lo)).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7           # -0 and negatives that round to 0 keep the sign
    out = code | sign
    return np.where(np.isnan(y), np.uint8(0x7F), out).astype(np.uint8)


def cache_rows_view(cache: np.ndarray) -> np.ndarray:
    """[pages, page_size, Hkv, D] -> [pages * page_size, Hkv, D] token rows."""
    return cache.reshape(-1, *cache.shape[2:])


def cache_append(k_cache: np.ndarray, v_cache: np.ndarray | None, k_new: np.ndarray,
                 v_new: np.ndarray | None, slot_mapping: np.ndarray, layer_base_rows: int,
                 cache_format: str = "bf16", k_scale: float = 1.0, v_scale: float = 1.0):
    """Return copies of the caches (token-row views [rows, Hkv, D]) with each
    new token written at row layer_base_rows + max(slot, 0).

    k_new / v_new are bfloat16 bit patterns (uint16) [N, Hkv, D]. A bf16
    cache receives the bits unchanged; an "e4m3fn" cache receives
    quantize_e4m3fn(value, scale). Tokens are written in order, so when two
    tokens address one row the later one is what this returns (the GPU
    leaves either; tests accept either).
    """
    k_out = k_cache.copy()
    v_out = None if v_cache is None else v_cache.copy()
    for b, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        row = int(layer_base_rows) + max(int(slot), 0)
        k_out[row] = _store(k_new[b], cache_format, k_scale)
        if v_out is not None:
            v_out[row] = _store(v_new[b], cache_format, v_scale)
    return k_out, v_out


def _store(bits: np.ndarray, cache_format: str, scale: float) -> np.ndarray:
    if cache_format == "bf16":
        return bits
    if cache_format == "e4m3fn":
        return quantize_e4m3fn(widen_bf16(bits), scale)
    raise ValueError(cache_format)


def mla_kv_pack(k_nope: np.ndarray, k_rope: np.ndarray, v: np.ndarray, k_scale: float, v_scale: float):
    """bf16 bit patterns k_nope [T, H, dn], k_rope [T, dr], v [T, H, dv] ->
    (K codes [T, H, dn + dr], V codes [T, H, dv]), E4M3."""
    t, h, _ = k_nope.shape
    rope = np.broadcast_to(widen_bf16(k_rope)[:, None, :], (t, h, k_rope.shape[-1]))
    k = np.concatenate([widen_bf16(k_nope), rope], axis=-1)
    return quantize_e4m3fn(k, k_scale), quantize_e4m3fn(widen_bf16(v), v_scale)
