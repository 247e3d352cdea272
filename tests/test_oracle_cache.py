"""Pins of the oracle's cache-append, FP8-quantise and MLA K/V-pack functions
against things other than themselves:
  * E4M3 codes the OCP format definition fixes (1.0, 2.0, 0.5, 448, the
    smallest normal and subnormal values, 240);
  * every midpoint between neighbouring E4M3 values (ties go to the even
    mantissa) and the floats right beside it, from the independently pinned
    decoder;
  * saturation above 448, signed zeros;
  * quotients whose binary32 rounding lands on a midpoint that the exact
    quotient misses (the binary32 reading of x / scale);
  * the append rule of "Writing Page Attention with PyPTO", section 4.3 (clamp
    the slot at zero, then add the layer base) and its section 10.2 checks:
    a cache canary and a nonzero layer base;
  * the pack's concatenation order and the rope part shared by all heads,
    on hand-written values.
"""

import numpy as np
import pytest

import oracle

CODES = np.arange(256, dtype=np.uint8)
FINITE = CODES[~np.isnan(oracle.widen_e4m3fn(CODES))]


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("value,code", [
    (1.0, 0x38), (2.0, 0x40), (0.5, 0x30), (-2.0, 0xC0), (448.0, 0x7E), (-448.0, 0xFE),
    (2.0 ** -6, 0x08), (7 * 2.0 ** -9, 0x07), (2.0 ** -9, 0x01), (240.0, 0x77), (0.0, 0x00), (1.125, 0x39),
])
def test_e4m3_known_codes(value, code):
    assert oracle.quantize_e4m3fn(np.array([value]))[0] == code


def test_every_code_round_trips():
    back = oracle.quantize_e4m3fn(oracle.widen_e4m3fn(FINITE))
    assert np.array_equal(back, FINITE)


def test_midpoints_go_to_the_even_mantissa_and_neighbours_to_the_nearer_code():
    pos = np.sort(oracle.widen_e4m3fn(FINITE[FINITE < 0x80]))
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2                                   # exact in float32 (one more bit)
        ca, cb = oracle.quantize_e4m3fn(np.array([a, b]))
        even = ca if ca % 2 == 0 else cb
        assert oracle.quantize_e4m3fn(np.array([mid]))[0] == even, (a, b)
        below = np.nextafter(np.float32(mid), np.float32(-1))
        above = np.nextafter(np.float32(mid), np.float32(1e9))
        assert oracle.quantize_e4m3fn(np.array([below]))[0] == ca
        assert oracle.quantize_e4m3fn(np.array([above]))[0] == cb
        assert oracle.quantize_e4m3fn(np.array([-mid]))[0] == (even | 0x80)


def test_saturation_and_signed_zero():
    q = oracle.quantize_e4m3fn(np.array([449.0, 464.0, 470.0, 1e6, np.inf, -1e6, -np.inf]))
    assert list(q) == [0x7E] * 5 + [0xFE] * 2
    q = oracle.quantize_e4m3fn(np.array([-0.0, -(2.0 ** -11), 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11]))
    assert list(q) == [0x80, 0x80, 0x00, 0x00, 0x01]      # 2^-10 is a tie between 0 and 2^-9: even


def test_scale_divides_before_rounding():
    assert oracle.quantize_e4m3fn(np.array([1.0, 3.0, -896.0]), 2.0).tolist() == [0x30, 0x3C, 0xFE]
    # 100 / 0.25 = 400 lies halfway between 384 (0x7C) and 416 (0x7D): even
    assert oracle.quantize_e4m3fn(np.array([100.0]), 0.25)[0] == 0x7C


@pytest.mark.parametrize("xbits,sbits,code", [
    (0x3EE73334, 0x3FD9999A, 40),     # binary32 quotient is the midpoint 0.265625 -> even 0x28
    (0x3F2ECCCC, 0x40133333, 42),     # binary32 quotient is the midpoint 0.296875 -> even 0x2A
    (0x405B4CCD, 0x414E6666, 40),
])
def test_quotient_is_rounded_in_binary32_first(xbits, sbits, code):
    # the exact quotient lies beside the midpoint and would round the other way
    assert oracle.quantize_e4m3fn(np.array([_f32(xbits)]), float(_f32(sbits)))[0] == code


# ------------------------------------------------------------ cache append --

def _bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_append_canary_only_addressed_rows_change():
    rows, hkv, d = 64, 2, 8
    canary = np.full((rows, hkv, d), 0x7FC1, dtype=np.uint16)
    k_new = _bf16_bits(np.arange(3 * hkv * d, dtype=np.float32).reshape(3, hkv, d) + 1)
    v_new = _bf16_bits(-np.arange(3 * hkv * d, dtype=np.float32).reshape(3, hkv, d) - 1)
    slots = np.array([5, 17, 30], dtype=np.int64)
    k, v = oracle.cache_append(canary, canary, k_new, v_new, slots, layer_base_rows=32)
    changed = np.where(np.any(k != canary, axis=(1, 2)))[0].tolist()
    assert changed == [37, 49, 62]
    assert np.array_equal(k[49], k_new[1]) and np.array_equal(v[62], v_new[2])
    assert np.array_equal(np.where(np.any(v != canary, axis=(1, 2)))[0], changed)


def test_append_clamps_the_slot_before_adding_the_layer_base():
    rows, base = 48, 16
    canary = np.zeros((rows, 1, 8), dtype=np.uint16)
    k_new = _bf16_bits(np.full((1, 1, 8), 3.0, dtype=np.float32))
    k, _ = oracle.cache_append(canary, None, k_new, None, np.array([-1]), layer_base_rows=base)
    assert np.any(k[base] != 0) and not np.any(k[base - 1] != 0)     # never the previous layer's last row
    assert np.count_nonzero(np.any(k != 0, axis=(1, 2))) == 1


def test_append_fp8_cache_stores_quantised_codes():
    k_new = _bf16_bits(np.array([[[1.0, -2.0, 0.5, 448.0, 1000.0, 0.0, 3.0, 1.0625]]], dtype=np.float32))
    cache = np.zeros((4, 1, 8), dtype=np.uint8)
    k, _ = oracle.cache_append(cache, None, k_new, None, np.array([2]), 0, "e4m3fn", k_scale=1.0)
    assert k[2, 0].tolist() == [0x38, 0xC0, 0x30, 0x7E, 0x7E, 0x00, 0x44, 0x38]
    k, _ = oracle.cache_append(cache, None, k_new, None, np.array([2]), 0, "e4m3fn", k_scale=2.0)
    assert k[2, 0, :3].tolist() == [0x30, 0xB8, 0x28]


def test_pack_concatenates_nope_then_the_shared_rope():
    t, h, dn, dr, dv = 2, 3, 4, 2, 4
    nope = np.zeros((t, h, dn), dtype=np.float32)
    for hh in range(h):
        nope[:, hh, :] = hh + 1                                  # head-dependent
    rope = np.array([[0.5, 2.0], [-0.5, -2.0]], dtype=np.float32)  # token-dependent, shared by heads
    v = np.full((t, h, dv), 0.25, dtype=np.float32)
    k8, v8 = oracle.mla_kv_pack(_bf16_bits(nope), _bf16_bits(rope), _bf16_bits(v), 1.0, 0.5)
    assert k8.shape == (t, h, dn + dr) and v8.shape == (t, h, dv)
    assert k8[0, 0].tolist() == [0x38] * 4 + [0x30, 0x40]        # 1.0 x4, then 0.5, 2.0
    assert k8[1, 2].tolist() == [0x44] * 4 + [0xB0, 0xC0]        # 3.0 x4, then -0.5, -2.0
    assert np.array_equal(k8[:, 0, dn:], k8[:, 2, dn:])
    assert np.all(v8 == 0x30)                                     # 0.25 / 0.5 = 0.5
