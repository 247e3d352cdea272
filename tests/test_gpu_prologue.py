"""GPU parity of the prologue kernels against the oracle, bit for bit: the
K/V cache append ("Writing Page Attention with PyPTO", sections 4.3, 9.2 and
10.2: clamp, layer base, cache canary) and the MLA K/V pack + FP8 quantise
("TokenSpeed-MLA", kernel capability summary).

Codes and copied bits are integer results, so every comparison is exact.
Where two new tokens address one row (warm-up slots of -1 all land on the
layer's row 0) the tokens race: each 8-element piece of that row must hold
the piece of one of them, and every other byte of the cache must equal the
oracle's.
"""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import bits

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run_append(case):
    c = case.to(DEV)
    kc, vc = c.k_cache.clone(), None if c.v_cache is None else c.v_cache.clone()
    sap.cache_append(c.k_new, c.v_new, kc, vc, c.slot_mapping, layer_base_rows=c.layer_base_rows,
                     k_scale=c.k_scale, v_scale=c.v_scale,
                     kv_dtype=None if case.kv_dtype == "bf16" else case.kv_dtype)
    torch.cuda.synchronize()
    return kc.cpu(), None if vc is None else vc.cpu()


def _check_append(case):
    k_gpu, v_gpu = _run_append(case)
    fmt = "bf16" if case.kv_dtype == "bf16" else "e4m3fn"
    k0 = oracle.cache_rows_view(bits(case.k_cache))
    v0 = None if case.v_cache is None else oracle.cache_rows_view(bits(case.v_cache))
    k_new, v_new = bits(case.k_new), None if case.v_new is None else bits(case.v_new)
    slots = case.slot_mapping.numpy()
    k_ref, v_ref = oracle.cache_append(k0, v0, k_new, v_new, slots, case.layer_base_rows, fmt,
                                       case.k_scale, case.v_scale)
    rows = case.layer_base_rows + np.maximum(slots, 0)
    uniq, counts = np.unique(rows, return_counts=True)
    shared = set(uniq[counts > 1].tolist())
    for got, ref, new, scale in ((oracle.cache_rows_view(bits(k_gpu)), k_ref, k_new, case.k_scale),
                                 (None if v_gpu is None else oracle.cache_rows_view(bits(v_gpu)), v_ref, v_new,
                                  case.v_scale)):
        if got is None:
            continue
        keep = np.ones(got.shape[0], dtype=bool)
        keep[list(shared)] = False
        assert np.array_equal(got[keep], ref[keep]), "cache differs outside shared rows"
        for r in shared:
            # the tokens race: every 8-element piece (one 16-byte load) of the
            # row must come from one of them
            cands = np.stack([oracle.cache_append(ref[r:r + 1] * 0, None, new[i:i + 1], None, np.array([0]), 0,
                                                  fmt, scale)[0][0] for i in np.where(rows == r)[0]])
            pieces = got[r].reshape(got.shape[1], -1, 8)
            cand_pieces = cands.reshape(len(cands), got.shape[1], -1, 8)
            match = (cand_pieces == pieces[None]).all(axis=-1).any(axis=0)
            assert match.all(), f"row {r}: a piece holds none of its tokens"
    return len(shared)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("page_size", [16, 128])
def test_append_qwen3_14b_shaped(kv_dtype, page_size):
    # one decode step of 64 requests, 8 KV heads of 128, into layer 1 of a
    # two-layer cache; three warm-up slots of -1 all land on the layer's row 0
    case = inputs.append_case(num_tokens=64, hkv=8, dk=128, dv=128, page_size=page_size,
                              pages_per_layer=4096 // page_size * 8, kv_dtype=kv_dtype, warmup_tokens=3,
                              seed=60 + page_size)
    print("append", kv_dtype, page_size, flush=True)
    assert _check_append(case) == 1


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_append_latent_cache(kv_dtype):
    # MLA latent cache: one 576-wide row per token, no separate V
    case = inputs.append_case(num_tokens=33, hkv=1, dk=576, dv=None, page_size=64, pages_per_layer=16,
                              kv_dtype=kv_dtype, seed=70)
    print("append latent", kv_dtype, flush=True)
    assert _check_append(case) == 0


def test_append_layer_zero_and_prefill_chunk():
    case = inputs.append_case(num_tokens=1500, hkv=2, dk=64, dv=64, page_size=16, pages_per_layer=128,
                              layers=1, layer=0, seed=71)
    assert _check_append(case) == 0


def test_append_rows_past_the_cache_are_not_written():
    case = inputs.append_case(num_tokens=8, hkv=2, dk=64, dv=64, page_size=16, pages_per_layer=4,
                              layers=2, layer=1, seed=72)
    # push two slots past the end of the cache (layer 1 is the last layer)
    case.slot_mapping[2] = 64 + 5
    case.slot_mapping[5] = 10 ** 9
    k_gpu, v_gpu = _run_append(case)
    keep = case.slot_mapping.clone()
    keep[[2, 5]] = -7                                   # marker: never written
    rows = oracle.cache_rows_view(bits(case.k_cache)).copy()
    ref = rows.copy()
    for i, s in enumerate(keep.tolist()):
        if s != -7:
            ref[case.layer_base_rows + max(s, 0)] = bits(case.k_new)[i]
    assert np.array_equal(oracle.cache_rows_view(bits(k_gpu)), ref)


def test_append_zero_tokens_is_a_no_op():
    case = inputs.append_case(num_tokens=1, hkv=1, dk=64, dv=64, page_size=16, pages_per_layer=2, seed=73)
    c = case.to(DEV)
    kc = c.k_cache.clone()
    sap.cache_append(c.k_new[:0], c.v_new[:0], kc, c.v_cache.clone(), c.slot_mapping[:0])
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc), bits(case.k_cache))       # bits: the canary holds NaN patterns


def _check_pack(case, k_out=None, v_out=None):
    c = case.to(DEV)
    k8, v8 = sap.mla_kv_pack_fp8(c.k_nope, c.k_rope, c.v, k_scale=c.k_scale, v_scale=c.v_scale,
                                 k_out=k_out, v_out=v_out)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.mla_kv_pack(bits(case.k_nope), bits(case.k_rope), bits(case.v), case.k_scale,
                                      case.v_scale)
    assert np.array_equal(bits(k8), k_ref) and np.array_equal(bits(v8), v_ref)


@pytest.mark.parametrize("strided", [False, True])
def test_pack_deepseek_shaped(strided):
    case = inputs.pack_case(num_tokens=257, heads=16, seed=80 + strided, strided=strided)
    _check_pack(case)


# head widths other than the MLA shape: K and V regions of different sizes
# (the shorter one runs out first in the shared loop), a rope row whose chunk
# count does not divide the workgroup (quantised per head), and no rope
@pytest.mark.parametrize("d_nope,d_rope,d_v,heads", [(64, 24, 96, 5), (128, 64, 512, 3), (256, 0, 64, 2),
                                                     (8, 8, 8, 33), (512, 40, 128, 1)])
def test_pack_other_widths(d_nope, d_rope, d_v, heads):
    case = inputs.pack_case(num_tokens=19, heads=heads, d_nope=d_nope, d_rope=d_rope, d_v=d_v, seed=83 + d_rope)
    _check_pack(case)


def test_pack_into_preallocated_strided_outputs_leaves_the_rest_alone():
    case = inputs.pack_case(num_tokens=40, heads=8, seed=82)
    kbuf = torch.full((40, 8, 256), 0x5A, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    vbuf = torch.full((40, 8, 136), 0xA5, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    _check_pack(case, k_out=kbuf[:, :, :192], v_out=vbuf[:, :, 8:])
    assert bool((kbuf.view(torch.uint8)[:, :, 192:] == 0x5A).all())
    assert bool((vbuf.view(torch.uint8)[:, :, :8] == 0xA5).all())


# scales: powers of two, amax/448-like values, and 24 log-uniform draws over
# 2^-24 .. 2^12 (the kernel divides through a reciprocal and one correction,
# which must give the binary32 quotient for every value and scale)
_SCALES = [1.0, 0.37109375, 3.1, 1.0 / 448.0, 2.0 ** -20, 0.0078125, 1.0000001, 0.99999994] + \
    [float(np.float32(2.0 ** x)) for x in np.random.Generator(np.random.PCG64(5)).uniform(-24, 12, 24)]


@pytest.mark.parametrize("scale", _SCALES)
def test_quantiser_on_every_bf16_value(scale):
    # every bf16 bit pattern except NaNs (infinities saturate), as k_nope and v
    pats = np.arange(1 << 16, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    pats = np.where(np.isnan(vals), 0, pats).astype(np.uint16)
    t, h = 128, 4                                          # 128 * 4 * 128 = 65536 values
    nope = torch.from_numpy(pats.view(np.int16).reshape(t, h, 128)).view(torch.bfloat16)
    v = torch.from_numpy(pats[::-1].copy().view(np.int16).reshape(t, h, 128)).view(torch.bfloat16)
    rope = torch.from_numpy(pats[: t * 64].view(np.int16).reshape(t, 64)).view(torch.bfloat16)
    case = inputs.PackCase(name="all-bf16", k_nope=nope, k_rope=rope, v=v, k_scale=scale, v_scale=scale, seed=0)
    _check_pack(case)


def test_pack_zero_tokens_is_a_no_op():
    k_nope = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=DEV)
    k_rope = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=DEV)
    k_out, v_out = sap.mla_kv_pack_fp8(k_nope, k_rope, v, k_scale=0.5, v_scale=0.25)
    torch.cuda.synchronize()
    assert tuple(k_out.shape) == (0, 4, 192) and tuple(v_out.shape) == (0, 4, 128)
