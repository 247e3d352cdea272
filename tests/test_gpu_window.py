"""GPU parity of the sliding window and of packed query rows ("TokenSpeed-MLA",
kernel capability summary: window_left; packed-query paragraph) against the
fp64 oracle, for the GQA decode, the latent (MLA) decode and the prefill.

Windows cover 0 (a row sees its causal block only), one tile, a tile
boundary, a window wider than the history, and windows whose start is not
tile-aligned; split counts force windows that begin inside a split and
splits that lie wholly before some rows' windows.
"""

import pytest
import torch

import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import TOL_BF16, TOL_FP8, compare, f64, oracle_decode, oracle_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda"
LENS = [1, 17, 33, 64, 100, 300, 700]


def _decode(case, num_splits=0):
    c = case.to(DEV)
    out, lse = sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, max_seq_len=c.max_seq_len,
                                softmax_scale=c.scale, causal=c.causal, head_dim_v=c.head_dim_v,
                                kv_dtype=None if c.kv_dtype == "bf16" else c.kv_dtype,
                                k_scale=c.kv_scale, v_scale=c.kv_scale, num_splits=num_splits, return_lse=True,
                                window_left=c.window_left, packed_q=c.packed_q)
    torch.cuda.synchronize()
    ref, lref = oracle_decode(case)
    tol = TOL_BF16 if case.kv_dtype == "bf16" else TOL_FP8
    return compare(f64(out.cpu()), ref, lse.cpu().numpy(), lref, tol)


def _prefill(case):
    c = case.to(DEV)
    kw = dict(max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale,
              causal=c.causal, return_lse=True, window_left=c.window_left)
    if c.paged:
        out, lse = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, seq_lens_kv=c.seq_lens_kv,
                               block_table=c.block_table, **kw)
    else:
        out, lse = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, cu_seqlens_kv=c.cu_seqlens_kv, **kw)
    torch.cuda.synchronize()
    ref, lref = oracle_prefill(case)
    return compare(f64(out.cpu()), ref, lse.cpu().numpy(), lref)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [0, 1, 31, 32, 90, 5000])
def test_gqa_decode_window(d, window):
    case = inputs.decode_case(batch=len(LENS), q_len=1, hq=8, hkv=2, d=d, dv=d, page_size=16, seq_lens=LENS,
                              seed=300 + d + window, layout="noncontiguous", window_left=window)
    print("gqa window", d, window, flush=True)
    for splits in (0, 1, 3, 8):
        _decode(case, splits)


@pytest.mark.parametrize("q_len,hq,hkv", [(4, 8, 2), (3, 20, 4), (4, 16, 1)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [0, 45, 200])
def test_gqa_decode_window_multi_token(q_len, hq, hkv, causal, window):
    case = inputs.decode_case(batch=len(LENS), q_len=q_len, hq=hq, hkv=hkv, d=128, dv=128, page_size=64,
                              seq_lens=LENS, seed=q_len * 10 + hq + window, causal=causal, window_left=window)
    print("gqa window multi", q_len, hq, hkv, causal, window, flush=True)
    for splits in (0, 1, 4):
        _decode(case, splits)


@pytest.mark.parametrize("q_len,hq,hkv", [(4, 20, 4), (4, 8, 1), (3, 12, 1), (2, 64, 4)])
@pytest.mark.parametrize("window", [-1, 60])
def test_gqa_decode_packed(q_len, hq, hkv, window):
    # G * q_len rows packed as token * G + head, in 16-row units (G = 5, q = 4
    # fills one unit and a quarter; G = 16, q = 2 fills two)
    case = inputs.decode_case(batch=len(LENS), q_len=q_len, hq=hq, hkv=hkv, d=128, dv=128, page_size=16,
                              seq_lens=LENS, seed=7 * q_len + hq, causal=True, window_left=window, packed_q=True)
    print("gqa packed", q_len, hq, hkv, window, flush=True)
    for splits in (0, 1, 3):
        _decode(case, splits)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("hq,q_len,window", [(128, 1, 0), (128, 1, 40), (16, 4, 70), (64, 2, 5000), (32, 4, 31)])
def test_mla_decode_window(kv_dtype, hq, q_len, window):
    case = inputs.decode_case(batch=len(LENS), q_len=q_len, hq=hq, hkv=1, d=576, dv=512, page_size=16,
                              seq_lens=LENS, seed=hq + q_len + window, kv_dtype=kv_dtype, latent=True,
                              scale=0.07216882, causal=True, layout="noncontiguous", window_left=window)
    print("mla window", kv_dtype, hq, q_len, window, flush=True)
    for splits in (0, 1, 3):
        _decode(case, splits)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("hq,q_len,window", [(96, 4, -1), (96, 4, 50), (40, 4, -1), (16, 3, -1)])
def test_mla_decode_packed(kv_dtype, hq, q_len, window):
    # 96 heads x 4 tokens = 384 packed rows: three 128-row tiles, the second
    # holding tokens 1 and 2 split at head 32 ("TokenSpeed-MLA", packed-query
    # paragraph)
    case = inputs.decode_case(batch=len(LENS), q_len=q_len, hq=hq, hkv=1, d=576, dv=512, page_size=64,
                              seq_lens=LENS, seed=hq * q_len + 3, kv_dtype=kv_dtype, latent=True,
                              scale=0.07216882, causal=True, window_left=window, packed_q=True)
    print("mla packed", kv_dtype, hq, q_len, window, flush=True)
    for splits in (0, 1, 3):
        _decode(case, splits)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [0, 63, 64, 130, 5000])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_window_dense(d, window, causal):
    # ragged: a prefill from empty, a chunk appended to a history (lq < lk),
    # and a request with more keys than queries by a non-tile amount
    case = inputs.prefill_case(q_lens=[300, 97, 1, 160], kv_lens=[300, 433, 70, 555], hq=8, hkv=2, d=d,
                               seed=400 + d + window, causal=causal, window_left=window)
    print("prefill window", d, window, causal, flush=True)
    _prefill(case)


@pytest.mark.parametrize("page_size", [16, 64, 128])
@pytest.mark.parametrize("window", [0, 100, 257])
def test_prefill_window_paged(page_size, window):
    case = inputs.prefill_case(q_lens=[300, 97, 1, 160], kv_lens=[300, 433, 70, 555], hq=4, hkv=4, d=128,
                               seed=500 + page_size + window, causal=True, paged=True, page_size=page_size,
                               layout="noncontiguous", window_left=window)
    print("prefill window paged", page_size, window, flush=True)
    _prefill(case)


@pytest.mark.parametrize("seed", range(16))
def test_random_decode_window_and_packing(seed):
    """Seeded random GQA and latent decodes with windows (from 0 to wider
    than the history), packed or folded query rows, 1-4 query tokens, causal
    or not, planned or with forced splits."""
    import numpy as np
    rng = np.random.default_rng(9000 + seed)
    latent = bool(rng.integers(2))
    batch = int(rng.integers(1, 12))
    q_len = int(rng.integers(1, 5))
    max_len = int(rng.choice([50, 600, 4000]))
    lens = rng.integers(0, max_len + 1, size=batch).tolist()
    window = int(rng.choice([0, 1, 31, 77, 300, 5000]))
    packed = bool(rng.integers(2))
    causal = bool(rng.integers(2))
    if latent:
        hq = int(rng.choice([16, 32, 96, 128]))
        case = inputs.decode_case(batch=batch, q_len=q_len, hq=hq, hkv=1, d=576, dv=512, page_size=64,
                                  seq_lens=lens, seed=9500 + seed, latent=True, scale=0.07216882, causal=causal,
                                  window_left=window, packed_q=packed, layout="random")
    else:
        hkv = int(rng.choice([1, 2, 4]))
        hq = hkv * int(rng.choice([1, 3, 5, 8]))
        d = int(rng.choice([64, 128]))
        case = inputs.decode_case(batch=batch, q_len=q_len, hq=hq, hkv=hkv, d=d, dv=d,
                                  page_size=int(rng.choice([16, 128])), seq_lens=lens, seed=9500 + seed,
                                  causal=causal, window_left=window, packed_q=packed, layout="random")
    splits = int(rng.choice([0, 0, 3]))
    print(f"seed {seed}: latent {latent} b{batch} q{q_len} hq{hq} window {window} packed {packed} causal {causal} "
          f"splits {splits}", _decode(case, splits), flush=True)
