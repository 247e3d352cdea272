"""The decode entry point that allocates nothing (attn_decode_paged_noalloc,
for callers that cannot call hipMalloc): its split partials live in the
library's static per-device scratch. Called through the C ABI, it must give
the output and LSE of attn_decode_paged bit for bit (the same plan and
kernels), on consecutive calls whose second input is smaller than the first
(the scratch keeps the first call's partials), and meet the oracle's bar.
A plan whose partials exceed the scratch is refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import _ffi, inputs
from helpers import TOL_BF16, TOL_FP8, compare, f64, oracle_decode

DEV = "cuda"


def _pair(case, **kw):
    c = case.to(DEV)
    args = (c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens)
    common = dict(max_seq_len=c.max_seq_len, softmax_scale=c.scale, causal=c.causal, head_dim_v=c.head_dim_v,
                  kv_dtype=None if c.kv_dtype == "bf16" else c.kv_dtype, k_scale=c.kv_scale, v_scale=c.kv_scale,
                  **kw)
    ref, lref = sap.decode_paged(*args, return_lse=True, **common)
    b, q_len, hq, _ = c.q.shape
    out = torch.full((b, q_len, hq, c.head_dim_v), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((b, q_len, hq), float("nan"), dtype=torch.float32, device=DEV)
    sap.decode_paged_noalloc(*args, out=out, lse=lse, **common)
    torch.cuda.synchronize()
    return ref.cpu(), lref.cpu(), out.cpu(), lse.cpu()


def _check(case, tol=TOL_BF16, **kw):
    ref, lref, out, lse = _pair(case, **kw)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lref.view(torch.int32))
    o, l = oracle_decode(case)
    return compare(f64(out), o, lse.numpy(), l, tol)


@pytest.mark.gpu
def test_noalloc_gqa_decode_two_calls_second_smaller():
    # first: the Qwen3-14B-shaped decode planned with the host's total of keys
    # (256 key ranges: 6.6 MB of partials); second: a smaller decode (3 splits)
    big = inputs.qwen3_14b_decode()
    print("call 1", big.name, flush=True)
    print(_check(big, total_kv_tokens=int(big.seq_lens.sum())))
    small = inputs.decode_case(batch=3, q_len=2, hq=8, hkv=2, d=128, dv=128, page_size=16,
                               seq_lens=[5, 300, 77], seed=91, causal=True, layout="noncontiguous")
    print("call 2", small.name, flush=True)
    print(_check(small, num_splits=3))


@pytest.mark.gpu
def test_noalloc_mla_decode_two_calls_second_smaller():
    big = inputs.decode_case(batch=4, q_len=4, hq=64, hkv=1, d=576, dv=512, page_size=64,
                             seq_lens=[4000, 1, 2500, 700], seed=92, kv_dtype="fp8_e4m3", latent=True,
                             scale=0.07216882, causal=True)
    print("call 1 mla fp8", flush=True)
    print(_check(big, tol=TOL_FP8, num_splits=4))
    small = inputs.decode_case(batch=2, q_len=1, hq=16, hkv=1, d=576, dv=512, page_size=16,
                               seq_lens=[300, 33], seed=93, latent=True, scale=0.07216882)
    print("call 2 mla bf16", flush=True)
    print(_check(small, num_splits=2))


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    """64 forced splits of the MLA 80K decode need 269 MB of partials, more
    than the 128 MiB scratch: refused on the host, nothing enqueued (the
    pointers are fake and never dereferenced)."""
    lib = _ffi.load()
    fake = 1 << 20
    p = _ffi.DecodeParams()
    for k, v in dict(q=fake, k_cache=fake, v_cache=fake, k_stride_page=64 * 576, k_stride_tok=576,
                     k_stride_head=576, v_stride_page=64 * 576, v_stride_tok=576, v_stride_head=576,
                     kv_dtype=_ffi.ATTN_BF16, k_scale=1.0, v_scale=1.0, seq_lens=fake, block_table=fake,
                     block_table_stride=1280, batch=8, q_len=4, num_q_heads=64, num_kv_heads=1,
                     head_dim_qk=576, head_dim_v=512, page_size=64, num_pages=10240, max_seq_len=81920,
                     softmax_scale=0.07216882, causal=1, num_splits=64, o=fake).items():
        setattr(p, k, v)
    assert lib.attn_decode_workspace_size(ctypes.byref(p)) == 64 * 8 * 4 * 64 * 513 * 4
    assert lib.attn_decode_paged_noalloc(ctypes.byref(p), None) == _ffi.ATTN_ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in lib.attn_last_error()
