"""GPU parity of paged decode (split kernel + LSE merge) against the fp64 oracle.

Every case calls the HIP library through the C ABI (via the ctypes binding)
and compares element by element with the oracle on the same seeded inputs.
"""

import dataclasses
import numpy as np
import pytest
import torch

import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import TOL_BF16, bits, compare, f64, oracle_decode

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(case, num_splits=0, return_lse=True, total_kv_tokens=0):
    c = case.to(DEV)
    out, lse = sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                                max_seq_len=c.max_seq_len, softmax_scale=c.scale, causal=c.causal,
                                head_dim_v=c.head_dim_v,
                                kv_dtype=c.kv_dtype if c.kv_dtype != "bf16" else None,
                                k_scale=c.kv_scale, v_scale=c.kv_scale, num_splits=num_splits,
                                return_lse=return_lse, window_left=c.window_left, packed_q=c.packed_q,
                                total_kv_tokens=total_kv_tokens)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(case, num_splits=0, tol=TOL_BF16):
    out, lse = _run(case, num_splits)
    ref, lref = oracle_decode(case)
    return compare(f64(out), ref, lse.numpy(), lref, tol)


def test_tiny_gqa_decode_matches_oracle():
    case = inputs.gqa_decode_tiny()
    print("case", case.name, flush=True)
    res = _check(case)
    print(res)


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 7])
def test_tiny_gqa_decode_forced_splits(splits):
    _check(inputs.gqa_decode_tiny(), num_splits=splits)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("page_size", [16, 64, 128])
def test_boundary_lengths(d, page_size):
    # page and tile boundaries on both sides, a 1-key request and an empty one
    lens = [1, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 256, 257, 511, 512, 513, 0]
    case = inputs.decode_case(batch=len(lens), q_len=1, hq=8, hkv=2, d=d, dv=d, page_size=page_size,
                              seq_lens=lens, seed=11 + d + page_size, layout="noncontiguous")
    print("boundary", d, page_size, flush=True)
    for splits in (0, 1, 3):
        _check(case, num_splits=splits)
    # planned from the host's total of the keys (one round of resident units)
    out, lse = _run(case, total_kv_tokens=sum(lens))
    ref, lref = oracle_decode(case)
    print(compare(f64(out), ref, lse.numpy(), lref))


@pytest.mark.parametrize("q_len,hq,hkv", [(2, 8, 2), (3, 8, 8), (4, 8, 2), (4, 20, 4), (4, 16, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_multi_token_fold(q_len, hq, hkv, causal):
    lens = [1, 2, 3, 5, 40, 300]
    case = inputs.decode_case(batch=len(lens), q_len=q_len, hq=hq, hkv=hkv, d=128, dv=128, page_size=16,
                              seq_lens=lens, seed=q_len * 100 + hq, causal=causal)
    for splits in (0, 1, 2):
        _check(case, num_splits=splits)


def test_layouts_are_bitwise_identical():
    outs = []
    for layout in ("identity", "random", "reverse", "noncontiguous"):
        case = inputs.decode_case(batch=3, q_len=1, hq=8, hkv=2, d=128, dv=128, page_size=16,
                                  seq_lens=[200, 77, 513], seed=21, layout=layout)
        outs.append(_run(case, num_splits=3))
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


def test_shared_prefix_layout_is_bitwise_identical():
    kw = dict(batch=3, q_len=1, hq=8, hkv=2, d=64, dv=64, page_size=16, seq_lens=[64, 100, 90],
              seed=22, shared_prefix_pages=2)
    a = _run(inputs.decode_case(layout="shared_prefix", **kw), num_splits=2)
    b = _run(inputs.decode_case(layout="identity", **kw), num_splits=2)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_repeat_runs_are_bitwise_identical():
    case = inputs.decode_case(batch=8, q_len=1, hq=40, hkv=8, d=128, dv=128, page_size=128,
                              seq_len_range=(256, 2048), seed=23)
    a, b = _run(case), _run(case)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_constant_v_and_single_key():
    case = inputs.decode_case(batch=3, q_len=1, hq=8, hkv=2, d=128, dv=128, page_size=16,
                              seq_lens=[1, 50, 333], seed=24, q_mult=4.0)
    # constant V per (request, kv head): every valid slot holds that request's row
    vc = case.v_cache.clone()
    bt = case.block_table
    const = torch.randn(3, 2, 128).to(torch.bfloat16)
    for b, n in enumerate([1, 50, 333]):
        for j in range(n):
            vc[int(bt[b, j // 16]), j % 16] = const[b]
    case.v_cache = vc
    out, lse = _run(case, num_splits=3)
    for b in range(3):
        for h in range(8):
            assert torch.equal(out[b, 0, h].view(torch.int16), const[b, h // 4].view(torch.int16))
    # single key: O is that key's V row, bitwise; LSE is its scaled score in base 2
    kc = f64(case.k_cache)
    qf = f64(case.q)
    p0 = int(bt[0, 0])
    for h in range(8):
        assert torch.equal(out[0, 0, h].view(torch.int16), vc[p0, 0, h // 4].view(torch.int16))
        s = case.scale * float(qf[0, 0, h] @ kc[p0, 0, h // 4])
        assert abs(float(lse[0, 0, h]) - s / np.log(2.0)) < 1e-3


def test_one_hot_v_rows_sum_to_one():
    lk = 96
    case = inputs.decode_case(batch=1, q_len=1, hq=4, hkv=1, d=128, dv=128, page_size=16,
                              seq_lens=[lk], seed=25)
    vc = case.v_cache.clone()
    for j in range(lk):
        row = torch.zeros(128)
        row[j] = 1.0
        vc[int(case.block_table[0, j // 16]), j % 16, 0] = row.to(torch.bfloat16)
    case.v_cache = vc
    out, _ = _run(case, num_splits=2)
    p = f64(out)[0, 0]
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-2
    ref, _ = oracle_decode(case)
    compare(p, ref[0, 0])


def test_peaky_scores_force_rescale():
    # Q x 8 makes scores large; a rising ramp in K forces a new max on every tile.
    case = inputs.decode_case(batch=2, q_len=1, hq=8, hkv=2, d=128, dv=128, page_size=16,
                              seq_lens=[700, 513], seed=26, q_mult=8.0)
    kc = case.k_cache.clone()
    bt = case.block_table
    for b, n in enumerate([700, 513]):
        for j in range(n):
            kc[int(bt[b, j // 16]), j % 16] += (0.004 * j)
    case.k_cache = kc
    for splits in (1, 4):
        _check(case, num_splits=splits)


_QWEN_REF = {}


@pytest.mark.parametrize("hint", [False, True])
def test_qwen3_14b_decode_every_row_full_size(hint):
    """The Qwen3-14B-shaped workload at full size, planned as the benchmark
    plans it (with the host's total of the keys) and without that hint:
    every one of its 2,560 (request, head) rows against the oracle."""
    case = inputs.qwen3_14b_decode()
    tokens = int(case.seq_lens.sum())
    print("case", case.name, "tokens", tokens, "hint", hint, flush=True)
    out, lse = _run(case, total_kv_tokens=tokens if hint else 0)
    if case.name not in _QWEN_REF:
        _QWEN_REF[case.name] = oracle_decode(case)
    ref, lref = _QWEN_REF[case.name]
    res = compare(f64(out), ref, lse.numpy(), lref)
    res["rows_checked"] = int(np.prod(lref.shape))
    print(res)


# ------------------------------------------------------------- key ranges --

def _lens(rng, n, lo, hi, zeros=0.0):
    return [0 if rng.random() < zeros else int(rng.integers(lo, hi + 1)) for _ in range(n)]


_KR = np.random.default_rng(5)
_KEY_RANGE_CASES = {
    # one request cut into 33 pieces (K = 257 tiles / 8)
    "one_long_request": dict(batch=1, q_len=1, hq=8, hkv=2, d=128, page_size=16, seq_lens=[8191]),
    # 300 short requests, a fifth of them empty: ranges of ~3 tiles hold
    # several whole requests each (written final) and cut others
    "many_short_with_empty": dict(batch=300, q_len=1, hq=8, hkv=2, d=64, page_size=16,
                                  seq_lens=_lens(_KR, 300, 1, 40, zeros=0.2), max_pages=32, bound=512),
    # two query groups per KV head (G 8, F 2), causal: the last tile of a
    # request is empty for the first query group's rows
    "causal_q4_two_groups": dict(batch=5, q_len=4, hq=16, hkv=2, d=128, page_size=16, causal=True,
                                 seq_lens=[1, 2, 3000, 33, 1500]),
    # the largest batch the kernels scan, and one past it (per-request splits)
    # (these three pass a max_seq_len bound of 512: with a bound of at most
    # 8 tiles the planner runs short requests unsplit)
    "batch_512": dict(batch=512, q_len=1, hq=4, hkv=1, d=64, page_size=16, seq_lens=_lens(_KR, 512, 0, 100),
                      max_pages=32, bound=512),
    "batch_513_splits": dict(batch=513, q_len=1, hq=4, hkv=1, d=64, page_size=16,
                             seq_lens=_lens(_KR, 513, 0, 100), max_pages=32, bound=512),
    "d256_ragged": dict(batch=9, q_len=1, hq=16, hkv=4, d=256, page_size=64,
                        seq_lens=[0, 4096, 17, 2000, 31, 32, 33, 700, 1]),
}


@pytest.mark.parametrize("name", list(_KEY_RANGE_CASES))
def test_key_ranges_match_oracle(name):
    kw = dict(_KEY_RANGE_CASES[name])
    d = kw.pop("d")
    bound = kw.pop("bound", 0)
    case = inputs.decode_case(dv=d, d=d, seed=300 + len(name), layout="noncontiguous", **kw)
    if bound:
        case = dataclasses.replace(case, max_seq_len=bound)
    c = case.to(DEV)
    plan = sap.decode_plan(sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                                             max_seq_len=c.max_seq_len, softmax_scale=c.scale, causal=c.causal))
    print(name, "key ranges", plan["key_ranges"], "splits", plan["num_splits"], flush=True)
    assert (plan["key_ranges"] > 0) == (kw["batch"] <= 512)
    res = _check(case)
    res["rows_checked"] = int(np.prod(case.q.shape[:3]))
    print(res)


def test_key_ranges_constant_v_and_single_key():
    # the exact-value invariants through the key-range plan: constant V comes
    # back bitwise (requests cut into pieces included), a single key's O is its
    # V row bitwise
    lens = [1, 50, 5000]
    case = inputs.decode_case(batch=3, q_len=1, hq=8, hkv=2, d=128, dv=128, page_size=16,
                              seq_lens=lens, seed=27, q_mult=4.0)
    vc = case.v_cache.clone()
    bt = case.block_table
    const = torch.randn(3, 2, 128).to(torch.bfloat16)
    for b, n in enumerate(lens):
        for j in range(n):
            vc[int(bt[b, j // 16]), j % 16] = const[b]
    case.v_cache = vc
    c = case.to(DEV)
    plan = sap.decode_plan(sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                                             max_seq_len=c.max_seq_len, softmax_scale=c.scale))
    assert plan["key_ranges"] > 1
    out, lse = _run(case)
    for b in range(3):
        for h in range(8):
            assert torch.equal(out[b, 0, h].view(torch.int16), const[b, h // 4].view(torch.int16))
    p0 = int(bt[0, 0])
    for h in range(8):
        assert torch.equal(out[0, 0, h].view(torch.int16), vc[p0, 0, h // 4].view(torch.int16))


@pytest.mark.parametrize("plan", ["key_ranges", "splits", "latent"])
def test_split_and_merge_phases_equal_the_whole_call(plan):
    # attn_decode_paged_split then attn_decode_paged_merge, with the same
    # out, lse and workspace, give attn_decode_paged's result bit for bit
    if plan == "latent":
        case = inputs.decode_case(batch=3, q_len=2, hq=32, hkv=1, d=576, dv=512, page_size=64, latent=True,
                                  seq_lens=[3000, 1, 900], seed=28, scale=0.07216882)
    else:
        case = inputs.decode_case(batch=6, q_len=1, hq=40, hkv=8, d=128, dv=128, page_size=128,
                                  seq_lens=[4000, 0, 300, 8000, 77, 2500], seed=29)
    c = case.to(DEV)
    kw = dict(max_seq_len=c.max_seq_len, softmax_scale=c.scale, head_dim_v=c.head_dim_v,
              num_splits=3 if plan != "key_ranges" else 0)
    args = (c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens)
    p = sap.decode_params(*args, **kw)
    info = sap.decode_plan(p)
    assert (info["key_ranges"] > 0) == (plan == "key_ranges") and info["workspace_bytes"] > 0
    ws = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device=DEV)
    ref, lref = sap.decode_paged(*args, workspace=ws, return_lse=True, **kw)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(lref, float("nan"))
    ws.fill_(0xFF)                                   # the split phase must write what the merge reads
    sap.decode_paged(*args, workspace=ws, out=out, lse=lse, phase="split", **kw)
    sap.decode_paged(*args, workspace=ws, out=out, lse=lse, phase="merge", **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lref.view(torch.int32))


# ------------------------------------------------------------------ merge --

@pytest.mark.parametrize("s,r,dv", [(1, 5, 128), (3, 100, 128), (16, 2560, 128), (7, 33, 512), (64, 10, 64)])
def test_merge_lse_matches_oracle(s, r, dv):
    import oracle
    g = torch.Generator().manual_seed(s * 1000 + r)
    o_parts = torch.randn(s, r, dv, generator=g)
    lse_parts = torch.randn(s, r, generator=g) * 8
    # some empty splits (-inf), and one row with every split empty
    mask = torch.rand(s, r, generator=g) < 0.2
    lse_parts[mask] = -float("inf")
    lse_parts[:, 0] = -float("inf")
    o_parts[mask] = float("nan")          # never read
    o_parts[:, 0] = float("nan")
    o, lse = sap.merge_lse(o_parts.to(DEV), lse_parts.to(DEV), out_dtype=torch.float32)
    ref, lref = oracle.merge_lse(o_parts.double().numpy(), lse_parts.double().numpy())
    res = compare(o.cpu().double().numpy(), ref, lse.cpu().double().numpy(), lref,
                  tol=dict(max_abs=1e-5, mean_abs=1e-6), lse_tol=1e-5)
    ob, _ = sap.merge_lse(o_parts.to(DEV), lse_parts.to(DEV), out_dtype=torch.bfloat16)
    compare(f64(ob.cpu()), ref)
    print(res)


@pytest.mark.parametrize("pool", [1, 0])
@pytest.mark.parametrize("latent", [False, True])
def test_no_request_has_keys(latent, pool):
    # every request empty: O = 0 and LSE = -inf exactly, planned and forced
    # split (a one-page pool, as a cache that has not been written yet, or
    # an empty cache)
    kw = dict(batch=3, q_len=2, page_size=16, seq_lens=[0, 0, 0], seed=23, pool_pages=pool, max_pages=1)
    if latent:
        case = inputs.decode_case(hq=64, hkv=1, d=576, dv=512, latent=True, scale=0.07216882, **kw)
    else:
        case = inputs.decode_case(hq=8, hkv=2, d=128, dv=128, **kw)
    for splits in (0, 2):
        c = case.to(DEV)
        out, lse = sap.decode_paged(c.q, c.k_cache, None if latent else c.v_cache, c.block_table, c.seq_lens,
                                    max_seq_len=c.max_seq_len, softmax_scale=c.scale, causal=c.causal,
                                    head_dim_v=c.head_dim_v, num_splits=splits, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu().float(), torch.zeros(out.shape))
        assert bool(torch.all(lse.cpu() == float("-inf")))


def test_empty_batch():
    # batch 0: nothing to compute, empty outputs, no error
    q = torch.empty((0, 1, 8, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((1, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((0, 1), dtype=torch.int32, device=DEV)
    sl = torch.zeros((0,), dtype=torch.int32, device=DEV)
    out, lse = sap.decode_paged(q, k, k.clone(), bt, sl, max_seq_len=16, softmax_scale=0.1, return_lse=True)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 1, 8, 128) and tuple(lse.shape) == (0, 1, 8)


def test_merge_lse_without_rows():
    o_parts = torch.empty((3, 0, 128), dtype=torch.float32, device=DEV)
    lse_parts = torch.empty((3, 0), dtype=torch.float32, device=DEV)
    o, lse = sap.merge_lse(o_parts, lse_parts)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (0, 128) and tuple(lse.shape) == (0,)


def test_binding_rejects_mismatched_tensors():
    """The binding checks what the C ABI cannot see (devices, ranks, the
    sizes the kernels index with) and raises before anything is enqueued."""
    case = inputs.decode_case(batch=2, q_len=1, hq=8, hkv=2, d=128, dv=128, page_size=16,
                              seq_lens=[37, 100], seed=5)
    c = case.to(DEV)
    kw = dict(max_seq_len=c.max_seq_len, softmax_scale=c.scale)
    bad = [
        dict(out=torch.empty((2, 1, 8, 64), dtype=torch.bfloat16, device=DEV)),     # too few channels
        dict(out=torch.empty((2, 1, 8, 128), dtype=torch.float32, device=DEV)),     # wrong dtype
        dict(out=torch.empty((2, 1, 8, 128), dtype=torch.bfloat16)),                # host memory
        dict(lse=torch.empty((2, 1, 4), dtype=torch.float32, device=DEV)),          # too few heads
    ]
    for extra in bad:
        with pytest.raises(ValueError):
            sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, **kw, **extra)
    with pytest.raises(ValueError):                                                 # K rows narrower than q
        sap.decode_paged(c.q, c.k_cache[..., :64], c.v_cache, c.block_table, c.seq_lens, **kw)
    with pytest.raises(ValueError):                                                 # a table row short
        sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table[:1], c.seq_lens, **kw)
    with pytest.raises(ValueError):
        sap.decode_paged_noalloc(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, **kw,
                                 out=torch.empty((2, 1, 8, 64), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        sap.merge_lse(torch.zeros((2, 4, 128), device=DEV), torch.zeros((2, 4), device=DEV),
                      out=torch.empty((4, 64), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    # the same call with matching tensors runs
    out = sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, **kw)
    ref, _ = oracle_decode(case)
    compare(f64(out.cpu()), ref)
