"""GPU parity of ragged prefill (dense and paged KV) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import block_edge_rows, compare, f64, oracle_prefill, oracle_prefill_cached

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(case):
    c = case.to(DEV)
    kw = dict(max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale,
              causal=c.causal, return_lse=True, window_left=c.window_left)
    if c.paged:
        out, lse = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, seq_lens_kv=c.seq_lens_kv,
                               block_table=c.block_table, **kw)
    else:
        out, lse = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, cu_seqlens_kv=c.cu_seqlens_kv, **kw)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(case):
    out, lse = _run(case)
    ref, lref = oracle_prefill(case)
    return compare(f64(out), ref, lse.numpy(), lref)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 2), (4, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_ragged(d, hq, hkv, causal):
    lens = [1, 37, 128, 200, 129]
    case = inputs.prefill_case(q_lens=lens, kv_lens=lens, hq=hq, hkv=hkv, d=d, seed=d + hq + 7 * causal,
                               causal=causal)
    print("dense", d, hq, hkv, causal, flush=True)
    print(_check(case))


@pytest.mark.parametrize("d", [64, 128])
def test_chunked_bottom_right(d):
    # fewer queries than keys (chunked prefill), and more queries than keys
    # (the first rows see no key: O = 0, LSE = -inf)
    case = inputs.prefill_case(q_lens=[5, 64, 130, 40, 1], kv_lens=[300, 64, 1000, 17, 0], hq=8, hkv=2, d=d,
                               seed=31 + d, causal=True)
    print(_check(case))
    case = inputs.prefill_case(q_lens=[5, 64, 130, 40], kv_lens=[300, 64, 1000, 17], hq=8, hkv=2, d=d,
                               seed=32 + d, causal=False)
    print(_check(case))


@pytest.mark.parametrize("page_size", [16, 64])
@pytest.mark.parametrize("layout", ["random", "noncontiguous", "reverse"])
def test_paged_matches_oracle_and_dense_bitwise(page_size, layout):
    q_lens, kv_lens = [3, 100, 64, 257], [500, 100, 77, 1024]
    kw = dict(q_lens=q_lens, kv_lens=kv_lens, hq=8, hkv=2, d=128, seed=41, causal=True)
    paged = inputs.prefill_case(paged=True, page_size=page_size, layout=layout, **kw)
    dense = inputs.prefill_case(**kw)
    assert torch.equal(paged.q, dense.q)
    po, pl = _run(paged)
    do, dl = _run(dense)
    assert torch.equal(po.view(torch.int16), do.view(torch.int16)) and torch.equal(pl, dl)
    ref, lref = oracle_prefill(paged)
    print(compare(f64(po), ref, pl.numpy(), lref))


@pytest.mark.parametrize("page_size", [16, 128])
def test_paged_d64(page_size):
    # pages smaller than a 64-key tile (rows find their own pages) and
    # larger (a tile lies in one page); ragged tails in both
    case = inputs.prefill_case(q_lens=[7, 190, 64], kv_lens=[450, 190, 1100], hq=8, hkv=4, d=64, seed=43,
                               causal=True, paged=True, page_size=page_size, layout="random")
    print(_check(case))


def test_constant_v_and_single_key():
    case = inputs.prefill_case(q_lens=[70], kv_lens=[70], hq=2, hkv=1, d=128, seed=51, causal=True, q_mult=4.0)
    const = torch.randn(128).to(torch.bfloat16)
    case.v = const.expand_as(case.v).contiguous()
    out, lse = _run(case)
    # O is normalised by the FP32 sum of P while P itself is rounded to bf16
    # for the product: a constant V comes back within one bf16 step.
    cf = const.float().expand_as(out)
    assert torch.all((out.float() - cf).abs() <= cf.abs() * 2.0 ** -7)
    # causal row 0 sees only key 0: its LSE is that score in base 2
    qf, kf = f64(case.q), f64(case.k)
    for h in range(2):
        s = case.scale * float(qf[0, h] @ kf[0, 0])
        assert abs(float(lse[0, h]) - s / np.log(2.0)) < 1e-3


@pytest.mark.parametrize("paged", [False, True])
def test_batch_without_queries(paged):
    # every request has keys but no query token: nothing to compute, an
    # empty result, no error (dense and paged)
    case = inputs.prefill_case(q_lens=[0, 0, 0], kv_lens=[5, 300, 0], hq=4, hkv=2, d=128, seed=17, causal=True,
                               paged=paged, page_size=16)
    out, lse = _run(case)
    assert tuple(out.shape) == (0, 4, 128) and tuple(lse.shape) == (0, 4)


def test_negative_scale():
    case = inputs.prefill_case(q_lens=[33, 70], kv_lens=[100, 70], hq=4, hkv=2, d=128, seed=53, causal=True,
                               scale=-0.09)
    print(_check(case))


def test_peaky_scores():
    case = inputs.prefill_case(q_lens=[300, 77], kv_lens=[700, 77], hq=4, hkv=4, d=128, seed=52, causal=True,
                               q_mult=8.0)
    print(_check(case))


def _sampled(case, n_rows, seed=0):
    out, lse = _run(case)
    rng = np.random.default_rng(seed)
    tq, hq = case.q.shape[0], case.q.shape[1]
    rows = [(int(rng.integers(tq)), int(rng.integers(hq))) for _ in range(n_rows)]
    rows += [(0, 0), (tq - 1, hq - 1)]
    ref, lref = oracle_prefill(case, rows)
    got = np.stack([f64(out[t, h]) for t, h in rows])
    gl = np.array([float(lse[t, h]) for t, h in rows])
    return compare(got, ref, gl, lref)


def _edge_rows_check(case, out, lse):
    rows = block_edge_rows(case.cu_seqlens_q.numpy(), case.q.shape[1])
    ref, lref = oracle_prefill_cached(case, rows)
    got = np.stack([f64(out[t, h]) for t, h in rows])
    gl = np.array([float(lse[t, h]) for t, h in rows])
    res = compare(got, ref, gl, lref)
    res["rows_checked"] = len(rows)
    return res


@pytest.mark.parametrize("d", [128, 256])
def test_dense_causal_prefill_8k_block_edges(d):
    """The dense causal 8K workload at full size: the first and last row of
    every 32-row wave block of every head (16,384 rows, every workgroup's
    first and last row among them) against the oracle; and row 0 of each
    head, which sees key 0 alone, equals V[0] bit for bit (p = 1 and l = 1
    up to rounding far below a bf16 step)."""
    case = inputs.dense_causal_prefill(d=d)
    print("case", case.name, flush=True)
    out, lse = _run(case)
    print(_edge_rows_check(case, out, lse))
    assert torch.equal(out[0].view(torch.int16), case.v[0].view(torch.int16))


def test_ragged_paged_prefill_80k_block_edges():
    """The 4-request 80K-key chunked prefill as the planner runs it (four key
    splits): the first and last row of every 32-row block of every head
    (6,144 rows). Every row's causal bound lies past the last split boundary
    (keys 20480, 40960, 61440), so each checked row merges all four splits."""
    case = inputs.ragged_paged_prefill()
    print("case", case.name, flush=True)
    out, lse = _run(case)
    print(_edge_rows_check(case, out, lse))


def test_binding_rejects_mismatched_tensors():
    """Prefill's binding checks devices, ranks and sizes before anything is
    enqueued (the C ABI sees only pointers and strides)."""
    case = inputs.prefill_case(q_lens=[40], kv_lens=[90], hq=4, hkv=2, d=128, seed=61, causal=True)
    c = case.to(DEV)
    kw = dict(max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale, causal=True,
              cu_seqlens_kv=c.cu_seqlens_kv)
    with pytest.raises(ValueError):                                   # output with too few rows
        sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, **kw, out=torch.empty((39, 4, 128), dtype=torch.bfloat16,
                                                                         device=DEV))
    with pytest.raises(ValueError):                                   # K narrower than Q
        sap.prefill(c.q, c.k[..., :64], c.v, c.cu_seqlens_q, **kw)
    with pytest.raises(ValueError):                                   # K and V of different lengths
        sap.prefill(c.q, c.k, c.v[:-1], c.cu_seqlens_q, **kw)
    with pytest.raises(ValueError):                                   # K on the host
        sap.prefill(c.q, c.k.cpu(), c.v, c.cu_seqlens_q, **kw)
    out, lse = _run(case)
    ref, lref = oracle_prefill(case)
    compare(f64(out.cpu()), ref, lse.cpu().numpy(), lref)
