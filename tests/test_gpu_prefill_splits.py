"""GPU parity of key-split prefill against the fp64 oracle: each query tile's
keys walked by several workgroups whose normalised partials are merged by
log-sum-exp ("TokenSpeed-MLA", split-KV with an LSE merge; prefill use cases
with few query rows over long keys).

Forced split counts put split boundaries inside requests, at requests shorter
than one split (splits with no keys), under causal masks whose rows end
before a split starts, and inside sliding windows. Results must meet the
same tolerance as the unsplit path and agree with it within rounding.
"""

import numpy as np
import pytest
import torch

import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import block_edge_rows, compare, f64, oracle_prefill, oracle_prefill_cached

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(case, kv_splits, workspace=None, return_lse=True):
    c = case.to(DEV)
    kw = dict(max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale,
              causal=c.causal, return_lse=return_lse, window_left=c.window_left, kv_splits=kv_splits,
              workspace=workspace)
    if c.paged:
        res = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, seq_lens_kv=c.seq_lens_kv, block_table=c.block_table, **kw)
    else:
        res = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, cu_seqlens_kv=c.cu_seqlens_kv, **kw)
    torch.cuda.synchronize()
    return (res[0].cpu(), res[1].cpu()) if return_lse else (res.cpu(), None)


def _check(case, splits):
    ref, lref = oracle_prefill(case)
    base, lbase = _run(case, 1)
    for s in splits:
        print("case", case.name, "splits", s, flush=True)
        out, lse = _run(case, s)
        print(compare(f64(out), ref, lse.numpy(), lref))
        # split and unsplit sum the same terms in another order
        assert np.abs(f64(out) - f64(base)).max() <= 2e-2
        a, b = lse.numpy(), lbase.numpy()
        fin = np.isfinite(b)
        assert np.array_equal(np.isfinite(a), fin) and np.array_equal(a[~fin], b[~fin])   # rows without keys
        assert np.abs(a[fin] - b[fin]).max() <= 1e-3


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_ragged_forced_splits(d, causal):
    case = inputs.prefill_case(q_lens=[1, 37, 128, 200, 129], kv_lens=[1, 37, 128, 900, 1300], hq=8, hkv=2, d=d,
                               seed=300 + d + causal, causal=causal, name=f"dense-d{d}-c{int(causal)}")
    _check(case, [2, 3, 5, 16])


@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_forced_splits(page_size):
    case = inputs.prefill_case(q_lens=[5, 64, 130, 40, 1], kv_lens=[300, 64, 2000, 17, 0], hq=8, hkv=2, d=128,
                               seed=310 + page_size, paged=True, page_size=page_size, name=f"paged-p{page_size}")
    _check(case, [2, 4, 7])


def test_gqa_group_of_one_and_odd_heads():
    case = inputs.prefill_case(q_lens=[33, 96], kv_lens=[1500, 700], hq=6, hkv=6, d=128, seed=320,
                               name="mha-6")
    _check(case, [2, 3])


@pytest.mark.parametrize("window", [0, 63, 200, 700])
def test_window_forced_splits(window):
    case = inputs.prefill_case(q_lens=[70, 128, 1], kv_lens=[1200, 128, 900], hq=8, hkv=2, d=128,
                               seed=330 + window, window_left=window, name=f"window-{window}")
    _check(case, [2, 3, 6])


def test_without_lse_and_with_a_caller_workspace():
    case = inputs.prefill_case(q_lens=[100, 20], kv_lens=[2100, 900], hq=4, hkv=1, d=128, seed=340, name="ws")
    ref, _ = oracle_prefill(case)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
    out, _ = _run(case, 4, workspace=ws, return_lse=False)
    print(compare(f64(out), ref))
    # a second call of another shape through the same workspace
    case2 = inputs.prefill_case(q_lens=[9], kv_lens=[3000], hq=8, hkv=2, d=64, seed=341, name="ws2")
    ref2, lref2 = oracle_prefill(case2)
    out2, lse2 = _run(case2, 8, workspace=ws)
    print(compare(f64(out2), ref2, lse2.numpy(), lref2))


def test_planner_splits_launches_of_few_long_units():
    def ws(q_lens, kv_lens, hq=32, hkv=8):
        case = inputs.prefill_case(q_lens=q_lens, kv_lens=kv_lens, hq=hq, hkv=hkv, d=128, seed=1, paged=True,
                                   page_size=64, name="plan")
        c = case.to(DEV)
        return sap.prefill_workspace_size(c.q, c.k, c.v, c.cu_seqlens_q, seq_lens_kv=c.seq_lens_kv,
                                          block_table=c.block_table, max_seqlen_q=c.max_seqlen_q,
                                          max_seqlen_kv=c.max_seqlen_kv, causal=True)
    row = 32 * 129 * 4                     # bytes of one query token's partials per split
    # one request of 512 queries over 40K keys: 16 query tiles x 8 head
    # groups = 128 workgroups, a quarter of the 512 slots: four splits
    assert ws([512], [40000]) == 4 * 512 * row
    # ... over 24K keys: no split under 8192 keys, so two
    assert ws([512], [24000]) == 2 * 512 * row
    # 1024 queries: 256 workgroups, half the slots: two splits
    assert ws([1024], [40000]) == 2 * 1024 * row
    # 512 + 1024 queries: 384 workgroups, between half and one round: unsplit
    assert ws([512, 1024], [40000, 40000]) == 0
    # four requests of 512-1024 queries over 80K keys: 768 workgroups over 512
    # slots, the second round half full: four splits
    assert ws([512, 1024, 512, 1024], [81920] * 4) == 4 * 3072 * row
    # 1024 workgroups are two whole rounds: unsplit
    assert ws([1024] * 4, [40000] * 4) == 0
    # short keys are never split
    assert ws([64], [8000]) == 0


def test_planner_split_matches_the_oracle():
    case = inputs.prefill_case(q_lens=[300], kv_lens=[40000], hq=8, hkv=2, d=128, seed=350, paged=True,
                               page_size=64, name="planned")
    c = case.to(DEV)
    assert sap.prefill_workspace_size(c.q, c.k, c.v, c.cu_seqlens_q, seq_lens_kv=c.seq_lens_kv,
                                      block_table=c.block_table, max_seqlen_q=c.max_seqlen_q,
                                      max_seqlen_kv=c.max_seqlen_kv, causal=True) > 0
    ref, lref = oracle_prefill(case)
    out, lse = _run(case, 0)
    print(compare(f64(out), ref, lse.numpy(), lref))


def _sampled(case, kv_splits, n_rows, seed=0):
    out, lse = _run(case, kv_splits)
    rng = np.random.default_rng(seed)
    tq, hq = case.q.shape[0], case.q.shape[1]
    rows = [(int(rng.integers(tq)), int(rng.integers(hq))) for _ in range(n_rows)] + [(0, 0), (tq - 1, hq - 1)]
    ref, lref = oracle_prefill(case, rows)
    got = np.stack([f64(out[t, h]) for t, h in rows])
    return compare(got, ref, np.array([float(lse[t, h]) for t, h in rows]), lref)


def test_ragged_paged_prefill_80k_forced_two_splits_block_edges():
    """The 4-request, 80K-key chunked prefill (512/1024 queries each) with its
    keys split in two (the boundary at key 40960 falls inside every
    request's visible keys): the first and last row of every 32-row block of
    every head (6,144 rows) against the oracle."""
    case = inputs.ragged_paged_prefill()
    print("case", case.name, flush=True)
    out, lse = _run(case, 2)
    rows = block_edge_rows(case.cu_seqlens_q.numpy(), case.q.shape[1])
    ref, lref = oracle_prefill_cached(case, rows)
    got = np.stack([f64(out[t, h]) for t, h in rows])
    res = compare(got, ref, np.array([float(lse[t, h]) for t, h in rows]), lref)
    res["rows_checked"] = len(rows)
    print(res)


def test_single_request_80k_planner_split_sampled():
    # one 512-query chunk over 80K keys: 128 workgroups unsplit, so the
    # planner splits the keys four ways
    case = inputs.single_chunk_prefill()
    print("case", case.name, flush=True)
    print(_sampled(case, 0, 48))
