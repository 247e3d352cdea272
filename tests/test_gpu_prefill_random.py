"""GPU parity of ragged prefill on seeded random shapes: request counts,
query and key lengths (chunks appended to histories, empty requests), head
counts and GQA groups, head dims, causal or not, sliding windows, dense or
paged K/V with random page sizes, and key splits forced or planned, against
the fp64 oracle on every row."""

import numpy as np
import pytest

import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import compare, f64, oracle_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(seed):
    rng = np.random.default_rng(3000 + seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 4]))
    batch = int(rng.integers(1, 6))
    q_lens = rng.integers(0, 260, size=batch).tolist()
    q_lens[int(rng.integers(batch))] = int(rng.integers(1, 260))
    kv_lens = [q + int(rng.integers(0, 2500)) for q in q_lens]
    causal = bool(rng.integers(2))
    window = int(rng.choice([-1, -1, 0, 40, 300]))
    paged = bool(rng.integers(2))
    page = int(rng.choice([16, 64, 128]))
    splits = int(rng.choice([0, 1, 2, 5]))
    case = inputs.prefill_case(q_lens=q_lens, kv_lens=kv_lens, hq=hkv * group, hkv=hkv, d=d, seed=4000 + seed,
                               causal=causal, paged=paged, page_size=page, window_left=window,
                               name=f"random-{seed}")
    return case, splits


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(seed):
    case, splits = _case(seed)
    c = case.to(DEV)
    kw = dict(max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale, causal=c.causal,
              return_lse=True, window_left=c.window_left, kv_splits=splits)
    kv = dict(seq_lens_kv=c.seq_lens_kv, block_table=c.block_table) if c.paged else dict(cu_seqlens_kv=c.cu_seqlens_kv)
    print(f"seed {seed}: q {case.cu_seqlens_q.tolist()} kv {case.seq_lens_kv.tolist()} heads {c.q.shape[1]}/"
          f"{(c.k.shape[2] if c.paged else c.k.shape[1])} d {c.q.shape[2]} causal {c.causal} window {c.window_left} "
          f"paged {c.paged} splits {splits}", flush=True)
    out, lse = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, **kv, **kw)
    ref, lref = oracle_prefill(case)
    print(compare(f64(out.cpu()), ref, lse.cpu().numpy(), lref))


@pytest.mark.parametrize("seed", range(12))
def test_random_prefill_short_histories(seed):
    """Key lengths drawn apart from the query lengths: requests with fewer
    keys than queries (bottom-right causal rows that see no key: O = 0, LSE =
    -inf) and requests with no keys at all, causal or not, dense or paged."""
    rng = np.random.default_rng(7000 + seed)
    batch = int(rng.integers(1, 6))
    q_lens = rng.integers(1, 300, size=batch).tolist()
    kv_lens = rng.integers(0, 400, size=batch).tolist()
    kv_lens[int(rng.integers(batch))] = 0
    hkv, group = int(rng.choice([1, 2])), int(rng.choice([1, 4]))
    case = inputs.prefill_case(q_lens=q_lens, kv_lens=kv_lens, hq=hkv * group, hkv=hkv, d=int(rng.choice([64, 128])),
                               seed=8000 + seed, causal=bool(rng.integers(2)), paged=bool(rng.integers(2)),
                               page_size=16, name=f"short-{seed}")
    c = case.to(DEV)
    kw = dict(max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale, causal=c.causal,
              return_lse=True, kv_splits=int(rng.choice([0, 2])))
    kv = dict(seq_lens_kv=c.seq_lens_kv, block_table=c.block_table) if c.paged else dict(cu_seqlens_kv=c.cu_seqlens_kv)
    print(f"seed {seed}: q {q_lens} kv {kv_lens} causal {c.causal} paged {c.paged}", flush=True)
    out, lse = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, **kv, **kw)
    ref, lref = oracle_prefill(case)
    print(compare(f64(out.cpu()), ref, lse.cpu().numpy(), lref))


@pytest.mark.parametrize("splits", [0, 3])
def test_many_short_chunks(splits):
    """A serving-shaped batch: 64 requests of 1-20 new tokens each over
    histories of up to 1500 keys (GQA 32/8, paged), so almost every query
    tile is partial and most workgroups of the grid find no rows. Every row
    against the oracle."""
    rng = np.random.default_rng(5000 + splits)
    q_lens = rng.integers(1, 21, size=64).tolist()
    kv_lens = [q + int(rng.integers(0, 1501)) for q in q_lens]
    case = inputs.prefill_case(q_lens=q_lens, kv_lens=kv_lens, hq=32, hkv=8, d=128, seed=6000 + splits, causal=True,
                               paged=True, page_size=64, name=f"chunks-{splits}")
    c = case.to(DEV)
    out, lse = sap.prefill(c.q, c.k, c.v, c.cu_seqlens_q, seq_lens_kv=c.seq_lens_kv, block_table=c.block_table,
                           max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale,
                           causal=True, return_lse=True, kv_splits=splits)
    ref, lref = oracle_prefill(case)
    print(f"splits {splits}: {sum(q_lens)} query tokens", compare(f64(out.cpu()), ref, lse.cpu().numpy(), lref))
