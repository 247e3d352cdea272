"""GPU parity of paged decode on seeded random shapes, planned with and
without the host's total of the keys: the planners pick split lengths from
the shape (one round of resident units, or a fixed number of units per CU),
so random batches, lengths, head counts and query lengths reach split plans
the fixed workloads do not. Every case is checked against the fp64 oracle on
sampled rows (all rows of the small ones)."""

import numpy as np
import pytest

import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import compare, f64, oracle_decode

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _shape(seed):
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 5, 8]))
    batch = int(rng.integers(1, 97))
    q_len = int(rng.integers(1, 5))
    max_len = int(rng.choice([64, 700, 3000, 9000, 20000]))
    lens = rng.integers(0, max_len + 1, size=batch).tolist()
    lens[int(rng.integers(batch))] = max_len              # one request at the bound
    page = int(rng.choice([16, 64, 128]))
    causal = bool(rng.integers(2))
    return dict(batch=batch, q_len=q_len, hq=hkv * group, hkv=hkv, d=d, dv=d, page_size=page, seq_lens=lens,
                seed=2000 + seed, causal=causal, layout="random"), rng


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_with_and_without_the_total_hint(seed):
    kw, rng = _shape(seed)
    case = inputs.decode_case(**kw)
    c = case.to(DEV)
    b, q_len, hq = kw["batch"], kw["q_len"], kw["hq"]
    n = b * q_len * hq
    rows = None if n <= 4096 else [(int(rng.integers(b)), int(rng.integers(q_len)), int(rng.integers(hq)))
                                   for _ in range(512)]
    ref, lref = oracle_decode(case, rows)
    for total in (0, int(sum(kw["seq_lens"]))):
        p = sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, max_seq_len=c.max_seq_len,
                              softmax_scale=c.scale, causal=c.causal, total_kv_tokens=total)
        plan = sap.decode_plan(p)
        print(f"seed {seed} b{b} q{q_len} hq{hq}/{kw['hkv']} d{kw['d']} page {kw['page_size']} max "
              f"{max(kw['seq_lens'])} total {total}: {plan['num_splits']} x {plan['split_tokens']}, "
              f"{plan['key_ranges']} key ranges", flush=True)
        out, lse = sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, max_seq_len=c.max_seq_len,
                                    softmax_scale=c.scale, causal=c.causal, return_lse=True, total_kv_tokens=total)
        out, lse = out.cpu(), lse.cpu()
        if rows is None:
            print(compare(f64(out), ref, lse.numpy(), lref))
        else:
            got = np.stack([f64(out[i, t, h]) for i, t, h in rows])
            gl = np.array([float(lse[i, t, h]) for i, t, h in rows])
            print(compare(got, ref, gl, lref))


@pytest.mark.parametrize("batch", [512, 513, 700])
def test_batches_at_and_past_the_key_range_limit(batch):
    """Key ranges serve up to 512 requests (the kernels scan seq_lens, eight
    entries per lane); a larger batch is planned as per-request splits, with
    and without the host's total of the keys. Every row against the oracle."""
    rng = np.random.default_rng(3000 + batch)
    lens = rng.integers(0, 700, size=batch).tolist()
    lens[int(rng.integers(batch))] = 700
    case = inputs.decode_case(batch=batch, q_len=1, hq=8, hkv=2, d=64, dv=64, page_size=16, seq_lens=lens,
                              seed=4000 + batch, layout="random")
    c = case.to(DEV)
    ref, lref = oracle_decode(case)
    for total in (0, int(sum(lens))):
        p = sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, max_seq_len=c.max_seq_len,
                              softmax_scale=c.scale, total_kv_tokens=total)
        plan = sap.decode_plan(p)
        print(f"batch {batch} total {total}: {plan['num_splits']} x {plan['split_tokens']}, "
              f"{plan['key_ranges']} key ranges", flush=True)
        assert (plan["key_ranges"] > 0) == (batch <= 512)
        out, lse = sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, max_seq_len=c.max_seq_len,
                                    softmax_scale=c.scale, return_lse=True, total_kv_tokens=total)
        print(compare(f64(out.cpu()), ref, lse.cpu().numpy(), lref))
