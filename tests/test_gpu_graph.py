"""HIP-graph capture of the entry points ("TokenSpeed-MLA": the decode and
its LSE reducer are meant to run under CUDA-graph replay; the library neither
allocates nor synchronises, so a call with caller-owned outputs and
workspace captures as plain kernel launches).

Each test captures one call, then replays the graph several times with new
input values copied into the captured buffers between replays (eager work
and a synchronisation in between), and checks every replay bit for bit
against an eager call on the same inputs, and the first one against the
fp64 oracle.
"""

import numpy as np
import pytest
import torch

import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import bits, compare, f64, oracle_decode, oracle_prefill

pytestmark = pytest.mark.gpu

DEV = "cuda"
REPLAYS = 4


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                      # warm the launch path outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("num_splits", [3, 0])
def test_decode_graph_replays_match_eager(num_splits):
    # 3: per-request splits and the merge kernel; 0: key ranges, merged in
    # the split kernel through arrival counters that every replay (same
    # captured epoch) must find reset by the previous one
    case = inputs.decode_case(batch=6, q_len=2, hq=8, hkv=2, d=128, dv=128, page_size=16,
                              seq_lens=[1, 40, 300, 511, 777, 64], seed=901, causal=True)
    c = case.to(DEV)
    kw = dict(max_seq_len=c.max_seq_len, softmax_scale=c.scale, causal=True, num_splits=num_splits)
    plan = sap.decode_plan(sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, **kw))
    assert (plan["key_ranges"] > 1) == (num_splits == 0)
    ws = torch.empty(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((6, 2, 8, 128), dtype=torch.bfloat16, device=DEV)
    q = c.q.clone()
    graph = _capture(lambda: sap.decode_paged(q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, workspace=ws,
                                              out=out, **kw))
    gen = torch.Generator().manual_seed(5)
    for i in range(REPLAYS):
        if i:
            q.copy_(torch.randn(q.shape, generator=gen).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = sap.decode_paged(q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(eager)), f"replay {i} differs from the eager call"
        if i == 0:
            ref, _ = oracle_decode(case)
            print(compare(f64(got), ref))


def test_split_prefill_graph_replays_match_eager():
    case = inputs.prefill_case(q_lens=[40, 100], kv_lens=[3000, 2200], hq=8, hkv=2, d=128, seed=902, paged=True,
                               page_size=64, name="graph")
    c = case.to(DEV)
    kw = dict(max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, causal=True, kv_splits=3,
              seq_lens_kv=c.seq_lens_kv, block_table=c.block_table)
    need = sap.prefill_workspace_size(c.q, c.k, c.v, c.cu_seqlens_q, **kw)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(c.q)
    q = c.q.clone()
    graph = _capture(lambda: sap.prefill(q, c.k, c.v, c.cu_seqlens_q, softmax_scale=c.scale, out=out, workspace=ws,
                                         **kw))
    gen = torch.Generator().manual_seed(6)
    for i in range(REPLAYS):
        if i:
            q.copy_(torch.randn(q.shape, generator=gen).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = sap.prefill(q, c.k, c.v, c.cu_seqlens_q, softmax_scale=c.scale, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(eager)), f"replay {i} differs from the eager call"
        if i == 0:
            ref, _ = oracle_prefill(case)
            print(compare(f64(got), ref))


def test_concurrent_calls_on_two_streams_with_their_own_workspaces():
    """The library keeps no state between calls: two key-range decodes with
    split partials, each on its own stream and workspace and running at the
    same time, give the same bits as each run alone."""
    cases = [inputs.decode_case(batch=24, q_len=1, hq=16, hkv=4, d=128, dv=128, page_size=64,
                                seq_len_range=(100, 6000), seed=s, layout="random") for s in (41, 42)]
    devs = [c.to("cuda") for c in cases]

    def call(c, ws, out, lse):
        tokens = int(c.seq_lens.sum())
        sap.decode_paged(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens, max_seq_len=c.max_seq_len,
                         softmax_scale=c.scale, workspace=ws, out=out, lse=lse, total_kv_tokens=tokens)

    bufs = []
    for c in devs:
        plan = sap.decode_plan(sap.decode_params(c.q, c.k_cache, c.v_cache, c.block_table, c.seq_lens,
                                                 max_seq_len=c.max_seq_len, softmax_scale=c.scale,
                                                 total_kv_tokens=int(c.seq_lens.sum())))
        assert plan["key_ranges"] > 1 and plan["workspace_bytes"] > 0
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
        out = torch.empty((c.q.shape[0], 1, 16, 128), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((c.q.shape[0], 1, 16), dtype=torch.float32, device="cuda")
        bufs.append((ws, out, lse))
    alone = []
    for c, (ws, out, lse) in zip(devs, bufs):
        call(c, ws, out, lse)
        torch.cuda.synchronize()
        alone.append((out.clone(), lse.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(5):
        for c, (ws, out, lse), st in zip(devs, bufs, streams):
            with torch.cuda.stream(st):
                call(c, ws, out, lse)
        torch.cuda.synchronize()
        for (out, lse), (o0, l0) in zip([(b[1], b[2]) for b in bufs], alone):
            assert torch.equal(out.view(torch.int16), o0.view(torch.int16)) and torch.equal(lse, l0)
    for c, case, (o0, l0) in zip(devs, cases, alone):
        ref, lref = oracle_decode(case)
        print(compare(f64(o0.cpu()), ref, l0.cpu().numpy(), lref))
