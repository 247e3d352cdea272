"""GPU parity of the FP8 (E4M3) MLA-shaped prefill (q, k 192 wide, v 128
wide, per-tensor scales, bf16 output) against the fp64 oracle on the same
codes ("TokenSpeed-MLA": the FP8 prefill command and the kernel capability
summary).

Tolerance: the scores of E4M3 codes are exact products summed in FP32 and P
is rounded to bf16 before P.V, as in the bf16 prefill, so the bf16 bar
applies (max 2e-2, mean 2e-3, LSE 1e-3).
"""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import TOL_BF16, bits, compare, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(case):
    c = case.to(DEV)
    f8 = lambda t: t.view(torch.float8_e4m3fn)
    out, lse = sap.prefill(f8(c.q), f8(c.k), f8(c.v), c.cu_seqlens_q, cu_seqlens_kv=c.cu_seqlens_kv,
                           max_seqlen_q=c.max_seqlen_q, max_seqlen_kv=c.max_seqlen_kv, softmax_scale=c.scale,
                           causal=c.causal, return_lse=True, window_left=c.window_left,
                           q_scale=c.q_scale, k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(case):
    out, lse = _run(case)
    ref, lref = oracle.prefill_dense_fp8(bits(case.q), bits(case.k), bits(case.v), case.q_scale, case.k_scale,
                                         case.v_scale, case.cu_seqlens_q.numpy(), case.cu_seqlens_kv.numpy(),
                                         case.scale, case.causal, case.window_left)
    return compare(f64(out), ref, lse.numpy(), lref, TOL_BF16)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 2), (3, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged(hq, hkv, causal):
    # a prefill from empty, a chunk over a longer history, a one-token request,
    # an empty request, and tails that are not tile multiples
    case = inputs.fp8_prefill_case(q_lens=[300, 97, 1, 0, 160], kv_lens=[300, 433, 70, 5, 555], hq=hq, hkv=hkv,
                                   seed=hq * 10 + hkv + causal, causal=causal)
    print("fp8 ragged", hq, hkv, causal, _check(case), flush=True)


@pytest.mark.parametrize("window", [0, 63, 130, 5000])
def test_window(window):
    case = inputs.fp8_prefill_case(q_lens=[300, 97, 160], kv_lens=[300, 433, 555], hq=4, hkv=4, seed=200 + window,
                                   window_left=window)
    print("fp8 window", window, _check(case), flush=True)


def test_more_queries_than_keys_and_negative_scale():
    case = inputs.fp8_prefill_case(q_lens=[70, 40], kv_lens=[20, 40], hq=2, hkv=2, seed=7, scale=-0.09)
    _check(case)


def test_peaky_scores_force_rescales():
    case = inputs.fp8_prefill_case(q_lens=[200], kv_lens=[700], hq=2, hkv=2, seed=8, q_mult=8.0)
    _check(case)


def test_fp8_mla_prefill_8k_sampled():
    # the full workload (8K x 8K causal, 128 heads) at sampled rows: the first
    # and last rows, tile boundaries, and random rows of several heads
    case = inputs.fp8_mla_prefill()
    out, lse = _run(case)
    r = np.random.Generator(np.random.PCG64(11))
    toks = [0, 1, 63, 64, 127, 128, 4095, 8191] + r.integers(0, 8192, 24).tolist()
    rows = [(int(t), int(hh)) for t in toks for hh in (0, 77, 127)]
    ref, lref = oracle.prefill_dense_fp8_rows(bits(case.q), bits(case.k), bits(case.v), case.q_scale, case.k_scale,
                                              case.v_scale, case.cu_seqlens_q.numpy(), case.cu_seqlens_kv.numpy(),
                                              case.scale, True, rows)
    got = np.stack([f64(out[t, hh]) for t, hh in rows])
    glse = np.array([float(lse[t, hh]) for t, hh in rows])
    print(compare(got, ref, glse, lref, TOL_BF16))


@pytest.mark.parametrize("seed", range(10))
def test_random_fp8_prefill(seed):
    """Seeded random ragged batches: request count, query and key lengths
    (chunks over histories, empty and one-token requests), head groups,
    causality and windows, every row against the oracle."""
    rng = np.random.default_rng(5000 + seed)
    batch = int(rng.integers(1, 7))
    q_lens = [int(x) for x in rng.integers(0, 700, size=batch)]
    kv_lens = [q + int(rng.integers(0, 900)) for q in q_lens]
    q_lens[int(rng.integers(batch))] = int(rng.choice([0, 1]))
    hq, hkv = [(4, 4), (8, 2), (16, 16), (6, 3)][int(rng.integers(4))]
    causal = bool(rng.integers(2))
    window = int(rng.choice([-1, -1, 0, 100, 700]))
    case = inputs.fp8_prefill_case(q_lens=q_lens, kv_lens=kv_lens, hq=hq, hkv=hkv, seed=6000 + seed, causal=causal,
                                   window_left=window)
    print(f"seed {seed}: q {q_lens} kv {kv_lens} h {hq}/{hkv} causal {causal} window {window}", _check(case),
          flush=True)
