"""GPU parity of the MLA-shaped latent decode (576-wide K, V = first 512 columns,
bf16 or fp8 e4m3 KV with a per-tensor scale) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_paged_amd as sap
from softmax_attention_paged_amd import inputs
from helpers import TOL_BF16, TOL_FP8, compare, f64, oracle_decode

pytestmark = pytest.mark.gpu

DEV = "cuda"


# KV dtype, with "+q" for the FP8 path whose query is FP8 too
DTYPES = ["bf16", "fp8_e4m3", "fp8_e4m3+q"]


def _dt(name):
    return dict(kv_dtype=name.split("+")[0], q_dtype="fp8_e4m3" if name.endswith("+q") else "bf16")


def _qvalues(case):
    """The query's values as float64 (bf16 bits, or E4M3 codes times q_scale)."""
    if case.q_dtype == "bf16":
        return f64(case.q)
    return oracle.widen_e4m3fn(case.q.numpy(), case.q_scale)


def _run(case, num_splits=0):
    c = case.to(DEV)
    out, lse = sap.decode_paged(c.q, c.k_cache, None, c.block_table, c.seq_lens, max_seq_len=c.max_seq_len,
                                softmax_scale=c.scale, causal=c.causal, head_dim_v=512,
                                kv_dtype=None if c.kv_dtype == "bf16" else c.kv_dtype,
                                k_scale=c.kv_scale, v_scale=c.kv_scale, num_splits=num_splits, return_lse=True,
                                window_left=c.window_left, packed_q=c.packed_q,
                                q_scale=None if c.q_dtype == "bf16" else c.q_scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(case, num_splits=0):
    out, lse = _run(case, num_splits)
    ref, lref = oracle_decode(case)
    return compare(f64(out), ref, lse.numpy(), lref, TOL_BF16 if case.kv_dtype == "bf16" else TOL_FP8)


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("hq,q_len", [(64, 4), (16, 4), (128, 1), (8, 3), (32, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_latent_decode_small(kv_dtype, hq, q_len, causal):
    case = inputs.decode_case(batch=3, q_len=q_len, hq=hq, hkv=1, d=576, dv=512, page_size=16,
                              seq_lens=[3, 37, 300], seed=hq + q_len, latent=True,
                              scale=0.07216882, causal=causal, layout="noncontiguous", **_dt(kv_dtype))
    print(kv_dtype, hq, q_len, causal, flush=True)
    for splits in (0, 1, 3):
        print(_check(case, splits))


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_latent_layouts_bitwise(kv_dtype):
    outs = []
    for layout in ("identity", "random", "reverse"):
        case = inputs.decode_case(batch=2, q_len=4, hq=64, hkv=1, d=576, dv=512, page_size=64,
                                  seq_lens=[1000, 129], seed=61, latent=True,
                                  scale=0.07216882, causal=True, layout=layout, **_dt(kv_dtype))
        outs.append(_run(case, num_splits=2))
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16)) and torch.equal(l, outs[0][1])


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("causal", [True, False])
def test_mla_decode_80k_every_row(kv_dtype, causal):
    """The MLA-shaped workload at full size (batch 8, 4 tokens, 64 heads,
    kv_len 81920), planned as the benchmark plans it: every one of its 2,048
    (request, token, head) rows against the oracle."""
    case = inputs.mla_decode(causal=causal, **_dt(kv_dtype))
    print("case", case.name, flush=True)
    out, lse = _run(case)
    ref, lref = oracle_decode(case)
    res = compare(f64(out), ref, lse.numpy(), lref, TOL_BF16 if case.kv_dtype == "bf16" else TOL_FP8)
    res["rows_checked"] = int(np.prod(lref.shape))
    print(res)


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("splits", [0, 3])
def test_static_anchor_restart(kv_dtype, splits):
    """One latent row gives the row (token 0, head 0) a score of about 150-175
    log2 units, about 145 above its first tile's max: without a restart its
    exponential would overflow FP32. The running-sum check fails, the split
    restarts with a raised anchor, and the result matches the oracle. bf16:
    the large values sit in the 64 rope columns (K only, so V and the output
    keep their usual size); fp8: the whole row is 3 x the query, clamped to
    the e4m3 range."""
    case = inputs.decode_case(batch=2, q_len=4, hq=64, hkv=1, d=576, dv=512, page_size=64,
                              seq_lens=[700, 300], seed=71, latent=True,
                              scale=0.07216882, causal=True, layout="random", **_dt(kv_dtype))
    j = 500                                            # logical key of request 0
    page = int(case.block_table[0, j // 64])
    q00 = torch.from_numpy(_qvalues(case)[0, 0, 0]).float()
    if case.kv_dtype == "bf16":
        case.k_cache[page, j % 64, 0, 512:] = (28.0 * q00[512:]).to(torch.bfloat16)
    else:
        codes = (3.0 * q00 / case.kv_scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        case.k_cache[page, j % 64, 0] = codes
    res = _check(case, splits)
    print(res)


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("splits", [1, 3])
def test_window_anchor_ignores_hidden_keys(kv_dtype, splits):
    """A sliding window whose start lies 30 keys into the first walked tile:
    those 30 keys are hidden from every row, and rows of tokens 2 and 3 see
    no key of that tile at all. The hidden keys are planted to score at
    least 150 log2 units above every key a row may see; the static anchor
    must come from the row's own visible scores ("Flywheel Attention",
    Appendix A: the anchor is one of the row's scores, so its sum is at
    least 1), else every visible exponential underflows and the row comes
    back empty. Queries are made positive where the planted keys are large
    (rope columns for bf16, every column for fp8, whose planted codes are
    the largest E4M3 value)."""
    lens, q_len, window = [700, 444], 4, 346      # 700 - 4 - 346 = 350 = 320 + 30; 444 - 4 - 346 = 94 = 64 + 30
    case = inputs.decode_case(batch=2, q_len=q_len, hq=64, hkv=1, d=576, dv=512, page_size=64,
                              seq_lens=lens, seed=83, latent=True,
                              scale=0.07216882, causal=True, layout="random", window_left=window, **_dt(kv_dtype))
    kv_dtype = case.kv_dtype
    cols = slice(512, 576) if kv_dtype == "bf16" else slice(0, 576)
    if case.q_dtype == "bf16":
        case.q[..., cols] = case.q[..., cols].abs()
    else:
        case.q[..., cols] = case.q[..., cols] & 0x7F        # E4M3 codes: clear the sign bit
    for b, lk in enumerate(lens):
        start = lk - q_len - window                  # first key row 0 sees
        base = start & ~31                           # first key of the walk
        assert start - base == 30
        for j in range(base, start):                 # hidden from every row
            page = int(case.block_table[b, j // 64])
            if kv_dtype == "bf16":
                case.k_cache[page, j % 64, 0, 512:] = 48.0
            else:
                case.k_cache[page, j % 64, 0] = 0x7E     # E4M3 448
    # precondition: every hidden score exceeds every visible one by >= 150 log2 units
    kc = f64(case.k_cache) if kv_dtype == "bf16" else oracle.widen_e4m3fn(case.k_cache.numpy(), case.kv_scale)
    qf = _qvalues(case)
    for b, lk in enumerate(lens):
        start = lk - q_len - window
        keys = np.stack([kc[int(case.block_table[b, j // 64]), j % 64, 0] for j in range(start & ~31, lk)])
        s2 = qf[b].reshape(-1, 576) @ keys.T * case.scale / np.log(2.0)
        hidden = s2[:, : start - (start & ~31)].min()
        visible = s2[:, start - (start & ~31):].max()
        assert hidden - visible >= 150.0, (hidden, visible)
    print("window anchor", kv_dtype, splits, flush=True)
    print(_check(case, splits))


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("splits", [1, 3])
def test_static_anchor_second_restart(kv_dtype, splits):
    """Two planted keys for the row (token 0, head 0), the second scoring far
    above the first: the first check fails at key 200 (anchor raised to its
    score), the restarted walk fails again at key 240, and the pass that sets
    every anchor to its row's max runs before the last walk. Both keys lie
    in the first split when there are three."""
    case = inputs.decode_case(batch=2, q_len=4, hq=64, hkv=1, d=576, dv=512, page_size=64,
                              seq_lens=[700, 300], seed=72, latent=True,
                              scale=0.07216882, causal=True, layout="random", **_dt(kv_dtype))
    q00 = torch.from_numpy(_qvalues(case)[0, 0, 0]).float()
    for j, mult in ((200, 1.0), (240, 2.0)):
        page = int(case.block_table[0, j // 64])
        if case.kv_dtype == "bf16":
            case.k_cache[page, j % 64, 0, 512:] = (28.0 * mult * q00[512:]).to(torch.bfloat16)
        else:
            codes = (1.5 * mult * q00 / case.kv_scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            case.k_cache[page, j % 64, 0] = codes.view(torch.uint8)
    print("second restart", kv_dtype, splits, flush=True)
    print(_check(case, splits))


def _random_mla_shape(seed):
    rng = np.random.default_rng(3000 + seed)
    batch = int(rng.integers(1, 9))
    q_len = int(rng.integers(1, 5))
    hq = int(rng.choice([8, 16, 32, 64, 128]))
    max_len = int(rng.choice([40, 700, 3000, 12000]))
    lens = rng.integers(0, max_len + 1, size=batch).tolist()
    lens[int(rng.integers(batch))] = max_len              # one request at the bound
    return dict(batch=batch, q_len=q_len, hq=hq, hkv=1, d=576, dv=512, page_size=int(rng.choice([16, 64, 128])),
                seq_lens=lens, seed=4000 + seed, latent=True, scale=0.07216882, causal=bool(rng.integers(2)),
                layout="random", **_dt(DTYPES[seed % len(DTYPES)]))


@pytest.mark.parametrize("seed", range(12))
def test_random_latent_decode(seed):
    """Seeded random batches, lengths, query tokens, head counts (folded
    tokens F = 1, 2 or 4 per 128-row unit), page sizes and causality, in all
    three dtypes, planned and with forced splits, every row against the
    oracle."""
    kw = _random_mla_shape(seed)
    case = inputs.decode_case(**kw)
    print(f"seed {seed}: b{kw['batch']} q{kw['q_len']} hq{kw['hq']} page {kw['page_size']} max "
          f"{max(kw['seq_lens'])} causal {kw['causal']} {kw['kv_dtype']}/{kw['q_dtype']}", flush=True)
    for splits in (0, 2):
        print(_check(case, splits))
