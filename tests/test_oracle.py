"""Pins of the fp64 oracle against things other than itself.

Each test is chosen so that a plausible slip in the oracle (a dropped scale,
a transposed operand, a wrong mask offset, a wrong KV-head map, a wrong page
lookup, a wrong LSE base) fails at least one of them:
  * a library routine (torch's scaled_dot_product_attention in float64 on
    the CPU; scipy's logsumexp);
  * pure-Python brute force on tiny inputs;
  * closed forms and special cases (constant V, one-hot V, one key, two keys
    with a known ratio);
  * the pages' own worked examples (tests/golden/);
  * a different algorithm from the pages (the online recurrence) agreeing
    with the two-pass definition.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- formats --

def test_widen_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.widen_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0


def test_widen_e4m3fn_scale_multiplies():
    codes = np.array([0x38, 0xB8, 0x40], dtype=np.uint8)   # 1, -1, 2
    assert np.array_equal(oracle.widen_e4m3fn(codes, 0.25), [0.25, -0.25, 0.5])


def test_widen_bf16_matches_torch():
    bits = _rng(0).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    ours = oracle.widen_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])


# ------------------------------------------------------ library routines --

def _sdpa(q, k, v, scale, causal):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), scale=scale, is_causal=causal)[0, 0].numpy()


@pytest.mark.parametrize("lq,lk,d,dv,scale", [(7, 7, 16, 16, 0.25), (5, 33, 24, 8, 1.7),
                                              (1, 100, 64, 64, 0.125), (9, 9, 40, 56, 0.09)])
def test_rows_match_torch_sdpa_noncausal(lq, lk, d, dv, scale):
    r = _rng(lq * 1000 + lk)
    q, k, v = r.standard_normal((lq, d)), r.standard_normal((lk, d)), r.standard_normal((lk, dv))
    o, _ = oracle.attention_rows(q, k, v, scale)
    assert np.max(np.abs(o - _sdpa(q, k, v, scale, False))) < 1e-12


@pytest.mark.parametrize("n,d,dv,scale", [(1, 8, 8, 1.0), (13, 32, 16, 0.3), (64, 16, 48, 0.7)])
def test_causal_square_matches_torch_sdpa(n, d, dv, scale):
    r = _rng(n)
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    bound = oracle.attention.causal_key_bound(np.arange(n), n, n)
    o, _ = oracle.attention_rows(q, k, v, scale, bound)
    assert np.max(np.abs(o - _sdpa(q, k, v, scale, True))) < 1e-12


def test_lse_is_base2_logsumexp_scipy():
    r = _rng(3)
    q, k, v = r.standard_normal((6, 16)), r.standard_normal((50, 16)), r.standard_normal((50, 4))
    _, lse2 = oracle.attention_rows(q, k, v, 0.4)
    ref = logsumexp(0.4 * (q @ k.T), axis=1) / math.log(2.0)
    assert np.max(np.abs(lse2 - ref)) < 1e-12


# ---------------------------------------------------------- brute force --

def test_tiny_brute_force_pure_python():
    r = _rng(4)
    lq, lk, d, dv, scale = 3, 5, 4, 3, 0.6
    q, k, v = r.standard_normal((lq, d)), r.standard_normal((lk, d)), r.standard_normal((lk, dv))
    o, lse2 = oracle.attention_rows(q, k, v, scale)
    for i in range(lq):
        s = [scale * sum(q[i][x] * k[j][x] for x in range(d)) for j in range(lk)]
        z = sum(math.exp(sj) for sj in s)
        for c in range(dv):
            ref = sum(math.exp(s[j]) / z * v[j][c] for j in range(lk))
            assert abs(o[i][c] - ref) < 1e-12
        assert abs(lse2[i] - math.log2(z)) < 1e-12


# ----------------------------------------------------------- closed forms --

def test_constant_v_returns_constant():
    r = _rng(5)
    q, k = r.standard_normal((8, 32)) * 4, r.standard_normal((70, 32))
    v = np.tile(r.standard_normal((1, 16)), (70, 1))
    o, _ = oracle.attention_rows(q, k, v, 0.2)
    assert np.max(np.abs(o - v[0])) < 1e-13


def test_one_hot_v_gives_probabilities_summing_to_one():
    r = _rng(6)
    lk = 24
    q, k = r.standard_normal((5, 8)), r.standard_normal((lk, 8))
    o, lse2 = oracle.attention_rows(q, k, np.eye(lk), 0.9)
    assert np.max(np.abs(o.sum(axis=1) - 1.0)) < 1e-13
    assert np.all(o > 0)
    s = 0.9 * (q @ k.T)
    # p_j = exp(s_j) / 2**lse2
    assert np.max(np.abs(o - np.exp(s) / np.exp2(lse2)[:, None])) < 1e-13


def test_single_key_returns_its_value_and_score():
    r = _rng(7)
    q, k, v = r.standard_normal((4, 16)), r.standard_normal((1, 16)), r.standard_normal((1, 8))
    o, lse2 = oracle.attention_rows(q, k, v, 0.5)
    assert np.array_equal(o, np.tile(v, (4, 1)))
    assert np.max(np.abs(lse2 - 0.5 * (q @ k[0]) / math.log(2.0))) < 1e-13


def test_two_keys_known_ratio():
    # scores 0 and ln 3 -> weights 1/4 and 3/4; lse2 = log2(1 + 3) = 2
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    v = np.array([[4.0, 0.0], [0.0, 8.0]])
    o, lse2 = oracle.attention_rows(q, k, v, 1.0)
    assert np.allclose(o, [[1.0, 6.0]], atol=1e-14, rtol=0)
    assert abs(lse2[0] - 2.0) < 1e-14


def test_rows_without_keys_are_zero_and_neg_inf():
    r = _rng(8)
    q, k, v = r.standard_normal((3, 4)), r.standard_normal((6, 4)), r.standard_normal((6, 5))
    o, lse2 = oracle.attention_rows(q, k, v, 1.0, key_bound=np.array([0, 3, 0]))
    assert np.all(o[[0, 2]] == 0) and np.all(np.isneginf(lse2[[0, 2]]))
    o1, l1 = oracle.attention_rows(q[1:2], k[:3], v[:3], 1.0)
    assert np.max(np.abs(o[1] - o1[0])) < 1e-13 and abs(lse2[1] - l1[0]) < 1e-13
    o0, l0 = oracle.attention_rows(q, k[:0], v[:0], 1.0)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


# ------------------------------------------------------------ sliding window --
# "TokenSpeed-MLA", kernel capability summary, window_left: row i of a block
# of q_len rows over K keys sees keys from max(0, K - q_len - window_left + i)
# up to its causal bound -- the whole block plus window_left keys of context.

def test_window_zero_leaves_the_diagonal_key_only():
    # causal with no context: each row sees exactly its own key j = K - q_len + i,
    # so o = v_j and lse2 = scale * <q, k_j> / ln 2
    r = _rng(31)
    lq, lk, scale = 4, 19, 0.37
    q, k, v = r.standard_normal((lq, 6)), r.standard_normal((lk, 6)), r.standard_normal((lk, 5))
    i = np.arange(lq)
    bound = oracle.attention.causal_key_bound(i, lq, lk)
    start = oracle.window_key_start(i, lq, lk, 0)
    o, lse2 = oracle.attention_rows(q, k, v, scale, bound, start)
    for row in range(lq):
        j = lk - lq + row
        assert np.max(np.abs(o[row] - v[j])) < 1e-14
        assert abs(lse2[row] - scale * float(q[row] @ k[j]) / math.log(2.0)) < 1e-13


def test_window_visible_keys_are_block_plus_context():
    # one-hot V turns o into the softmax weights: the nonzero columns are the
    # keys each row sees. With causal and window W: W + 1 keys per row, and
    # the block's rows together see its q_len keys plus W keys of context.
    r = _rng(32)
    lq, lk, w = 4, 40, 9
    q, k = r.standard_normal((lq, 8)) * 0.1, r.standard_normal((lk, 8))
    i = np.arange(lq)
    o, _ = oracle.attention_rows(q, k, np.eye(lk), 0.5, oracle.attention.causal_key_bound(i, lq, lk),
                                 oracle.window_key_start(i, lq, lk, w))
    seen = [set(np.nonzero(o[row] > 0)[0].tolist()) for row in range(lq)]
    assert all(len(sv) == w + 1 for sv in seen)
    assert set().union(*seen) == set(range(lk - lq - w, lk))
    assert all(max(sv) == lk - lq + row for row, sv in enumerate(seen))


def test_window_wider_than_history_is_full_history():
    r = _rng(33)
    lq, lk = 3, 12
    q, k, v = r.standard_normal((lq, 4)), r.standard_normal((lk, 4)), r.standard_normal((lk, 4))
    i = np.arange(lq)
    bound = oracle.attention.causal_key_bound(i, lq, lk)
    o_w, l_w = oracle.attention_rows(q, k, v, 0.8, bound, oracle.window_key_start(i, lq, lk, lk + 5))
    o_f, l_f = oracle.attention_rows(q, k, v, 0.8, bound)
    assert np.max(np.abs(o_w - o_f)) < 1e-14 and np.max(np.abs(l_w - l_f)) < 1e-14
    assert np.all(oracle.window_key_start(i, lq, lk, -1) == 0)


def test_window_row_equals_attention_over_its_key_slice():
    # a windowed row is unwindowed attention over the keys it may see
    r = _rng(34)
    lq, lk, w = 5, 30, 7
    q, k, v = r.standard_normal((lq, 6)), r.standard_normal((lk, 6)), r.standard_normal((lk, 3))
    i = np.arange(lq)
    o, lse2 = oracle.attention_rows(q, k, v, 0.4, oracle.attention.causal_key_bound(i, lq, lk),
                                    oracle.window_key_start(i, lq, lk, w))
    for row in range(lq):
        a, b = lk - lq - w + row, lk - lq + row + 1
        o1, l1 = oracle.attention_rows(q[row:row + 1], k[a:b], v[a:b], 0.4)
        assert np.max(np.abs(o[row] - o1[0])) < 1e-13 and abs(lse2[row] - l1[0]) < 1e-13


def test_decode_window_matches_prefill_window_on_the_same_rows():
    # the decode and the dense-prefill entry points apply the same window
    # bound to a q_len block appended after the cache (dense cache, one page each)
    r = _rng(35)
    q_len, lk, d, w = 3, 20, 8, 4
    qd = r.standard_normal((1, q_len, 2, d))
    kc = r.standard_normal((1, 32, 1, d))
    vc = r.standard_normal((1, 32, 1, d))
    od, ld = oracle.decode_paged(qd, kc, vc, np.array([[0]]), np.array([lk]), 32, 0.3, True, d,
                                 window_left=w)
    op, lp = oracle.prefill_dense(qd[0], kc[0, :lk], vc[0, :lk], np.array([0, q_len]), np.array([0, lk]),
                                  0.3, True, window_left=w)
    assert np.max(np.abs(od[0] - op)) < 1e-13 and np.max(np.abs(ld[0] - lp)) < 1e-13


# ------------------------------------------------------------ causal mask --

def test_bottom_right_last_row_sees_everything():
    r = _rng(9)
    lq, lk = 4, 21
    q, k, v = r.standard_normal((lq, 8)), r.standard_normal((lk, 8)), r.standard_normal((lk, 8))
    bound = oracle.attention.causal_key_bound(np.arange(lq), lq, lk)
    assert list(bound) == [18, 19, 20, 21]
    o, _ = oracle.attention_rows(q, k, v, 0.3, bound)
    full, _ = oracle.attention_rows(q[-1:], k, v, 0.3)
    assert np.max(np.abs(o[-1] - full[0])) < 1e-13


def test_chunked_causal_row_equals_decode_of_its_prefix():
    # Row i of a causal chunk (Lq rows appended after Lk - Lq cached keys)
    # is the non-causal attention of that token over its own prefix.
    r = _rng(10)
    lq, lk, d = 6, 15, 8
    q, k, v = r.standard_normal((lq, d)), r.standard_normal((lk, d)), r.standard_normal((lk, d))
    o, lse2 = oracle.prefill_dense(q[:, None], k[:, None], v[:, None], [0, lq], [0, lk], 0.4, True)
    for i in range(lq):
        n = lk - lq + i + 1
        oi, li = oracle.attention_rows(q[i:i + 1], k[:n], v[:n], 0.4)
        assert np.max(np.abs(o[i, 0] - oi[0])) < 1e-13 and abs(lse2[i, 0] - li[0]) < 1e-13


def test_causal_more_queries_than_keys_leaves_empty_rows():
    r = _rng(11)
    lq, lk = 5, 3
    q, k, v = r.standard_normal((lq, 4)), r.standard_normal((lk, 4)), r.standard_normal((lk, 4))
    o, lse2 = oracle.prefill_dense(q[:, None], k[:, None], v[:, None], [0, lq], [0, lk], 1.0, True)
    assert np.all(o[:2] == 0) and np.all(np.isneginf(lse2[:2]))
    assert np.all(np.isfinite(lse2[2:]))


# ------------------------------------------------------- online vs 2-pass --

@pytest.mark.parametrize("seed", range(6))
def test_online_recurrence_equals_two_pass_on_random_partitions(seed):
    r = _rng(100 + seed)
    lk = int(r.integers(1, 60))
    q = r.standard_normal((4, 12)) * 3
    k, v = r.standard_normal((lk, 12)), r.standard_normal((lk, 7))
    cuts = sorted(set(r.integers(1, lk, size=int(r.integers(0, 6))).tolist())) if lk > 1 else []
    edges = [0] + cuts + [lk]
    o_on, l_on = oracle.online_softmax_blocks(q, k, v, 0.35, edges)
    o_tp, l_tp = oracle.attention_rows(q, k, v, 0.35)
    assert np.max(np.abs(o_on - o_tp)) <= 1e-12 * max(1.0, np.max(np.abs(o_tp)))
    assert np.max(np.abs(l_on - l_tp)) < 1e-12


def test_online_recurrence_with_rising_ramp():
    # Each block raises the max, so every block rescales.
    lk = 40
    k = np.arange(lk, dtype=np.float64)[:, None] * 0.7
    q = np.ones((1, 1))
    v = np.random.default_rng(1).standard_normal((lk, 3))
    edges = list(range(0, lk + 1, 5))
    o_on, l_on = oracle.online_softmax_blocks(q, k, v, 1.0, edges)
    o_tp, l_tp = oracle.attention_rows(q, k, v, 1.0)
    assert np.max(np.abs(o_on - o_tp)) < 1e-12 and abs(l_on[0] - l_tp[0]) < 1e-12


# ------------------------------------------------------------------ merge --

@pytest.mark.parametrize("seed", range(5))
def test_merge_of_split_partials_equals_unsplit(seed):
    r = _rng(200 + seed)
    lk = int(r.integers(2, 90))
    q = r.standard_normal((6, 16)) * 2
    k, v = r.standard_normal((lk, 16)), r.standard_normal((lk, 10))
    n_split = int(r.integers(1, 7))
    cuts = np.sort(r.integers(0, lk + 1, size=n_split - 1))
    edges = [0] + cuts.tolist() + [lk]          # empty splits allowed
    o_parts, l_parts = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        o_i, l_i = oracle.attention_rows(q, k[a:b], v[a:b], 0.25)
        o_parts.append(o_i)
        l_parts.append(l_i)
    o, lse2 = oracle.merge_lse(np.stack(o_parts), np.stack(l_parts))
    o_ref, l_ref = oracle.attention_rows(q, k, v, 0.25)
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse2 - l_ref)) < 1e-12


def test_merge_identity_associativity_and_empty():
    r = _rng(300)
    o_parts = r.standard_normal((3, 5, 4))
    l_parts = r.standard_normal((3, 5)) * 10
    o1, l1 = oracle.merge_lse(o_parts[:1], l_parts[:1])
    assert np.array_equal(o1, o_parts[0]) and np.allclose(l1, l_parts[0], atol=1e-14, rtol=0)
    oa, la = oracle.merge_lse(o_parts[:2], l_parts[:2])
    ob, lb = oracle.merge_lse(np.stack([oa, o_parts[2]]), np.stack([la, l_parts[2]]))
    oc, lc = oracle.merge_lse(o_parts, l_parts)
    assert np.max(np.abs(ob - oc)) < 1e-12 and np.max(np.abs(lb - lc)) < 1e-12
    empty = np.full((2, 5), -np.inf)
    oe, le = oracle.merge_lse(r.standard_normal((2, 5, 4)), empty)
    assert np.all(oe == 0) and np.all(np.isneginf(le))


# ------------------------------------------------------------------ paging --

def test_paged_decode_equals_contiguous_and_ignores_unused_pages():
    g = _golden("pypto_seq700_pages.json")
    ps, hkv, head = g["page_size"], g["kv_heads"], g["kv_head"]
    lk, table = g["seq_len"], g["block_table"]
    r = _rng(400)
    d, group = 16, 5
    n_pages = 48
    k_cache = np.full((n_pages, ps, hkv, d), np.nan)
    v_cache = np.full((n_pages, ps, hkv, d), np.nan)
    k_seq, v_seq = r.standard_normal((lk, hkv, d)), r.standard_normal((lk, hkv, d))
    for logical, phys in enumerate(table):
        take = min(ps, lk - logical * ps)
        k_cache[phys, :take] = k_seq[logical * ps:logical * ps + take]
        v_cache[phys, :take] = v_seq[logical * ps:logical * ps + take]
    bt = np.array([table + [-1] * 4])                   # entries past the last page are -1
    q = r.standard_normal((1, 1, hkv * group, d))
    o, lse2 = oracle.decode_paged(q, k_cache, v_cache, bt, np.array([lk]), ps, 0.3, False, d)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse2))
    for h in range(hkv * group):
        ref, lref = oracle.attention_rows(q[0, 0, h][None], k_seq[:, h // group], v_seq[:, h // group], 0.3)
        assert np.max(np.abs(o[0, 0, h] - ref[0])) < 1e-13 and abs(lse2[0, 0, h] - lref[0]) < 1e-13


def test_gqa_head_map_matches_pypto_task_example():
    g = _golden("pypto_task9_mapping.json")
    batch, kv_head, first = oracle.decode_task_mapping(g["task"], g["num_kv_heads"], g["group"])
    assert (batch, kv_head) == (g["expect_batch"], g["expect_kv_head"])
    assert list(range(first, first + g["group"])) == g["expect_q_heads"]
    # The oracle's decode sends exactly those query heads to that KV head:
    # give every KV head a constant, distinct V and read back which one each
    # query head averaged.
    hkv, group, ps = g["num_kv_heads"], g["group"], 16
    v_cache = np.zeros((1, ps, hkv, 4))
    for h in range(hkv):
        v_cache[0, :, h, :] = h
    k_cache = _rng(1).standard_normal((1, ps, hkv, 4))
    q = _rng(2).standard_normal((1, 1, hkv * group, 4))
    o, _ = oracle.decode_paged(q, k_cache, v_cache, np.array([[0]]), np.array([ps]), ps, 1.0, False, 4)
    owner = o[0, 0, :, 0].round().astype(int)
    assert [h for h in range(hkv * group) if owner[h] == kv_head] == g["expect_q_heads"]


def test_paged_prefill_equals_dense_prefill():
    r = _rng(500)
    ps, hq, hkv, d, dv = 8, 4, 2, 16, 16
    q_lens, kv_lens = [3, 5, 1], [11, 5, 20]
    cu_q = np.concatenate([[0], np.cumsum(q_lens)])
    cu_k = np.concatenate([[0], np.cumsum(kv_lens)])
    q = r.standard_normal((cu_q[-1], hq, d))
    k, v = r.standard_normal((cu_k[-1], hkv, d)), r.standard_normal((cu_k[-1], hkv, dv))
    n_pages = sum(-(-n // ps) for n in kv_lens)
    perm = r.permutation(n_pages)
    k_cache = np.full((n_pages, ps, hkv, d), np.nan)
    v_cache = np.full((n_pages, ps, hkv, dv), np.nan)
    bt = np.full((3, 4), -1)
    nxt = 0
    for b, n in enumerate(kv_lens):
        for logical in range(-(-n // ps)):
            phys = perm[nxt]
            nxt += 1
            bt[b, logical] = phys
            take = min(ps, n - logical * ps)
            k_cache[phys, :take] = k[cu_k[b] + logical * ps: cu_k[b] + logical * ps + take]
            v_cache[phys, :take] = v[cu_k[b] + logical * ps: cu_k[b] + logical * ps + take]
    for causal in (False, True):
        od, ld = oracle.prefill_dense(q, k, v, cu_q, cu_k, 0.3, causal)
        op, lp = oracle.prefill_paged(q, k_cache, v_cache, cu_q, np.array(kv_lens), bt, ps, 0.3, causal, dv)
        assert np.max(np.abs(od - op)) < 1e-13
        fin = np.isfinite(ld)
        assert np.array_equal(fin, np.isfinite(lp)) and np.max(np.abs(ld[fin] - lp[fin])) < 1e-13


def test_sampled_rows_equal_full_decode():
    r = _rng(600)
    b, q_len, hq, hkv, d, ps = 3, 2, 6, 2, 8, 4
    lens = np.array([9, 0, 13])
    pool = 12
    k_cache, v_cache = r.standard_normal((pool, ps, hkv, d)), r.standard_normal((pool, ps, hkv, d))
    bt = r.permutation(pool)[:12].reshape(3, 4)
    q = r.standard_normal((b, q_len, hq, d))
    o, lse2 = oracle.decode_paged(q, k_cache, v_cache, bt, lens, ps, 0.5, True, d)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse2[1]))
    rows = [(2, 1, 5), (0, 0, 0), (1, 1, 3)]
    o_s, l_s = oracle.decode_paged_rows(q, k_cache, v_cache, bt, lens, ps, 0.5, True, d, rows)
    for n, (bb, t, h) in enumerate(rows):
        assert np.max(np.abs(o_s[n] - o[bb, t, h])) < 1e-13
        assert l_s[n] == lse2[bb, t, h] or abs(l_s[n] - lse2[bb, t, h]) < 1e-13


# ------------------------------------------------------ host-side formulas --

def test_pypto_page_and_stack_counts():
    g = _golden("pypto_seq700_pages.json")
    pages, stacks, last = oracle.page_stack_counts(g["seq_len"], g["page_size"], g["pages_per_stack"])
    assert pages == g["expect_pages"] and stacks == g["expect_stacks"]
    assert last == g["expect_stack_tokens"][-1]
    assert len(g["block_table"]) == pages


def test_tokenspeed_fold_and_packed_tiles():
    g = _golden("tokenspeed_fold.json")
    for ex in g["fold_examples"]:
        f = oracle.fold_factor(ex["num_heads"], ex["q_len"])
        assert f == ex["expect_F"]
        assert ex["num_heads"] * f == ex["expect_H_eff"] and ex["q_len"] // f == ex["expect_q_eff"]
    for ex in g["packed_tile_examples"]:
        assert oracle.packed_query_tiles(ex["num_heads"], ex["q_len"]) == ex["expect_tiles"]
    assert oracle.fold_factor(96, 4) == 1            # no factor > 1 fits 128 rows
    assert oracle.fold_factor(16, 4) == 4
    assert oracle.mla_packed_workspace_bytes(4, 96, 4, 1) == 0
    assert oracle.mla_packed_workspace_bytes(4, 96, 4, 2) == 4 * 128 * 3 * 2 * 513 * 4


def test_flywheel_static_anchor_tau():
    g = _golden("flywheel_static_anchor.json")
    tau = oracle.static_anchor_tau(g["n_keys"], g["v_max"], g["delta"])
    assert abs(tau - g["expect_tau_nats_about"]) < g["about_tolerance"]
    assert abs(tau - math.log(g["n_keys"]) - g["expect_tau_minus_lnN_about"]) < g["about_tolerance"]
    assert round(tau / math.log(10)) == g["expect_exp_tau_about_pow10"]
    assert oracle.static_anchor_tau(2 ** 40, 2.0 ** 60, 2.0) < g["refuse_below_nats"]


# ------------------------------------------------------------ FP8 prefill --

def _e4m3_codes(r, shape):
    c = r.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, np.uint8(0x38), c)          # no NaN codes


def _torch_values(codes, scale):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_prefill_matches_sdpa_on_torch_decoded_values(causal):
    # the MLA prefill shape (q, k 192 wide, v 128 wide), one square request
    r = _rng(91)
    n, h = 40, 2
    q, k, v = _e4m3_codes(r, (n, h, 192)), _e4m3_codes(r, (n, h, 192)), _e4m3_codes(r, (n, h, 128))
    qs, ks, vs, scale = 0.011, 0.013, 0.7, 0.0721
    cu = np.array([0, n])
    o, _ = oracle.prefill_dense_fp8(q, k, v, qs, ks, vs, cu, cu, scale, causal)
    for hh in range(h):
        ref = _sdpa(_torch_values(q[:, hh], qs), _torch_values(k[:, hh], ks), _torch_values(v[:, hh], vs), scale, causal)
        assert np.max(np.abs(o[:, hh] - ref)) < 1e-10


def test_fp8_prefill_scales_enter_as_the_pages_describe():
    r = _rng(92)
    q, k, v = _e4m3_codes(r, (12, 1, 192)), _e4m3_codes(r, (30, 1, 192)), _e4m3_codes(r, (30, 1, 128))
    cu_q, cu_k = np.array([0, 5, 12]), np.array([0, 14, 30])
    o1, l1 = oracle.prefill_dense_fp8(q, k, v, 0.02, 0.01, 1.0, cu_q, cu_k, 0.07, True)
    o2, l2 = oracle.prefill_dense_fp8(q, k, v, 0.04, 0.01, 1.0, cu_q, cu_k, 0.035, True)   # q_scale x softmax_scale
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
    o3, l3 = oracle.prefill_dense_fp8(q, k, v, 0.02, 0.01, 2.5, cu_q, cu_k, 0.07, True)     # v_scale scales o only
    assert np.allclose(o3, 2.5 * o1, atol=1e-12) and np.array_equal(l3, l1)


def test_fp8_prefill_sampled_rows_equal_full():
    r = _rng(93)
    q, k, v = _e4m3_codes(r, (20, 4, 192)), _e4m3_codes(r, (50, 2, 192)), _e4m3_codes(r, (50, 2, 128))
    cu_q, cu_k = np.array([0, 7, 20]), np.array([0, 21, 50])
    o, l = oracle.prefill_dense_fp8(q, k, v, 0.03, 0.02, 0.5, cu_q, cu_k, 0.09, True, window_left=9)
    rows = [(0, 0), (6, 3), (7, 1), (19, 2), (12, 0)]
    orow, lrow = oracle.prefill_dense_fp8_rows(q, k, v, 0.03, 0.02, 0.5, cu_q, cu_k, 0.09, True, rows, window_left=9)
    for n, (t, hh) in enumerate(rows):
        assert np.allclose(orow[n], o[t, hh], atol=1e-12) and abs(lrow[n] - l[t, hh]) < 1e-12


# ------------------------------------------------- FP8 query, latent decode --

def test_fp8_query_latent_decode_matches_sdpa_on_torch_decoded_values():
    # the FP8 decode path: E4M3 query codes and an E4M3 latent cache (K the
    # 576-wide row, V its first 512), each with its own scale; one query
    # token, non-causal, against torch's own decoding of the codes and SDPA
    r = _rng(94)
    h, ps, lens = 4, 16, [5, 40, 1]
    q = _e4m3_codes(r, (3, 1, h, 576))
    logical = [_e4m3_codes(r, (n, 576)) for n in lens]
    pages = sum(-(-n // ps) for n in lens)
    perm = r.permutation(pages)
    cache = np.zeros((pages, ps, 1, 576), dtype=np.uint8)
    bt = np.full((3, 3), -1, dtype=np.int64)
    used = 0
    for b, n in enumerate(lens):
        for j in range(-(-n // ps)):
            bt[b, j] = perm[used]
            rows = logical[b][j * ps:(j + 1) * ps]
            cache[perm[used], :len(rows), 0] = rows
            used += 1
    qs, kvs, scale = 0.021, 0.017, 0.0417
    o, lse2 = oracle.decode_paged(q, cache, cache, bt, np.array(lens), ps, scale, False, 512, "e4m3fn", kvs,
                                  "e4m3fn", q_scale=qs)
    for b, n in enumerate(lens):
        kv = _torch_values(logical[b], kvs)
        for hh in range(h):
            qv = _torch_values(q[b, 0, hh][None], qs)
            ref = _sdpa(qv, kv, kv[:, :512], scale, False)[0]
            assert np.max(np.abs(o[b, 0, hh] - ref)) < 1e-10
            want = logsumexp(scale * (qv @ kv.T)[0]) / math.log(2.0)
            assert abs(lse2[b, 0, hh] - want) < 1e-10


def test_fp8_query_scale_enters_as_a_product_with_the_softmax_scale():
    r = _rng(95)
    q = _e4m3_codes(r, (1, 2, 2, 576))
    cache = _e4m3_codes(r, (2, 16, 1, 576))
    bt, lens = np.array([[1, 0]]), np.array([20])
    a = oracle.decode_paged(q, cache, cache, bt, lens, 16, 0.05, True, 512, "e4m3fn", 0.01, "e4m3fn", q_scale=0.03)
    b = oracle.decode_paged(q, cache, cache, bt, lens, 16, 0.1, True, 512, "e4m3fn", 0.01, "e4m3fn", q_scale=0.015)
    assert np.allclose(a[0], b[0], atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)
