"""Pins for the fp64 oracle: closed forms, the pages' printed examples,
invariants, a library special case and brute force on tiny inputs.

Each test checks the oracle against something other than itself, chosen so
that a plausible slip (a dropped term, a wrong sign, a transposed operand, an
off-by-one causal boundary, a wrong GQA head map) fails at least one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import cascade_ref as ref


def _paged_single(keys, values, page_size, perm_seed=0, extra_pages=3):
    """Scatter one request's [L, Hkv, d] K/V into a shuffled paged cache."""
    L, hkv, d = keys.shape
    n_pages = -(-L // page_size)
    total = n_pages + extra_pages
    rng = np.random.default_rng(perm_seed)
    ids = rng.permutation(total)[:n_pages]
    kc = np.full((total, page_size, hkv, d), np.nan)
    vc = np.full((total, page_size, hkv, d), np.nan)
    for t in range(L):
        kc[ids[t // page_size], t % page_size] = keys[t]
        vc[ids[t // page_size], t % page_size] = values[t]
    bt = np.concatenate([ids, rng.integers(0, total, 2)])[None, :]
    return kc, vc, bt


# ----------------------------------------------------------------- closed forms

def test_hand_softmax():
    # d=1, scale=1, q=1, k=(0, ln2, ln3): weights 1/6, 2/6, 3/6.
    # v=(6, 12, 18) -> o = (6 + 24 + 54) / 6 = 14, lse = ln(1 + 2 + 3) = ln 6.
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(2.0)], [math.log(3.0)]])
    v = np.array([[6.0], [12.0], [18.0]])
    o, lse = oracle.attend(q, k, v, 1.0)
    assert abs(o[0, 0] - 14.0) < 1e-12
    assert abs(lse[0] - math.log(6.0)) < 1e-12


def test_hand_softmax_through_paged_path():
    # Same numbers through block tables, shuffled pages and the causal rule:
    # one request, seq_len 3, one query at position 2 sees all three keys.
    keys = np.array([[0.0], [math.log(2.0)], [math.log(3.0)]])[:, None, :]
    vals = np.array([[6.0], [12.0], [18.0]])[:, None, :]
    kc, vc, bt = _paged_single(keys, vals, page_size=2)
    q = np.ones((1, 1, 1))
    out, lse = oracle.attention_full(q, kc, vc, bt, [0, 1], [3], 2, scale=1.0)
    assert abs(out[0, 0, 0] - 14.0) < 1e-12
    assert abs(lse[0, 0] - math.log(6.0)) < 1e-12


def test_causal_boundary():
    # num_computed = 0, three queries: query i sees keys 0..i only.
    rng = np.random.default_rng(1)
    L, d = 3, 4
    keys = rng.standard_normal((L, 1, d))
    vals = rng.standard_normal((L, 1, d))
    q = rng.standard_normal((L, 1, d))
    kc, vc, bt = _paged_single(keys, vals, page_size=2)
    scale = 0.7
    out, lse = oracle.attention_full(q, kc, vc, bt, [0, L], [L], 2, scale=scale)
    # query 0: exactly one visible key
    assert np.allclose(out[0, 0], vals[0, 0], atol=1e-14, rtol=0)
    assert abs(lse[0, 0] - scale * float(q[0, 0] @ keys[0, 0])) < 1e-13
    # query 1: two keys, written out by hand
    s = np.array([scale * q[1, 0] @ keys[t, 0] for t in range(2)])
    w = np.exp(s - s.max())
    exp_o = (w[0] * vals[0, 0] + w[1] * vals[1, 0]) / w.sum()
    assert np.allclose(out[1, 0], exp_o, atol=1e-13, rtol=0)
    assert abs(lse[1, 0] - (s.max() + math.log(w.sum()))) < 1e-13


def test_constant_values_give_that_value():
    rng = np.random.default_rng(2)
    L, hkv, d = 37, 2, 8
    keys = rng.standard_normal((L, hkv, d)) * 3
    vals = np.broadcast_to(rng.standard_normal((1, hkv, d)), (L, hkv, d)).copy()
    kc, vc, bt = _paged_single(keys, vals, page_size=16)
    q = rng.standard_normal((5, 4, d))
    out, _ = oracle.attention_full(q, kc, vc, bt, [0, 5], [L], 16)
    for h in range(4):
        assert np.allclose(out[:, h], vals[0, h // 2][None, :], atol=1e-13, rtol=0)


def test_zero_query_is_mean_of_visible_values():
    rng = np.random.default_rng(3)
    L, d = 21, 8
    keys = rng.standard_normal((L, 1, d))
    vals = rng.standard_normal((L, 1, d))
    kc, vc, bt = _paged_single(keys, vals, page_size=4)
    qn = 4
    q = np.zeros((qn, 1, d))
    out, lse = oracle.attention_full(q, kc, vc, bt, [0, qn], [L], 4)
    for i in range(qn):
        pos = L - qn + i
        assert np.allclose(out[i, 0], vals[:pos + 1, 0].mean(axis=0), atol=1e-13, rtol=0)
        assert abs(lse[i, 0] - math.log(pos + 1)) < 1e-13


def test_gqa_head_mapping():
    # Hq=4, Hkv=2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1.
    # KV head 0 has constant V = +1, KV head 1 has constant V = -1.
    rng = np.random.default_rng(4)
    L, d = 9, 4
    keys = rng.standard_normal((L, 2, d))
    vals = np.zeros((L, 2, d))
    vals[:, 0] = 1.0
    vals[:, 1] = -1.0
    kc, vc, bt = _paged_single(keys, vals, page_size=4)
    q = rng.standard_normal((1, 4, d))
    out, _ = oracle.attention_full(q, kc, vc, bt, [0, 1], [L], 4)
    assert np.allclose(out[0, 0:2], 1.0) and np.allclose(out[0, 2:4], -1.0)


# ------------------------------------------------------------ library routine

def _dense_kv(batch, r):
    """Independent gather of a request's dense K/V [L, Hkv, d] (page loop)."""
    ps = batch.workload.page_size
    L = int(batch.seq_lens[r])
    k = torch.empty(L, batch.k_cache.shape[2], batch.k_cache.shape[3], dtype=torch.float64)
    v = torch.empty_like(k)
    for p in range(-(-L // ps)):
        page = int(batch.block_table[r, p])
        n = min(ps, L - p * ps)
        k[p * ps:p * ps + n] = batch.k_cache[page, :n].to(torch.float64)
        v[p * ps:p * ps + n] = batch.v_cache[page, :n].to(torch.float64)
    return k, v


def _small_batch(seed=7, n=5, prefix=40, suffix=(3, 30), q=(1, 6), hq=4, hkv=2, d=16, ps=8):
    w = workloads.Workload("small", n, prefix, suffix, q, hq, hkv, d, page_size=ps, seed=seed)
    return workloads.make_batch(w)


@pytest.mark.parametrize("seed", [7, 8])
def test_matches_torch_sdpa_fp64(seed):
    b = _small_batch(seed)
    w = b.workload
    G = w.num_q_heads // w.num_kv_heads
    out, lse = oracle.attention_full(
        b.q.float().numpy(), b.k_cache.float().numpy(), b.v_cache.float().numpy(),
        b.block_table.numpy(), b.query_start_loc.numpy(), b.seq_lens.numpy(), w.page_size)
    for r in range(w.num_reqs):
        q0, q1 = int(b.query_start_loc[r]), int(b.query_start_loc[r + 1])
        k, v = _dense_kv(b, r)
        L = k.shape[0]
        qq = b.q[q0:q1].to(torch.float64).transpose(0, 1)          # [Hq, q, d]
        kk = k.repeat_interleave(G, dim=1).transpose(0, 1)          # [Hq, L, d]
        vv = v.repeat_interleave(G, dim=1).transpose(0, 1)
        ql = q1 - q0
        mask = torch.ones(ql, L, dtype=torch.bool).tril(diagonal=L - ql)
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=mask, scale=w.softmax_scale)
        s = (qq @ kk.transpose(1, 2)) * w.softmax_scale
        l = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
        assert np.abs(out[q0:q1] - o.transpose(0, 1).numpy()).max() < 1e-12
        assert np.abs(lse[q0:q1] - l.transpose(0, 1).numpy()).max() < 1e-12


# ------------------------------------------------------------------- merging

@pytest.mark.parametrize("parts", [2, 3, 5])
def test_merge_of_partition_equals_union(parts):
    rng = np.random.default_rng(10 + parts)
    m, n, d = 6, 50, 8
    q = rng.standard_normal((m, d)) * 2
    k = rng.standard_normal((n, d)) * 2
    v = rng.standard_normal((n, d))
    o_all, l_all = oracle.attend(q, k, v, 0.5)
    label = rng.integers(0, parts, n)
    label[:parts] = np.arange(parts)                       # no part empty
    outs, lses = [], []
    for p in range(parts):
        sel = label == p
        o_p, l_p = oracle.attend(q, k[sel], v[sel], 0.5)
        outs.append(o_p)
        lses.append(l_p)
    o_m, l_m = oracle.merge_states(outs, lses)
    assert np.abs(o_m - o_all).max() < 1e-12
    assert np.abs(l_m - l_all).max() < 1e-12


def test_merge_with_empty_partial_and_all_empty():
    rng = np.random.default_rng(20)
    q = rng.standard_normal((3, 4))
    k = rng.standard_normal((7, 4))
    v = rng.standard_normal((7, 4))
    o_all, l_all = oracle.attend(q, k, v, 1.0)
    o_e, l_e = oracle.attend(q, k[:0], v[:0], 1.0)
    assert np.all(np.isneginf(l_e)) and np.all(o_e == 0)
    o_m, l_m = oracle.merge_states([o_e, o_all], [l_e, l_all])
    assert np.abs(o_m - o_all).max() < 1e-14 and np.abs(l_m - l_all).max() < 1e-14
    o_z, l_z = oracle.merge_states([o_e, o_e], [l_e, l_e])
    assert np.all(o_z == 0) and np.all(np.isneginf(l_z))


def test_cascade_split_equals_full_attention():
    """The decomposition the pages describe, done with the oracle's own
    pieces: non-causal attention of every query over the capped shared
    prefix, causal attention over each request's suffix, LSE merge. Checked
    against full attention (a different computation of the same values)."""
    b = _small_batch(seed=11, n=6, prefix=48, suffix=(5, 25), q=(1, 5), ps=8)
    w = b.workload
    G = w.num_q_heads // w.num_kv_heads
    kc, vc = b.k_cache.float().numpy(), b.v_cache.float().numpy()
    bt, qsl, sl = b.block_table.numpy(), b.query_start_loc.numpy(), b.seq_lens.numpy()
    full_o, full_l = oracle.attention_full(b.q.float().numpy(), kc, vc, bt, qsl, sl, w.page_size)
    blocks = oracle.common_prefix_blocks(bt, sl, w.page_size)
    pc = oracle.cascade_prefix_len(blocks, w.page_size, b.num_computed.numpy())
    assert pc == 48
    for r in range(w.num_reqs):
        q0, q1 = int(qsl[r]), int(qsl[r + 1])
        k, v = _dense_kv(b, r)
        nc = int(b.num_computed[r])
        for h in range(w.num_q_heads):
            g = h // G
            rows = b.q[q0:q1, h].double().numpy()
            o_p, l_p = oracle.attend(rows, k[:pc, g].numpy(), v[:pc, g].numpy(), w.softmax_scale)
            t = np.arange(pc, k.shape[0])
            vis = t[None, :] <= (nc + np.arange(q1 - q0))[:, None]
            o_s, l_s = oracle.attend(rows, k[pc:, g].numpy(), v[pc:, g].numpy(), w.softmax_scale, vis)
            o_m, l_m = oracle.merge_states([o_p, o_s], [l_p, l_s])
            assert np.abs(o_m - full_o[q0:q1, h]).max() < 1e-12
            assert np.abs(l_m - full_l[q0:q1, h]).max() < 1e-12


# ---------------------------------------------------------------- invariances

def _run(b, requests=None):
    return oracle.attention_full(
        b.q.float().numpy(), b.k_cache.float().numpy(), b.v_cache.float().numpy(),
        b.block_table.numpy(), b.query_start_loc.numpy(), b.seq_lens.numpy(),
        b.workload.page_size, requests=requests)


def _reorder(b, order):
    qsl = b.query_start_loc
    qs = [b.q[int(qsl[r]):int(qsl[r + 1])] for r in order]
    lens = torch.tensor([int(qsl[r + 1] - qsl[r]) for r in order])
    new_qsl = torch.zeros(len(order) + 1, dtype=torch.int32)
    new_qsl[1:] = torch.cumsum(lens, 0)
    return workloads.Batch(b.workload, torch.cat(qs), b.k_cache, b.v_cache,
                           b.block_table[order], new_qsl, b.seq_lens[order], b.num_computed[order])


def test_request_permutation_and_subset_are_bitwise_invariant():
    b = _small_batch(seed=12)
    out, lse = _run(b)
    qsl = b.query_start_loc
    order = [3, 0, 4, 1, 2]
    out_p, lse_p = _run(_reorder(b, order))
    qslp = _reorder(b, order).query_start_loc
    for new_r, r in enumerate(order):
        a = slice(int(qsl[r]), int(qsl[r + 1]))
        c = slice(int(qslp[new_r]), int(qslp[new_r + 1]))
        assert np.array_equal(out[a], out_p[c]) and np.array_equal(lse[a], lse_p[c])
    alone_o, alone_l = _run(_reorder(b, [2]))
    a = slice(int(qsl[2]), int(qsl[3]))
    assert np.array_equal(out[a], alone_o) and np.array_equal(lse[a], alone_l)


def test_page_relabel_is_bitwise_invariant():
    b = _small_batch(seed=13)
    out, lse = _run(b)
    n = b.num_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(5))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(n)
    b2 = workloads.Batch(b.workload, b.q, b.k_cache[inv], b.v_cache[inv],
                         perm[b.block_table.long()].to(torch.int32),
                         b.query_start_loc, b.seq_lens, b.num_computed)
    out2, lse2 = _run(b2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_oracle_never_reads_poison():
    b = _small_batch(seed=14)
    out, lse = _run(b)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


# ------------------------------------------------------------- host decisions

def test_r1_r2_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "r1r2_example.json")))
    tok = ex["tokens"]
    bt = [[tok[x] for x in row] for row in ex["block_table"]]
    blocks = oracle.common_prefix_blocks(bt, ex["seq_lens"], ex["page_size"])
    assert blocks == ex["expected_common_blocks"]
    pc = oracle.cascade_prefix_len(blocks, ex["page_size"], ex["num_computed_tokens"])
    assert pc == ex["expected_prefix_len"]
    assert bt[0][:pc] == [tok[x] for x in ex["expected_prefix"]]
    for r in range(2):
        assert bt[r][pc:ex["seq_lens"][r]] == [tok[x] for x in ex["expected_suffix"][r]]


def test_cap_and_floor(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "cap_floor.json")))["cases"]
    for c in cases:
        assert oracle.cascade_prefix_len(c["blocks"], c["page_size"], c["num_computed"]) == c["prefix_len"], c


def test_gates(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "gates.json")))
    assert oracle.MIN_PREFIX_TOKENS == g["min_prefix_tokens"]
    assert oracle.MIN_NUM_REQS == g["min_num_reqs"]
    for c in g["cases"]:
        assert oracle.passes_cascade_gates(c["prefix_len"], c["num_reqs"]) == c["pass"], c


def test_worked_example_kv_tokens(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    n, p, s = ex["num_reqs"], ex["prefix"], ex["suffix"]
    lens = [p + s] * n
    assert oracle.kv_tokens_standard(lens) == ex["kv_tokens_standard"]
    assert oracle.kv_tokens_cascade(p, lens) == ex["kv_tokens_cascade"]
    assert oracle.kv_tokens_cascade(p, lens) - p == ex["kv_tokens_cascade_suffix"]
    assert round(ex["kv_tokens_standard"] / ex["kv_tokens_cascade"]) == ex["reduction"]


def test_common_blocks_hand_cases():
    ps = 4
    # identical leading pages, then divergence at column 2
    assert oracle.common_prefix_blocks([[5, 6, 7, 9], [5, 6, 8, 9]], [16, 16], ps) == 2
    # divergence at column 0
    assert oracle.common_prefix_blocks([[1, 6], [5, 6]], [8, 8], ps) == 0
    # a short request: its padding column equals the other's real page, but
    # padding never counts (limit = ceil(5/4) = 2 columns)
    assert oracle.common_prefix_blocks([[5, 6, 7], [5, 6, 7]], [12, 5], ps) == 2
    # a single request shares all of its pages with itself
    assert oracle.common_prefix_blocks([[3, 4, 2]], [9], ps) == 3
    # match resumes after a mismatch: still only the contiguous run counts
    assert oracle.common_prefix_blocks([[1, 2, 3], [1, 9, 3]], [12, 12], ps) == 1


def test_common_blocks_brute_force_tiny():
    """Exhaustive check on tiny tables against a differently written rule:
    the largest C such that the first C columns, restricted to real pages,
    form one identical row."""
    rng = np.random.default_rng(30)
    for _ in range(2000):
        n = int(rng.integers(1, 4))
        cols = int(rng.integers(1, 5))
        ps = int(rng.integers(1, 4))
        bt = rng.integers(0, 3, (n, cols)).tolist()
        lens = rng.integers(1, cols * ps + 1, n).tolist()
        limit = min(-(-x // ps) for x in lens)
        best = 0
        for c in range(limit + 1):
            if len({tuple(row[:c]) for row in bt}) == 1:
                best = c
        assert oracle.common_prefix_blocks(bt, lens, ps) == best


# ------------------------------------------------------ second shared level

# Seven requests, page size 4. Pages 0 and 1 are shared by all (level 0,
# 8 tokens). Requests 0-2 also share pages 10 and 11 (0 and 1 share page 12
# too); requests 4-6 share page 40 (4 and 5 also page 41); request 3 shares
# nothing more. Row 1's padding column copies row 0's real page 21.
_L1_BT = [[0, 1, 10, 11, 12, 20, 21],
          [0, 1, 10, 11, 12, 22, 21],
          [0, 1, 10, 11, 13, 23, 0],
          [0, 1, 30, 31, 0, 0, 0],
          [0, 1, 40, 41, 42, 0, 0],
          [0, 1, 40, 41, 43, 0, 0],
          [0, 1, 40, 50, 0, 0, 0]]
_L1_SEQ = [26, 24, 22, 16, 20, 18, 14]


def test_level1_groups_hand_case():
    """Worked by hand. Adjacent shared pages: (0,1) 5, (1,2) 4, (2,3) 2,
    (3,4) 2, (4,5) 4, (5,6) 3; the runs sharing more than the 2 level-0
    pages are requests 0-2 (4 pages = 16 tokens) and 4-6 (3 pages = 12
    tokens). Caps (num_computed = seq - 1): 0-2 min 21 -> 16; 4-6 min 13 ->
    12."""
    nc = [s - 1 for s in _L1_SEQ]
    assert oracle.common_prefix_blocks(_L1_BT, _L1_SEQ, 4) == 2
    assert oracle.level1_groups(_L1_BT, _L1_SEQ, nc, 4, 8, min_extra_tokens=4) == [(0, 3, 16), (4, 7, 12)]
    # the gate on the extra length: 4-6 adds only 4 tokens
    assert oracle.level1_groups(_L1_BT, _L1_SEQ, nc, 4, 8, min_extra_tokens=5) == [(0, 3, 16)]
    # the cap binds: request 2 has computed only 14 tokens -> floor(14 / 4) * 4 = 12
    nc2 = list(nc)
    nc2[2] = 14
    assert oracle.level1_groups(_L1_BT, _L1_SEQ, nc2, 4, 8, min_extra_tokens=4) == [(0, 3, 12), (4, 7, 12)]
    # members: a group needs two requests, so 4-6 split at 5 leaves none there
    bt3 = [row[:] for row in _L1_BT]
    bt3[5][2] = 44
    assert oracle.level1_groups(bt3, _L1_SEQ, nc, 4, 8, min_extra_tokens=4) == [(0, 3, 16)]
    # nothing nested: no group
    flat = [[0, 1, 100 + r, 0] for r in range(4)]
    assert oracle.level1_groups(flat, [13] * 4, [12] * 4, 4, 8, min_extra_tokens=1) == []


def test_level1_groups_brute_force_tiny():
    """Random tiny tables against a differently written rule: rows a..b-1
    share c columns when their first c real columns form one tuple; a run is
    extended while some c above the level-0 pages is shared."""
    rng = np.random.default_rng(31)
    for _ in range(1500):
        n = int(rng.integers(1, 6))
        cols = int(rng.integers(2, 6))
        ps = int(rng.integers(1, 4))
        bt = rng.integers(0, 3, (n, cols)).tolist()
        for row in bt:
            row[0] = 7                           # one level-0 page
        lens = rng.integers(ps + 1, cols * ps + 1, n).tolist()
        nc = [int(rng.integers(1, x + 1)) for x in lens]
        level0 = ps

        def shared(a, b):
            limit = min(-(-x // ps) for x in lens[a:b])
            return max(c for c in range(limit + 1) if len({tuple(bt[r][:c]) for r in range(a, b)}) == 1)

        want, a = [], 0
        while a < n:
            b = a + 1
            while b < n and shared(a, b + 1) > 1:
                b += 1
            if b - a >= 2:
                length = min(shared(a, b) * ps, min(nc[a:b])) // ps * ps
                if length - level0 >= 1:
                    want.append((a, b, length))
            a = b
        assert oracle.level1_groups(bt, lens, nc, ps, level0, min_extra_tokens=1) == want


def test_multilevel_split_equals_full_attention():
    """Three levels with the oracle's own pieces -- every query over the
    level-0 prefix, each group's queries over the group's extra positions
    (both non-causal), each request over the rest (causal), LSE merge --
    equal full attention (every shared position is at or below every member
    query's position because of the cap)."""
    w = workloads.Workload("nested", 7, 16, (3, 20), (1, 4), 4, 2, 16, page_size=8, seed=17,
                           groups=((3, 20), (2, 37)))
    b = workloads.make_batch(w)
    G = w.num_q_heads // w.num_kv_heads
    bt, qsl, sl = b.block_table.numpy(), b.query_start_loc.numpy(), b.seq_lens.numpy()
    full_o, full_l = oracle.attention_full(b.q.float().numpy(), b.k_cache.float().numpy(),
                                           b.v_cache.float().numpy(), bt, qsl, sl, w.page_size)
    nc = b.num_computed.numpy()
    p0 = oracle.cascade_prefix_len(oracle.common_prefix_blocks(bt, sl, 8), 8, nc)
    groups = oracle.level1_groups(bt, sl, nc, 8, p0, min_extra_tokens=1)
    assert p0 == 16 and groups == [(0, 3, 32), (3, 5, 48)]   # whole shared pages only
    start = [p0] * w.num_reqs
    for a, e, length in groups:
        for r in range(a, e):
            start[r] = length
    for r in range(w.num_reqs):
        q0, q1 = int(qsl[r]), int(qsl[r + 1])
        k, v = _dense_kv(b, r)
        pos = int(nc[r]) + np.arange(q1 - q0)
        for h in range(w.num_q_heads):
            g = h // G
            rows = b.q[q0:q1, h].double().numpy()
            parts = [oracle.attend(rows, k[:p0, g].numpy(), v[:p0, g].numpy(), w.softmax_scale),
                     oracle.attend(rows, k[p0:start[r], g].numpy(), v[p0:start[r], g].numpy(), w.softmax_scale)]
            t = np.arange(start[r], k.shape[0])
            vis = t[None, :] <= pos[:, None]
            parts.append(oracle.attend(rows, k[start[r]:, g].numpy(), v[start[r]:, g].numpy(), w.softmax_scale, vis))
            o_m, l_m = oracle.merge_states([p[0] for p in parts], [p[1] for p in parts])
            assert np.abs(o_m - full_o[q0:q1, h]).max() < 1e-12
            assert np.abs(l_m - full_l[q0:q1, h]).max() < 1e-12


def test_kv_tokens_multilevel_hand():
    # level 0: 16; group (0, 2) shares 48 (32 extra); suffixes 12 + 22 + 14
    assert oracle.kv_tokens_multilevel(16, [(0, 2, 48)], [60, 70, 30]) == 16 + 32 + 12 + 22 + 14
    assert oracle.kv_tokens_multilevel(16, [], [60, 70, 30]) == oracle.kv_tokens_cascade(16, [60, 70, 30])


# ------------------------------------------------------- prefix-tree levels

# Seven requests, page size 1 (so pages are tokens), level 0 = the 2 pages
# P0 P1 every row starts with. Requests 0, 2 and 4 (not consecutive) share a
# document A A A (pages 10-12); within it 0 and 4 share a chapter C C (20,
# 21); requests 1 and 3 share a document B B B (30-32); request 5 shares one
# page (40) with request 6, and then 5 and 6 part.
_T_BT = [[0, 1, 10, 11, 12, 20, 21, 50, 0],
         [0, 1, 30, 31, 32, 51, 0, 0, 0],
         [0, 1, 10, 11, 12, 52, 0, 0, 0],
         [0, 1, 30, 31, 32, 53, 54, 0, 0],
         [0, 1, 10, 11, 12, 20, 21, 55, 56],
         [0, 1, 40, 57, 0, 0, 0, 0, 0],
         [0, 1, 40, 58, 59, 0, 0, 0, 0]]
_T_SEQ = [8, 6, 6, 7, 9, 4, 5]


def test_tree_groups_hand_case():
    """Worked by hand (min_extra_tokens 2, every request computed all but its
    last token). Level 0 is 2 pages. At column 2 the rows split into {0, 2,
    4} (page 10), {1, 3} (page 30) and {5, 6} (page 40). {0, 2, 4} shares 5
    pages -> 5 tokens, 3 more than level 0: a level-1 group; inside it, at
    column 5, {0, 4} (page 20) shares 7 -> 7 tokens, 2 more: a level-2 group.
    {1, 3} shares 5 -> level 1. {5, 6} shares 3 pages, 1 more than level 0:
    not a group (and its rows part at column 3)."""
    nc = [s - 1 for s in _T_SEQ]
    want = [((0, 2, 4), 2, 5, 1), ((0, 4), 5, 7, 2), ((1, 3), 2, 5, 1)]
    assert oracle.tree_groups(_T_BT, _T_SEQ, nc, 1, 2, min_extra_tokens=2) == want
    # two shared levels at most: the chapter is not formed
    assert oracle.tree_groups(_T_BT, _T_SEQ, nc, 1, 2, min_extra_tokens=2, max_levels=2) == [want[0], want[2]]
    # the cap: request 4 has computed only 6 tokens, so {0, 4} shares 6, 1
    # more than its document -- not a group
    nc2 = list(nc)
    nc2[4] = 6
    assert oracle.tree_groups(_T_BT, _T_SEQ, nc2, 1, 2, min_extra_tokens=2) == [want[0], want[2]]
    # a gate of 3 leaves the documents; with 4 neither document passes, but
    # the chapter {0, 4}, 5 tokens past level 0, becomes a level-1 group;
    # with 6 nothing is left
    assert oracle.tree_groups(_T_BT, _T_SEQ, nc, 1, 2, min_extra_tokens=3) == [want[0], want[2]]
    assert oracle.tree_groups(_T_BT, _T_SEQ, nc, 1, 2, min_extra_tokens=4) == [((0, 4), 2, 7, 1)]
    assert oracle.tree_groups(_T_BT, _T_SEQ, nc, 1, 2, min_extra_tokens=6) == []
    # KV positions: level 0 (2) + A's 3 + C's 2 + B's 3 + each request past its innermost group
    rest = [8 - 7, 6 - 5, 6 - 5, 7 - 5, 9 - 7, 4 - 2, 5 - 2]
    assert oracle.kv_tokens_tree(2, want, _T_SEQ) == 2 + 3 + 2 + 3 + sum(rest)


def test_tree_groups_look_past_a_small_split():
    """Four requests share one page beyond level 0 (too little for a group);
    inside it two pairs share three more each: the pairs are groups one level
    below level 0, their extra length counted from level 0."""
    bt = [[0, 1, 9, 10, 11, 12, 60], [0, 1, 9, 10, 11, 12, 61], [0, 1, 9, 20, 21, 22, 62], [0, 1, 9, 20, 21, 22, 63]]
    seq = [7, 7, 7, 7]
    nc = [6] * 4
    assert oracle.tree_groups(bt, seq, nc, 1, 2, min_extra_tokens=3) == [((0, 1), 2, 6, 1), ((2, 3), 2, 6, 1)]


def _tree_brute(bt, seq, nc, ps, level0, min_extra, max_levels):
    """Declarative form: a set of >= 2 requests (not the whole batch) is a
    candidate if no other request shares all the pages its members share;
    candidates are taken largest first, each measured against the smallest
    accepted group that contains it (or level 0)."""
    n = len(bt)
    sets = []
    for mask in range(1, 1 << n):
        S = [r for r in range(n) if mask >> r & 1]
        if len(S) < 2 or len(S) == n:
            continue
        c = oracle.common_prefix_blocks([bt[r] for r in S], [seq[r] for r in S], ps)
        closed = all(oracle.common_prefix_blocks([bt[r] for r in S + [o]], [seq[r] for r in S + [o]], ps) < c
                     for o in range(n) if o not in S)
        if closed:
            sets.append((S, c))
    sets.sort(key=lambda x: -len(x[0]))
    accepted = []
    for S, c in sets:
        parent_len, level = level0, 0
        for T, plen, tlen, tlev in sorted(accepted, key=lambda g: len(g[0])):
            if set(S) < set(T):
                parent_len, level = tlen, tlev
                break
        length = oracle.cascade_prefix_len(c, ps, [nc[r] for r in S])
        if length - parent_len >= min_extra and level + 1 <= max_levels - 1:
            accepted.append((tuple(S), parent_len, length, level + 1))
    return sorted(accepted)


def test_tree_groups_brute_force_tiny():
    rng = np.random.default_rng(43)
    checked = 0
    for _ in range(1200):
        n = int(rng.integers(2, 7))
        cols = int(rng.integers(3, 7))
        ps = int(rng.integers(1, 3))
        bt = rng.integers(0, 3, (n, cols)).tolist()
        for row in bt:
            row[0] = 7
        lens = rng.integers(ps + 1, cols * ps + 1, n).tolist()
        nc = [int(rng.integers(1, x + 1)) for x in lens]
        level0 = oracle.cascade_prefix_len(oracle.common_prefix_blocks(bt, lens, ps), ps, nc)
        ml = int(rng.integers(2, 5))
        got = sorted(oracle.tree_groups(bt, lens, nc, ps, level0, min_extra_tokens=1, max_levels=ml))
        assert got == _tree_brute(bt, lens, nc, ps, level0, 1, ml)
        checked += bool(got)
    assert checked > 100


def test_tree_groups_match_the_consecutive_runs():
    """On batches whose documents are consecutive runs, the tree's level-1
    groups are the runs the second-level rule finds."""
    for name in ("multi_doc", "multi_doc_prefill"):
        b = workloads.make_batch(workloads.get(name))
        bt, sl, nc = b.block_table.numpy(), b.seq_lens.numpy(), b.num_computed.numpy()
        p0 = oracle.cascade_prefix_len(oracle.common_prefix_blocks(bt, sl, 16), 16, nc)
        runs = oracle.level1_groups(bt, sl, nc, 16, p0)
        tree = oracle.tree_groups(bt, sl, nc, 16, p0)
        assert [(m[0], m[-1] + 1, L) for m, _, L, lev in tree if lev == 1] == runs
        assert all(lev == 1 for *_, lev in tree)


def test_tree_split_equals_full_attention():
    """A three-level tree with interleaved members, computed with the
    oracle's own pieces -- every query over the level-0 prefix, each group's
    queries over its positions beyond the group it lies in (non-causal), each
    request over the rest (causal), LSE merge -- equals full attention."""
    w = workloads.Workload("tree", 8, 16, (3, 20), (1, 4), 4, 2, 16, page_size=8, seed=23,
                           docs=(((0, 2, 4, 6), 24), ((1, 3, 5), 16), ((0, 4), 19), ((3, 5), 21)))
    b = workloads.make_batch(w)
    G = w.num_q_heads // w.num_kv_heads
    bt, qsl, sl = b.block_table.numpy(), b.query_start_loc.numpy(), b.seq_lens.numpy()
    full_o, full_l = oracle.attention_full(b.q.float().numpy(), b.k_cache.float().numpy(),
                                           b.v_cache.float().numpy(), bt, qsl, sl, w.page_size)
    nc = b.num_computed.numpy()
    p0 = oracle.cascade_prefix_len(oracle.common_prefix_blocks(bt, sl, 8), 8, nc)
    groups = oracle.tree_groups(bt, sl, nc, 8, p0, min_extra_tokens=1)
    # whole shared pages only: the chapters (19, 21 tokens) share 16 each
    assert p0 == 16 and groups == [((0, 2, 4, 6), 16, 40, 1), ((0, 4), 40, 56, 2), ((1, 3, 5), 16, 32, 1),
                                   ((3, 5), 32, 48, 2)]
    assert oracle.kv_tokens_tree(p0, groups, sl) == 16 + 24 + 16 + 16 + 16 + sum(
        int(sl[r]) - s for r, s in enumerate([56, 32, 40, 48, 56, 48, 40, 16]))
    for r in range(w.num_reqs):
        q0, q1 = int(qsl[r]), int(qsl[r + 1])
        k, v = _dense_kv(b, r)
        pos = int(nc[r]) + np.arange(q1 - q0)
        bounds = [0, p0] + [L for m, _, L, _ in groups if r in m]
        for h in range(w.num_q_heads):
            g = h // G
            rows = b.q[q0:q1, h].double().numpy()
            parts = [oracle.attend(rows, k[a:e, g].numpy(), v[a:e, g].numpy(), w.softmax_scale)
                     for a, e in zip(bounds[:-1], bounds[1:])]
            t = np.arange(bounds[-1], k.shape[0])
            vis = t[None, :] <= pos[:, None]
            parts.append(oracle.attend(rows, k[bounds[-1]:, g].numpy(), v[bounds[-1]:, g].numpy(), w.softmax_scale,
                                       vis))
            o_m, l_m = oracle.merge_states([p[0] for p in parts], [p[1] for p in parts])
            assert np.abs(o_m - full_o[q0:q1, h]).max() < 1e-12
            assert np.abs(l_m - full_l[q0:q1, h]).max() < 1e-12


# ------------------------------------------------- sinks and sliding window

def test_sink_hand_case():
    """d=1, scale 1, one key with score 0 and value 6, sink ln 2: weights
    1 / (1 + 2) for the key, so o = 2 and lse = ln 3."""
    o, lse = oracle.attend([[1.0]], [[0.0]], [[6.0]], 1.0, sink=math.log(2.0))
    assert abs(o[0, 0] - 2.0) < 1e-15 and abs(lse[0] - math.log(3.0)) < 1e-15
    # a sink of -inf is no sink at all
    q, k, v = np.random.default_rng(3).normal(size=(3, 4, 8))
    a = oracle.attend(q, k, v, 0.5)
    b = oracle.attend(q, k, v, 0.5, sink=-np.inf)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sink_is_one_more_partial_in_the_merge():
    """The way the merge applies a sink: an extra partial state with
    lse = sink and o = 0, merged with the key partials, equals attention with
    the sink over the union of the keys."""
    rng = np.random.default_rng(4)
    q, k, v = rng.normal(size=(5, 16)), rng.normal(size=(9, 16)), rng.normal(size=(9, 16))
    sink = 0.7
    full_o, full_l = oracle.attend(q, k, v, 0.25, sink=sink)
    parts = [oracle.attend(q, k[:4], v[:4], 0.25), oracle.attend(q, k[4:], v[4:], 0.25),
             (np.zeros((5, 16)), np.full(5, sink))]
    o_m, l_m = oracle.merge_states([p[0] for p in parts], [p[1] for p in parts])
    assert np.abs(o_m - full_o).max() < 1e-12 and np.abs(l_m - full_l).max() < 1e-12


def test_window_special_cases_and_sdpa():
    """A window of one key gives each query its own position's value; a
    window longer than every sequence is plain causal attention; other
    windows match torch SDPA in float64 with the explicit band mask."""
    b = _small_batch(seed=21, n=4, prefix=24, suffix=(5, 20), q=(1, 6), ps=8)
    w = b.workload
    args = (b.q.float().numpy(), b.k_cache.float().numpy(), b.v_cache.float().numpy(), b.block_table.numpy(),
            b.query_start_loc.numpy(), b.seq_lens.numpy(), w.page_size)
    causal = oracle.attention_full(*args)
    wide = oracle.attention_full(*args, window=int(b.seq_lens.max()))
    assert np.array_equal(causal[0], wide[0]) and np.array_equal(causal[1], wide[1])
    one_o, one_l = oracle.attention_full(*args, window=1)
    G = w.num_q_heads // w.num_kv_heads
    for r in range(w.num_reqs):
        q0, q1 = int(b.query_start_loc[r]), int(b.query_start_loc[r + 1])
        k, v = _dense_kv(b, r)
        nc = int(b.num_computed[r])
        for i in range(q1 - q0):
            for h in range(w.num_q_heads):
                assert np.abs(one_o[q0 + i, h] - v[nc + i, h // G].numpy()).max() < 1e-12
        for win in (3, 11):
            o, l = oracle.attention_full(*args, window=win, requests=[r])
            L = k.shape[0]
            pos = nc + torch.arange(q1 - q0)
            t = torch.arange(L)
            mask = (t[None, :] <= pos[:, None]) & (t[None, :] > (pos - win)[:, None])
            for h in range(w.num_q_heads):
                qq = b.q[q0:q1, h].double()[None, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, k[None, None, :, h // G], v[None, None, :, h // G], attn_mask=mask[None, None],
                    scale=w.softmax_scale)[0, 0]
                assert np.abs(o[q0:q1, h] - ref.numpy()).max() < 1e-12


# ------------------------------------------------------------- fp8 caches

def test_fp8_e4m3_hand_values():
    """Codes worked by hand from the E4M3 layout (sign, 4-bit exponent with
    bias 7, 3-bit mantissa; exponent 0 subnormal; S.1111.111 NaN)."""
    cases = {0x00: 0.0, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0xB8: -1.0, 0xC4: -3.0, 0x30: 0.5, 0x77: 240.0}
    got = oracle.fp8_e4m3_decode(np.array(list(cases), dtype=np.uint8))
    assert got.tolist() == list(cases.values())
    nan = oracle.fp8_e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(nan).all()
    z = oracle.fp8_e4m3_decode(np.array([0x80], dtype=np.uint8))
    assert z[0] == 0.0 and np.signbit(z[0])


def test_fp8_e4m3_matches_torch_on_every_code():
    """A library routine as a second reading of the format: torch's
    float8_e4m3fn dtype, every one of the 256 codes."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(oracle.fp8_e4m3_decode(codes), ref, equal_nan=True)


def test_fp8_workload_codes_dequantise_to_the_values():
    """The fp8 batch recipe: the decoded codes times the scale are the bf16
    batch's values rounded to the fp8 grid (within half a step, 2^-4
    relative, or the subnormal step), and the poison stays NaN."""
    base = dict(num_reqs=4, prefix=32, suffix=(3, 10), q_len=(1, 2), num_q_heads=4, num_kv_heads=2, head_dim=128,
                seed=5)
    b16 = workloads.make_batch(workloads.Workload("t", **base))
    b8 = workloads.make_batch(workloads.Workload("t", **base, kv_dtype="fp8", k_scale=0.125, v_scale=0.0625))
    assert torch.equal(b16.block_table, b8.block_table) and torch.equal(b16.q, b8.q)
    for c16, c8, sc in ((b16.k_cache, b8.k_cache, 0.125), (b16.v_cache, b8.v_cache, 0.0625)):
        x = c16.double().numpy()
        y = oracle.fp8_e4m3_decode(c8.numpy()) * sc
        assert np.array_equal(np.isnan(x), np.isnan(y))
        ok = ~np.isnan(x)
        assert (np.abs(y[ok] - x[ok]) <= np.maximum(np.abs(x[ok]) * 2.0 ** -4, sc * 2.0 ** -10) + 1e-12).all()


# --------------------------------------------------------------- input recipe

def test_workload_structure_matches_recipe():
    b = workloads.make_batch(workloads.get("tiny_decode"))
    w = b.workload
    assert b.q.shape == (8, 4, 64) and b.q.dtype == torch.bfloat16
    assert b.seq_lens.tolist() == [272] * 8
    assert b.num_computed.tolist() == [271] * 8
    shared = w.prefix // w.page_size
    assert (b.block_table[:, :shared] == b.block_table[0, :shared]).all()
    assert len(set(b.block_table[:, shared].tolist())) == 8
    out, lse = _run(b)
    assert np.isfinite(out).all()
