"""fp64 reference for shared-prefix (cascade) attention -- test infrastructure.

This module is the oracle. It is plain, slow and written to be checked by eye
against the pages; it must never be imported by the product path (the HIP
library and its Python binding). Inputs are numpy arrays (any float dtype for
Q/K/V, upcast to float64 here; bf16 values are exactly representable).

Conventions (the readings of the pages that this module fixes):

* ``seq_lens[r]`` counts every KV position of request r, including this
  step's query tokens, which are its last ``q_len_r`` positions. Reading of
  [p2] section 5, whose standard-path count N x (P + S) = 270,336 for
  N=64, P=4096, S=128 only comes out with the query inside S.
* ``num_computed_r = seq_lens[r] - q_len_r``: the tokens already in the cache
  before this step ([p2] section 4 table, column "already computed KV").
* Causal alignment is bottom-right: query i of request r (0-based within the
  request) sees KV positions t <= num_computed_r + i ([p2] section 4: the
  queries follow the already computed tokens).
* GQA: query head h reads KV head h // (Hq // Hkv) (the pages are silent; the
  plainest reading, consecutive query heads share a KV head).
* LSE is the natural log of the softmax normaliser of the *scaled* scores.
* Default softmax scale 1/sqrt(head_dim).
* KV cache layout handed to the oracle: ``[num_pages, page_size, Hkv, d]``.
"""

from __future__ import annotations

import math

import numpy as np

# [p2] section 3, trigger-condition table: common prefix >= 256 tokens and
# batch >= 8 requests (section 3 also lists "< 8 requests" as not benefiting).
MIN_PREFIX_TOKENS = 256
MIN_NUM_REQS = 8


def attend(q_rows, keys, values, scale, visible=None, sink=None):
    """Softmax attention of query rows over an explicit key set, in fp64.

    The plain definition ([p2] section 1: cascade is "mathematically
    equivalent to standard attention"): s = scale * q.k, o = sum softmax(s) v,
    lse = log sum exp(s).

    q_rows [m, d], keys [n, d], values [n, d]; ``visible`` optional bool
    [m, n] (True = key visible). ``sink``: optional attention-sink logit
    ([p2] section 9 names the sinks parameter every backend receives; the
    reading here is one logit per query head that joins the softmax
    normaliser and carries no value): it is one more score, with value 0,
    so lse = log(sum exp(s) + exp(sink)). Returns (o [m, d], lse [m]). A row
    that sees no key (and has no sink) gets o = 0 and lse = -inf.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    m = q_rows.shape[0]
    d = q_rows.shape[1]
    if sink is not None:
        keys = np.concatenate([keys, np.zeros((1, d))])
        values = np.concatenate([values, np.zeros((1, d))])
        vis = np.ones((m, keys.shape[0] - 1), dtype=bool) if visible is None else np.asarray(visible, dtype=bool)
        visible = np.concatenate([vis, np.ones((m, 1), dtype=bool)], axis=1)
    if keys.shape[0] == 0:
        return np.zeros((m, d)), np.full(m, -np.inf)
    s = (q_rows @ keys.T) * float(scale)
    if sink is not None:
        s[:, -1] = float(sink)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    row_max = s.max(axis=1)
    empty = ~np.isfinite(row_max)
    safe_max = np.where(empty, 0.0, row_max)
    w = np.exp(s - safe_max[:, None])          # exp(-inf) == 0 for hidden keys
    z = w.sum(axis=1)
    o = np.zeros((m, d))
    live = ~empty
    o[live] = (w[live] @ values) / z[live, None]
    lse = np.full(m, -np.inf)
    lse[live] = safe_max[live] + np.log(z[live])
    return o, lse


def merge_states(outs, lses):
    """Combine partial attention states over disjoint key sets.

    [p2] section 1 step 3 and section 8 Step 5 (merge_attn_states): the two
    partial outputs are combined by log-sum-exp rescaling. Written out:
    M = max_s lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s,
    lse = M + log sum w_s. Partials with lse = -inf carry weight 0; if every
    partial is empty the result is o = 0, lse = -inf (the pages are silent on
    this case).

    outs: list of arrays [..., d]; lses: list of arrays [...].
    """
    lse_stack = np.stack([np.asarray(x, dtype=np.float64) for x in lses])
    o_stack = np.stack([np.asarray(x, dtype=np.float64) for x in outs])
    big = lse_stack.max(axis=0)
    empty = ~np.isfinite(big)
    safe = np.where(empty, 0.0, big)
    w = np.exp(lse_stack - safe)                 # [S, ...]
    wsum = w.sum(axis=0)
    o = np.zeros(o_stack.shape[1:])
    num = (w[..., None] * np.where(w[..., None] > 0, o_stack, 0.0)).sum(axis=0)
    live = ~empty
    o[live] = num[live] / wsum[live][..., None]
    lse = np.where(live, safe + np.log(np.where(live, wsum, 1.0)), -np.inf)
    return o, lse


def _request_kv(cache, block_table_row, seq_len, page_size, kv_head):
    """Gather one request's KV sequence for one KV head from the paged cache.

    [p2] section 5 / section 8 Step 5: ``block_table[seq_id]`` lists the
    physical pages holding the request's KV positions in order; position t
    lives in page block_table[t // page_size], slot t % page_size.
    """
    n_pages = -(-int(seq_len) // page_size)
    assert n_pages <= len(block_table_row)
    t = np.arange(int(seq_len))
    pages = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
    slots = t % page_size
    return np.asarray(cache[pages, slots, kv_head], dtype=np.float64)


def attention_full(q, k_cache, v_cache, block_table, query_start_loc, seq_lens,
                   page_size, scale=None, requests=None, window=0, sinks=None):
    """Full (non-cascade) causal attention of every request over its whole KV.

    This is the plain definition the cascade path must reproduce ([p2]
    section 1: equivalent to standard attention; section 8 Step 4: the
    standard path is one varlen attention over the full block tables; [p1]
    states that the option leaves results mathematically unchanged).

    q [T, Hq, d]; k_cache, v_cache [num_pages, page_size, Hkv, d];
    block_table [N, stride]; query_start_loc [N+1]; seq_lens [N].
    ``requests``: optional iterable of request indices to compute (rows of
    other requests are left NaN). ``window`` > 0: sliding-window attention, a
    query at position p sees positions p - window < t <= p (the pages list
    sliding window among the features cascade does not support, [p2]
    section 3). ``sinks``: optional [Hq] attention-sink logits (see
    ``attend``). Returns (out [T, Hq, d], lse [T, Hq]) fp64.
    """
    q = np.asarray(q)
    T, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    out = np.full((T, Hq, d), np.nan)
    lse = np.full((T, Hq), np.nan)
    reqs = range(len(lens)) if requests is None else requests
    for r in reqs:
        q0, q1 = int(qsl[r]), int(qsl[r + 1])
        q_len = q1 - q0
        seq_len = int(lens[r])
        num_computed = seq_len - q_len
        for g in range(Hkv):
            keys = _request_kv(k_cache, bt[r], seq_len, page_size, g)
            vals = _request_kv(v_cache, bt[r], seq_len, page_size, g)
            t = np.arange(seq_len)
            for j in range(group):
                h = g * group + j
                rows = np.asarray(q[q0:q1, h, :], dtype=np.float64)
                pos = num_computed + np.arange(q_len)
                visible = t[None, :] <= pos[:, None]
                if window > 0:
                    visible &= t[None, :] > (pos - int(window))[:, None]
                o_h, l_h = attend(rows, keys, vals, scale, visible, None if sinks is None else sinks[h])
                out[q0:q1, h, :] = o_h
                lse[q0:q1, h] = l_h
    return out, lse


def common_prefix_blocks(block_table, seq_lens, page_size):
    """Number of leading KV pages shared by every request of the batch.

    [p2] section 8 Step 1: walk the block tables and count the physical
    blocks shared by all running requests, matching contiguously from block
    0. [p3]: only the running requests count (the batch rows here), not
    reference counts that stale requests may still hold. A column is only
    compared inside every request's own pages (j < ceil(seq_len / page_size)),
    so padding entries of a block table never count.
    """
    bt = [list(map(int, row)) for row in block_table]
    n = len(bt)
    if n == 0:
        return 0
    limit = min(-(-int(s) // page_size) for s in seq_lens)
    count = 0
    for j in range(limit):
        first = bt[0][j]
        if all(bt[r][j] == first for r in range(n)):
            count += 1
        else:
            break
    return count


def cascade_prefix_len(num_common_blocks, page_size, num_computed_tokens):
    """Shared-prefix length used by the cascade split.

    [p2] section 8 Step 2: length = blocks * block_size, capped at the
    minimum num_computed_tokens (section 4 and section 11: the cap avoids
    attention-mask leakage), then floored to a whole block.
    """
    length = int(num_common_blocks) * int(page_size)
    length = min(length, min(int(x) for x in num_computed_tokens))
    length = (length // int(page_size)) * int(page_size)
    return length


def passes_cascade_gates(prefix_len, num_reqs):
    """[p2] section 3 trigger table: prefix >= 256 tokens and >= 8 requests."""
    return int(prefix_len) >= MIN_PREFIX_TOKENS and int(num_reqs) >= MIN_NUM_REQS


def kv_tokens_standard(seq_lens):
    """KV positions read by the standard path: every request reads its whole
    sequence ([p2] section 5: N x (P + S))."""
    return int(sum(int(s) for s in seq_lens))


def kv_tokens_cascade(prefix_len, seq_lens):
    """KV positions read by cascade: the prefix once plus each request's
    suffix ([p2] section 5: P + N x S)."""
    return int(prefix_len) + int(sum(int(s) - int(prefix_len) for s in seq_lens))


def level1_groups(block_table, seq_lens, num_computed_tokens, page_size, level0_len,
                  min_members=2, min_extra_tokens=MIN_PREFIX_TOKENS):
    """Request groups of a second shared level, as (first, end, shared_len).

    FlashInfer's cascade runs any number of levels ([p2] section 7 table) and
    the workloads of [p2] section 3 nest (a system prompt shared by all, a
    document shared by some). The pages give no detector for the inner
    level, so this is the plainest extension of the batch-wide rule
    ([p2] section 8 Steps 1-2) to runs of consecutive requests: starting
    from request a, extend the run while all its requests still share more
    leading pages than the batch-wide prefix (common_prefix_blocks of the
    run), then give the run the pages all of it shares, capped at its
    smallest num_computed_tokens and floored to a page. A run is a group if
    it has at least ``min_members`` requests and shares at least
    ``min_extra_tokens`` more positions than the batch-wide prefix (the
    prefix-length gate of section 3 by default).
    """
    bt = [list(map(int, row)) for row in block_table]
    sl = [int(s) for s in seq_lens]
    nc = [int(x) for x in num_computed_tokens]
    n = len(bt)
    level0_pages = int(level0_len) // int(page_size)
    groups = []
    a = 0
    while a < n:
        b = a + 1
        while b < n and common_prefix_blocks(bt[a:b + 1], sl[a:b + 1], page_size) > level0_pages:
            b += 1
        if b - a >= min_members:
            blocks = common_prefix_blocks(bt[a:b], sl[a:b], page_size)
            length = cascade_prefix_len(blocks, page_size, nc[a:b])
            if length - int(level0_len) >= min_extra_tokens:
                groups.append((a, b, length))
        a = b
    return groups


def kv_tokens_multilevel(level0_len, groups, seq_lens):
    """KV positions read with a second shared level: the batch-wide prefix
    once, each group's extra positions once, and each request's remaining
    positions ([p2] section 5's accounting, one level deeper)."""
    start = [int(level0_len)] * len(seq_lens)
    extra = 0
    for a, b, length in groups:
        extra += int(length) - int(level0_len)
        for r in range(a, b):
            start[r] = int(length)
    return int(level0_len) + extra + int(sum(int(s) - st for s, st in zip(seq_lens, start)))


def tree_groups(block_table, seq_lens, num_computed_tokens, page_size, level0_len, min_members=2,
                min_extra_tokens=MIN_PREFIX_TOKENS, max_levels=4):
    """Nested request groups of a multi-level cascade, found with a prefix tree.

    FlashInfer's cascade takes any number of levels ([p2] section 7) and the
    workloads of [p2] section 3 nest (a system prompt shared by all, a
    document shared by some, a chapter by fewer). The pages give the
    batch-wide rule only ([p2] section 8 Steps 1-2: shared leading pages,
    capped at the smallest num_computed_tokens, floored to a page); this
    applies it at every node of the prefix tree of the requests' page-id
    sequences. Starting from all requests (the batch-wide prefix,
    ``level0_len``, is level 0): let C be the number of leading pages every
    member shares; split the members (those with more than C pages) by their
    page at column C. A part of at least ``min_members`` requests gets its
    shared length L = its own shared pages in tokens, capped at its smallest
    num_computed_tokens, floored to a page. If L exceeds the length of the
    group it lies in by at least ``min_extra_tokens`` (the prefix-length gate
    of [p2] section 3) it is a group one level deeper, and its parts are
    examined against it; otherwise its parts are examined against the same
    enclosing group. Groups deeper than ``max_levels - 1`` are not formed.

    Returns (members, parent_len, shared_len, level) tuples in the order found
    (a group before the groups inside it); members in batch order.
    """
    bt = [list(map(int, row)) for row in block_table]
    sl = [int(s) for s in seq_lens]
    nc = [int(x) for x in num_computed_tokens]
    ps = int(page_size)
    pages = [-(-s // ps) for s in sl]
    found = []

    def shared_pages(members):
        return common_prefix_blocks([bt[r] for r in members], [sl[r] for r in members], ps)

    def visit(members, parent_len, level):
        c = shared_pages(members)
        parts = {}
        for r in members:
            if pages[r] > c:
                parts.setdefault(bt[r][c], []).append(r)
        for part in parts.values():
            if len(part) < min_members:
                continue
            length = cascade_prefix_len(shared_pages(part), ps, [nc[r] for r in part])
            if length - parent_len >= min_extra_tokens and level + 1 <= max_levels - 1:
                found.append((tuple(part), int(parent_len), int(length), level + 1))
                visit(part, length, level + 1)
            else:
                visit(part, parent_len, level)

    if bt:
        visit(list(range(len(bt))), int(level0_len), 0)
    return found


def kv_tokens_tree(level0_len, groups, seq_lens):
    """KV positions read by a multi-level cascade: the batch-wide prefix once,
    each group's positions beyond the group it lies in once, and each
    request's positions past its innermost group ([p2] section 5's
    accounting, applied at every level)."""
    start = [int(level0_len)] * len(seq_lens)
    extra = 0
    for members, parent_len, length, _ in groups:
        extra += int(length) - int(parent_len)
        for r in members:
            start[r] = max(start[r], int(length))
    return int(level0_len) + extra + int(sum(int(s) - st for s, st in zip(seq_lens, start)))


def fp8_e4m3_decode(codes):
    """Values of fp8 e4m3 codes (uint8) as float64.

    The format of the OCP 8-bit floating-point specification, E4M3 variant:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
    encodes subnormals 2^-6 * m/8; the all-ones pattern S.1111.111 is NaN and
    there is no infinity, so the largest value is 2^8 * 1.75 = 448. The pages
    name FP8 KV caches only as a feature FlashInfer's cascade lacked ([p2]
    section 6); the caches here are dequantised as code value * scale.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 7) == 7), np.nan, out)
