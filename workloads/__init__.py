"""Seeded synthetic batches for shared-prefix attention (inputs only).

This module builds inputs -- query tensors, a paged bf16 KV cache, block
tables and per-request lengths -- for both the HIP library and the oracle.
It holds none of the method's arithmetic: it never computes a common prefix,
a cascade decision, a softmax or a merge.

Batch structure (the shapes of the workloads the pages discuss: many requests
behind one shared system prompt or document, each with its own continuation):

* every request's KV sequence is the shared prefix (P tokens, identical
  values) followed by its own tokens; ``seq_len = P + S_r`` and the last
  ``q_len_r`` positions are this step's query tokens, so
  ``num_computed = seq_len - q_len``;
* the ``P // page_size`` full prefix pages are physically shared (the same
  page ids in every block-table row); a partial last prefix page is copied
  into each request's own first page (same values), since only whole pages
  can be shared;
* physical page ids are a seeded permutation of the pool; ~5 % spare pages;
* spare pages and the unused tail slots of each request's last page hold
  bf16 NaN, so any read outside a request's KV range poisons the result;
* block-table padding columns hold random *valid* page ids;
* Q, K, V ~ N(0, 1) in fp32, optionally with a Bernoulli outlier mask scaled
  by a factor, then rounded to bf16.
* fp8 caches (``kv_dtype="fp8"``): K / V are stored as fp8 e4m3 codes (uint8)
  of value / k_scale and value / v_scale (clamped to +-448, rounded to
  nearest by torch's float8_e4m3fn cast); the poison is the NaN code 0x7f.

Nested sharing (``groups``): consecutive runs of requests additionally share
a document of L_g tokens after the batch-wide prefix (system prompt ->
document -> own tokens). Members get ``seq_len = P + L_g + S_r``; the
document's full pages are physically shared by the members and a partial
last document page is copied into each member's own first page.

Documents in a tree (``docs``): any sets of requests, not only consecutive
ones, each sharing a document after the prefix and after the documents of
every earlier-listed set that contains it (the sets must nest or be
disjoint: system prompt -> document -> chapter -> own tokens). A request's
sequence is the prefix, its documents outermost first, then its own tokens.
Documents that contain others must fill whole pages; the innermost may end
in a partial page, which is copied into each member's own first page.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_reqs: int
    prefix: int                      # shared prefix tokens P
    suffix: Tuple[int, int]          # S_r ~ U[lo, hi] inclusive (includes the queries)
    q_len: Tuple[int, int]           # q_r ~ U[lo, hi] inclusive
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 16
    seed: int = 0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    # request index -> (seq_len, q_len), applied after the random draws
    override: Tuple[Tuple[int, int, int], ...] = ()
    extra_stride: int = 1            # padding columns in the block table
    # (members, shared tokens): runs of consecutive requests from request 0
    # that share a document after the prefix; remaining requests share none
    groups: Tuple[Tuple[int, int], ...] = ()
    # (member request indices, shared tokens): documents of a prefix tree, outer
    # documents first; the member sets nest or are disjoint
    docs: Tuple[Tuple[Tuple[int, ...], int], ...] = ()
    kv_dtype: str = "bf16"           # "bf16" or "fp8" (e4m3 codes, dequantised by the scales)
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def _w(name, n, p, s, q, hq, hkv, d, seed, **kw) -> Workload:
    return Workload(name=name, num_reqs=n, prefix=p, suffix=s, q_len=q,
                    num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seed=seed, **kw)


# The five workloads: tiny decode; the pages' worked example (N=64, P=4096,
# S=128); mixed chunked prefill; many-sample self-consistency decode; long
# shared document (+ at the 8-request threshold, + with a 255-token prefix).
# Then two batches with nested sharing (system prompt -> document ->
# request): decode and chunked prefill, some requests in no group. Then the
# worked example and the prefill mix with fp8 e4m3 caches.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        _w("tiny_decode", 8, 256, (16, 16), (1, 1), 4, 4, 64, 1000),
        _w("worked_decode", 64, 4096, (128, 128), (1, 1), 32, 8, 128, 1001),
        _w("mixed_prefill", 32, 2048, (64, 512), (1, 64), 32, 8, 128, 1002),
        # request 0 has computed only 2040 tokens and brings 40 queries, so
        # the minimum num_computed (2040) is below the shared pages (2048).
        _w("mixed_prefill_capped", 32, 2048, (64, 512), (1, 64), 32, 8, 128, 1012,
           override=((0, 2080, 40),)),
        _w("self_consistency", 256, 8192, (1, 1024), (1, 1), 64, 8, 128, 1003,
           outlier_frac=0.01, outlier_scale=8.0),
        _w("long_doc", 16, 32768, (256, 256), (1, 1), 32, 8, 128, 1004),
        _w("long_doc_n8", 8, 32768, (256, 256), (1, 1), 32, 8, 128, 1014),
        _w("long_doc_p255", 16, 255, (256, 256), (1, 1), 32, 8, 128, 1024),
        _w("multi_doc", 32, 1024, (32, 160), (1, 1), 32, 8, 128, 1005,
           groups=((8, 2048), (8, 2048), (6, 3072), (6, 1000))),
        _w("multi_doc_prefill", 24, 512, (32, 200), (1, 24), 32, 8, 128, 1006,
           groups=((6, 1024), (6, 768), (4, 2000))),
        _w("worked_decode_fp8", 64, 4096, (128, 128), (1, 1), 32, 8, 128, 1007,
           kv_dtype="fp8", k_scale=0.125, v_scale=0.0625),
        _w("mixed_prefill_fp8", 32, 2048, (64, 512), (1, 64), 32, 8, 128, 1008,
           kv_dtype="fp8", k_scale=0.125, v_scale=0.0625),
        _w("self_consistency_fp8", 256, 8192, (1, 1024), (1, 1), 64, 8, 128, 1009,
           outlier_frac=0.01, outlier_scale=8.0, kv_dtype="fp8", k_scale=0.125, v_scale=0.0625),
    ]
}


@dataclasses.dataclass
class Batch:
    workload: Workload
    q: torch.Tensor                  # [T, Hq, d] bf16
    k_cache: torch.Tensor            # [num_pages, page_size, Hkv, d] bf16, or uint8 fp8 codes
    v_cache: torch.Tensor            # [num_pages, page_size, Hkv, d] bf16, or uint8 fp8 codes
    block_table: torch.Tensor        # [N, stride] int32
    query_start_loc: torch.Tensor    # [N+1] int32
    seq_lens: torch.Tensor           # [N] int32
    num_computed: torch.Tensor       # [N] int32

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])


def _randn(shape, gen, frac, scale):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if frac > 0.0:
        mask = torch.rand(shape, generator=gen) < frac
        x = torch.where(mask, x * scale, x)
    return x.to(torch.bfloat16)


def make_batch(w: Workload, seed: Optional[int] = None) -> Batch:
    """Build the seeded synthetic batch for workload ``w`` (CPU tensors)."""
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    n, ps, hkv, d = w.num_reqs, w.page_size, w.num_kv_heads, w.head_dim
    s_lo, s_hi = w.suffix
    q_lo, q_hi = w.q_len
    suffix = torch.randint(s_lo, s_hi + 1, (n,), generator=gen)
    qlen = torch.randint(q_lo, q_hi + 1, (n,), generator=gen)
    qlen = torch.minimum(qlen, suffix)
    # documents: the consecutive runs of `groups`, then the tree of `docs`
    docs = []
    r = 0
    for members, tokens in w.groups:
        docs.append((tuple(range(r, r + members)), tokens))
        r += members
    assert r <= n
    docs += [(tuple(m), t) for m, t in w.docs]
    chain = [[] for _ in range(n)]     # documents of each request, outermost first
    for di, (members, _) in enumerate(docs):
        for m in members:
            if chain[m]:   # nested: the enclosing document holds every member of this one
                assert set(members) <= set(docs[chain[m][-1]][0]), "document sets must nest or be disjoint"
            chain[m].append(di)
    assert not docs or w.prefix % ps == 0
    for r in range(n):
        for di in chain[r][:-1]:
            assert docs[di][1] % ps == 0, "a document that contains others must fill whole pages"
    doc_tokens = [sum(docs[di][1] for di in chain[r]) for r in range(n)]
    doc = torch.tensor(doc_tokens, dtype=suffix.dtype)
    seq = suffix + w.prefix + doc
    for r, sl, ql in w.override:
        seq[r] = sl
        qlen[r] = ql
    seq_l = [int(x) for x in seq]
    q_l = [int(x) for x in qlen]

    shared_pages = w.prefix // ps
    doc_pages = [t // ps for _, t in docs]          # full document pages, shared by the members
    lead = [shared_pages + sum(doc_pages[di] for di in chain[r]) for r in range(n)]   # shared columns
    own_pages = [-(-s // ps) - lead[r] for r, s in enumerate(seq_l)]
    used = shared_pages + sum(doc_pages) + sum(own_pages)
    num_pages = used + max(1, int(math.ceil(0.05 * used)))
    perm = torch.randperm(num_pages, generator=gen)
    shared_ids = perm[:shared_pages]
    pos = shared_pages
    doc_ids = []
    for k in doc_pages:
        doc_ids.append(perm[pos:pos + k])
        pos += k
    own_ids = []
    for k in own_pages:
        own_ids.append(perm[pos:pos + k])
        pos += k

    stride = max(-(-s // ps) for s in seq_l) + w.extra_stride
    block_table = torch.randint(0, num_pages, (n, stride), generator=gen, dtype=torch.int64)
    for r in range(n):
        block_table[r, :shared_pages] = shared_ids
        col = shared_pages
        for di in chain[r]:
            block_table[r, col:col + doc_pages[di]] = doc_ids[di]
            col += doc_pages[di]
        block_table[r, lead[r]:lead[r] + own_pages[r]] = own_ids[r]

    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    caches = []
    for _ in range(2):                                   # K then V (values; fp8 codes below)
        cache = torch.full((num_pages, ps, hkv, d), nan.item(), dtype=torch.bfloat16)
        prefix_vals = _randn((w.prefix, hkv, d), gen, w.outlier_frac, w.outlier_scale)
        if shared_pages:
            cache[shared_ids] = prefix_vals[:shared_pages * ps].reshape(shared_pages, ps, hkv, d)
        doc_vals = []
        for di, (_, L) in enumerate(docs):
            vals = _randn((L, hkv, d), gen, w.outlier_frac, w.outlier_scale)
            if doc_pages[di]:
                cache[doc_ids[di]] = vals[:doc_pages[di] * ps].reshape(doc_pages[di], ps, hkv, d)
            doc_vals.append(vals)
        for r in range(n):
            start = lead[r] * ps
            n_tok = seq_l[r] - start
            if n_tok <= 0:
                continue
            own_vals = _randn((n_tok, hkv, d), gen, w.outlier_frac, w.outlier_scale)
            t = torch.arange(start, seq_l[r])
            in_prefix = t < w.prefix
            if bool(in_prefix.any()):
                own_vals[in_prefix] = prefix_vals[t[in_prefix]]
            if chain[r]:   # the partial last page of the innermost document
                leaf = chain[r][-1]
                d0 = w.prefix + sum(docs[di][1] for di in chain[r][:-1])
                in_doc = (t >= d0) & (t < d0 + docs[leaf][1])
                if bool(in_doc.any()):
                    own_vals[in_doc] = doc_vals[leaf][t[in_doc] - d0]
            pages = own_ids[r][(t - start) // ps]
            cache[pages, t % ps] = own_vals
        caches.append(cache)

    if w.kv_dtype == "fp8":
        def codes(cache, scale):
            x = cache.float() / scale
            x = torch.where(torch.isnan(x), x, x.clamp(-448.0, 448.0))
            return x.to(torch.float8_e4m3fn).view(torch.uint8)
        caches = [codes(caches[0], w.k_scale), codes(caches[1], w.v_scale)]
    total_q = sum(q_l)
    q = _randn((total_q, w.num_q_heads, d), gen, w.outlier_frac, w.outlier_scale)
    qsl = torch.zeros(n + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(q_l), 0).to(torch.int32)
    seq_t = torch.tensor(seq_l, dtype=torch.int32)
    return Batch(
        workload=w, q=q, k_cache=caches[0], v_cache=caches[1],
        block_table=block_table.to(torch.int32), query_start_loc=qsl,
        seq_lens=seq_t, num_computed=seq_t - torch.tensor(q_l, dtype=torch.int32),
    )


def get(name: str) -> Workload:
    return WORKLOADS[name]
