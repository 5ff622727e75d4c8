"""Seeded random batches through every plan option at once: shapes (request
count, shared prefix, ragged suffixes and query lengths, head layout,
head_dim), fp8 caches, nested groups, and the planner's overrides (mode,
prefix splits, heads per item, shared levels, partial-state dtype, dispatch
order), with sliding windows on the non-cascade path and attention sinks.
Every output row is checked against the oracle."""

import numpy as np
import pytest
import torch

import workloads
from workloads import Workload
from parity_util import DeviceBatch, assert_close, log, oracle_ref, rows_of, run

pytestmark = pytest.mark.gpu

HEADS = [(4, 4), (8, 2), (16, 2), (32, 8), (8, 8), (16, 4)]


def setup_module():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(i):
    rng = np.random.default_rng(7000 + i)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = 64 if rng.random() < 0.3 else 128
    fp8 = d == 128 and rng.random() < 0.3
    n = int(rng.integers(1, 25))
    prefix = int(rng.choice([0, 16, 240, 256, 512, 1000, 1024]))
    q_hi = int(rng.choice([1, 1, 4, 24]))
    s_lo = max(q_hi, int(rng.integers(1, 60)))
    s_hi = s_lo + int(rng.integers(0, 300))
    groups = ()
    if prefix % 16 == 0 and prefix > 0 and n >= 4 and rng.random() < 0.35:
        groups = ((int(rng.integers(2, n // 2 + 1)), int(rng.choice([256, 400, 640]))),)
    w = Workload(f"random_{i}", n, prefix, (s_lo, s_hi), (1, q_hi), hq, hkv, d, seed=7000 + i, groups=groups,
                 kv_dtype="fp8" if fp8 else "bf16", k_scale=0.125 if fp8 else 1.0, v_scale=0.0625 if fp8 else 1.0,
                 outlier_frac=0.01 if rng.random() < 0.2 else 0.0, outlier_scale=8.0)
    mode = str(rng.choice(["auto", "on", "on", "off"]))
    kw = dict(mode=mode,
              prefix_splits=int(rng.choice([0, 0, 1, 3, 8])),
              heads_per_item=int(rng.choice([0, 0, 1] + ([2] if hkv % 2 == 0 else []))),
              max_levels=int(rng.choice([0, 1])),
              partials_fp32=bool(rng.random() < 0.3),
              suffix_order=int(rng.random() < 0.3))
    window = 0
    if mode != "on" and rng.random() < 0.25:
        window = int(rng.integers(1, 400))
    sinks = None
    if rng.random() < 0.25:
        sinks = rng.normal(0.0, 2.0, size=hq).astype(np.float32)
    return w, kw, window, sinks


@pytest.mark.parametrize("i", range(40))
def test_random_batches(i):
    w, kw, window, sinks = _case(i)
    log(f"[random {i}] N={w.num_reqs} P={w.prefix} S={w.suffix} q={w.q_len} heads={w.num_q_heads}/{w.num_kv_heads} "
        f"d={w.head_dim} {w.kv_dtype} groups={w.groups} W={window} sinks={sinks is not None} {kw}")
    b = workloads.make_batch(w)
    if kw["mode"] == "on" and int(b.num_computed.min()) < 16:
        kw["mode"] = "auto"            # nothing is shared: a forced cascade plan has no prefix to run
    ref_o, ref_l = oracle_ref(b, window=window, sinks=sinks)
    out, lse, info = run(DeviceBatch(b), sinks=sinks, sliding_window=window, **kw)
    log(f"  plan: cascade={info['use_cascade']} P_c={info['common_prefix_len']} psplit={info['prefix_splits']} "
        f"groups={info['num_level1_groups']} schunks={info['suffix_chunks']} heads={info['suffix_heads_per_item']} "
        f"slots={info['num_partial_slots']} fp32={info['partials_fp32']} order={info['suffix_longest_first']}")
    assert_close(out, lse, ref_o, ref_l, what=f"random {i}")


def _random_docs(rng, n, ps):
    """A random prefix tree of documents over requests [0, n): disjoint
    sibling sets of >= 2 members, up to three levels, members scattered over
    the batch; documents with children fill whole pages."""
    docs = []

    def node(members, depth):
        kids = []
        pool = [int(x) for x in rng.permutation(members)]
        if depth < 3 and len(pool) >= 4:
            for _ in range(int(rng.integers(0, 3))):
                if len(pool) < 2:
                    break
                size = int(rng.integers(2, max(3, len(pool) // 2 + 1)))
                kids.append(sorted(pool[:size]))
                pool = pool[size:]
        tokens = int(rng.choice([256, 512])) if kids else int(rng.choice([40, 100, 256, 300, 640]))
        docs.append((tuple(sorted(members)), tokens))
        for k in kids:
            node(k, depth + 1)

    pool = [int(x) for x in rng.permutation(n)]
    for _ in range(int(rng.integers(1, 4))):
        if len(pool) < 2:
            break
        size = int(rng.integers(2, max(3, len(pool) // 2 + 1)))
        node(pool[:size], 1)
        pool = pool[size:]
    return tuple(docs)


def _tree_case(i):
    rng = np.random.default_rng(9000 + i)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = 64 if rng.random() < 0.3 else 128
    fp8 = d == 128 and rng.random() < 0.3
    n = int(rng.integers(4, 25))
    prefix = int(rng.choice([256, 512, 512]))
    q_hi = int(rng.choice([1, 1, 3, 8]))
    s_lo = max(q_hi, int(rng.integers(1, 40)))
    s_hi = s_lo + int(rng.integers(0, 200))
    docs = _random_docs(rng, n, 16)
    w = Workload(f"random_tree_{i}", n, prefix, (s_lo, s_hi), (1, q_hi), hq, hkv, d, seed=9000 + i, docs=docs,
                 kv_dtype="fp8" if fp8 else "bf16", k_scale=0.125 if fp8 else 1.0, v_scale=0.0625 if fp8 else 1.0)
    kw = dict(mode=str(rng.choice(["auto", "on", "on"])),
              max_levels=int(rng.integers(0, 5)),
              merge_mode=int(rng.integers(0, 3)),
              separate_phases=bool(rng.random() < 0.3),
              prefix_splits=int(rng.choice([0, 0, 2])),
              partials_fp32=bool(rng.random() < 0.2))
    return w, kw


@pytest.mark.parametrize("i", range(16))
def test_random_tree_batches(i):
    """Random prefix trees of documents (members scattered over the batch, up
    to three levels below the batch-wide prefix, some requests in none),
    with every shared-level limit, merge placement and phase split: every
    output row against the oracle."""
    w, kw = _tree_case(i)
    log(f"[random tree {i}] N={w.num_reqs} P={w.prefix} S={w.suffix} q={w.q_len} "
        f"heads={w.num_q_heads}/{w.num_kv_heads} d={w.head_dim} {w.kv_dtype} docs={w.docs} {kw}")
    b = workloads.make_batch(w)
    if kw["mode"] == "on" and int(b.num_computed.min()) < 16:
        kw["mode"] = "auto"            # nothing is shared by the whole batch
    ref_o, ref_l = oracle_ref(b)
    out, lse, info = run(DeviceBatch(b), **kw)
    log(f"  plan: cascade={info['use_cascade']} P_c={info['common_prefix_len']} levels={info['shared_levels']} "
        f"groups={info['num_level1_groups']} merge_in_launch={info['merge_in_launch']} "
        f"slots={info['num_partial_slots']}")
    assert_close(out, lse, ref_o, ref_l, what=f"random tree {i}")


def _large_case(i):
    rng = np.random.default_rng(9500 + i)
    hq, hkv = [(32, 8), (64, 8), (16, 2)][int(rng.integers(3))]
    fp8 = rng.random() < 0.3
    n = int(rng.integers(64, 301))
    prefix = int(rng.choice([1024, 2048, 4096, 8192]))
    q_hi = int(rng.choice([1, 1, 4, 16]))
    s_lo = max(q_hi, int(rng.integers(1, 200)))
    s_hi = s_lo + int(rng.integers(0, 1500))
    w = Workload(f"random_large_{i}", n, prefix, (s_lo, s_hi), (1, q_hi), hq, hkv, 128, seed=9500 + i,
                 kv_dtype="fp8" if fp8 else "bf16", k_scale=0.125 if fp8 else 1.0, v_scale=0.0625 if fp8 else 1.0,
                 outlier_frac=0.01 if rng.random() < 0.3 else 0.0, outlier_scale=8.0)
    return w, str(rng.choice(["auto", "on", "off"]))


@pytest.mark.parametrize("i", range(6))
def test_random_large_batches(i):
    """Larger random batches (64-300 requests, 1k-8k shared tokens, suffixes up
    to ~1,700 tokens, up to 16 queries per request, 16-64 query heads, fp8 in
    some): every row of eight requests (first, last, shortest, longest and
    four random ones) against the oracle."""
    w, mode = _large_case(i)
    log(f"[random large {i}] N={w.num_reqs} P={w.prefix} S={w.suffix} q={w.q_len} "
        f"heads={w.num_q_heads}/{w.num_kv_heads} {w.kv_dtype} mode={mode}")
    b = workloads.make_batch(w)
    seq = b.seq_lens.numpy()
    rng = np.random.default_rng(9600 + i)
    reqs = sorted({0, w.num_reqs - 1, int(seq.argmin()), int(seq.argmax())}
                  | {int(x) for x in rng.choice(w.num_reqs, 4, replace=False)})
    ref_o, ref_l = oracle_ref(b, requests=reqs)
    out, lse, info = run(DeviceBatch(b), mode=mode)
    log(f"  plan: cascade={info['use_cascade']} psplit={info['prefix_splits']} row tile={info['prefix_row_tile']} "
        f"schunks={info['suffix_chunks']} heads={info['suffix_heads_per_item']} requests={reqs}")
    assert_close(out, lse, ref_o, ref_l, rows=rows_of(b, reqs), what=f"random large {i}")
