"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and its host planner agrees with the oracle's definitions (no kernel runs)."""

import ctypes
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import shared_prefix_attention_amd as spa
from shared_prefix_attention_amd import _lib


@pytest.fixture(scope="module", autouse=True)
def _library_built():
    """A checkout without the built library builds it here (host compile
    only) rather than skipping the boundary and planner tests."""
    if not os.path.exists(_lib.LIB_PATH):
        from shared_prefix_attention_amd.build import build
        build()


def test_library_exports_every_header_symbol():
    lib = spa.load()
    names = _lib.header_symbols()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
        ctypes.cast(getattr(lib, n), ctypes.c_void_p)


def _plan(b, mode="auto", **kw):
    w = b.workload
    return spa.plan_batch(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                          k_cache=b.k_cache, block_table=b.block_table, query_start_loc=b.query_start_loc,
                          seq_lens=b.seq_lens, num_computed_tokens=b.num_computed, mode=mode,
                          num_cus=256, **kw)


def test_detector_matches_oracle_on_random_tables():
    rng = np.random.default_rng(40)
    for _ in range(3000):
        n = int(rng.integers(1, 5))
        cols = int(rng.integers(1, 6))
        ps = int(rng.integers(1, 5))
        base = rng.integers(0, 3, cols)
        bt = np.tile(base, (n, 1))
        # perturb a few entries so rows diverge at random columns
        for _ in range(int(rng.integers(0, 4))):
            bt[rng.integers(0, n), rng.integers(0, cols)] = rng.integers(0, 3)
        lens = rng.integers(1, cols * ps + 1, n)
        got = spa.cascade_attn_num_common_prefix_blocks(bt, lens, ps)
        assert got == oracle.common_prefix_blocks(bt.tolist(), lens.tolist(), ps)


def test_detector_r1_r2_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "r1r2_example.json")))
    tok = ex["tokens"]
    bt = [[tok[x] for x in row] for row in ex["block_table"]]
    assert spa.cascade_attn_num_common_prefix_blocks(bt, ex["seq_lens"], ex["page_size"]) == \
        ex["expected_common_blocks"]


def test_plan_r1_r2_example_scaled_to_pages(golden_dir):
    """The section-4 example with every token of it scaled to one 16-token page:
    shared pages A..E, R1 computed 3 pages, R2 computed 4 -> prefix 3 pages."""
    ex = json.load(open(os.path.join(golden_dir, "r1r2_example.json")))
    tok = ex["tokens"]
    bt = np.array([[tok[x] for x in row] for row in ex["block_table"]], dtype=np.int32)
    ps = 16
    seq = np.array(ex["seq_lens"]) * ps
    nc = np.array(ex["num_computed_tokens"]) * ps
    qsl = np.concatenate([[0], np.cumsum(seq - nc)])
    pl = spa.cascade_attn_plan(num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=ps, num_pages=7,
                               kv_strides=(ps * 64, 64, 64), block_table=bt, query_start_loc=qsl,
                               seq_lens=seq, num_computed_tokens=nc, mode="on", num_cus=256)
    assert pl.info["num_common_prefix_blocks"] == ex["expected_common_blocks"]
    assert pl.info["common_prefix_len"] == ex["expected_prefix_len"] * ps
    assert pl.info["use_cascade"] == 1


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_plan_matches_oracle_on_workloads(name):
    b = workloads.make_batch(workloads.get(name))
    pl = _plan(b)
    info = pl.info
    ps = b.workload.page_size
    blocks = oracle.common_prefix_blocks(b.block_table.tolist(), b.seq_lens.tolist(), ps)
    plen = oracle.cascade_prefix_len(blocks, ps, b.num_computed.tolist())
    assert info["num_common_prefix_blocks"] == blocks
    assert info["common_prefix_len"] == plen
    assert info["gates_pass"] == int(oracle.passes_cascade_gates(plen, b.workload.num_reqs))
    assert info["kv_tokens_noncascade"] == oracle.kv_tokens_standard(b.seq_lens.tolist())
    groups = oracle.tree_groups(b.block_table.tolist(), b.seq_lens.tolist(), b.num_computed.tolist(), ps, plen)
    assert info["kv_tokens_cascade"] == oracle.kv_tokens_tree(plen, groups, b.seq_lens.tolist())
    if not groups:
        assert info["kv_tokens_cascade"] == oracle.kv_tokens_cascade(plen, b.seq_lens.tolist())
    assert info["total_q"] == b.total_q
    if plen > 0:
        assert _tree_of(_plan(b, mode="on")) == groups
    if plen < 256 or b.workload.num_reqs < 2:   # AUTO's gate
        assert info["use_cascade"] == 0
    on = _plan(b, mode="on").info
    off = _plan(b, mode="off").info
    assert on["use_cascade"] == int(plen > 0)
    assert off["use_cascade"] == 0


def test_expected_prefix_lengths_of_the_workloads():
    expect = {"tiny_decode": 256, "worked_decode": 4096, "mixed_prefill": 2048,
              "mixed_prefill_capped": 2032, "self_consistency": 8192, "long_doc": 32768,
              "long_doc_n8": 32768, "long_doc_p255": 240}
    for name, plen in expect.items():
        b = workloads.make_batch(workloads.get(name))
        assert _plan(b).info["common_prefix_len"] == plen, name


def test_auto_decisions_at_the_gates():
    # P=255 -> 240 shared tokens: below 256, AUTO must fall back
    assert _plan(workloads.make_batch(workloads.get("long_doc_p255"))).info["use_cascade"] == 0
    # N = 8 with a 32768-token document: at the threshold, gates pass
    info = _plan(workloads.make_batch(workloads.get("long_doc_n8"))).info
    assert info["gates_pass"] == 1
    # the pages' worked example: cascade
    assert _plan(workloads.make_batch(workloads.get("worked_decode"))).info["use_cascade"] == 1


def test_worked_example_accounting_through_the_planner(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    b = workloads.make_batch(workloads.get("worked_decode"))
    info = _plan(b).info
    assert info["kv_tokens_noncascade"] == ex["kv_tokens_standard"]
    assert info["kv_tokens_cascade"] == ex["kv_tokens_cascade"]


def test_seven_requests_fail_the_pages_gate():
    """Seven requests fail the pages' request gate (reported in gates_pass);
    AUTO's own gate (two or more requests) passes, and its cost model
    decides."""
    w = workloads.Workload("seven", 7, 1024, (32, 32), (1, 1), 8, 2, 64, seed=5)
    b = workloads.make_batch(w)
    info = _plan(b).info
    assert info["common_prefix_len"] == 1024 and info["gates_pass"] == 0
    assert info["use_cascade"] == int(info["est_us_cascade"] < info["est_us_noncascade"])


def test_one_request_never_takes_the_cascade_path():
    """A single request shares with nobody: AUTO keeps the non-cascade path
    whatever the prefix (forcing the cascade still runs it)."""
    w = workloads.Workload("one", 1, 4096, (16, 16), (1, 1), 32, 8, 128, seed=5)
    b = workloads.make_batch(w)
    assert _plan(b).info["use_cascade"] == 0
    assert _plan(b, mode="on").info["use_cascade"] == 1


def _meta(n=3, seq=40, q=2, stride=4):
    bt = np.arange(n * stride, dtype=np.int32).reshape(n, stride)
    qsl = np.arange(n + 1, dtype=np.int32) * q
    sl = np.full(n, seq, dtype=np.int32)
    return bt, qsl, sl


def _try(**kw):
    bt, qsl, sl = _meta()
    args = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, num_pages=64,
                kv_strides=(16 * 2 * 64, 2 * 64, 64), block_table=bt, query_start_loc=qsl, seq_lens=sl,
                num_cus=256)
    args.update(kw)
    return spa.cascade_attn_plan(**args)


def test_error_codes():
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(head_dim=96)
    assert e.value.status == _lib.CA_EUNSUPPORTED
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(page_size=8)
    assert e.value.status == _lib.CA_EUNSUPPORTED
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(num_q_heads=6, num_kv_heads=4)
    assert e.value.status == _lib.CA_EUNSUPPORTED
    bt, qsl, sl = _meta()
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(num_computed_tokens=sl - 1)          # q_len is 2, not 1
    assert e.value.status == _lib.CA_EMETA
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(num_pages=5)                          # page ids up to 11 referenced
    assert e.value.status == _lib.CA_EMETA
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(seq_lens=np.full(3, 80, dtype=np.int32))   # needs 5 pages, stride 4
    assert e.value.status == _lib.CA_EMETA
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(query_start_loc=np.array([0, 2, 2, 4], dtype=np.int32))   # empty request
    assert e.value.status == _lib.CA_EMETA
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(kv_strides=(16 * 2 * 64, 2 * 64, 60))
    assert e.value.status == _lib.CA_EUNSUPPORTED
    assert "stride" in _lib.load().cascade_attn_last_error().decode()
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(heads_per_item=3)                     # must divide num_kv_heads (2)
    assert e.value.status == _lib.CA_EINVAL
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(heads_per_item=-1)
    assert e.value.status == _lib.CA_EINVAL
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(separate_phases=2)
    assert e.value.status == _lib.CA_EINVAL
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(max_levels=5)
    assert e.value.status == _lib.CA_EINVAL
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(kv_dtype=2)
    assert e.value.status == _lib.CA_EINVAL
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(kv_dtype="fp8")                       # head_dim 64
    assert e.value.status == _lib.CA_EUNSUPPORTED
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(kv_dtype="fp8", head_dim=128, kv_strides=(16 * 2 * 128, 2 * 128, 120))
    assert e.value.status == _lib.CA_EUNSUPPORTED
    with pytest.raises(spa.CascadeAttnError) as e:
        _try(kv_dtype="fp8", head_dim=128, kv_strides=(16 * 2 * 128, 2 * 128, 128), k_scale=float("nan"))
    assert e.value.status == _lib.CA_EINVAL


def test_plan_partition_is_consistent():
    for name in workloads.WORKLOADS:
        b = workloads.make_batch(workloads.get(name))
        for mode in ("on", "off"):
            info = _plan(b, mode=mode).info
            T, hq, d = b.q.shape
            slots = info["num_partial_slots"]
            assert info["partials_fp32"] == 0
            assert info["workspace_bytes"] >= slots * T * hq * (d * 2 + 4)
            # fp32 partials (the cost model prices their bytes, so the split count may differ)
            wide = _plan(b, mode=mode, partials_fp32=True).info
            assert wide["partials_fp32"] == 1
            assert wide["workspace_bytes"] >= wide["num_partial_slots"] * T * hq * (d + 1) * 4
            if info["use_cascade"]:
                if info["shared_levels"] <= 2:
                    assert slots == info["prefix_splits"] + info["level1_splits"] + info["suffix_chunks"]
                else:
                    assert slots > info["prefix_splits"] + info["level1_splits"] + info["suffix_chunks"]
                assert (info["level1_splits"] > 0) == (info["num_level1_groups"] > 0)
                assert (info["shared_levels"] > 1) == (info["num_level1_groups"] > 0)
                assert info["prefix_splits"] >= 1
            assert info["suffix_chunk_tokens"] % 64 == 0
            assert 0 < info["suffix_chunk_tokens"] <= 8192
            assert info["suffix_stages"] in (2, 4)
            h = info["suffix_heads_per_item"]
            assert h >= 1 and b.workload.num_kv_heads % h == 0
            if info["suffix_kernel"] != 1:
                assert h == 1


def test_heads_per_item_choice_and_override():
    """Auto grouping for the worked example (two heads per decode item keeps
    the launch within two work-groups per CU); the explicit setting is
    reported as given and ignored for items of more than 16 rows."""
    wd = workloads.make_batch(workloads.get("worked_decode"))
    assert _plan(wd, mode="on").info["suffix_heads_per_item"] == 2
    assert _plan(wd, mode="off").info["suffix_heads_per_item"] == 1
    assert _plan(wd, mode="on", heads_per_item=8).info["suffix_heads_per_item"] == 8
    mp = workloads.make_batch(workloads.get("mixed_prefill"))
    assert _plan(mp, mode="on", heads_per_item=2).info["suffix_heads_per_item"] == 1
    # 2,048 one-head decode items need four rounds of two work-groups per CU:
    # two heads per item; fp8 plans keep one
    sc = workloads.make_batch(workloads.get("self_consistency"))
    assert _plan(sc, mode="on").info["suffix_heads_per_item"] == 2
    sc8 = workloads.make_batch(workloads.get("self_consistency_fp8"))
    assert _plan(sc8, mode="on").info["suffix_heads_per_item"] == 1
    # the long document's 64 items per head fit one round with two heads per item
    ld = workloads.make_batch(workloads.get("long_doc"))
    assert _plan(ld, mode="on").info["suffix_heads_per_item"] == 2


def test_separate_phases_changes_only_the_launch_count():
    """Asking for the cascade phases as two launches (which then need the
    merge as a launch of its own) leaves the partition as it was; a
    non-cascade plan ignores it. merge_mode=1 keeps one attention launch but
    moves the merge to a launch of its own, the partition again unchanged."""
    wd = workloads.make_batch(workloads.get("worked_decode"))
    fused, split = _plan(wd, mode="on").info, _plan(wd, mode="on", separate_phases=1).info
    sep_merge = _plan(wd, mode="on", merge_mode=1).info
    in_launch = _plan(wd, mode="on", merge_mode=2).info
    assert fused["separate_phases"] == 0 and split["separate_phases"] == 1
    assert in_launch["merge_in_launch"] == 1 and split["merge_in_launch"] == 0 and sep_merge["merge_in_launch"] == 0
    assert _plan(wd, mode="on", separate_phases=1, merge_mode=2).info["merge_in_launch"] == 0
    launch_only = ("separate_phases", "merge_in_launch", "est_us_cascade")
    assert {k: v for k, v in fused.items() if k not in launch_only} == \
        {k: v for k, v in split.items() if k not in launch_only}
    assert {k: v for k, v in fused.items() if k not in launch_only} == \
        {k: v for k, v in sep_merge.items() if k not in launch_only}
    assert {k: v for k, v in fused.items() if k not in launch_only} == \
        {k: v for k, v in in_launch.items() if k not in launch_only}
    assert _plan(wd, mode="off", separate_phases=1).info["separate_phases"] == 0
    with pytest.raises(spa.CascadeAttnError) as e:
        _plan(wd, mode="on", merge_mode=3)
    assert e.value.status == _lib.CA_EINVAL


def test_workspace_layout_reserves_the_merge_counters():
    """Every plan with partial states reserves the merge counters at the
    workspace's start, whatever its merge mode; direct plans need none."""
    for name, mode in (("worked_decode", "on"), ("mixed_prefill", "on"), ("long_doc_n8", "off"),
                       ("self_consistency", "off")):
        b = workloads.make_batch(workloads.get(name))
        for mm in (1, 2):
            info = _plan(b, mode=mode, merge_mode=mm).info
            w = b.workload
            T = int(b.total_q)
            slots = info["num_partial_slots"]
            assert slots > 0
            o = -(-slots * T * w.num_q_heads * w.head_dim * 2 // 256) * 256
            l = -(-slots * T * w.num_q_heads * 4 // 256) * 256
            assert info["workspace_bytes"] == _lib.WORKSPACE_COUNTER_BYTES + o + l
            assert info["merge_in_launch"] == (mm - 1)
    tiny = _plan(workloads.make_batch(workloads.get("tiny_decode")), mode="off").info
    assert tiny["num_partial_slots"] == 0 and tiny["workspace_bytes"] == 0 and tiny["merge_in_launch"] == 0


def test_auto_takes_the_measured_faster_path():
    """AUTO's cost model (constants fitted to this library's kernels on
    MI355X) picks, for each workload, the path that measured faster when both
    were timed on the device: cascade for the worked example, the mixed and
    capped prefill batches, self-consistency and both long-document batches;
    non-cascade where the gates fail (255-token prefix) or the two paths tie
    (the tiny batch)."""
    expect = {"worked_decode": 1, "mixed_prefill": 1, "mixed_prefill_capped": 1, "self_consistency": 1,
              "long_doc": 1, "long_doc_n8": 1, "long_doc_p255": 0}
    for name, casc in expect.items():
        b = workloads.make_batch(workloads.get(name))
        assert _plan(b, mode="auto").info["use_cascade"] == casc, name


# Shapes of the device decision sweep (seed 7; decode shapes one query
# token) where one path was faster in every run of the sweep, by 15 % or more
# in at least one (µs per step in the latest run, cascade / non-cascade):
# (name, N, P, suffix range, query range, cascade?). 32 / 8 heads,
# head_dim 128, bf16:
SWEEP_CLEAR = [
    ("decode_n2_p4096_s16", 2, 4096, (16, 16), (1, 1), 1),        # 14.4 / 18.5
    ("decode_n4_p1024_s16", 4, 1024, (16, 16), (1, 1), 1),        # 15.0 / 15.8
    ("decode_n4_p4096_s512", 4, 4096, (512, 512), (1, 1), 1),     # 15.4 / 23.6
    ("decode_n8_p256_s16", 8, 256, (16, 16), (1, 1), 0),          # 12.2 / 10.5
    ("decode_n8_p1024_s16", 8, 1024, (16, 16), (1, 1), 1),        # 15.2 / 17.2
    ("decode_n16_p4096_s16", 16, 4096, (16, 16), (1, 1), 1),      # 15.5 / 27.6
    ("decode_n64_p256_s16", 64, 256, (16, 16), (1, 1), 0),        # 15.2 / 15.0
    ("decode_n64_p1024_s512", 64, 1024, (512, 512), (1, 1), 1),   # 37.4 / 41.8
    ("decode_n256_p1024_s16", 256, 1024, (16, 16), (1, 1), 1),    # 31.0 / 71.3
    ("prefill_n8_p2048", 8, 2048, (64, 512), (1, 64), 1),         # 32.1 / 43.5
    ("prefill_n32_p256", 32, 256, (64, 512), (1, 64), 0),         # 45.9 / 41.2
    ("prefill_n128_p256", 128, 256, (64, 512), (1, 64), 0),       # 152.7 / 135.7
]

# The wider families (decode, one query token): 64 / 8 heads; head_dim 64;
# fp8 e4m3 caches; two interleaved documents (1024 tokens for the even
# requests, 2048 for the odd ones) after the prefix. (name, family, N, P, S,
# cascade?)
SWEEP_CLEAR_WIDE = [
    ("h64_n4_p1024_s512", "h64", 4, 1024, 512, 1),       # 15.0 / 17.3
    ("h64_n16_p8192_s16", "h64", 16, 8192, 16, 1),       # 21.6 / 44.4
    ("h64_n64_p1024_s16", "h64", 64, 1024, 16, 1),       # 20.3 / 22.7
    ("h64_n256_p8192_s512", "h64", 256, 8192, 512, 1),   # 153.1 / 480.8
    ("d64_n16_p4096_s16", "d64", 16, 4096, 16, 1),       # 15.4 / 20.4
    ("d64_n64_p4096_s512", "d64", 64, 4096, 512, 1),     # 26.8 / 55.1
    ("fp8_n16_p4096_s512", "fp8", 16, 4096, 512, 1),     # 19.9 / 26.5
    ("fp8_n64_p1024_s16", "fp8", 64, 1024, 16, 1),       # 18.5 / 19.7
    ("fp8_n64_p4096_s16", "fp8", 64, 4096, 16, 1),       # 22.0 / 56.1
    ("docs_n32_p256_s16", "docs", 32, 256, 16, 1),       # 21.2 / 28.6
    ("docs_n32_p1024_s256", "docs", 32, 1024, 256, 1),   # 25.8 / 36.6
]


@pytest.mark.parametrize("name,n,p,s,q,casc", SWEEP_CLEAR, ids=[c[0] for c in SWEEP_CLEAR])
def test_auto_matches_the_decision_sweep(name, n, p, s, q, casc):
    """Where the device sweep found one path clearly faster, AUTO picks it
    (host-only plan; the cost model is fitted to the kernels' measured
    per-item, per-stage and per-launch costs), also below the pages'
    8-request gate."""
    w = workloads.Workload(name=name, num_reqs=n, prefix=p, suffix=s, q_len=q, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, seed=7)
    info = _plan(workloads.make_batch(w), mode="auto").info
    assert info["gates_pass"] == int(n >= 8)
    assert info["use_cascade"] == casc, (info["est_us_cascade"], info["est_us_noncascade"])


@pytest.mark.parametrize("name,fam,n,p,s,casc", SWEEP_CLEAR_WIDE, ids=[c[0] for c in SWEEP_CLEAR_WIDE])
def test_auto_matches_the_wider_decision_sweep(name, fam, n, p, s, casc):
    kw = dict(num_reqs=n, prefix=p, suffix=(s, s), q_len=(1, 1), num_q_heads=32, num_kv_heads=8, head_dim=128,
              seed=7)
    if fam == "h64":
        kw["num_q_heads"] = 64
    elif fam == "d64":
        kw["head_dim"] = 64
    elif fam == "fp8":
        kw.update(kv_dtype="fp8", k_scale=0.125, v_scale=0.0625)
    else:
        kw["docs"] = ((tuple(range(0, n, 2)), 1024), (tuple(range(1, n, 2)), 2048))
    w = workloads.Workload(name=name, **kw)
    b = workloads.make_batch(w)
    info = _plan(b, mode="auto").info
    assert info["use_cascade"] == casc, (info["est_us_cascade"], info["est_us_noncascade"])
    if fam == "docs":
        assert info["shared_levels"] == 2 and info["num_level1_groups"] == 2


def _tree_of(pl):
    """The plan's nested groups in the oracle's form: (members in batch
    order, enclosing length, shared length, level), parents first."""
    groups, deepest = spa.cascade_attn_plan_groups(pl)
    members = [[] for _ in groups]
    for r, g in enumerate(deepest):
        while g >= 0:
            members[g].append(r)
            g = groups[g][1]
    return [(tuple(sorted(members[j])), kb, ke, lev) for j, (lev, _, kb, ke) in enumerate(groups)]


def _nested_tables(rng, n, ps=16, depth=1, shuffle=False):
    """Random block tables with a level-0 prefix, runs of requests sharing
    extra pages (sometimes only some of a run), nested `depth` levels deep,
    and random lengths; with `shuffle`, the requests in random order (group
    members not adjacent)."""
    level0 = int(rng.integers(16, 20))
    rows, seq, nxt = [], [], [1000]

    def fresh(k):
        ids = list(range(nxt[0], nxt[0] + k))
        nxt[0] += k
        return ids

    def fill(prefix, count, lvl):
        r = 0
        while r < count:
            m = min(int(rng.integers(1, 5)), count - r)
            extra = fresh(int(rng.integers(0, 40)))
            if lvl < depth and m >= 2 and rng.random() < 0.6:
                fill(prefix + extra, m, lvl + 1)
            else:
                for _ in range(m):
                    keep = len(extra) if rng.random() < 0.8 else int(rng.integers(0, len(extra) + 1))
                    row = prefix + extra[:keep] + fresh(int(rng.integers(1, 6)))
                    rows.append(row)
                    seq.append((len(row) - 1) * ps + int(rng.integers(1, ps + 1)))
            r += m

    fill(fresh(level0), n, 1)
    order = rng.permutation(n) if shuffle else np.arange(n)
    rows = [rows[i] for i in order]
    seq = [seq[i] for i in order]
    stride = max(len(x) for x in rows) + 1
    bt = np.zeros((n, stride), dtype=np.int32)
    for i, row in enumerate(rows):
        bt[i, :len(row)] = row
        bt[i, len(row):] = row[0]
    seq = np.array(seq, dtype=np.int32)
    q = np.minimum(rng.integers(1, 40, n), seq - level0 * ps).astype(np.int32)
    return bt, seq, q, nxt[0]


@pytest.mark.parametrize("depth,shuffle", [(1, False), (1, True), (3, False), (3, True)])
def test_tree_groups_match_oracle_on_random_batches(depth, shuffle):
    rng = np.random.default_rng(41 + 10 * depth + int(shuffle))
    deep_seen = 0
    for _ in range(150):
        n = int(rng.integers(1, 40))
        bt, seq, q, pages = _nested_tables(rng, n, depth=depth, shuffle=shuffle)
        nc = seq - q
        qsl = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
        kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, num_pages=pages,
                  kv_strides=(16 * 2 * 128, 2 * 128, 128), block_table=bt, query_start_loc=qsl, seq_lens=seq,
                  num_computed_tokens=nc, mode="on", num_cus=256)
        pl = spa.cascade_attn_plan(**kw)
        info = pl.info
        plen = info["common_prefix_len"]
        want = oracle.tree_groups(bt.tolist(), seq.tolist(), nc.tolist(), 16, plen)
        assert _tree_of(pl) == want
        assert info["num_level1_groups"] == len(want)
        assert info["shared_levels"] == 1 + max([g[3] for g in want], default=0)
        assert info["kv_tokens_cascade"] == oracle.kv_tokens_tree(plen, want, seq.tolist())
        deep_seen += info["shared_levels"] >= 3
        for levels in (1, 2, 3):
            lim = spa.cascade_attn_plan(**kw, max_levels=levels)
            want_l = oracle.tree_groups(bt.tolist(), seq.tolist(), nc.tolist(), 16, plen, max_levels=levels)
            assert _tree_of(lim) == want_l
            assert lim.info["shared_levels"] <= levels
    if depth > 1:
        assert deep_seen >= 10


def test_tree_keeps_the_64_groups_that_save_most():
    """100 pairs of requests, each pair sharing its own document of a
    different length beyond the batch prefix, interleaved (pair i is
    requests i and i + 100): the plan keeps 64 groups, the ones whose
    documents are longest (saving = extra tokens), in the order found."""
    ps, level0 = 16, 16
    rows, seq = [None] * 200, [None] * 200
    nxt = 1000
    doc_pages = [17 + (i * 37) % 50 for i in range(100)]
    for i in range(100):
        doc = list(range(nxt, nxt + doc_pages[i]))
        nxt += doc_pages[i]
        for r in (i, i + 100):
            row = list(range(level0)) + doc + [nxt]
            nxt += 1
            rows[r] = row
            seq[r] = len(row) * ps
    stride = max(len(x) for x in rows)
    bt = np.zeros((200, stride), dtype=np.int32)
    for i, row in enumerate(rows):
        bt[i, :len(row)] = row
    seq = np.array(seq, dtype=np.int32)
    qsl = np.arange(201, dtype=np.int32)
    pl = spa.cascade_attn_plan(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=ps, num_pages=nxt,
                               kv_strides=(ps * 2 * 128, 2 * 128, 128), block_table=bt, query_start_loc=qsl,
                               seq_lens=seq, mode="on", num_cus=256)
    got = _tree_of(pl)
    every = oracle.tree_groups(bt.tolist(), seq.tolist(), (seq - 1).tolist(), ps, level0 * ps)
    assert len(every) == 100 and len(got) == 64
    by_saving = sorted(every, key=lambda g: -(g[2] - g[1]))
    assert sorted(got) == sorted(by_saving[:64])
    assert got == [g for g in every if g in got]   # order found
    assert all(len(g[0]) == 2 and g[0][1] == g[0][0] + 100 for g in got)


def test_tree_batches_beyond_the_order_table_use_one_level():
    """More than 512 requests: no nested levels (the kernels' tree-order
    table holds 512 positions); the batch-wide prefix still applies."""
    n = 600
    rows = []
    nxt = 100000
    for r in range(n):
        rows.append(list(range(20)) + list(range(1000 + 40 * (r % 7), 1000 + 40 * (r % 7) + 30)) + [nxt])
        nxt += 1
    bt = np.array(rows, dtype=np.int32)
    seq = np.full(n, bt.shape[1] * 16, dtype=np.int32)
    qsl = np.arange(n + 1, dtype=np.int32)
    pl = spa.cascade_attn_plan(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, num_pages=nxt,
                               kv_strides=(16 * 2 * 128, 2 * 128, 128), block_table=bt, query_start_loc=qsl,
                               seq_lens=seq, mode="on", num_cus=256)
    assert pl.info["use_cascade"] == 1 and pl.info["common_prefix_len"] == 320
    assert pl.info["num_level1_groups"] == 0 and pl.info["shared_levels"] == 1


def test_fp8_plans():
    """fp8 caches: the same decisions and partition as bf16 except the byte
    count the cost model uses, four pipeline stages in the same LDS, and one
    KV head per work item (an explicit heads_per_item is not applied)."""
    b16 = workloads.make_batch(workloads.get("worked_decode"))
    b8 = workloads.make_batch(workloads.get("worked_decode_fp8"))
    i16, i8 = _plan(b16, mode="on").info, _plan(b8, mode="on").info
    assert i8["kv_dtype"] == _lib.KV_FP8_E4M3 and i16["kv_dtype"] == _lib.KV_BF16
    assert i8["prefix_stages"] == 4 and i8["suffix_stages"] == 4 and i8["suffix_heads_per_item"] == 1
    assert i8["common_prefix_len"] == i16["common_prefix_len"] == 4096
    assert i8["kv_tokens_cascade"] == i16["kv_tokens_cascade"]
    assert _plan(b8, mode="on", heads_per_item=2).info["suffix_heads_per_item"] == 1
    off = _plan(b8, mode="off").info
    assert off["suffix_stages"] == 4 and off["suffix_heads_per_item"] == 1


def test_sliding_window_decisions():
    """A window that hides positions from some query rules cascade out
    (AUTO falls back, FORCE_ON refuses); one longer than every sequence
    never binds and is dropped."""
    wd = workloads.make_batch(workloads.get("worked_decode"))
    assert _plan(wd, mode="auto", sliding_window=1024).info["use_cascade"] == 0
    assert _plan(wd, mode="auto", sliding_window=1024).info["sliding_window"] == 1024
    with pytest.raises(spa.CascadeAttnError) as e:
        _plan(wd, mode="on", sliding_window=1024)
    assert e.value.status == _lib.CA_EUNSUPPORTED
    wide = _plan(wd, mode="auto", sliding_window=4096 + 128).info
    assert wide["sliding_window"] == 0 and wide["use_cascade"] == 1
    assert _plan(wd, mode="off", sliding_window=100).info["sliding_window"] == 100
    with pytest.raises(spa.CascadeAttnError) as e:
        _plan(wd, mode="auto", sliding_window=-1)
    assert e.value.status == _lib.CA_EINVAL


def test_prefix_split_override():
    """An explicit prefix split count is applied, limited to one 64-key tile
    per split and raised so no item exceeds 8192 keys."""
    wd = workloads.make_batch(workloads.get("worked_decode"))       # 4096-token prefix: 64 tiles
    assert _plan(wd, mode="on", prefix_splits=4).info["prefix_splits"] == 4
    assert _plan(wd, mode="on", prefix_splits=1000).info["prefix_splits"] == 64
    ld = workloads.make_batch(workloads.get("long_doc"))            # 32768 tokens: at least 4 splits
    assert _plan(ld, mode="on", prefix_splits=1).info["prefix_splits"] == 4
    with pytest.raises(spa.CascadeAttnError) as e:
        _plan(wd, mode="on", prefix_splits=-1)
    assert e.value.status == _lib.CA_EINVAL
    spa.cascade_attn_autotune_reset()      # host-only: callable without a device


def test_suffix_order():
    """Per-request work items of a ragged batch start with the longest key
    range; batches whose requests already come longest first, suffix_order=1
    and batches of more than 512 requests keep batch order."""
    sc = workloads.make_batch(workloads.get("self_consistency"))   # suffixes U[1, 1024]
    assert _plan(sc, mode="on").info["suffix_longest_first"] == 1
    assert _plan(sc, mode="off").info["suffix_longest_first"] == 1
    assert _plan(sc, mode="on", suffix_order=1).info["suffix_longest_first"] == 0
    wd = workloads.make_batch(workloads.get("worked_decode"))      # every suffix 128 tokens
    assert _plan(wd, mode="on").info["suffix_longest_first"] == 0
    big = workloads.make_batch(workloads.Workload("many_requests", 600, 256, (1, 200), (1, 1), 1, 1, 64, seed=77))
    assert _plan(big, mode="on").info["suffix_longest_first"] == 0
    with pytest.raises(spa.CascadeAttnError) as e:
        _plan(wd, mode="on", suffix_order=2)
    assert e.value.status == _lib.CA_EINVAL


def test_noncascade_chunking_pays_for_the_merge():
    """The non-cascade path splits a request's KV range only when that saves
    more than the merge launch it adds: small batches run one direct launch
    (no partial slots); 8 requests of 33k tokens keep their chunks."""
    for name in ("tiny_decode", "long_doc_p255", "multi_doc_prefill"):
        info = _plan(workloads.make_batch(workloads.get(name)), mode="off").info
        assert info["suffix_chunks"] == 1 and info["num_partial_slots"] == 0, name
    info = _plan(workloads.make_batch(workloads.get("long_doc_n8")), mode="off").info
    assert info["suffix_chunks"] > 1 and info["num_partial_slots"] == info["suffix_chunks"]


def test_auto_is_a_function_of_the_batch_unless_tuning_is_asked_for():
    """A recorded tuning choice never changes a default AUTO plan: the same
    batch planned before and after the record gets identical plans. Only a
    plan that opts in (use_tuned) takes the record, and a reset forgets it.
    ("Diary - vLLM's cascade attention": output that depends on what else
    happened in the process is the failure to avoid.)"""
    wd = workloads.make_batch(workloads.get("worked_decode"))
    w = wd.workload
    kw = dict(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
              num_pages=wd.num_pages, kv_strides=spa.kv_strides(wd.k_cache), block_table=wd.block_table,
              query_start_loc=wd.query_start_loc, seq_lens=wd.seq_lens, num_computed_tokens=wd.num_computed,
              num_cus=256)
    try:
        spa.cascade_attn_autotune_reset()
        before = _plan(wd, mode="auto").info
        before_opt_in = _plan(wd, mode="auto", use_tuned=True).info
        assert before_opt_in == before and before["use_cascade"] == 1
        spa.cascade_attn_autotune_record(mode="off", **kw)
        assert _plan(wd, mode="auto").info == before
        tuned = _plan(wd, mode="auto", use_tuned=True).info
        assert tuned["use_cascade"] == 0
        # an explicit setting keeps the record out even when opted in
        assert _plan(wd, mode="auto", use_tuned=True, max_levels=1).info["use_cascade"] == 1
        spa.cascade_attn_autotune_record(mode="on", prefix_splits=4, **kw)
        tuned = _plan(wd, mode="auto", use_tuned=True).info
        assert tuned["use_cascade"] == 1 and tuned["prefix_splits"] == 4
        assert _plan(wd, mode="auto").info == before
        spa.cascade_attn_autotune_reset()
        assert _plan(wd, mode="auto", use_tuned=True).info == before
        for bad in (dict(mode="auto"), dict(mode="on", prefix_splits=-1), dict(mode="on", max_levels=5)):
            with pytest.raises(spa.CascadeAttnError) as e:
                spa.cascade_attn_autotune_record(**bad, **kw)
            assert e.value.status == _lib.CA_EINVAL
        with pytest.raises(spa.CascadeAttnError) as e:
            _plan(wd, mode="auto", use_tuned=2)
        assert e.value.status == _lib.CA_EINVAL
    finally:
        spa.cascade_attn_autotune_reset()
