"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test compares every output row and LSE with the oracle: the small
batches, and the full-size workloads at the sizes and launch configurations
the benchmark times (the oracle runs once per full workload). Tolerances: |out - ref| <= 2e-2 + 1e-2 |ref| elementwise, |lse - ref|
<= 1e-3. Inputs carry NaN in unused pages and in the tail slots of each
request's last page, so any out-of-range read shows up as a non-finite output.
"""

import numpy as np
import pytest
import torch

import workloads
from workloads import Workload
from parity_util import DeviceBatch, assert_close, log, oracle_ref, run

pytestmark = pytest.mark.gpu

SMALL = {
    w.name: w for w in [
        workloads.get("tiny_decode"),
        Workload("decode_ragged", 16, 512, (33, 47), (1, 1), 32, 8, 128, seed=2001),
        Workload("prefill_mix", 8, 256, (20, 100), (1, 20), 8, 2, 128, seed=2002),
        # request 0 computed only 238 tokens: the cap binds (256 -> 224)
        Workload("prefill_capped", 8, 256, (20, 100), (1, 20), 8, 2, 128, seed=2003, override=((0, 250, 12),)),
        Workload("gqa8_outliers", 24, 1024, (1, 100), (1, 1), 16, 2, 128, seed=2004,
                 outlier_frac=0.01, outlier_scale=8.0),
        Workload("long_prefix_split", 8, 4096, (64, 64), (1, 1), 8, 2, 128, seed=2005),
        Workload("many_rows", 16, 768, (24, 40), (8, 16), 16, 4, 128, seed=2006),
        Workload("d64_gqa", 10, 320, (5, 60), (1, 4), 8, 2, 64, seed=2007),
        Workload("single_request", 1, 0, (70, 70), (3, 3), 8, 2, 128, seed=2008),
        Workload("fresh_prefill", 4, 0, (30, 50), (30, 50), 4, 1, 64, seed=2009),
        Workload("partial_page_prefix", 9, 250, (10, 30), (1, 2), 4, 2, 128, seed=2010),
        Workload("one_page_suffix", 12, 512, (1, 1), (1, 1), 8, 8, 128, seed=2011),
        # second shared level: groups of consecutive requests share a document
        Workload("nested_decode", 12, 256, (1, 40), (1, 1), 8, 2, 128, seed=2012,
                 groups=((4, 512), (3, 300), (2, 1000))),
        Workload("nested_prefill", 10, 256, (5, 60), (1, 12), 8, 2, 128, seed=2013,
                 groups=((3, 400), (4, 640))),
        Workload("nested_d64", 9, 256, (1, 30), (1, 3), 16, 4, 64, seed=2014,
                 groups=((5, 300), (2, 700))),
        Workload("nested_all_grouped", 8, 256, (1, 20), (1, 1), 8, 2, 128, seed=2015,
                 groups=((4, 512), (4, 512))),
        # request 1 has computed only 601 tokens: the group's share is capped (896 -> 592)
        Workload("nested_capped", 8, 256, (10, 30), (1, 4), 8, 2, 128, seed=2016,
                 groups=((4, 640),), override=((1, 901, 300),)),
        # fp8 e4m3 caches (head_dim 128), scales 1/8 (K) and 1/16 (V)
        Workload("fp8_decode", 16, 512, (33, 47), (1, 1), 32, 8, 128, seed=2017,
                 kv_dtype="fp8", k_scale=0.125, v_scale=0.0625),
        Workload("fp8_prefill", 8, 256, (20, 100), (1, 20), 8, 2, 128, seed=2018,
                 kv_dtype="fp8", k_scale=0.125, v_scale=0.0625),
        Workload("fp8_gqa8_outliers", 24, 1024, (1, 100), (1, 1), 16, 2, 128, seed=2019,
                 outlier_frac=0.01, outlier_scale=8.0, kv_dtype="fp8", k_scale=0.125, v_scale=0.0625),
        Workload("fp8_nested", 12, 256, (1, 40), (1, 3), 8, 2, 128, seed=2020,
                 groups=((4, 512), (3, 300)), kv_dtype="fp8", k_scale=0.25, v_scale=0.125),
        Workload("fp8_fresh_prefill", 4, 0, (30, 50), (30, 50), 4, 1, 128, seed=2021,
                 kv_dtype="fp8", k_scale=0.125, v_scale=0.0625),
        # nested levels in a tree: members not adjacent in the batch, up to
        # four shared levels (prefix -> document -> chapter -> section)
        Workload("tree_decode", 16, 256, (1, 40), (1, 1), 8, 2, 128, seed=2023,
                 docs=(((0, 3, 5, 8, 11, 14), 512), ((3, 8, 14), 256), ((8, 14), 300), ((1, 6, 9), 640))),
        Workload("tree_prefill", 12, 256, (5, 60), (1, 12), 8, 2, 128, seed=2024,
                 docs=(((1, 4, 7, 10), 768), ((4, 10), 512), ((2, 11), 400))),
        Workload("tree_d64", 10, 256, (1, 30), (1, 3), 16, 4, 64, seed=2025,
                 docs=(((0, 2, 4, 6, 8), 512), ((2, 6), 300), ((1, 9), 700))),
        Workload("tree_fp8", 14, 256, (1, 40), (1, 3), 8, 2, 128, seed=2026,
                 docs=(((0, 2, 4, 6, 8, 10, 12), 512), ((2, 6, 10), 512), ((6, 10), 256), ((1, 13), 300)),
                 kv_dtype="fp8", k_scale=0.25, v_scale=0.125),
        # every request in a group, interleaved halves
        Workload("tree_all_grouped", 8, 256, (1, 20), (1, 1), 8, 2, 128, seed=2027,
                 docs=(((0, 2, 4, 6), 512), ((1, 3, 5, 7), 512), ((2, 6), 256), ((1, 5), 512))),
    ]
}


def setup_module():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("mode", ["auto", "on", "off"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name, mode):
    log(f"[parity] {name} mode={mode}")
    b = workloads.make_batch(SMALL[name])
    ref_o, ref_l = oracle_ref(b)
    out, lse, info = run(DeviceBatch(b), mode=mode)
    log(f"  plan: cascade={info['use_cascade']} P_c={info['common_prefix_len']} "
        f"psplit={info['prefix_splits']} groups={info['num_level1_groups']}x{info['level1_splits']} "
        f"levels={info['shared_levels']} schunks={info['suffix_chunks']}")
    if mode == "on" and (SMALL[name].groups or SMALL[name].docs):
        assert info["num_level1_groups"] > 0
    assert_close(out, lse, ref_o, ref_l, what=f"{name}/{mode}")


GROUPED = [("tiny_decode", 2), ("tiny_decode", 4), ("decode_ragged", 8), ("gqa8_outliers", 2),
           ("long_prefix_split", 2), ("d64_gqa", 2), ("one_page_suffix", 4), ("prefill_mix", 2)]


@pytest.mark.parametrize("mode", ["on", "off"])
@pytest.mark.parametrize("name,heads", GROUPED)
def test_grouped_heads(name, heads, mode):
    """Decode-shaped items that run several KV heads each (one continuous
    pipeline over consecutive heads of a request). prefill_mix has items of
    more than 16 rows, where the setting does not apply."""
    log(f"[parity] {name} mode={mode} heads/item={heads}")
    b = workloads.make_batch(SMALL[name])
    ref_o, ref_l = oracle_ref(b)
    out, lse, info = run(DeviceBatch(b), mode=mode, heads_per_item=heads)
    log(f"  plan: cascade={info['use_cascade']} heads/item={info['suffix_heads_per_item']} "
        f"kernel={info['suffix_kernel']} schunks={info['suffix_chunks']}")
    assert info["suffix_heads_per_item"] == (heads if info["suffix_kernel"] == 1 else 1)
    assert_close(out, lse, ref_o, ref_l, what=f"{name}/{mode}/h{heads}")


@pytest.mark.parametrize("name", ["decode_ragged", "prefill_mix", "d64_gqa", "fp8_decode", "fp8_prefill",
                                  "tree_prefill", "tree_fp8"])
def test_small_hnd_layout(name):
    log(f"[parity] {name} HND")
    b = workloads.make_batch(SMALL[name])
    ref_o, ref_l = oracle_ref(b)
    for mode in ("on", "off"):
        out, lse, _ = run(DeviceBatch(b, layout="HND"), mode=mode)
        assert_close(out, lse, ref_o, ref_l, what=f"{name}/HND/{mode}")


_ORACLE = {}


def oracle_cached(name, b):
    """The fp64 oracle over every request of a named workload, computed once
    per test session and shared by the tests that compare against it."""
    if name not in _ORACLE:
        log(f"  oracle: {name} ({b.workload.num_reqs} requests, every row)")
        _ORACLE[name] = oracle_ref(b)
    return _ORACLE[name]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size_every_row_parity(name):
    """Every full-size workload, every output row and LSE against the fp64
    oracle, on the AUTO plan, the forced cascade plan and the forced
    non-cascade plan (the launch configurations the benchmark times)."""
    w = workloads.get(name)
    log(f"[parity-full] {name}")
    b = workloads.make_batch(w)
    ref_o, ref_l = oracle_cached(name, b)
    db = DeviceBatch(b)
    for mode in ("auto", "on", "off"):
        out, lse, info = run(db, mode=mode)
        log(f"  {mode}: cascade={info['use_cascade']} P_c={info['common_prefix_len']} "
            f"psplit={info['prefix_splits']} row tile={info['prefix_row_tile']} schunks={info['suffix_chunks']}")
        assert_close(out, lse, ref_o, ref_l, what=f"{name}/{mode}")


def test_128_row_prefix_tile_every_row():
    """A batch small enough for an every-row check whose packed prefix rows
    (T * G = 2,304 per KV head) select the 128-row MFMA prefix tile, with
    ragged query and suffix lengths; cascade forced on and under AUTO."""
    w = Workload("prefix_128row_tile", 16, 512, (48, 96), (32, 40), 32, 8, 128, seed=2022)
    b = workloads.make_batch(w)
    assert int(b.total_q) * 4 >= 2048
    ref_o, ref_l = oracle_ref(b)
    db = DeviceBatch(b)
    for mode in ("on", "auto"):
        out, lse, info = run(db, mode=mode)
        log(f"[128-row tile] mode={mode} cascade={info['use_cascade']} row tile={info['prefix_row_tile']} "
            f"psplit={info['prefix_splits']}")
        if mode == "on":
            assert info["prefix_row_tile"] == 128
        assert_close(out, lse, ref_o, ref_l, what=f"prefix_128row_tile/{mode}")


SEPARATE = ["tiny_decode", "prefill_mix", "prefill_capped", "gqa8_outliers", "many_rows", "d64_gqa",
            "nested_decode", "nested_prefill", "fp8_decode", "fp8_prefill", "fp8_nested", "worked_decode",
            "mixed_prefill", "self_consistency", "multi_doc", "worked_decode_fp8"]


@pytest.mark.parametrize("name", SEPARATE)
def test_separate_phase_launches_match_fused(name):
    """The prefix and suffix phases as two launches run the same work items
    as the single launch, so the results are bitwise the same."""
    log(f"[separate] {name}")
    w = SMALL[name] if name in SMALL else workloads.get(name)
    db = DeviceBatch(workloads.make_batch(w))
    fo, fl, finfo = run(db, mode="on")
    so, sl, sinfo = run(db, mode="on", separate_phases=True)
    assert finfo["use_cascade"] == 1 and finfo["separate_phases"] == 0 and sinfo["separate_phases"] == 1
    log(f"  prefix row tile {sinfo['prefix_row_tile']}, suffix kernel {sinfo['suffix_kernel']}, "
        f"heads/item {sinfo['suffix_heads_per_item']}")
    assert np.array_equal(fo, so) and np.array_equal(fl, sl), f"{name}: separate launches differ from the fused one"
    if name in SMALL:
        ref_o, ref_l = oracle_ref(db.b)
        assert_close(so, sl, ref_o, ref_l, what=f"{name}/separate")


@pytest.mark.parametrize("name", ["nested_decode", "nested_prefill", "nested_capped", "multi_doc"])
def test_second_level_against_single_level(name):
    """The same batch with the second shared level and with the batch-wide
    prefix only: both match the oracle (they split the keys differently, so
    they are not bitwise equal) and agree with each other within the bar."""
    log(f"[levels] {name}")
    w = SMALL[name] if name in SMALL else workloads.get(name)
    b = workloads.make_batch(w)
    db = DeviceBatch(b)
    o2, l2, i2 = run(db, mode="on")
    o1, l1, i1 = run(db, mode="on", max_levels=1)
    assert i2["num_level1_groups"] > 0 and i1["num_level1_groups"] == 0
    log(f"  groups {i2['num_level1_groups']} x {i2['level1_splits']} splits; slots {i2['num_partial_slots']} "
        f"vs {i1['num_partial_slots']}")
    ref_o, ref_l = oracle_ref(b) if name in SMALL else oracle_cached(name, b)
    assert_close(o2, l2, ref_o, ref_l, what=f"{name}/two-level")
    assert_close(o1, l1, ref_o, ref_l, what=f"{name}/one-level")
    assert np.all(np.abs(o2 - o1) <= 2e-2 + 1e-2 * np.abs(o1)) and np.abs(l2 - l1).max() <= 1e-3


WINDOWS = [("decode_ragged", 1), ("decode_ragged", 37), ("prefill_mix", 17), ("prefill_mix", 200),
           ("d64_gqa", 64), ("fresh_prefill", 9), ("fp8_prefill", 50), ("long_prefix_split", 1000),
           ("many_rows", 130)]


@pytest.mark.parametrize("name,window", WINDOWS)
def test_sliding_window(name, window):
    """Sliding window: AUTO takes the non-cascade path (the window binds),
    stages wholly below a row's window are skipped, the rest is masked."""
    log(f"[window] {name} W={window}")
    b = workloads.make_batch(SMALL[name])
    ref_o, ref_l = oracle_ref(b, window=window)
    out, lse, info = run(DeviceBatch(b), mode="auto", sliding_window=window)
    assert info["use_cascade"] == 0 and info["sliding_window"] == window
    assert_close(out, lse, ref_o, ref_l, what=f"{name}/W{window}")


def _sinks(hq, seed):
    z = np.random.default_rng(seed).normal(0.0, 2.0, hq).astype(np.float32)
    z[0] = -np.inf                     # a head without a sink
    if hq > 2:
        z[1] = 8.0                     # a sink that outweighs most keys
    return z


SINKS = [(name, mode) for name in ["tiny_decode", "prefill_mix", "gqa8_outliers", "nested_decode", "fp8_decode",
                                   "long_prefix_split", "single_request"]
         for mode in ("on", "off") if mode == "off" or SMALL[name].prefix > 0]   # single_request shares nothing


@pytest.mark.parametrize("name,mode", SINKS)
def test_attention_sinks(name, mode):
    """Attention sinks through the merge (cascade, split KV) and through the
    direct epilogue (non-cascade with one chunk per request)."""
    w = SMALL[name]
    log(f"[sinks] {name} mode={mode}")
    b = workloads.make_batch(w)
    z = _sinks(w.num_q_heads, w.seed)
    ref_o, ref_l = oracle_ref(b, sinks=z)
    out, lse, info = run(DeviceBatch(b), mode=mode, sinks=z)
    log(f"  cascade={info['use_cascade']} slots={info['num_partial_slots']}")
    assert_close(out, lse, ref_o, ref_l, what=f"{name}/{mode}/sinks")


def test_window_with_sinks():
    b = workloads.make_batch(SMALL["prefill_mix"])
    z = _sinks(b.workload.num_q_heads, 7)
    ref_o, ref_l = oracle_ref(b, window=33, sinks=z)
    out, lse, _ = run(DeviceBatch(b), mode="auto", sliding_window=33, sinks=z)
    assert_close(out, lse, ref_o, ref_l, what="prefill_mix/W33/sinks")


def _rising_keys(b, per_token):
    """Scales every cached key by 1 + t * per_token, t its position (shared
    pages hold the same positions in every request), so each row's running
    maximum keeps rising by many units of log2 along the sequence."""
    f = torch.ones(b.k_cache.shape[0], b.k_cache.shape[1])
    ps = b.workload.page_size
    for r in range(b.workload.num_reqs):
        n = int(b.seq_lens[r])
        t = torch.arange(n)
        pages = b.block_table[r, t // ps].long()
        f[pages, t % ps] = 1.0 + t.float() * per_token
    b.k_cache = (b.k_cache.float() * f[:, :, None, None]).to(torch.bfloat16)
    return b


@pytest.mark.parametrize("mode", ["on", "off"])
@pytest.mark.parametrize("name,per_token", [("tiny_decode", 1 / 16), ("prefill_mix", 1 / 16),
                                            ("long_prefix_split", 1 / 256), ("d64_gqa", 1 / 8),
                                            ("many_rows", 1 / 32)])
def test_rising_row_maximum(name, per_token, mode):
    """Scores whose maximum grows by far more than the online softmax's
    rescale slack over a row's keys: the reference maximum is raised many
    times inside one work item and across splits."""
    log(f"[parity] {name} rising keys x{per_token:.4f}/token mode={mode}")
    b = _rising_keys(workloads.make_batch(SMALL[name]), per_token)
    ref_o, ref_l = oracle_ref(b)
    out, lse, _ = run(DeviceBatch(b), mode=mode)
    assert_close(out, lse, ref_o, ref_l, what=f"{name}/rising/{mode}")


@pytest.mark.parametrize("name,mode", [("prefill_mix", "on"), ("prefill_mix", "off"), ("gqa8_outliers", "on"),
                                       ("gqa8_outliers", "off"), ("nested_decode", "off"), ("nested_capped", "on"),
                                       ("fp8_gqa8_outliers", "on"), ("fp8_prefill", "off")])
def test_longest_first_order_changes_no_result(name, mode):
    """Starting per-request items longest first only reorders the dispatch:
    outputs and LSE are bitwise those of batch order."""
    log(f"[order] {name} mode={mode}")
    b = workloads.make_batch(SMALL[name])
    db = DeviceBatch(b)
    o1, l1, i1 = run(db, mode=mode)
    o2, l2, i2 = run(db, mode=mode, suffix_order=1)
    assert i1["suffix_longest_first"] == 1 and i2["suffix_longest_first"] == 0
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ref_o, ref_l = oracle_ref(b)
    assert_close(o1, l1, ref_o, ref_l, what=f"{name}/{mode}/longest-first")


@pytest.mark.parametrize("name,mode", [("prefill_mix", "on"), ("gqa8_outliers", "on"), ("nested_prefill", "on"),
                                       ("long_prefix_split", "off"), ("fp8_prefill", "on"), ("d64_gqa", "on")])
def test_fp32_partials(name, mode):
    """Partial outputs kept in fp32 (partials_fp32): the same plan shape,
    the merge reading fp32 states; parity with the oracle."""
    log(f"[parity] {name} mode={mode} fp32 partials")
    b = workloads.make_batch(SMALL[name])
    db = DeviceBatch(b)
    o32, l32, i32 = run(db, mode=mode, partials_fp32=True)
    assert i32["partials_fp32"] == 1 and i32["num_partial_slots"] > 0
    ref_o, ref_l = oracle_ref(b)
    assert_close(o32, l32, ref_o, ref_l, what=f"{name}/{mode}/fp32-partials")


@pytest.mark.parametrize("num_reqs,ordered", [(512, 1), (600, 0)])
def test_request_order_table_limits(num_reqs, ordered):
    """Decode batches at the request-order table's size: 512 requests fill
    it (longest first), 600 run in batch order; every row against the
    oracle, cascade and non-cascade."""
    w = Workload(f"many_requests_{num_reqs}", num_reqs, 256, (1, 200), (1, 1), 8, 2, 64, seed=3000 + num_reqs)
    b = workloads.make_batch(w)
    ref_o, ref_l = oracle_ref(b)
    db = DeviceBatch(b)
    for mode in ("on", "off"):
        out, lse, info = run(db, mode=mode)
        log(f"[order] N={num_reqs} mode={mode} longest_first={info['suffix_longest_first']}")
        assert info["suffix_longest_first"] == ordered
        assert_close(out, lse, ref_o, ref_l, what=f"N={num_reqs}/{mode}")


@pytest.mark.parametrize("num_reqs", [2, 3])
def test_few_requests_take_the_cascade_under_auto(num_reqs):
    """Two or three decode requests behind a 4,096-token prefix: AUTO's
    request gate (two or more) lets the cost model pick the cascade path,
    which matches the oracle."""
    w = Workload(f"few{num_reqs}", num_reqs, 4096, (16, 40), (1, 1), 32, 8, 128, seed=77 + num_reqs)
    b = workloads.make_batch(w)
    ref_o, ref_l = oracle_ref(b)
    out, lse, info = run(DeviceBatch(b), mode="auto")
    log(f"[few requests] N={num_reqs} cascade={info['use_cascade']} gates_pass={info['gates_pass']} "
        f"psplit={info['prefix_splits']}")
    assert info["gates_pass"] == 0 and info["use_cascade"] == 1
    assert_close(out, lse, ref_o, ref_l, what=f"few{num_reqs}/auto")


@pytest.mark.parametrize("mode", ["on", "off"])
def test_long_prefill_chunks(mode):
    """Four requests with 1,100-1,600 query tokens each over a 2,048-token
    shared prefix (5,833 tokens, 23,332 packed prefix rows per KV head): many
    row tiles per request on the per-request phase, a large prefix phase.
    Every row against the oracle."""
    w = Workload("long_prefill", 4, 2048, (1500, 2500), (1000, 2000), 32, 8, 128, seed=4242)
    b = workloads.make_batch(w)
    ref_o, ref_l = oracle_ref(b)
    out, lse, info = run(DeviceBatch(b), mode=mode)
    log(f"[long prefill] mode={mode} cascade={info['use_cascade']} psplit={info['prefix_splits']} "
        f"row tile={info['prefix_row_tile']} schunks={info['suffix_chunks']}")
    assert info["use_cascade"] == (1 if mode == "on" else 0)
    assert_close(out, lse, ref_o, ref_l, what=f"long_prefill/{mode}")


TREE_LEVELS = {"tree_decode": 4, "tree_prefill": 3, "tree_d64": 3, "tree_fp8": 4, "tree_all_grouped": 3}


@pytest.mark.parametrize("separate", [0, 1])
@pytest.mark.parametrize("name", list(TREE_LEVELS))
def test_tree_levels_every_depth(name, separate):
    """The same batch with 1 to 4 shared levels allowed (fewer levels: a
    request's positions past its innermost kept group are its own), one
    launch or one launch per role: every row against the oracle."""
    b = workloads.make_batch(SMALL[name])
    ref_o, ref_l = oracle_ref(b)
    db = DeviceBatch(b)
    for levels in (1, 2, 3, 4):
        log(f"[tree] {name} max_levels={levels} separate={separate}")
        out, lse, info = run(db, mode="on", max_levels=levels, separate_phases=separate)
        assert info["shared_levels"] == min(levels, TREE_LEVELS[name])
        assert_close(out, lse, ref_o, ref_l, what=f"{name}/levels{levels}/sep{separate}")
