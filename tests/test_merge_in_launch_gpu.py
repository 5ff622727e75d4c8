"""The merge inside the attention launch (merge_mode=2, or the planner's
choice where it pays): the work item that completes a row block's partial
states merges it, in the same slot order as the stand-alone merge kernel. So
its outputs and LSEs equal, bit for bit, those of the same plan with a
separate merge launch (merge_mode=1), run after run (the arrival counters go
back to zero), and match the oracle. Plans with nested shared levels merge
in a launch of their own whatever merge_mode asks; batches with documents
are run here with the batch-wide level only (max_levels=1)."""

import numpy as np
import pytest
import torch

import workloads
from workloads import Workload
import shared_prefix_attention_amd as spa
from parity_util import DeviceBatch, assert_close, log, oracle_ref, plan, run

pytestmark = pytest.mark.gpu

SMALL = {
    "prefill_capped": Workload("prefill_capped", 8, 256, (20, 100), (1, 20), 8, 2, 128, seed=2003,
                               override=((0, 250, 12),)),
    "nested_prefill": Workload("nested_prefill", 10, 256, (5, 60), (1, 12), 8, 2, 128, seed=2013,
                               groups=((3, 400), (4, 640))),
    "fp8_nested": Workload("fp8_nested", 12, 256, (1, 40), (1, 3), 8, 2, 128, seed=2020,
                           groups=((4, 512), (3, 300)), kv_dtype="fp8", k_scale=0.25, v_scale=0.125),
    "many_rows": Workload("many_rows", 16, 768, (24, 40), (8, 16), 16, 4, 128, seed=2006),
    "d64_gqa": Workload("d64_gqa", 10, 320, (5, 60), (1, 4), 8, 2, 64, seed=2007),
    "long_prefix_split": Workload("long_prefix_split", 8, 4096, (64, 64), (1, 1), 8, 2, 128, seed=2005),
}

CASES = [("tiny_decode", "on", {}), ("worked_decode", "on", {}), ("worked_decode", "auto", {}),
         ("mixed_prefill", "on", {}), ("mixed_prefill_capped", "on", {}), ("self_consistency", "on", {}),
         ("long_doc", "on", {}), ("multi_doc", "on", {}), ("multi_doc_prefill", "on", {}),
         ("worked_decode_fp8", "on", {}), ("long_doc_n8", "off", {}), ("self_consistency", "off", {}),
         ("prefill_capped", "on", {}), ("nested_prefill", "on", {}), ("fp8_nested", "on", {}),
         ("many_rows", "on", {}), ("d64_gqa", "on", {}), ("long_prefix_split", "on", {}),
         ("long_prefix_split", "off", {}), ("many_rows", "on", {"partials_fp32": True}),
         ("worked_decode", "on", {"heads_per_item": 1}), ("d64_gqa", "on", {"partials_fp32": True})]


def setup_module():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _batch(name):
    return workloads.make_batch(SMALL[name] if name in SMALL else workloads.get(name))


@pytest.mark.parametrize("name,mode,kw", CASES)
def test_merge_in_launch_equals_merge_launch(name, mode, kw):
    log(f"[merge in launch] {name} mode={mode} {kw}")
    b = _batch(name)
    if b.workload.groups or b.workload.docs:
        kw = dict(kw, max_levels=1)
    db = DeviceBatch(b)
    o1, l1, i1 = run(db, mode=mode, merge_mode=2, **kw)
    o2, l2, i2 = run(db, mode=mode, merge_mode=1, **kw)
    o3, l3, _ = run(db, mode=mode, merge_mode=2, **kw)
    log(f"  cascade={i1['use_cascade']} slots={i1['num_partial_slots']} in-launch={i1['merge_in_launch']} "
        f"psplit={i1['prefix_splits']} groups={i1['num_level1_groups']} schunks={i1['suffix_chunks']}")
    assert i1["merge_in_launch"] == 1 and i2["merge_in_launch"] == 0 and i1["num_partial_slots"] > 0
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "in-launch merge differs from the merge kernel"
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3), "second run differs"
    if b.workload.num_reqs <= 16 and b.workload.prefix <= 4096:
        ref_o, ref_l = oracle_ref(b)
        assert_close(o1, l1, ref_o, ref_l, what=f"{name}/{mode}/in-launch")


@pytest.mark.parametrize("name,mode", [("tiny_decode", "on"), ("prefill_capped", "on"), ("long_prefix_split", "on"),
                                       ("nested_prefill", "on")])
def test_merge_in_launch_with_sinks(name, mode):
    b = _batch(name)
    z = np.random.default_rng(5).normal(0.0, 2.0, b.workload.num_q_heads).astype(np.float32)
    z[0] = -np.inf
    db = DeviceBatch(b)
    o1, l1, i1 = run(db, mode=mode, sinks=z, merge_mode=2, max_levels=1)
    o2, l2, _ = run(db, mode=mode, sinks=z, merge_mode=1, max_levels=1)
    assert i1["merge_in_launch"] == 1
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ref_o, ref_l = oracle_ref(b, sinks=z)
    assert_close(o1, l1, ref_o, ref_l, what=f"{name}/{mode}/sinks/in-launch")


def test_planner_keeps_small_merges_in_the_launch():
    """By default the planner merges inside the launch only where that is
    priced below a merge launch (small batches: few rows per completing item,
    few slots), as measured; the worked example keeps its merge launch."""
    assert plan(_batch("tiny_decode"), mode="on").info["merge_in_launch"] == 1
    assert plan(_batch("worked_decode"), mode="on").info["merge_in_launch"] == 0


def test_counters_return_to_zero_and_workspace_init():
    """A workspace full of garbage, cleared by cascade_attn_workspace_init,
    serves a sequence of different plans; after each run the counter region
    is zero again."""
    seq = [("worked_decode", "on"), ("mixed_prefill", "on"), ("worked_decode", "on"), ("long_doc_n8", "off")]
    batches = {n: _batch(n) for n, _ in seq}
    need = max(plan(batches[n], mode=m, merge_mode=2).workspace_bytes for n, m in seq)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    spa.cascade_attn_workspace_init(ws)
    torch.cuda.synchronize()
    assert int(ws[:spa._lib.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
    for name, mode in seq:
        b = batches[name]
        db = DeviceBatch(b)
        pl = plan(b, mode=mode, k_cache=db.k, merge_mode=2)
        assert pl.info["merge_in_launch"] == 1
        out = torch.empty_like(db.q)
        lse = torch.empty(db.q.shape[0], db.q.shape[1], dtype=torch.float32, device="cuda")
        spa.cascade_attn_run(pl, db.q, db.k, db.v, db.bt, db.qsl, db.sl, out, lse, ws)
        torch.cuda.synchronize()
        assert int(ws[:spa._lib.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0, f"{name}: counters not reset"
        ref_o, ref_l = run(db, mode=mode, merge_mode=1)[:2]
        assert np.array_equal(out.float().cpu().numpy(), ref_o) and np.array_equal(lse.cpu().numpy(), ref_l)


@pytest.mark.parametrize("name", ["nested_prefill", "fp8_nested", "multi_doc"])
def test_nested_levels_merge_in_a_launch_of_their_own(name):
    """merge_mode=2 on a plan with nested levels: the plan reports a separate
    merge, and the result equals merge_mode=1's bit for bit and the oracle."""
    b = _batch(name)
    db = DeviceBatch(b)
    o1, l1, i1 = run(db, mode="on", merge_mode=2)
    o2, l2, i2 = run(db, mode="on", merge_mode=1)
    assert i1["num_level1_groups"] > 0 and i1["merge_in_launch"] == 0 and i2["merge_in_launch"] == 0
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    if b.workload.num_reqs <= 16:
        ref_o, ref_l = oracle_ref(b)
        assert_close(o1, l1, ref_o, ref_l, what=f"{name}/nested/merge_mode=2")
