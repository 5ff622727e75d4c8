"""On-device autotuning: cascade_attn_autotune times candidate plans with the
caller's data and returns the fastest; the choice is recorded for the batch
shape, so a later AUTO plan of that shape that opts in (use_tuned) takes it,
while default AUTO plans stay a function of the batch alone. Every candidate
computes the same attention, so the tuned plan is checked against the oracle
like any other."""

import numpy as np
import pytest
import torch

import workloads
import shared_prefix_attention_amd as spa
from parity_util import DeviceBatch, assert_close, log, oracle_ref, plan

pytestmark = pytest.mark.gpu


def setup_module():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(autouse=True)
def _clean_tuning_table():
    """Every test starts and ends with an empty tuning table, pass or fail."""
    spa.cascade_attn_autotune_reset()
    yield
    spa.cascade_attn_autotune_reset()


def _plan_kw(b):
    w = b.workload
    kw = dict(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
              num_pages=b.num_pages, kv_strides=spa.kv_strides(b.k_cache), block_table=b.block_table,
              query_start_loc=b.query_start_loc, seq_lens=b.seq_lens, num_computed_tokens=b.num_computed,
              kv_dtype=w.kv_dtype)
    if w.kv_dtype == "fp8":
        kw.update(k_scale=w.k_scale, v_scale=w.v_scale)
    return kw


@pytest.mark.parametrize("name", ["tiny_decode", "worked_decode", "mixed_prefill", "multi_doc", "worked_decode_fp8"])
def test_autotune_picks_a_valid_plan_and_records_it(name):
    log(f"[autotune] {name}")
    b = workloads.make_batch(workloads.get(name))
    db = DeviceBatch(b)
    auto = plan(b, mode="auto")
    ws = torch.zeros(max(auto.workspace_bytes, 64 << 20), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(db.q)
    lse = torch.empty(b.total_q, b.workload.num_q_heads, dtype=torch.float32, device="cuda")
    tuned, us = spa.cascade_attn_autotune(db.q, db.k, db.v, db.bt, db.qsl, db.sl, out, lse, ws, iters=5,
                                          **_plan_kw(b))
    info = tuned.info
    log(f"  {us:.1f} us: cascade={info['use_cascade']} psplits={info['prefix_splits']} "
        f"heads/item={info['suffix_heads_per_item']} groups={info['num_level1_groups']} "
        f"(AUTO: cascade={auto.info['use_cascade']} psplits={auto.info['prefix_splits']})")
    assert us > 0
    # the tuned plan computes the batch's attention
    spa.cascade_attn_run(tuned, db.q, db.k, db.v, db.bt, db.qsl, db.sl, out, lse, ws)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_ref(b)
    assert_close(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, what=f"{name}/tuned")
    # a later AUTO plan of the same shape that opts in takes the recorded choice
    again = plan(b, mode="auto", use_tuned=True).info
    for k in ("use_cascade", "prefix_splits", "suffix_heads_per_item", "num_level1_groups", "num_partial_slots"):
        assert again[k] == info[k], k
    # a default AUTO plan ignores the record
    default = plan(b, mode="auto").info
    assert default == auto.info
    spa.cascade_attn_autotune_reset()
    fresh = plan(b, mode="auto", use_tuned=True).info
    assert fresh == auto.info


def test_autotune_skips_candidates_that_do_not_fit_the_workspace():
    """Without a workspace only plans that need none can run; the worked
    example's cascade plans all need one."""
    b = workloads.make_batch(workloads.get("tiny_decode"))
    db = DeviceBatch(b)
    out = torch.empty_like(db.q)
    lse = torch.empty(b.total_q, b.workload.num_q_heads, dtype=torch.float32, device="cuda")
    try:
        tuned, _ = spa.cascade_attn_autotune(db.q, db.k, db.v, db.bt, db.qsl, db.sl, out, lse, None, iters=2,
                                             **_plan_kw(b))
    except spa.CascadeAttnError as e:
        assert e.status == 4   # CA_EWORKSPACE: nothing fits
    else:
        assert tuned.workspace_bytes == 0
