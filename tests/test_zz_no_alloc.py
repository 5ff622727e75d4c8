"""The no-allocation entry point: cascade_attn_run_noalloc keeps the partial
states in the library's own per-GPU device array instead of a caller
workspace. Through the C ABI, its outputs equal cascade_attn_run's bitwise
(same plan, same kernels), on two calls in a row where the second batch is
smaller than the first, and a plan needing more than the array holds is
refused before anything runs."""

import numpy as np
import pytest
import torch

import workloads
from workloads import Workload
import shared_prefix_attention_amd as spa
from parity_util import DeviceBatch, assert_close, log, oracle_ref, plan

pytestmark = pytest.mark.gpu


def setup_module():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(b, mode):
    db = DeviceBatch(b)
    pl = plan(b, mode=mode, k_cache=db.k)
    T, hq = db.q.shape[0], db.q.shape[1]
    ws = torch.zeros(max(pl.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    o_ref = torch.empty_like(db.q)
    l_ref = torch.empty(T, hq, dtype=torch.float32, device="cuda")
    spa.cascade_attn_run(pl, db.q, db.k, db.v, db.bt, db.qsl, db.sl, o_ref, l_ref, ws)
    o = torch.full_like(db.q, float("nan"))
    l = torch.full((T, hq), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    spa.cascade_attn_run_noalloc(pl, db.q, db.k, db.v, db.bt, db.qsl, db.sl, o, l)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return pl.info, o_ref, l_ref, o, l


SEQUENCES = [
    # (first, mode), (second, mode): the second needs less workspace
    (("worked_decode", "on"), ("tiny_decode", "on")),
    (("mixed_prefill_capped", "on"), ("decode_ragged", "on")),
    (("long_doc", "auto"), ("decode_ragged", "off")),
    (("multi_doc", "on"), ("decode_ragged", "on")),   # nested levels, then none
]

SMALL = {
    "decode_ragged": Workload("decode_ragged", 16, 512, (33, 47), (1, 1), 32, 8, 128, seed=2001),
}


def _batch(name):
    return workloads.make_batch(SMALL[name] if name in SMALL else workloads.get(name))


@pytest.mark.parametrize("first,second", SEQUENCES)
def test_noalloc_matches_run_on_two_calls(first, second):
    sizes = []
    for name, mode in (first, second):
        log(f"[noalloc] {name} mode={mode}")
        b = _batch(name)
        info, o_ref, l_ref, o, l = _both(b, mode)
        sizes.append(info["workspace_bytes"])
        log(f"  cascade={info['use_cascade']} workspace={info['workspace_bytes']} slots={info['num_partial_slots']}")
        assert info["workspace_bytes"] <= spa._lib.NOALLOC_WORKSPACE_BYTES
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(l, l_ref)
        if b.workload.num_reqs <= 16:
            ref_o, ref_l = oracle_ref(b)
            assert_close(o.float().cpu().numpy(), l.cpu().numpy(), ref_o, ref_l, what=f"{name}/{mode}/noalloc")
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_a_plan_beyond_its_array():
    b = workloads.make_batch(workloads.get("mixed_prefill"))
    db = DeviceBatch(b)
    pl = plan(b, mode="on", k_cache=db.k, partials_fp32=True)
    assert pl.workspace_bytes > spa._lib.NOALLOC_WORKSPACE_BYTES
    out = torch.empty_like(db.q)
    with pytest.raises(spa.CascadeAttnError) as e:
        spa.cascade_attn_run_noalloc(pl, db.q, db.k, db.v, db.bt, db.qsl, db.sl, out)
    assert e.value.status == 4 and "at most" in str(e.value)
