"""A run captured in a HIP graph: cascade_attn_run performs no host
synchronisation, no host-to-device copy, no allocation and no memset, so a
caller can capture it once and replay it. Every replay is checked against the
eager result of the same inputs, with eager work (another run on other inputs,
a host synchronisation) between replays."""

import pytest
import torch

import workloads
import shared_prefix_attention_amd as spa
from parity_util import DeviceBatch, assert_close, log, oracle_ref, plan

pytestmark = pytest.mark.gpu


def setup_module():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name,mode", [("tiny_decode", "on"), ("worked_decode", "auto"),
                                       ("mixed_prefill", "on"), ("mixed_prefill", "off"),
                                       ("worked_decode_fp8", "auto"), ("multi_doc", "on")])
def test_graph_replays_match_eager(name, mode):
    log(f"[graph] {name} mode={mode}")
    b = workloads.make_batch(workloads.get(name))
    db = DeviceBatch(b)
    pl = plan(b, mode=mode)
    out = torch.empty_like(db.q)
    lse = torch.empty(b.total_q, b.workload.num_q_heads, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(pl.workspace_bytes, 256), dtype=torch.uint8, device="cuda")

    def run_into(o, l):
        spa.cascade_attn_run(pl, db.q, db.k, db.v, db.bt, db.qsl, db.sl, o, l, ws)

    eager_o, eager_l = torch.empty_like(out), torch.empty_like(lse)
    run_into(eager_o, eager_l)
    torch.cuda.synchronize()
    if name == "tiny_decode":   # small enough to pin the eager result to the oracle as well
        ref_o, ref_l = oracle_ref(b)
        assert_close(eager_o.float().cpu().numpy(), eager_l.cpu().numpy(), ref_o, ref_l, what=f"{name}/eager")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        run_into(out, lse)                 # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            run_into(out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = DeviceBatch(b)
    other.q = torch.flip(db.q, dims=[0]).contiguous()   # different inputs for the eager work in between
    other_o, other_l = torch.empty_like(out), torch.empty_like(lse)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o), f"replay {rep}: output differs from the eager run"
        assert torch.equal(lse, eager_l), f"replay {rep}: LSE differs from the eager run"
        spa.cascade_attn_run(pl, other.q, db.k, db.v, db.bt, db.qsl, db.sl, other_o, other_l, ws)
        torch.cuda.synchronize()
