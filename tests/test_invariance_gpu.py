"""GPU invariance tests: the failure the pages report is output that changes
with batch composition and tensor-parallel size ("Diary - vLLM's cascade
attention"). A request's result here must not depend on which other requests
share the batch, on their order, on physical page placement, or on how many
heads a GPU holds -- bitwise when the plan's partition is the same, within the
parity tolerance otherwise -- and runs must be deterministic."""

import numpy as np
import pytest
import torch

import workloads
from parity_util import DeviceBatch, assert_close, log, oracle_ref, run, rows_of

pytestmark = pytest.mark.gpu


def setup_module():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _reorder(b, order):
    qsl = b.query_start_loc
    qs = [b.q[int(qsl[r]):int(qsl[r + 1])] for r in order]
    lens = torch.tensor([int(qsl[r + 1] - qsl[r]) for r in order])
    new_qsl = torch.zeros(len(order) + 1, dtype=torch.int32)
    new_qsl[1:] = torch.cumsum(lens, 0)
    return workloads.Batch(b.workload, torch.cat(qs), b.k_cache, b.v_cache, b.block_table[order].contiguous(),
                           new_qsl, b.seq_lens[order].contiguous(), b.num_computed[order].contiguous())


SCALARS = ("use_cascade", "common_prefix_len", "prefix_splits", "prefix_row_tile", "suffix_chunks",
           "suffix_chunk_tokens", "suffix_kernel")


@pytest.mark.parametrize("name", ["worked_decode", "mixed_prefill"])
def test_run_twice_is_bitwise_identical(name):
    log(f"[invariance] determinism {name}")
    db = DeviceBatch(workloads.make_batch(workloads.get(name)))
    for mode in ("on", "off"):
        o1, l1, _ = run(db, mode=mode)
        o2, l2, _ = run(db, mode=mode)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", ["worked_decode", "mixed_prefill", "multi_doc", "multi_doc_prefill"])
def test_request_permutation_is_bitwise_invariant(name):
    """Shuffled requests give every request bitwise the same rows. For the
    batches with documents the shuffle scatters each document's requests
    over the batch, so the permuted plan's nested groups have members that
    are not adjacent (the prefix tree puts them in its own order)."""
    log(f"[invariance] permutation {name}")
    b = workloads.make_batch(workloads.get(name))
    n = b.workload.num_reqs
    order = list(np.random.default_rng(3).permutation(n))
    b2 = _reorder(b, order)
    for mode in ("on", "off"):
        o1, l1, i1 = run(DeviceBatch(b), mode=mode)
        o2, l2, i2 = run(DeviceBatch(b2), mode=mode)
        assert all(i1[k] == i2[k] for k in SCALARS)
        q1, q2 = b.query_start_loc, b2.query_start_loc
        for new_r, r in enumerate(order):
            a = slice(int(q1[r]), int(q1[r + 1]))
            c = slice(int(q2[new_r]), int(q2[new_r + 1]))
            assert np.array_equal(o1[a], o2[c]) and np.array_equal(l1[a], l2[c])


def test_page_relabel_is_bitwise_invariant():
    log("[invariance] page relabel")
    b = workloads.make_batch(workloads.get("worked_decode"))
    n = b.num_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(9))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(n)
    b2 = workloads.Batch(b.workload, b.q, b.k_cache[inv].contiguous(), b.v_cache[inv].contiguous(),
                         perm[b.block_table.long()].to(torch.int32), b.query_start_loc, b.seq_lens, b.num_computed)
    for mode in ("on", "off"):
        o1, l1, _ = run(DeviceBatch(b), mode=mode)
        o2, l2, _ = run(DeviceBatch(b2), mode=mode)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


_FULL_REF = {}


@pytest.mark.parametrize("n_sub", [8, 16, 50, 63])
def test_batch_size_does_not_change_a_request(n_sub):
    """Sub-batches of the worked example (the report saw breakage at batch 50
    but not 100): every request of the sub-batch matches the full batch and,
    row by row, the oracle."""
    log(f"[invariance] sub-batch {n_sub}")
    b = workloads.make_batch(workloads.get("worked_decode"))
    sub = _reorder(b, list(range(n_sub)))
    o_full, l_full, _ = run(DeviceBatch(b), mode="auto")
    o_sub, l_sub, info = run(DeviceBatch(sub), mode="auto")
    rows = rows_of(b, range(n_sub))
    assert np.all(np.abs(o_sub - o_full[rows]) <= 2e-2 + 1e-2 * np.abs(o_full[rows]))
    assert np.abs(l_sub - l_full[rows]).max() <= 1e-3
    # the sub-batch's requests are the full batch's first n_sub (same inputs)
    if "worked_decode" not in _FULL_REF:
        _FULL_REF["worked_decode"] = oracle_ref(b)
    ref_o, ref_l = _FULL_REF["worked_decode"]
    assert_close(o_sub, l_sub, ref_o[rows], ref_l[rows], what=f"sub{n_sub}")


def test_tensor_parallel_head_slice():
    """One GPU's share under tensor parallelism: the KV heads [2, 4) and their
    query heads, run alone, equal those heads of the full run."""
    log("[invariance] TP head slice")
    b = workloads.make_batch(workloads.get("worked_decode"))
    w = b.workload
    G = w.num_q_heads // w.num_kv_heads
    g0, g1 = 2, 4
    w2 = workloads.Workload("tp_slice", w.num_reqs, w.prefix, w.suffix, w.q_len, (g1 - g0) * G, g1 - g0,
                            w.head_dim, seed=w.seed)
    b2 = workloads.Batch(w2, b.q[:, g0 * G:g1 * G].contiguous(), b.k_cache[:, :, g0:g1].contiguous(),
                         b.v_cache[:, :, g0:g1].contiguous(), b.block_table, b.query_start_loc, b.seq_lens,
                         b.num_computed)
    for mode in ("on", "off"):
        o1, l1, i1 = run(DeviceBatch(b), mode=mode)
        o2, l2, i2 = run(DeviceBatch(b2), mode=mode)
        ref1, ref2 = o1[:, g0 * G:g1 * G], l1[:, g0 * G:g1 * G]
        same_partition = all(i1[k] == i2[k] for k in SCALARS)
        log(f"  {mode}: same partition {same_partition}")
        if same_partition:
            assert np.array_equal(o2, ref1) and np.array_equal(l2, ref2)
        else:
            assert np.all(np.abs(o2 - ref1) <= 2e-2 + 1e-2 * np.abs(ref1))
            assert np.abs(l2 - ref2).max() <= 1e-3
