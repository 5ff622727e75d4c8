"""Helpers for GPU parity tests: device transfer, running the library through
its C ABI, oracle evaluation and the tolerance check."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import shared_prefix_attention_amd as spa

OUT_ABS, OUT_REL, LSE_ABS = 2e-2, 1e-2, 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceBatch:
    def __init__(self, b, layout="NHD", device="cuda"):
        self.b = b
        self.layout = layout
        self.q = b.q.to(device)
        if layout == "NHD":
            self.k = b.k_cache.to(device)
            self.v = b.v_cache.to(device)
        else:   # HND: [pages, Hkv, page_size, d]
            self.k = b.k_cache.permute(0, 2, 1, 3).contiguous().to(device)
            self.v = b.v_cache.permute(0, 2, 1, 3).contiguous().to(device)
        self.bt = b.block_table.to(device)
        self.qsl = b.query_start_loc.to(device)
        self.sl = b.seq_lens.to(device)


def plan(b, mode="auto", layout="NHD", k_cache=None, **kw):
    w = b.workload
    if w.kv_dtype == "fp8":
        kw.setdefault("k_scale", w.k_scale)
        kw.setdefault("v_scale", w.v_scale)
    cache = b.k_cache if layout == "NHD" else b.k_cache.permute(0, 2, 1, 3).contiguous()
    if k_cache is not None:
        cache = k_cache
    return spa.plan_batch(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                          k_cache=cache, block_table=b.block_table, query_start_loc=b.query_start_loc,
                          seq_lens=b.seq_lens, num_computed_tokens=b.num_computed, layout=layout, mode=mode, **kw)


def run(db: DeviceBatch, mode="auto", sinks=None, **kw):
    pl = plan(db.b, mode=mode, layout=db.layout, k_cache=db.k, **kw)
    sinks_d = None if sinks is None else torch.as_tensor(sinks, dtype=torch.float32).cuda().contiguous()
    out, lse = spa.run_batch(pl, db.q, db.k, db.v, db.bt, db.qsl, db.sl, sinks=sinks_d)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), pl.info


def oracle_kv(b):
    """The caches' values for the oracle: bf16 as is, fp8 codes decoded by the
    oracle's own E4M3 decoder times the scales."""
    w = b.workload
    if w.kv_dtype == "fp8":
        return (oracle.fp8_e4m3_decode(b.k_cache.numpy()) * w.k_scale,
                oracle.fp8_e4m3_decode(b.v_cache.numpy()) * w.v_scale)
    return b.k_cache.float().numpy(), b.v_cache.float().numpy()


def oracle_ref(b, requests=None, window=0, sinks=None):
    k, v = oracle_kv(b)
    return oracle.attention_full(b.q.float().numpy(), k, v,
                                 b.block_table.numpy(), b.query_start_loc.numpy(), b.seq_lens.numpy(),
                                 b.workload.page_size, scale=b.workload.softmax_scale, requests=requests,
                                 window=window, sinks=None if sinks is None else np.asarray(sinks, dtype=np.float64))


def rows_of(b, requests):
    qsl = b.query_start_loc
    idx = []
    for r in requests:
        idx.extend(range(int(qsl[r]), int(qsl[r + 1])))
    return np.array(idx, dtype=np.int64)


def assert_close(out, lse, ref_o, ref_l, rows=None, what=""):
    if rows is not None:
        out, lse, ref_o, ref_l = out[rows], lse[rows], ref_o[rows], ref_l[rows]
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    assert np.isfinite(lse).all(), f"{what}: non-finite lse"
    err = np.abs(out - ref_o)
    bound = OUT_ABS + OUT_REL * np.abs(ref_o)
    bad = err > bound
    lerr = np.abs(lse - ref_l)
    big = np.abs(ref_o) > OUT_ABS
    max_rel = float((err[big] / np.abs(ref_o[big])).max()) if big.any() else 0.0
    log(f"  {what}: out max-abs {err.max():.3e} max-rel {max_rel:.3e}; lse max-abs {lerr.max():.3e}")
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside 2e-2 + 1e-2|ref| (max abs {err.max():.3e})"
    assert lerr.max() <= LSE_ABS, f"{what}: lse max-abs {lerr.max():.3e} > 1e-3"
