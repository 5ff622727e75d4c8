"""Convenience wrappers over the C ABI for torch tensors (marshalling only)."""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from ._lib import Plan, cascade_attn_plan, cascade_attn_run


def kv_strides(cache: torch.Tensor, layout: str = "NHD") -> Tuple[int, int, int]:
    """(page, token-slot, head) element strides of a paged cache tensor.

    NHD: cache is [num_pages, page_size, Hkv, d]; HND: [num_pages, Hkv, page_size, d].
    """
    if cache.stride(-1) != 1:
        raise ValueError("head_dim must be contiguous")
    if layout == "NHD":
        return cache.stride(0), cache.stride(1), cache.stride(2)
    if layout == "HND":
        return cache.stride(0), cache.stride(2), cache.stride(1)
    raise ValueError(layout)


def plan_batch(*, num_q_heads: int, num_kv_heads: int, head_dim: int, k_cache: torch.Tensor,
               block_table, query_start_loc, seq_lens, num_computed_tokens=None, page_size: int = 16,
               layout: str = "NHD", mode="auto", softmax_scale: float = 0.0, num_cus: int = 0,
               heads_per_item: int = 0, separate_phases: bool = False, max_levels: int = 0,
               kv_dtype=None, k_scale: float = 0.0, v_scale: float = 0.0, sliding_window: int = 0,
               prefix_splits: int = 0, suffix_order: int = 0, partials_fp32: bool = False,
               use_tuned: bool = False, merge_mode: int = 0) -> Plan:
    """Plan from host metadata; strides and pool size are read off ``k_cache``.

    kv_dtype: "bf16" or "fp8"; by default taken from ``k_cache`` (bf16, or a
    one-byte dtype for fp8 e4m3 bytes).
    """
    if kv_dtype is None:
        kv_dtype = "bf16" if k_cache.element_size() == 2 else "fp8"
    return cascade_attn_plan(
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
        num_pages=k_cache.shape[0], kv_strides=kv_strides(k_cache, layout), block_table=block_table,
        query_start_loc=query_start_loc, seq_lens=seq_lens, num_computed_tokens=num_computed_tokens,
        softmax_scale=softmax_scale, mode=mode, num_cus=num_cus, heads_per_item=heads_per_item,
        separate_phases=separate_phases, max_levels=max_levels, kv_dtype=kv_dtype, k_scale=k_scale,
        v_scale=v_scale, sliding_window=sliding_window, prefix_splits=prefix_splits, suffix_order=suffix_order,
        partials_fp32=partials_fp32, use_tuned=use_tuned, merge_mode=merge_mode)


def run_batch(plan: Plan, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              block_table_d: torch.Tensor, query_start_loc_d: torch.Tensor, seq_lens_d: torch.Tensor,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None, sinks: Optional[torch.Tensor] = None):
    """Run the plan; allocates out / lse / workspace with torch when not given
    (the workspace zeroed, as its merge counters must start at zero)."""
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    if workspace is None and plan.workspace_bytes > 0:
        workspace = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=q.device)
    cascade_attn_run(plan, q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d, out, lse,
                     workspace, stream, sinks)
    return out, lse
