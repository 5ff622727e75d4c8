"""ctypes binding of ``include/cascade_attn.h`` (argument marshalling only).

Every computation happens in ``libcascade_attn.so`` (host planner + HIP
kernels). Loading fails loudly when the library has not been built; there is
no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcascade_attn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "cascade_attn.h")

CA_OK, CA_EINVAL, CA_EUNSUPPORTED, CA_EMETA, CA_EWORKSPACE, CA_EHIP = range(6)
MODE_AUTO, MODE_FORCE_ON, MODE_FORCE_OFF = 0, 1, 2
KV_BF16, KV_FP8_E4M3 = 0, 1
_KV_DTYPES = {"bf16": KV_BF16, "fp8": KV_FP8_E4M3, "fp8_e4m3": KV_FP8_E4M3}
_MODES = {"auto": MODE_AUTO, "on": MODE_FORCE_ON, "off": MODE_FORCE_OFF}
KERNEL_KINDS = ("cascade_phases", "attention", "merge", "decode", "prefix", "suffix", "level1")


class CascadeAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"cascade_attn status {status}: {message}")
        self.status = status


class ca_params_t(ctypes.Structure):
    _fields_ = [
        ("num_reqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("separate_phases", ctypes.c_int32),
        ("kv_stride_page", ctypes.c_int64),
        ("kv_stride_token", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("mode", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("heads_per_item", ctypes.c_int32),
        ("max_levels", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("sliding_window", ctypes.c_int32),
        ("prefix_splits", ctypes.c_int32),
        ("suffix_order", ctypes.c_int32),
        ("partials_fp32", ctypes.c_int32),
        ("merge_mode", ctypes.c_int32),
        ("use_tuned", ctypes.c_int32),
    ]


class ca_plan_info_t(ctypes.Structure):
    _fields_ = [
        ("use_cascade", ctypes.c_int32),
        ("num_common_prefix_blocks", ctypes.c_int32),
        ("common_prefix_len", ctypes.c_int32),
        ("gates_pass", ctypes.c_int32),
        ("prefix_splits", ctypes.c_int32),
        ("prefix_row_tile", ctypes.c_int32),
        ("suffix_chunks", ctypes.c_int32),
        ("suffix_chunk_tokens", ctypes.c_int32),
        ("suffix_kernel", ctypes.c_int32),
        ("num_partial_slots", ctypes.c_int32),
        ("prefix_stages", ctypes.c_int32),
        ("suffix_stages", ctypes.c_int32),
        ("merge_in_launch", ctypes.c_int32),
        ("suffix_heads_per_item", ctypes.c_int32),
        ("separate_phases", ctypes.c_int32),
        ("num_level1_groups", ctypes.c_int32),
        ("level1_splits", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("suffix_longest_first", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("kv_tokens_cascade", ctypes.c_int64),
        ("kv_tokens_noncascade", ctypes.c_int64),
        ("est_us_cascade", ctypes.c_float),
        ("est_us_noncascade", ctypes.c_float),
        ("partials_fp32", ctypes.c_int32),
        ("shared_levels", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_i32p = ctypes.POINTER(ctypes.c_int32)
_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m shared_prefix_attention_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.cascade_attn_last_error.restype = ctypes.c_char_p
    lib.cascade_attn_num_common_prefix_blocks.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, _i32p,
                                                          ctypes.c_int32, _i32p]
    lib.cascade_attn_plan.argtypes = [ctypes.POINTER(ca_params_t), _i32p, _i32p, _i32p, _i32p,
                                      ctypes.POINTER(ctypes.c_void_p)]
    lib.cascade_attn_plan_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(ca_plan_info_t)]
    lib.cascade_attn_run.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 3 + [ctypes.c_void_p] * 3 + \
        [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.cascade_attn_run_noalloc.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 3 + [ctypes.c_void_p] * 3 + \
        [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.cascade_attn_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.cascade_attn_plan_groups.argtypes = [ctypes.c_void_p, ctypes.c_int32, _i32p, _i32p, _i32p]
    lib.cascade_attn_autotune.argtypes = [ctypes.POINTER(ca_params_t), _i32p, _i32p, _i32p, _i32p] + \
        [ctypes.c_void_p] * 10 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                  ctypes.POINTER(ctypes.c_float)]
    lib.cascade_attn_autotune_record.argtypes = [ctypes.POINTER(ca_params_t), _i32p, _i32p, _i32p, _i32p] + \
        [ctypes.c_int32] * 4
    lib.cascade_attn_autotune_reset.argtypes = []
    lib.cascade_attn_autotune_reset.restype = None
    lib.cascade_attn_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.cascade_attn_plan_destroy.restype = None
    lib.cascade_attn_profile_enable.argtypes = [ctypes.c_int32]
    lib.cascade_attn_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    for name in ("cascade_attn_num_common_prefix_blocks", "cascade_attn_plan", "cascade_attn_plan_info",
                 "cascade_attn_plan_groups", "cascade_attn_run", "cascade_attn_run_noalloc", "cascade_attn_workspace_init", "cascade_attn_autotune", "cascade_attn_autotune_record",
                 "cascade_attn_profile_enable", "cascade_attn_profile_read"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def header_symbols():
    """Function names declared in include/cascade_attn.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(cascade_attn_[a-z_]+)\s*\(", text)))


def _check(status: int):
    if status != CA_OK:
        msg = load().cascade_attn_last_error().decode(errors="replace")
        raise CascadeAttnError(status, msg)


def _host_i32(x):
    """Contiguous host int32 buffer (torch CPU tensor or numpy array) + pointer."""
    import numpy as np
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.int32).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    arr = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return arr, arr.ctypes.data_as(_i32p)


def cascade_attn_num_common_prefix_blocks(block_table, seq_lens, page_size: int) -> int:
    bt, bt_p = _host_i32(block_table)
    sl, sl_p = _host_i32(seq_lens)
    out = ctypes.c_int32(0)
    _check(load().cascade_attn_num_common_prefix_blocks(bt_p, int(bt.shape[0]), int(bt.shape[1]), sl_p,
                                                        int(page_size), ctypes.byref(out)))
    return int(out.value)


class Plan:
    """Owns a ``ca_plan_t`` handle; ``info`` holds ``cascade_attn_plan_info``."""

    def __init__(self, handle: int, num_reqs: int):
        self._h = ctypes.c_void_p(handle)
        self.num_reqs = int(num_reqs)
        info = ca_plan_info_t()
        _check(load().cascade_attn_plan_info(self._h, ctypes.byref(info)))
        self.info = info.as_dict()

    @property
    def handle(self):
        return self._h

    @property
    def workspace_bytes(self) -> int:
        return int(self.info["workspace_bytes"])

    def close(self):
        if self._h is not None and self._h.value:
            load().cascade_attn_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _params(*, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int, num_pages: int, kv_strides,
            block_table, query_start_loc, seq_lens, num_computed_tokens=None, softmax_scale: float = 0.0,
            mode="auto", num_cus: int = 0, heads_per_item: int = 0, separate_phases: bool = False,
            max_levels: int = 0, kv_dtype="bf16", k_scale: float = 0.0, v_scale: float = 0.0,
            sliding_window: int = 0, prefix_splits: int = 0, suffix_order: int = 0,
            partials_fp32: bool = False, use_tuned: bool = False, merge_mode: int = 0):
    """ca_params_t plus the host metadata arrays and their pointers."""
    bt, bt_p = _host_i32(block_table)
    qsl, qsl_p = _host_i32(query_start_loc)
    sl, sl_p = _host_i32(seq_lens)
    nc, nc_p = None, None
    if num_computed_tokens is not None:
        nc, nc_p = _host_i32(num_computed_tokens)
    if bt.ndim != 2 or qsl.shape[0] != bt.shape[0] + 1 or sl.shape[0] != bt.shape[0]:
        raise CascadeAttnError(CA_EINVAL, "block_table [N, stride], query_start_loc [N+1], seq_lens [N] expected")
    prm = ca_params_t()
    prm.num_reqs = int(bt.shape[0])
    prm.num_q_heads = int(num_q_heads)
    prm.num_kv_heads = int(num_kv_heads)
    prm.head_dim = int(head_dim)
    prm.page_size = int(page_size)
    prm.block_table_stride = int(bt.shape[1])
    prm.num_pages = int(num_pages)
    prm.kv_stride_page, prm.kv_stride_token, prm.kv_stride_head = (int(s) for s in kv_strides)
    prm.softmax_scale = float(softmax_scale)
    prm.mode = _MODES[mode] if isinstance(mode, str) else int(mode)
    prm.num_cus = int(num_cus)
    prm.heads_per_item = int(heads_per_item)
    prm.separate_phases = int(separate_phases)
    prm.max_levels = int(max_levels)
    prm.kv_dtype = _KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    prm.k_scale = float(k_scale)
    prm.v_scale = float(v_scale)
    prm.sliding_window = int(sliding_window)
    prm.prefix_splits = int(prefix_splits)
    prm.suffix_order = int(suffix_order)
    prm.partials_fp32 = int(partials_fp32)
    prm.use_tuned = int(use_tuned)
    prm.merge_mode = int(merge_mode)
    keep = (bt, qsl, sl, nc)   # the arrays behind the pointers
    return prm, (bt_p, qsl_p, sl_p, nc_p), keep


def cascade_attn_plan(**kw) -> Plan:
    """Host-only planner (see cascade_attn_plan in the header).

    Keywords: num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
    kv_strides ((page, token-slot, head) element strides of the caches),
    block_table, query_start_loc, seq_lens, num_computed_tokens (host int32
    arrays or CPU tensors), and the optional ca_params_t settings
    softmax_scale, mode, num_cus, heads_per_item, separate_phases,
    max_levels, kv_dtype, k_scale, v_scale, sliding_window, prefix_splits,
    suffix_order, partials_fp32, use_tuned, merge_mode.
    """
    prm, ptrs, keep = _params(**kw)
    h = ctypes.c_void_p(0)
    _check(load().cascade_attn_plan(ctypes.byref(prm), *ptrs, ctypes.byref(h)))
    del keep
    return Plan(h.value, prm.num_reqs)


def cascade_attn_autotune(q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d, out, lse_out,
                          workspace, iters: int = 10, stream=None, sinks=None, **kw):
    """Times candidate plans on the device and returns (best Plan, us per run);
    see cascade_attn_autotune in the header. ``kw`` as for cascade_attn_plan
    (host metadata and settings); device tensors as for cascade_attn_run."""
    import torch
    prm, ptrs, keep = _params(**kw)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    h = ctypes.c_void_p(0)
    us = ctypes.c_float(0.0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().cascade_attn_autotune(
        ctypes.byref(prm), *ptrs, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table_d.data_ptr(),
        query_start_loc_d.data_ptr(), seq_lens_d.data_ptr(), sinks.data_ptr() if sinks is not None else None,
        out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None,
        workspace.data_ptr() if workspace is not None else None, ws_bytes, s, int(iters), ctypes.byref(h),
        ctypes.byref(us)))
    del keep
    return Plan(h.value, prm.num_reqs), float(us.value)


def cascade_attn_autotune_record(mode="on", prefix_splits: int = 0, heads_per_item: int = 0, max_levels: int = 0,
                                 **kw) -> None:
    """Records a choice for the batch shape of ``kw`` (as for
    cascade_attn_plan) without timing; see the header."""
    prm, ptrs, keep = _params(**kw)
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    _check(load().cascade_attn_autotune_record(ctypes.byref(prm), *ptrs, m, int(prefix_splits), int(heads_per_item),
                                               int(max_levels)))
    del keep


def cascade_attn_autotune_reset() -> None:
    load().cascade_attn_autotune_reset()


def cascade_attn_plan_info(plan: Plan) -> dict:
    return dict(plan.info)


def cascade_attn_plan_groups(plan: Plan):
    """Nested shared levels of the plan: ([(level, parent, key_begin, key_end)]
    parents first, [innermost group of each request or -1])."""
    n = ctypes.c_int32(0)
    _check(load().cascade_attn_plan_groups(plan.handle, 0, None, None, ctypes.byref(n)))
    cap = int(n.value)
    buf = (ctypes.c_int32 * max(1, 4 * cap))()
    deepest = (ctypes.c_int32 * max(1, plan.num_reqs))()
    _check(load().cascade_attn_plan_groups(plan.handle, cap, buf, deepest, ctypes.byref(n)))
    groups = [tuple(buf[4 * j + i] for i in range(4)) for j in range(cap)]
    return groups, [deepest[r] for r in range(plan.num_reqs)]


def cascade_attn_run(plan: Plan, q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d,
                     out, lse_out=None, workspace=None, stream=None, sinks=None) -> None:
    """Launch one attention step on ``stream`` (default: torch's current stream).

    All tensors are device tensors (torch); see cascade_attn_run in the header
    for dtypes and layouts. ``sinks``: optional [num_q_heads] fp32 tensor.
    """
    import torch
    for name, t in (("q", q), ("out", out)):
        if not t.is_contiguous():
            raise CascadeAttnError(CA_EINVAL, f"{name} must be contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_contiguous()):
        raise CascadeAttnError(CA_EINVAL, "sinks must be a contiguous float32 tensor")
    _check(load().cascade_attn_run(
        plan.handle, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table_d.data_ptr(),
        query_start_loc_d.data_ptr(), seq_lens_d.data_ptr(), sinks.data_ptr() if sinks is not None else None,
        out.data_ptr(),
        lse_out.data_ptr() if lse_out is not None else None, ws_ptr, ws_bytes, s))


NOALLOC_WORKSPACE_BYTES = 32 << 20
WORKSPACE_COUNTER_BYTES = 256 << 10


def cascade_attn_workspace_init(workspace, stream=None) -> None:
    """Zeroes the merge counters at the start of ``workspace`` (a device
    tensor) on ``stream``; needed once unless it was allocated zeroed."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    _check(load().cascade_attn_workspace_init(workspace.data_ptr(), workspace.numel() * workspace.element_size(), s))


def cascade_attn_run_noalloc(plan: Plan, q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d,
                             out, lse_out=None, stream=None, sinks=None) -> None:
    """cascade_attn_run with the library's own per-GPU workspace (no device
    allocation anywhere in the call); see the header for its limit and for
    calls that overlap on one GPU."""
    import torch
    for name, t in (("q", q), ("out", out)):
        if not t.is_contiguous():
            raise CascadeAttnError(CA_EINVAL, f"{name} must be contiguous")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_contiguous()):
        raise CascadeAttnError(CA_EINVAL, "sinks must be a contiguous float32 tensor")
    _check(load().cascade_attn_run_noalloc(
        plan.handle, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table_d.data_ptr(),
        query_start_loc_d.data_ptr(), seq_lens_d.data_ptr(), sinks.data_ptr() if sinks is not None else None,
        out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None, s))


def cascade_attn_profile_enable(capacity: int = 4096) -> None:
    """Creates a pool of timing events for ``capacity`` kernel launches (0:
    timing off, pool freed); see the header."""
    _check(load().cascade_attn_profile_enable(int(capacity)))


def cascade_attn_profile_read():
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(load().cascade_attn_profile_read(ms, cnt))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_KINDS)}
