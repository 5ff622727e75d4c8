// Launcher: cascade_attn_run() and the kernel-timing hooks.
//
// Cascade path ("vLLM Cascade Attention：用法、场景与原理解析", beaiera.top,
// section 8 Step 5): prefix phase (all queries, shared pages, non-causal) ->
// suffix phase (per request, own pages, causal) -> LSE merge. Non-cascade
// path (Step 4): one attention over each request's whole block table, plus
// a merge when the plan splits the KV range. All launches go to the
// caller's stream in order; nothing here allocates or synchronises.

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <vector>

#include "attn_tile.hpp"
#include "merge.hpp"
#include "plan.h"

using namespace ca;

namespace {

enum KernelKind { K_PHASES = 0, K_ATTN = 1, K_MERGE = 2, K_DECODE = 3, K_PREFIX = 4, K_SUFFIX = 5, K_LEVEL1 = 6, K_KINDS = 7 };
static_assert(kMaxGroups == kMaxTreeGroups && kMaxLevels == kMaxShared && kMaxTreeOrder == kOrderCapacity, "group table size");
static_assert(kOrderCapacity == kMaxOrderedReqs, "request order table size");
static_assert(K_KINDS == CA_PROFILE_KINDS, "profile kinds");

// Kernel timing for measurement: a pool of HIP events created when timing
// is enabled (outside any timed region); each launch takes the next start /
// stop pair, recorded on the launch stream right before and right after it
// (hipEventRecord markers, events without a system-scope fence: no event is
// created and no host work is added between launches). When the pool is
// used up, further launches run untimed.
struct Profiler {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> pool;   // 2 * capacity events
  struct Rec {
    int kind;
    int slot;                     // events pool[2 slot], pool[2 slot + 1]
  };
  std::vector<Rec> recs;
  size_t next = 0;
  int64_t dropped = 0;            // launches past the pool's capacity
  void release() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
    pool.clear();
    recs.clear();
    next = 0;
    dropped = 0;
  }
};
Profiler g_prof;

template <typename K, typename... Args>
void launch(int kind, K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> g(g_prof.mu);
    if (g_prof.enabled) {
      if (2 * g_prof.next + 1 < g_prof.pool.size()) {
        a = g_prof.pool[2 * g_prof.next];
        b = g_prof.pool[2 * g_prof.next + 1];
        g_prof.recs.push_back({kind, (int)g_prof.next});
        ++g_prof.next;
      } else {
        ++g_prof.dropped;
      }
    }
  }
  if (a) (void)hipEventRecord(a, s);
  hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  if (b) (void)hipEventRecord(b, s);
}

ca_status_t fail(ca_status_t c, const std::string& m) {
  set_error(m);
  return c;
}

ca_status_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(CA_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return CA_OK;
}

template <int D, int RB, int RW, int KG, int NS, bool F8>
void launch_tile(const TileArgs& args, const GroupTable& gt, const ReqOrder& ro, const MergeTailArgs& mt, int grid,
                 hipStream_t s, int kind) {
  constexpr bool MH = (KG > 1) && !F8;
  // Launches whose role needs no sliding-window or sink code (shared-prefix
  // items never do; per-request items when the batch has neither) take a
  // variant without it and with the role fixed, which holds fewer scalar
  // registers through the stage loop. (128-row shared-prefix tiles measured
  // ~1.5 % slower that way and keep the general variant.)
  if constexpr (RB == 1 && RW == 4) {
    if (gt.n == 0 && args.prefix_mode == 1) {
      launch(kind, attn_tile_kernel<D, RB, RW, KG, NS, 64, MH, F8, false, false, 1>, dim3(grid), dim3(64 * RW * KG),
             s, args, NoGroupTable{}, ro, mt);
      return;
    }
  }
  if (gt.n > 0)
    launch(kind, attn_tile_kernel<D, RB, RW, KG, NS, 64, MH, F8, true>, dim3(grid), dim3(64 * RW * KG), s, args, gt,
           ro, mt);
  else if (args.window > 0 || args.sinks || args.prefix_mode != 0)
    launch(kind, attn_tile_kernel<D, RB, RW, KG, NS, 64, MH, F8, false>, dim3(grid), dim3(64 * RW * KG), s, args,
           NoGroupTable{}, ro, mt);
  else
    launch(kind, attn_tile_kernel<D, RB, RW, KG, NS, 64, MH, F8, false, false, 0>, dim3(grid), dim3(64 * RW * KG),
           s, args, NoGroupTable{}, ro, mt);
}

// bf16 caches: 2 or 4 stages of 64 keys; fp8 caches (head_dim 128 only):
// 4 stages, the same 64 KB of LDS.
template <int D, int RB, int RW, int KG>
void launch_tile_ns(const TileArgs& args, const GroupTable& gt, const ReqOrder& ro, const MergeTailArgs& mt, int ns,
                    bool f8, int grid, hipStream_t s, int kind) {
  if constexpr (D == 128) {
    if (f8) {
      launch_tile<D, RB, RW, KG, 4, true>(args, gt, ro, mt, grid, s, kind);
      return;
    }
  }
  if (ns == 4) launch_tile<D, RB, RW, KG, 4, false>(args, gt, ro, mt, grid, s, kind);
  else launch_tile<D, RB, RW, KG, 2, false>(args, gt, ro, mt, grid, s, kind);
}

bool item_ok(const PhaseTile& ph) { return ph.split_tokens > 0 && ph.split_tokens <= kMaxItemTokens && ph.split_tokens % kTileKeys == 0; }

// 4-wave work-group shapes (row_blocks, row_waves, key_groups):
// 0 = rows (1,4,1), 1 = MFMA (2,4,1), 2 = decode (1,1,4)
int shape_id(const PhaseTile& ph) {
  if (ph.row_blocks == 1 && ph.row_waves == 4 && ph.key_groups == 1) return 0;
  if (ph.row_blocks == 2 && ph.row_waves == 4 && ph.key_groups == 1) return 1;
  if (ph.row_blocks == 1 && ph.row_waves == 1 && ph.key_groups == 4) return 2;
  return -1;
}

template <int D>
ca_status_t run_tile(const TileArgs& args, const GroupTable& gt, const ReqOrder& ro, const MergeTailArgs& mt,
                     const PhaseTile& ph, int64_t grid, bool f8, hipStream_t s, int kind) {
  if (grid <= 0) return CA_OK;
  if (grid > 0x7fffffff) return fail(CA_EINVAL, "grid too large");
  if (!item_ok(ph)) return fail(CA_EINVAL, "work item exceeds the per-item KV limit");
  if (f8 && (D != 128 || ph.stages != 4)) return fail(CA_EINVAL, "fp8 plan needs head_dim 128 and 4 stages");
  switch (shape_id(ph)) {
    case 0: launch_tile_ns<D, 1, 4, 1>(args, gt, ro, mt, ph.stages, f8, (int)grid, s, kind); break;
    case 1: launch_tile_ns<D, 2, 4, 1>(args, gt, ro, mt, ph.stages, f8, (int)grid, s, kind); break;
    case 2: launch_tile_ns<D, 1, 1, 4>(args, gt, ro, mt, ph.stages, f8, (int)grid, s, kind); break;
    default: return fail(CA_EINVAL, "unsupported work-group shape in plan");
  }
  return check_launch("attention kernel launch");
}

// All roles 64-key stages in 64 KB of LDS (two work-groups per CU): 2 stages
// of bf16, or 4 of fp8.
template <int D, int P, int S, bool F8>
void launch_phases(const TileArgs& pa, const TileArgs& ga, const TileArgs& sa, int n_prefix, int n_group,
                   const GroupTable& gt, const ReqOrder& ro, const MergeTailArgs& mt, int grid, hipStream_t s) {
  constexpr int PRB = P == 1 ? 2 : 1;
  constexpr int SRW = S == 2 ? 1 : 4, SKG = S == 2 ? 4 : 1;
  constexpr int NS = F8 ? 4 : 2;
  if (gt.n > 0)
    launch(K_PHASES, cascade_phases_kernel<D, PRB, 4, 1, NS, 64, 1, SRW, SKG, NS, 64, F8, true>, dim3(grid),
           dim3(256), s, pa, ga, sa, n_prefix, n_group, gt, ro, mt);
  else
    launch(K_PHASES, cascade_phases_kernel<D, PRB, 4, 1, NS, 64, 1, SRW, SKG, NS, 64, F8, false>, dim3(grid),
           dim3(256), s, pa, ga, sa, n_prefix, 0, NoGroupTable{}, ro, mt);
}

template <int D, bool F8>
void launch_phases_shapes(int pid, int sid, const TileArgs& pa, const TileArgs& ga, const TileArgs& sa, int np,
                          int ng, const GroupTable& gt, const ReqOrder& ro, const MergeTailArgs& mt, int grid,
                          hipStream_t s) {
  if (sid == 0) {
    if (pid == 0) launch_phases<D, 0, 0, F8>(pa, ga, sa, np, ng, gt, ro, mt, grid, s);
    else launch_phases<D, 1, 0, F8>(pa, ga, sa, np, ng, gt, ro, mt, grid, s);
  } else {
    if (pid == 0) launch_phases<D, 0, 2, F8>(pa, ga, sa, np, ng, gt, ro, mt, grid, s);
    else launch_phases<D, 1, 2, F8>(pa, ga, sa, np, ng, gt, ro, mt, grid, s);
  }
}

template <int D>
ca_status_t run_phases(const TileArgs& pa, const PhaseTile& pp, int64_t n_prefix, const TileArgs& ga,
                       int64_t n_group, const GroupTable& gt, const ReqOrder& ro, const TileArgs& sa, const PhaseTile& sp,
                       int64_t n_suffix, const MergeTailArgs& mt, bool f8, hipStream_t s) {
  if (n_prefix + n_group + n_suffix > 0x7fffffff) return fail(CA_EINVAL, "grid too large");
  if (!item_ok(pp) || !item_ok(sp)) return fail(CA_EINVAL, "work item exceeds the per-item KV limit");
  const int pid = shape_id(pp), sid = shape_id(sp);
  const int ns = f8 ? 4 : 2;
  if ((pid != 0 && pid != 1) || (sid != 0 && sid != 2) || pp.stages != ns || sp.stages != ns || (f8 && D != 128))
    return fail(CA_EINVAL, "unsupported work-group shape in plan");
  const int grid = (int)(n_prefix + n_group + n_suffix);
  const int np = (int)n_prefix, ng = (int)n_group;
  if constexpr (D == 128) {
    if (f8) launch_phases_shapes<D, true>(pid, sid, pa, ga, sa, np, ng, gt, ro, mt, grid, s);
    else launch_phases_shapes<D, false>(pid, sid, pa, ga, sa, np, ng, gt, ro, mt, grid, s);
  } else {
    launch_phases_shapes<D, false>(pid, sid, pa, ga, sa, np, ng, gt, ro, mt, grid, s);
  }
  return check_launch("cascade phases kernel launch");
}

template <int D>
ca_status_t run_merge(const MergeArgs& args, bool f32, hipStream_t s) {
  // more than 16 slots: four slot groups per row, each one batch of loads
  const int sg = args.slots > 16 ? 4 : 1;
  const int rpb = 256 / (D / (f32 ? 4 : 8)) / sg;   // a thread owns 4 fp32 or 8 bf16 values
  const int64_t grid = (args.rows + rpb - 1) / rpb;
  if (grid <= 0) return CA_OK;
  if (grid > 0x7fffffff) return fail(CA_EINVAL, "merge grid too large");
  const dim3 gr((unsigned)grid), bl(256);
  if (sg == 4) {
    if (f32) launch(K_MERGE, merge_kernel<D, true, 4>, gr, bl, s, args);
    else launch(K_MERGE, merge_kernel<D, false, 4>, gr, bl, s, args);
  } else {
    if (f32) launch(K_MERGE, merge_kernel<D, true, 1>, gr, bl, s, args);
    else launch(K_MERGE, merge_kernel<D, false, 1>, gr, bl, s, args);
  }
  return check_launch("merge kernel launch");
}

template <int D>
ca_status_t run_impl(const ca_plan* pl, const void* q, const void* k, const void* v, const int32_t* bt,
                     const int32_t* qsl, const int32_t* sl, const float* sinks, void* out, float* lse, void* ws,
                     hipStream_t s) {
  TileArgs base{};
  base.heads_per_item = 1;
  base.q = static_cast<const uint16_t*>(q);
  base.k = static_cast<const uint16_t*>(k);
  base.v = static_cast<const uint16_t*>(v);
  base.sp = pl->p.kv_stride_page;
  base.st = pl->p.kv_stride_token;
  base.sh = pl->p.kv_stride_head;
  base.bt = bt;
  base.qsl = qsl;
  base.seq_lens = sl;
  base.bt_stride = pl->p.block_table_stride;
  base.hq = pl->hq;
  base.hkv = pl->hkv;
  base.group = pl->group;
  base.scale_log2 = pl->scale * pl->k_scale * kLog2e;   // k dequantisation folded into the scores
  base.v_scale = pl->v_scale;
  base.sinks = sinks;
  base.num_reqs = pl->num_reqs;
  base.slot_elems = pl->slot_elems;
  base.slot_rows = pl->total_q * pl->hq;
  base.out = static_cast<uint16_t*>(out);
  base.lse_out = lse;
  void* part_o = ws ? static_cast<char*>(ws) + pl->ws_o_offset : nullptr;
  float* part_lse = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + pl->ws_lse_offset) : nullptr;
  base.part_o = part_o;
  base.part_fp32 = pl->part_fp32;
  base.part_lse = part_lse;
  // merge inside the attention launch: counters at the workspace's start
  MergeTailArgs mt{};
  mt.counters = (pl->merge_in_launch && ws) ? static_cast<int32_t*>(ws) : nullptr;
  mt.qsl = qsl;
  mt.part_o = part_o;
  mt.part_lse = part_lse;
  mt.out = base.out;
  mt.lse_out = lse;
  mt.sinks = sinks;
  mt.slot_elems = base.slot_elems;
  mt.slot_rows = base.slot_rows;
  mt.part_fp32 = pl->part_fp32;
  mt.merge_slots = pl->num_slots;
  mt.hq = pl->hq;
  mt.hkv = pl->hkv;
  mt.group = pl->group;
  mt.num_reqs = pl->num_reqs;
  mt.m_pre_splits = pl->use_cascade ? pl->prefix.splits : 0;
  mt.m_pre_rows = pl->use_cascade ? pl->prefix.rows_per_wg() : 1;
  mt.m_suf_splits = pl->suffix.splits;
  mt.m_suf_rows = pl->suffix.rows_per_wg();
  mt.m_suf_mtiles = pl->suffix.mtiles;
  mt.uniform_q = pl->uniform_q;
  base.coherent = mt.counters ? 1 : 0;

  // nested shared levels (none: n = 0)
  GroupTable gt{};
  const Tree& T = pl->tree;
  gt.n = pl->use_cascade ? T.n : 0;
  gt.levels = gt.n > 0 ? T.levels : 1;
  gt.uniform_q = pl->uniform_q;
  if (gt.n > kMaxGroups || gt.levels > kMaxLevels || (gt.n > 0 && pl->num_reqs > kMaxTreeOrder))
    return fail(CA_EINVAL, "nested levels exceed the kernel's group table");
  if (gt.n > 0 && mt.counters) return fail(CA_EINVAL, "plans with nested levels merge in a launch of their own");
  for (int l = 0; l < gt.levels; ++l) {
    gt.level_splits[l] = T.level_splits[l];
    gt.level_slot_base[l] = T.level_slot_base[l];
  }
  for (int j = 0; j < gt.n; ++j) {
    gt.item_begin[j] = T.item_begin[j];
    gt.level[j] = T.level[j];
    gt.first_req[j] = T.first_req[j];
    gt.pos_begin[j] = T.pos_begin[j];
    gt.pos_end[j] = T.pos_end[j];
    gt.key_begin[j] = T.key_begin[j];
    gt.key_end[j] = T.key_end[j];
    gt.split_tokens[j] = T.split_tokens[j];
    gt.rows[j] = T.rows[j];
    if (T.split_tokens[j] <= 0 || T.split_tokens[j] > kMaxItemTokens || T.split_tokens[j] % kTileKeys)
      return fail(CA_EINVAL, "group work item exceeds the per-item KV limit");
    if (T.level[j] < 1 || T.level[j] >= gt.levels || T.pos_begin[j] < 0 || T.pos_end[j] > pl->num_reqs ||
        T.pos_begin[j] >= T.pos_end[j])
      return fail(CA_EINVAL, "malformed group table in plan");
  }
  gt.item_begin[gt.n] = gt.n > 0 ? T.item_begin[gt.n] : 0;
  if (gt.n > 0) {
    for (int r = 0; r < pl->num_reqs; ++r) {
      gt.pos_tok[r] = T.pos_tok[r];
      gt.pos_cum[r] = T.pos_cum[r];
      gt.deepest[r] = T.deepest[r];
    }
    gt.pos_cum[pl->num_reqs] = T.pos_cum[pl->num_reqs];
  }

  // dispatch order of the per-request items (n = 0: batch order)
  ReqOrder ro{};
  ro.n = pl->order_n;
  if (ro.n != 0 && ro.n != pl->num_reqs) return fail(CA_EINVAL, "request order does not cover the batch");
  for (int j = 0; j < ro.n; ++j) ro.req[j] = pl->order[j];

  const bool f8 = pl->kv_fp8 != 0;
  if (f8 && pl->suffix.heads_per_item != 1) return fail(CA_EINVAL, "fp8 plans run one KV head per item");

  ca_status_t st;
  TileArgs sa = base;
  sa.prefix_mode = 0;
  sa.key_start = pl->key_start;
  sa.mtiles = pl->suffix.mtiles;
  sa.splits = pl->suffix.splits;
  sa.split_tokens = pl->suffix.split_tokens;
  sa.heads_per_item = pl->suffix.heads_per_item;
  sa.slot_base = pl->use_cascade ? pl->prefix.splits + (gt.n > 0 ? T.slots() : 0) : 0;
  sa.direct = pl->direct_out ? 1 : 0;
  sa.window = pl->use_cascade ? 0 : pl->window;
  // several KV heads per item only in the decode shape (its waves split the keys)
  if (sa.heads_per_item < 1 || pl->hkv % sa.heads_per_item != 0 ||
      (sa.heads_per_item > 1 && pl->suffix.key_groups == 1))
    return fail(CA_EINVAL, "invalid heads per item in plan");
  const int64_t n_suffix = (int64_t)pl->num_reqs * sa.mtiles * (pl->hkv / sa.heads_per_item) * sa.splits;
  if (pl->use_cascade) {
    TileArgs pa = base;
    pa.prefix_mode = 1;
    pa.total_rows = (int32_t)(pl->total_q * pl->group);
    pa.prefix_len = pl->prefix_len;
    pa.mtiles = pl->prefix.mtiles;
    pa.splits = pl->prefix.splits;
    pa.split_tokens = pl->prefix.split_tokens;
    pa.slot_base = 0;
    pa.direct = 0;
    const int64_t n_prefix = (int64_t)pa.mtiles * pl->hkv * pa.splits;
    TileArgs ga = base;   // nested levels: prefix-shaped items over each group's extra pages
    ga.prefix_mode = 2;
    ga.splits = 1;                 // per level, key ranges and slots per group: in the table
    ga.split_tokens = kTileKeys;
    ga.direct = 0;
    const int64_t n_group = gt.n > 0 ? gt.item_begin[gt.n] : 0;
    if (pl->separate_phases) {
      st = run_tile<D>(pa, gt, ro, mt, pl->prefix, n_prefix, f8, s, K_PREFIX);
      if (st == CA_OK) st = run_tile<D>(ga, gt, ro, mt, pl->prefix, n_group, f8, s, K_LEVEL1);
      if (st == CA_OK) st = run_tile<D>(sa, gt, ro, mt, pl->suffix, n_suffix, f8, s, K_SUFFIX);
    } else {
      st = run_phases<D>(pa, pl->prefix, n_prefix, ga, n_group, gt, ro, sa, pl->suffix, n_suffix, mt, f8, s);
    }
  } else {
    st = run_tile<D>(sa, gt, ro, mt, pl->suffix, n_suffix, f8, s, pl->suffix.kernel == 1 ? K_DECODE : K_ATTN);
  }
  if (st != CA_OK) return st;
  if (!pl->direct_out && !mt.counters) {
    MergeArgs ma{};
    ma.part_o = part_o;
    ma.part_lse = part_lse;
    ma.slots = pl->num_slots;
    ma.rows = pl->total_q * pl->hq;
    ma.slot_elems = pl->slot_elems;
    ma.out = static_cast<uint16_t*>(out);
    ma.lse_out = lse;
    ma.sinks = sinks;
    ma.hq = pl->hq;
    st = run_merge<D>(ma, pl->part_fp32 != 0, s);
    if (st != CA_OK) return st;
  }
  return CA_OK;
}

// Sets n 32-bit words to zero (a kernel rather than a memset, so that it can
// be recorded in a HIP graph like any launch).
__global__ __launch_bounds__(256) void zero_words_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

ca_status_t zero_counters(void* ws, int64_t bytes, hipStream_t s) {
  const int64_t n = std::min<int64_t>(bytes, kCounterBytes) / 4;
  if (n <= 0) return CA_OK;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, static_cast<int32_t*>(ws), n);
  return check_launch("workspace init launch");
}

}  // namespace

extern "C" ca_status_t cascade_attn_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace && workspace_bytes > 0) return fail(CA_EINVAL, "null workspace");
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255)) return fail(CA_EINVAL, "workspace must be 256-byte aligned");
  return zero_counters(workspace, (int64_t)workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" int ca_query_num_cus(int32_t* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
  *out = n;
  return 0;
}

extern "C" ca_status_t cascade_attn_run(ca_plan_t pl, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_table_d, const int32_t* query_start_loc_d,
                                        const int32_t* seq_lens_d, const float* sinks_d, void* out,
                                        float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!pl) return fail(CA_EINVAL, "null plan");
  if (!q || !k_cache || !v_cache || !block_table_d || !query_start_loc_d || !seq_lens_d || !out)
    return fail(CA_EINVAL, "null tensor argument");
  if ((int64_t)workspace_bytes < pl->workspace_bytes || (pl->workspace_bytes > 0 && !workspace))
    return fail(CA_EWORKSPACE, "workspace smaller than the plan requires (" + std::to_string(pl->workspace_bytes) +
                                   " bytes)");
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(CA_EINVAL, "workspace must be 256-byte aligned");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
       reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(CA_EINVAL, "q, k_cache, v_cache and out must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pl->d == 128)
    return run_impl<128>(pl, q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d, sinks_d, out,
                         lse_out, workspace, s);
  return run_impl<64>(pl, q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d, sinks_d, out, lse_out,
                      workspace, s);
}

// ------------------------------------------------- run without allocation
//
// Workspace for cascade_attn_run_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the device address that
// hipGetSymbolAddress returns for the current device, kept per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up once per device,
// with that device current). The array starts zeroed (static storage); its
// merge counters are also cleared once here, by a kernel on the caller's
// stream, ahead of the first run on this device; runs leave them zero.
ca_status_t scratch_for_current_device(void** out, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(CA_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(CA_EINVAL, "device index beyond the scratch table");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(CA_EHIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
    const ca_status_t st = zero_counters(p, kCounterBytes, s);
    if (st != CA_OK) return st;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CA_OK;
}
}  // namespace

extern "C" ca_status_t cascade_attn_run_noalloc(ca_plan_t pl, const void* q, const void* k_cache,
                                                const void* v_cache, const int32_t* block_table_d,
                                                const int32_t* query_start_loc_d, const int32_t* seq_lens_d,
                                                const float* sinks_d, void* out, float* lse_out, void* stream) {
  if (!pl) return fail(CA_EINVAL, "null plan");
  if (pl->workspace_bytes > (int64_t)kScratchBytes)
    return fail(CA_EWORKSPACE, "plan needs " + std::to_string(pl->workspace_bytes) +
                                   " bytes of workspace; cascade_attn_run_noalloc holds at most " +
                                   std::to_string(kScratchBytes) + " (use cascade_attn_run with a workspace)");
  void* ws = nullptr;
  if (pl->workspace_bytes > 0) {
    const ca_status_t st = scratch_for_current_device(&ws, static_cast<hipStream_t>(stream));
    if (st != CA_OK) return st;
  }
  // the kernels overwrite every partial state they read back, and the merge
  // counters at the array's start return to zero at the end of every run
  return cascade_attn_run(pl, q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d, sinks_d, out,
                          lse_out, ws, ws ? kScratchBytes : 0, stream);
}

extern "C" ca_status_t cascade_attn_profile_enable(int32_t capacity) {
  if (capacity < 0 || capacity > (1 << 20)) return fail(CA_EINVAL, "capacity must be in [0, 2^20]");
  std::lock_guard<std::mutex> g(g_prof.mu);
  g_prof.release();
  g_prof.enabled = false;
  if (capacity == 0) return CA_OK;
  g_prof.pool.reserve(2 * (size_t)capacity);
  for (int32_t i = 0; i < 2 * capacity; ++i) {
    // no system-scope fence when an event is recorded: the events only time
    // kernels, and the fence's cache write-back / invalidation would slow
    // the launches around it
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      g_prof.release();
      return fail(CA_EHIP, "event creation failed");
    }
    g_prof.pool.push_back(e);
  }
  g_prof.recs.reserve(capacity);
  g_prof.enabled = true;
  return CA_OK;
}

extern "C" ca_status_t cascade_attn_profile_read(double* ms, int64_t* counts) {
  if (!ms || !counts) return fail(CA_EINVAL, "null output");
  std::lock_guard<std::mutex> g(g_prof.mu);
  for (int i = 0; i < K_KINDS; ++i) {
    ms[i] = 0.0;
    counts[i] = 0;
  }
  ca_status_t st = CA_OK;
  for (const auto& r : g_prof.recs) {
    float t = 0.f;
    hipEvent_t a = g_prof.pool[2 * r.slot], b = g_prof.pool[2 * r.slot + 1];
    if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&t, a, b) != hipSuccess) {
      st = fail(CA_EHIP, "event timing failed");
    } else {
      ms[r.kind] += t;
      counts[r.kind] += 1;
    }
  }
  // the pool is reused from its start; launches past its capacity were untimed
  g_prof.recs.clear();
  g_prof.next = 0;
  g_prof.dropped = 0;
  return st;
}

// ------------------------------------------------------------ autotuning

extern "C" ca_status_t cascade_attn_autotune(const ca_params_t* params, const int32_t* block_table_h,
                                             const int32_t* query_start_loc_h, const int32_t* seq_lens_h,
                                             const int32_t* num_computed_tokens_h, const void* q, const void* k_cache,
                                             const void* v_cache, const int32_t* block_table_d,
                                             const int32_t* query_start_loc_d, const int32_t* seq_lens_d,
                                             const float* sinks_d, void* out, float* lse_out, void* workspace,
                                             size_t workspace_bytes, void* stream, int32_t iters,
                                             ca_plan_t* out_plan, float* out_us) {
  if (!params || !out_plan) return fail(CA_EINVAL, "null pointer argument");
  *out_plan = nullptr;
  if (iters < 1 || iters > 1000) return fail(CA_EINVAL, "iters must be in [1, 1000]");
  ca_params_t base_p = *params;
  base_p.mode = CA_MODE_AUTO;
  base_p.prefix_splits = 0;
  base_p.heads_per_item = 0;
  base_p.max_levels = 0;
  base_p.use_tuned = 0;
  ca_plan_t base = nullptr;
  ca_status_t st = cascade_attn_plan(&base_p, block_table_h, query_start_loc_h, seq_lens_h, num_computed_tokens_h,
                                     &base);
  if (st != CA_OK) return st;
  // The shape signature is the AUTO plan's, whatever the table says: plan
  // it once more without the table's influence.
  std::vector<TunedChoice> cands;
  cands.push_back({CA_MODE_FORCE_OFF, 0, 0, 0});
  if (base->prefix_len > 0 && base->window == 0) {
    ca_params_t pp = base_p;
    pp.mode = CA_MODE_FORCE_ON;
    pp.max_levels = 4;   // every nested level; any explicit setting bypasses the table
    ca_plan_t on = nullptr;
    st = cascade_attn_plan(&pp, block_table_h, query_start_loc_h, seq_lens_h, num_computed_tokens_h, &on);
    if (st != CA_OK) {
      cascade_attn_plan_destroy(base);
      return st;
    }
    const int32_t s0 = on->prefix.splits;
    const int32_t h0 = on->suffix.heads_per_item;
    const int32_t lv0 = on->tree.n > 0 ? on->tree.levels : 1;
    // two heads per decode item is a candidate whenever the plan's items are
    // decode-shaped bf16 ones (fp8 plans run one head per item)
    const bool two_heads = on->suffix.kernel == 1 && !on->kv_fp8 && on->hkv % 2 == 0 && h0 != 2;
    cascade_attn_plan_destroy(on);
    std::vector<int32_t> splits{s0};
    if (s0 >= 2) splits.push_back(s0 / 2);
    splits.push_back(s0 * 2);
    std::vector<int32_t> heads{0};
    if (h0 > 1) heads.push_back(1);
    if (two_heads) heads.push_back(2);
    // shared levels: all the detector finds, the batch-wide prefix only,
    // and two when it finds more
    std::vector<int32_t> levels{0};
    if (lv0 > 1) levels.push_back(1);
    if (lv0 > 2) levels.push_back(2);
    for (int32_t sp : splits)
      for (int32_t hd : heads)
        for (int32_t lv : levels) cands.push_back({CA_MODE_FORCE_ON, sp, hd, lv});
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    cascade_attn_plan_destroy(base);
    return fail(CA_EHIP, "event creation failed");
  }
  ca_plan_t best = nullptr;
  TunedChoice best_c;
  float best_us = 0.f;
  for (const TunedChoice& c : cands) {
    ca_params_t cp = base_p;
    cp.mode = c.mode;
    cp.prefix_splits = c.prefix_splits;
    cp.heads_per_item = c.heads_per_item;
    // an explicit level count keeps the table out of the candidate's plan
    cp.max_levels = c.max_levels > 0 ? c.max_levels : 4;
    ca_plan_t cand = nullptr;
    if (cascade_attn_plan(&cp, block_table_h, query_start_loc_h, seq_lens_h, num_computed_tokens_h, &cand) != CA_OK)
      continue;
    if ((int64_t)workspace_bytes < cand->workspace_bytes) {
      cascade_attn_plan_destroy(cand);
      continue;
    }
    st = CA_OK;
    for (int i = 0; i < 2 && st == CA_OK; ++i)
      st = cascade_attn_run(cand, q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d, sinks_d, out,
                            lse_out, workspace, workspace_bytes, stream);
    if (st == CA_OK && hipEventRecord(e0, s) != hipSuccess) st = fail(CA_EHIP, "event record failed");
    for (int i = 0; i < iters && st == CA_OK; ++i)
      st = cascade_attn_run(cand, q, k_cache, v_cache, block_table_d, query_start_loc_d, seq_lens_d, sinks_d, out,
                            lse_out, workspace, workspace_bytes, stream);
    float ms = 0.f;
    if (st == CA_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                        hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
      st = fail(CA_EHIP, "event timing failed");
    if (st != CA_OK) {
      cascade_attn_plan_destroy(cand);
      cascade_attn_plan_destroy(best);
      cascade_attn_plan_destroy(base);
      (void)hipEventDestroy(e0);
      (void)hipEventDestroy(e1);
      return st;
    }
    const float us = ms * 1000.f / iters;
    if (!best || us < best_us) {
      cascade_attn_plan_destroy(best);
      best = cand;
      best_c = c;
      best_c.max_levels = cp.max_levels;
      best_us = us;
    } else {
      cascade_attn_plan_destroy(cand);
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (!best) {
    cascade_attn_plan_destroy(base);
    return fail(CA_EWORKSPACE, "no candidate plan fits the workspace");
  }
  tune_record(*base, best_c);
  cascade_attn_plan_destroy(base);
  *out_plan = best;
  if (out_us) *out_us = best_us;
  return CA_OK;
}
