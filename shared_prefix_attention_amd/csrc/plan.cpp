// Host planner: common-prefix detection, prefix-length cap, cascade decision
// and the work partition of each kernel. Pure host C++ (no HIP calls except
// the optional CU-count query in cascade_attn_plan, kept in run.hip).
//
// Method references: "vLLM Cascade Attention：用法、场景与原理解析"
// (beaiera.top), section 8 Steps 1-3 (detector, cap/floor, metadata) and
// section 3 (trigger thresholds); "resolve async KV transfer bug in cascade
// attention #23485" (the detector counts running requests only).

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <string>
#include <vector>

#include "plan.h"

namespace ca {

static thread_local std::string g_err;

void set_error(const std::string& msg) { g_err = msg; }

static ca_status_t fail(ca_status_t code, const std::string& msg) {
  set_error(msg);
  return code;
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// [p2] section 8 Step 1 / [p3]: leading block-table columns whose physical
// page id is the same in every row, stopping at the first column that
// differs; only columns inside every request's own pages are compared.
static int32_t count_common_blocks(const int32_t* bt, int32_t n, int32_t stride, const int32_t* seq_lens,
                                   int32_t ps) {
  int64_t limit = stride;
  for (int32_t r = 0; r < n; ++r) limit = std::min<int64_t>(limit, cdiv(seq_lens[r], ps));
  int32_t count = 0;
  for (int64_t j = 0; j < limit; ++j) {
    const int32_t first = bt[j];
    bool same = true;
    for (int32_t r = 1; r < n && same; ++r) same = (bt[(int64_t)r * stride + j] == first);
    if (!same) break;
    ++count;
  }
  return count;
}

// Cost model of this library's own kernels on `cus` compute units. The pages
// give only the shape of such a model (section 9 of [p2]: count the work
// tiles of each path and the waves of them the SMs must run; cascade only
// when it beats the plain path) and ask that it be re-derived per kernel
// family ([p4] "Update Cascade Attention Heuristics for FA3"). Constants are
// effective rates of these kernels on MI355X, not spec-sheet peaks.
struct CostModel {
  double hbm_bw = 5.5e12;         // bytes/s streamed from HBM by the attention kernels
  double cu_bw = 40.0e9;          // bytes/s one CU's work-groups pull when few CUs are busy
  double item_latency_us = 4.0;   // fixed start / drain latency of one work item
  double mall_bw = 11.0e12;       // bytes/s for re-reads that hit L2 / Infinity Cache
  double cu_mfma = 4.0e12;        // flop/s of one CU, 128-row tiles (2 row blocks per wave)
  double cu_mfma_rows = 1.8e12;   // flop/s of one CU, 64-row tiles and prefill suffixes (causal, ragged)
  double reread_bw = 14.0e12;     // bytes/s of the non-cascade path's shared-prefix re-reads (L2 / MALL)
  double launch_us = 2.5;         // per kernel launch on one stream
  double merge_trip_us = 1.5;     // the merge's one memory round trip
  double decode_stage_us = 0.5;   // one 64-key stage of a decode-shaped item
  double rows_stage_us = 1.4;     // one 64-key stage of a 64-row item
  // CU time of work items, for launches bound by their items' stage chains
  // rather than by bytes (two work-groups per CU overlap, so these are per
  // CU, not per work-group): a fixed part per item (start-up, combine,
  // store) and a part per 64-key stage by work-group shape.
  double item_cu_us = 5.2;        // 64- / 128-row items; decode-shaped items half of it
  double rows_stage_cu_us = 0.94; // 64-row stage
  double mfma_stage_cu_us = 0.91; // 128-row stage
  double decode_stage_cu_us = 0.25;
  double kernel_floor_us = 7.5;   // shortest attention launch: dispatch, page-table and first-stage round trips, store
  double chunked_floor_us = 11.0; // shortest launch of KV-chunked decode items (partial states out)
  double merge_floor_us = 3.5;    // shortest merge launch (its bytes move at hbm_bw on top)
  double inlaunch_merge_us = 3.0; // merge inside the attention launch: waiting for the partial states' stores
                                  // and counting at the end of the last item of a row block
  double inlaunch_trip_us = 2.0;  // one dependent round trip of that item's merge loads
  double inlaunch_item_us = 2.5;  // every item's own end: its stores complete, then it is counted
  double mall_bytes = 256.0e6;    // Infinity Cache capacity
};

// Work-group shapes of the tiled kernel (all 64-key stages):
//   kRowsConfig   64 rows (4 waves x 16); for packed prefix rows and
//                 prefill suffixes;
//   kMfmaConfig   128 rows (4 waves x 32), one key group; when the prefix
//                 is large enough to be bound by the MFMA rate;
//   kDecodeConfig 16 rows (1 wave), each stage split over 4 key groups;
//                 for suffixes whose rows (q_len * G) fit one MFMA block.
static PhaseTile rows_config() { PhaseTile t; t.row_blocks = 1; t.row_waves = 4; t.key_groups = 1; return t; }
static PhaseTile mfma_config() { PhaseTile t; t.row_blocks = 2; t.row_waves = 4; t.key_groups = 1; return t; }
static PhaseTile decode_config() {
  PhaseTile t;
  t.row_blocks = 1;
  t.row_waves = 1;
  t.key_groups = 4;
  t.kernel = 1;
  return t;
}

// Pipeline depth: 4 stages when the grid leaves CUs with a single
// work-group (more bytes in flight per work-group), else 2 (two work-groups
// per CU fit in LDS).
static int32_t pick_stages(int64_t items, int32_t cus) { return items >= 2 * (int64_t)cus ? 2 : 4; }

// Prefix phase: rows = T*G packed (token, head-in-group) rows per KV head,
// keys = the capped shared prefix. Chooses the KV split count.
static PhaseTile choose_prefix(const ca_plan& pl, int32_t cus, const CostModel& cm, double* est_us) {
  const int64_t rows = pl.total_q * pl.group;
  PhaseTile t = rows >= 2048 ? mfma_config() : rows_config();
  const int64_t bm = t.rows_per_wg();
  const int64_t mtiles = cdiv(rows, bm);
  const int64_t ntiles = cdiv(pl.prefix_len, kTileKeys);
  const int64_t max_tiles = kMaxItemTokens / kTileKeys;
  const double bpt = 2.0 * pl.kv_bytes() * pl.hkv * pl.d;       // K+V bytes per token
  const double part_per_split = (double)pl.total_q * pl.hq * pl.part_row_bytes();
  double best = 1e30;
  t.mtiles = (int32_t)mtiles;
  t.splits = 1;
  t.split_tokens = (int32_t)(ntiles * kTileKeys);
  for (int64_t s = 1; s <= ntiles; s *= 2) {
    const int64_t tiles_per = cdiv(ntiles, s);
    if (tiles_per > max_tiles) continue;
    // an item of one stage has nothing to overlap its start-up with
    if (s > 1 && tiles_per < 2) break;
    const int64_t splits = cdiv(ntiles, tiles_per);
    const int64_t items = mtiles * pl.hkv * splits;
    const double active = (double)std::min<int64_t>(items, cus);
    const double item_flops = 4.0 * bm * pl.d * (double)tiles_per * kTileKeys;
    const double waves_of_items = std::ceil((double)items / cus);
    const double t_mfma = waves_of_items * item_flops / (t.row_blocks > 1 ? cm.cu_mfma : cm.cu_mfma_rows);
    const double hbm = bpt * pl.prefix_len + part_per_split * splits + (double)pl.total_q * pl.hq * pl.d * 2.0;
    const double t_hbm = hbm / std::min(cm.hbm_bw, active * cm.cu_bw);
    // every round of items on the CUs pays the start / drain latency again
    const double est =
        (std::max(t_mfma, t_hbm) + part_per_split * splits / cm.mall_bw) * 1e6 + waves_of_items * cm.item_latency_us;
    if (est < best) {
      best = est;
      t.splits = (int32_t)splits;
      t.split_tokens = (int32_t)(tiles_per * kTileKeys);
      t.stages = pick_stages(items, cus);
    }
    if (splits == ntiles) break;
  }
  *est_us = best;
  return t;
}

// Suffix (or only) phase: per request r the rows are q_len_r*G and the keys
// [key_start, seq_len_r). `fill` asks for enough chunks per request to give
// the grid ~2 work-groups per CU; otherwise the fewest chunks the per-item
// token cap allows (one chunk lets the cascade suffix kernel do the merge).
static PhaseTile choose_suffix(const ca_plan& pl, int32_t cus, bool fill) {
  PhaseTile t = ((int64_t)pl.max_q_len * pl.group <= 16) ? decode_config() : rows_config();
  const int64_t mt = cdiv((int64_t)pl.max_q_len * pl.group, t.rows_per_wg());
  const int64_t base = (int64_t)pl.num_reqs * mt * pl.hkv;
  const int64_t ntiles = std::max<int64_t>(1, cdiv(pl.max_suffix_len, kTileKeys));
  const int64_t max_tiles = kMaxItemTokens / kTileKeys;
  int64_t chunks = cdiv(ntiles, max_tiles);
  if (fill) chunks = std::max(chunks, std::min(ntiles, std::max<int64_t>(1, cdiv(2 * (int64_t)cus, base))));
  const int64_t tiles_per = cdiv(ntiles, chunks);
  chunks = cdiv(ntiles, tiles_per);
  t.mtiles = (int32_t)mt;
  t.splits = (int32_t)chunks;
  t.split_tokens = (int32_t)(tiles_per * kTileKeys);
  t.stages = pick_stages(base * chunks, cus);
  return t;
}

// Per-request work items start with the longest key ranges (in 64-key
// tiles; ties keep batch order): greedy list scheduling that leaves the short
// items for the end of the launch, where they fill the CUs freed by the long
// ones. Only the dispatch order changes, never an item's work.
static void order_requests(ca_plan& pl, const ca_params_t& p, const int32_t* seq_lens, const int64_t* kstart) {
  pl.order_n = 0;
  const int32_t n = pl.num_reqs;
  if (p.suffix_order != 0 || n > kOrderCapacity) return;
  std::vector<int64_t> tiles(n);
  for (int32_t r = 0; r < n; ++r) tiles[r] = cdiv(std::max<int64_t>(0, seq_lens[r] - kstart[r]), kTileKeys);
  std::vector<int32_t> idx(n);
  for (int32_t r = 0; r < n; ++r) idx[r] = r;
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return tiles[a] > tiles[b]; });
  bool identity = true;
  for (int32_t r = 0; r < n; ++r) identity = identity && idx[r] == r;
  if (identity) return;
  pl.order_n = n;
  for (int32_t r = 0; r < n; ++r) pl.order[r] = (uint16_t)idx[r];
}

// Decode-shaped items may run several consecutive KV heads of one request as
// one stage pipeline (same pages and key range). Worth it when that keeps the
// whole cascade launch within two resident work-groups per CU (no item waits
// for a slot, and each item's first round trips are paid once for all its
// heads) and the grouped item stays at most half as long as a prefix item: a
// decode stage costs about one memory round trip, so longer chains become the
// launch's critical path. Failing that, two heads per item when the suffix
// items alone need more than two rounds; otherwise one head per item.
static int32_t pick_heads_per_item(const ca_plan& pl, int64_t prefix_items, int64_t prefix_stages,
                                   const PhaseTile& suf, int32_t cus) {
  if (suf.kernel != 1) return 1;
  if (pl.p.heads_per_item > 0) return pl.p.heads_per_item;
  const int64_t per_head = (int64_t)pl.num_reqs * suf.mtiles * suf.splits;
  const int64_t suffix_stages = suf.split_tokens / kTileKeys;
  for (int32_t h = 1; h <= pl.hkv && h <= 8; ++h) {
    if (pl.hkv % h) continue;
    if (prefix_items + per_head * (pl.hkv / h) <= 2 * (int64_t)cus) {
      if (h * suffix_stages <= std::max<int64_t>(1, prefix_stages / 2)) return h;
      break;
    }
  }
  // Suffix items alone fill more than two rounds of two work-groups per CU:
  // two heads per item halve the item start-ups (the second head's first
  // stages are already in flight when the first head finishes).
  if (per_head * pl.hkv > 4 * (int64_t)cus && pl.hkv % 2 == 0) return 2;
  return 1;
}

// CU time (µs) of a per-request phase's items: request r runs
// ceil(q_len_r * G / rows) row tiles per KV head, each split in `chunks`
// items that together walk its positions [start_r, seq_len_r).
static double items_cu_us(const ca_plan& pl, const PhaseTile& t, const int32_t* qsl, const int32_t* seq_lens,
                          const int64_t* start, const CostModel& cm, int32_t heads_per_item = 1) {
  const bool dec = t.kernel == 1;
  const double a = (dec ? 0.5 * cm.item_cu_us : cm.item_cu_us) / heads_per_item;
  const double x = dec ? cm.decode_stage_cu_us : (t.row_blocks > 1 ? cm.mfma_stage_cu_us : cm.rows_stage_cu_us);
  double us = 0.0;
  for (int32_t r = 0; r < pl.num_reqs; ++r) {
    const int64_t mt = cdiv((int64_t)(qsl[r + 1] - qsl[r]) * pl.group, t.rows_per_wg());
    const int64_t tiles = cdiv(std::max<int64_t>(0, seq_lens[r] - (start ? start[r] : 0)), kTileKeys);
    us += (double)(mt * pl.hkv) * ((double)t.splits * a + (double)tiles * x);
  }
  return us;
}

// The merge as a launch of its own, reading and writing `bytes` (partial
// states in, output out): a fixed floor plus the bytes at the streaming rate,
// plus the launch.
static double est_merge_launch_us(double bytes, const CostModel& cm) {
  return cm.merge_floor_us + bytes / cm.hbm_bw * 1e6 + cm.launch_us;
}

// The merge inside the attention launch: the item that completes a row
// block merges every row it wrote (up to `winner_rows`), each thread two
// 16-byte chunks of a row, slots in batches of 8 per slot group, one memory
// round trip per batch and pass of the work-group's 256 threads, after the
// wait for its own stores and the count. Every item also ends by waiting
// for its stores and being counted, which lengthens each round of items on
// the CUs (`items` work items, two resident per CU).
static double est_merge_in_launch_us(const ca_plan& pl, int64_t winner_rows, int32_t slots, int64_t items,
                                     int32_t cus, const CostModel& cm) {
  const int64_t tpr = pl.d * (pl.part_fp32 ? 4 : 2) / 32;
  const int64_t passes = cdiv(winner_rows * tpr, kThreads);
  const int64_t sg = slots > 16 ? 4 : 1;
  const int64_t batches = sg * cdiv(cdiv(slots, sg), 8);
  const int64_t rounds = cdiv(std::max<int64_t>(items, 1), 2 * (int64_t)cus);
  return cm.inlaunch_merge_us + cm.inlaunch_trip_us * (double)(passes * batches) +
         cm.inlaunch_item_us * (double)(rounds - 1);
}

// Where a plan merges: inside the attention launch when asked (merge_mode 2)
// or, by default, when the model prices it below the merge launch; never
// with separate phase launches or when the per-request tiles need more
// counters than the workspace reserves.
static bool merges_in_launch(const ca_params_t& p, int64_t num_reqs, int64_t mtiles, int64_t hkv, double in_us,
                             double launch_us) {
  if (p.merge_mode == 1 || p.separate_phases != 0 || num_reqs * mtiles * hkv > kMaxCounters) return false;
  return p.merge_mode == 2 || in_us < launch_us;
}

// Per-request phase over KV positions [key_start, seq_len): HBM bytes for the
// KV actually streamed, plus the MFMA work of 16-row padded query blocks, but
// no less than `floor_us` (the launch's item rounds; 0 when the phase overlaps
// another in one launch).
static double est_suffix_us(const ca_plan& pl, int64_t kv_tokens, double padded_flops, int32_t chunks, bool merge,
                            double merge_us, int32_t cus, const CostModel& cm, double extra_mall_bytes,
                            double floor_us) {
  const double bpt = 2.0 * pl.kv_bytes() * pl.hkv * pl.d;
  const double io = (double)pl.total_q * pl.hq * pl.d * 2.0 * 2.0;
  const double t_bytes = (bpt * kv_tokens + io) / cm.hbm_bw + extra_mall_bytes / cm.reread_bw;
  const double t_mfma = padded_flops / ((double)cus * cm.cu_mfma_rows);
  double us = std::max(std::max(t_bytes, t_mfma) * 1e6, floor_us) + cm.launch_us;
  if (merge) us += merge_us;
  (void)chunks;
  return us;
}

// MFMA work of the per-request phase: every KV head of request r runs
// ceil(q_len*G / 16) blocks of 16 rows over its keys from key_start[r] (null:
// from 0) (causal rows stop early,
// counted here as the mean of the first and last row's key count).
static double suffix_padded_flops(const ca_plan& pl, const int32_t* qsl, const int32_t* seq_lens,
                                  const int64_t* key_start) {
  double f = 0.0;
  for (int32_t r = 0; r < pl.num_reqs; ++r) {
    const int64_t ql = (int64_t)qsl[r + 1] - qsl[r];
    const int64_t keys_last = seq_lens[r] - (key_start ? key_start[r] : 0);
    const int64_t keys_first = keys_last - (ql - 1);
    const double blocks = (double)cdiv(ql * pl.group, 16);
    f += blocks * 16.0 * 0.5 * (double)(keys_first + keys_last);
  }
  return f * 4.0 * pl.d * pl.hkv;
}

// Nested shared levels. FlashInfer's cascade runs any number of levels
// ([p2] section 7), and the workloads of [p2] section 3 nest: a system
// prompt shared by every request, then a document shared by some, a chapter
// by fewer, then each request's own tokens. The batch-wide rule of [p2]
// section 8 Steps 1-2 (shared leading pages, capped at the members' smallest
// num_computed, floored to a page) is applied at every node of the prefix
// tree of the requests' page-id sequences: members that share every page up
// to column c are split by their page at column c; a part of >= 2 requests
// whose shared length exceeds its enclosing group's by >= 256 tokens (the
// pages' prefix-length gate, [p2] section 3) is a group one level deeper,
// and its parts are examined against it; otherwise its parts are examined
// against the same enclosing group. Members need not be consecutive.
struct TreeCand {
  std::vector<int32_t> members;   // batch order
  int32_t parent_len, len, level, parent;
  int64_t saving() const { return (int64_t)(members.size() - 1) * (len - parent_len); }
};

static int64_t shared_columns(const int32_t* bt, int32_t stride, const int32_t* seq_lens, int32_t ps,
                              const std::vector<int32_t>& members) {
  int64_t limit = stride;
  for (int32_t r : members) limit = std::min<int64_t>(limit, cdiv(seq_lens[r], ps));
  const int32_t* first = bt + (int64_t)members[0] * stride;
  int64_t c = 0;
  for (; c < limit; ++c) {
    bool same = true;
    for (size_t k = 1; k < members.size() && same; ++k) same = bt[(int64_t)members[k] * stride + c] == first[c];
    if (!same) break;
  }
  return c;
}

static void tree_visit(const int32_t* bt, int32_t stride, const int32_t* seq_lens, const int32_t* qsl, int32_t ps,
                       const std::vector<int32_t>& members, int32_t parent_len, int32_t level, int32_t parent,
                       int32_t max_levels, std::vector<TreeCand>& out) {
  const int64_t c = shared_columns(bt, stride, seq_lens, ps, members);
  // parts by the page at column c, in order of first appearance
  std::vector<std::pair<int32_t, std::vector<int32_t>>> parts;
  for (int32_t r : members) {
    if (cdiv(seq_lens[r], ps) <= c) continue;
    const int32_t page = bt[(int64_t)r * stride + c];
    auto it = std::find_if(parts.begin(), parts.end(), [&](const auto& x) { return x.first == page; });
    if (it == parts.end()) parts.push_back({page, {r}});
    else it->second.push_back(r);
  }
  for (const auto& part : parts) {
    const std::vector<int32_t>& m = part.second;
    if (m.size() < 2) continue;
    int64_t len = shared_columns(bt, stride, seq_lens, ps, m) * ps;
    for (int32_t r : m) len = std::min<int64_t>(len, seq_lens[r] - (qsl[r + 1] - qsl[r]));
    len = len / ps * ps;
    if (len - parent_len >= 256 && level + 1 <= max_levels - 1) {
      out.push_back({m, parent_len, (int32_t)len, level + 1, parent});
      tree_visit(bt, stride, seq_lens, qsl, ps, m, (int32_t)len, level + 1, (int32_t)out.size() - 1, max_levels, out);
    } else {
      tree_visit(bt, stride, seq_lens, qsl, ps, m, parent_len, level, parent, max_levels, out);
    }
  }
}

// At most kMaxTreeGroups groups: level by level, the groups that save the
// most KV reads ((members - 1) x extra length) among those whose enclosing
// group was kept. A dropped group's members fall back to the nearest kept
// enclosing level (results are exact either way).
static std::vector<TreeCand> limit_tree(std::vector<TreeCand> all) {
  if ((int)all.size() <= kMaxTreeGroups) return all;
  std::vector<int32_t> keep_idx;
  std::vector<char> kept(all.size(), 0);
  for (int32_t lev = 1; lev < kMaxShared && (int)keep_idx.size() < kMaxTreeGroups; ++lev) {
    std::vector<int32_t> cand;
    for (int32_t g = 0; g < (int32_t)all.size(); ++g)
      if (all[g].level == lev && (all[g].parent < 0 || kept[all[g].parent])) cand.push_back(g);
    std::stable_sort(cand.begin(), cand.end(), [&](int32_t a, int32_t b) { return all[a].saving() > all[b].saving(); });
    for (int32_t g : cand) {
      if ((int)keep_idx.size() >= kMaxTreeGroups) break;
      kept[g] = 1;
      keep_idx.push_back(g);
    }
  }
  std::sort(keep_idx.begin(), keep_idx.end());   // parents before children, as found
  std::vector<int32_t> remap(all.size(), -1);
  std::vector<TreeCand> out;
  for (int32_t g : keep_idx) {
    remap[g] = (int32_t)out.size();
    TreeCand t = all[g];
    t.parent = t.parent >= 0 ? remap[t.parent] : -1;
    out.push_back(t);
  }
  return out;
}

// Autotuning table: shape signature -> recorded choice.
using ShapeKey = std::tuple<int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                            int32_t>;
static std::mutex g_tune_mu;
static std::map<ShapeKey, TunedChoice> g_tune;

static int32_t log2_bucket(int64_t x) { return x <= 0 ? -1 : 63 - __builtin_clzll((unsigned long long)x); }

static ShapeKey shape_key(const ca_plan& pl) {
  const int64_t mean_rest = (pl.sum_seq - (int64_t)pl.prefix_len * pl.num_reqs) / std::max(1, pl.num_reqs);
  return ShapeKey{pl.num_reqs, pl.hq, pl.hkv, pl.d, pl.kv_fp8, pl.window, log2_bucket(pl.prefix_len),
                  log2_bucket(pl.total_q), log2_bucket(pl.max_q_len), log2_bucket(mean_rest),
                  std::min(pl.cand_groups, 8)};
}

void tune_record(const ca_plan& pl, const TunedChoice& c) {
  if (c.mode == CA_MODE_AUTO) return;   // a recorded choice always fixes the path
  std::lock_guard<std::mutex> g(g_tune_mu);
  g_tune[shape_key(pl)] = c;
}

static bool tune_lookup(const ca_plan& pl, TunedChoice* c) {
  std::lock_guard<std::mutex> g(g_tune_mu);
  const auto it = g_tune.find(shape_key(pl));
  if (it == g_tune.end()) return false;
  *c = it->second;
  return true;
}

}  // namespace ca

using namespace ca;

extern "C" void cascade_attn_autotune_reset(void) {
  std::lock_guard<std::mutex> g(g_tune_mu);
  g_tune.clear();
}

extern "C" const char* cascade_attn_last_error(void) { return g_err.c_str(); }

extern "C" ca_status_t cascade_attn_num_common_prefix_blocks(const int32_t* block_table_h, int32_t num_reqs,
                                                             int32_t stride, const int32_t* seq_lens_h,
                                                             int32_t page_size, int32_t* out_blocks) {
  if (!block_table_h || !seq_lens_h || !out_blocks) return fail(CA_EINVAL, "null pointer argument");
  if (num_reqs <= 0 || stride <= 0 || page_size <= 0) return fail(CA_EINVAL, "num_reqs, stride and page_size must be > 0");
  for (int32_t r = 0; r < num_reqs; ++r) {
    if (seq_lens_h[r] < 0) return fail(CA_EMETA, "negative seq_len for request " + std::to_string(r));
    if (cdiv(seq_lens_h[r], page_size) > stride)
      return fail(CA_EMETA, "request " + std::to_string(r) + " needs more pages than block_table_stride");
  }
  *out_blocks = count_common_blocks(block_table_h, num_reqs, stride, seq_lens_h, page_size);
  return CA_OK;
}

// Defined in run.hip: CU count of the current device (host HIP call).
extern "C" int ca_query_num_cus(int32_t* out);

extern "C" ca_status_t cascade_attn_plan(const ca_params_t* prm, const int32_t* bt, const int32_t* qsl,
                                         const int32_t* seq_lens, const int32_t* num_computed,
                                         ca_plan_t* out_plan) {
  if (out_plan) *out_plan = nullptr;   // no plan on any error
  if (!prm || !bt || !qsl || !seq_lens || !out_plan) return fail(CA_EINVAL, "null pointer argument");
  const ca_params_t& p = *prm;
  if (p.num_reqs <= 0) return fail(CA_EINVAL, "num_reqs must be >= 1");
  if (p.num_q_heads <= 0 || p.num_kv_heads <= 0) return fail(CA_EINVAL, "head counts must be >= 1");
  if (p.num_q_heads % p.num_kv_heads != 0) return fail(CA_EUNSUPPORTED, "num_q_heads must be a multiple of num_kv_heads");
  if (p.head_dim != 64 && p.head_dim != 128) return fail(CA_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (p.page_size != 16) return fail(CA_EUNSUPPORTED, "page_size must be 16");
  if (p.block_table_stride <= 0) return fail(CA_EINVAL, "block_table_stride must be >= 1");
  if (p.num_pages <= 0) return fail(CA_EINVAL, "num_pages must be >= 1");
  if (p.kv_stride_page <= 0 || p.kv_stride_token <= 0 || p.kv_stride_head <= 0 || p.kv_stride_page % 8 ||
      p.kv_stride_token % 8 || p.kv_stride_head % 8)
    return fail(CA_EUNSUPPORTED, "KV strides must be positive multiples of 8 elements");
  if (p.kv_stride_token > (int64_t(1) << 26)) return fail(CA_EUNSUPPORTED, "kv_stride_token must be <= 2^26");
  if (p.mode < CA_MODE_AUTO || p.mode > CA_MODE_FORCE_OFF) return fail(CA_EINVAL, "unknown mode");
  if (p.heads_per_item < 0 || (p.heads_per_item > 0 && p.num_kv_heads % p.heads_per_item != 0))
    return fail(CA_EINVAL, "heads_per_item must be 0 or divide num_kv_heads");
  if (p.separate_phases != 0 && p.separate_phases != 1) return fail(CA_EINVAL, "separate_phases must be 0 or 1");
  if (p.max_levels < 0 || p.max_levels > kMaxShared) return fail(CA_EINVAL, "max_levels must be in [0, 4]");
  if (p.kv_dtype != CA_KV_BF16 && p.kv_dtype != CA_KV_FP8_E4M3) return fail(CA_EINVAL, "unknown kv_dtype");
  if (p.sliding_window < 0) return fail(CA_EINVAL, "sliding_window must be >= 0");
  if (p.prefix_splits < 0) return fail(CA_EINVAL, "prefix_splits must be >= 0");
  if (p.suffix_order != 0 && p.suffix_order != 1) return fail(CA_EINVAL, "suffix_order must be 0 or 1");
  if (p.partials_fp32 != 0 && p.partials_fp32 != 1) return fail(CA_EINVAL, "partials_fp32 must be 0 or 1");
  if (p.use_tuned != 0 && p.use_tuned != 1) return fail(CA_EINVAL, "use_tuned must be 0 or 1");
  if (p.merge_mode < 0 || p.merge_mode > 2) return fail(CA_EINVAL, "merge_mode must be 0, 1 or 2");
  if (!std::isfinite(p.k_scale) || !std::isfinite(p.v_scale)) return fail(CA_EINVAL, "k_scale / v_scale must be finite");
  if (p.kv_dtype == CA_KV_FP8_E4M3) {
    if (p.head_dim != 128) return fail(CA_EUNSUPPORTED, "fp8 caches need head_dim 128");
    if (p.kv_stride_page % 16 || p.kv_stride_token % 16 || p.kv_stride_head % 16)
      return fail(CA_EUNSUPPORTED, "fp8 KV strides must be multiples of 16 elements");
  }

  const int32_t n = p.num_reqs, ps = p.page_size, stride = p.block_table_stride;
  if (qsl[0] != 0) return fail(CA_EMETA, "query_start_loc[0] must be 0");
  int32_t max_q = 0, max_seq = 0;
  for (int32_t r = 0; r < n; ++r) {
    const int64_t ql = (int64_t)qsl[r + 1] - qsl[r];
    if (ql < 1) return fail(CA_EMETA, "request " + std::to_string(r) + " has no query token");
    if (seq_lens[r] < ql) return fail(CA_EMETA, "seq_len smaller than query length for request " + std::to_string(r));
    if (num_computed && num_computed[r] != seq_lens[r] - ql)
      return fail(CA_EMETA, "num_computed_tokens != seq_len - q_len for request " + std::to_string(r));
    const int64_t pages = cdiv(seq_lens[r], ps);
    if (pages > stride) return fail(CA_EMETA, "request " + std::to_string(r) + " needs more pages than block_table_stride");
    for (int64_t j = 0; j < pages; ++j) {
      const int32_t id = bt[(int64_t)r * stride + j];
      if (id < 0 || id >= p.num_pages)
        return fail(CA_EMETA, "page id out of range in request " + std::to_string(r));
    }
    max_q = std::max<int32_t>(max_q, (int32_t)ql);
    max_seq = std::max(max_seq, seq_lens[r]);
  }
  const int64_t total_q = qsl[n];

  int32_t cus = p.num_cus;
  if (cus <= 0) {
    if (ca_query_num_cus(&cus) != 0 || cus <= 0) return fail(CA_EHIP, "could not query the device CU count");
  }

  ca_plan* pl = new (std::nothrow) ca_plan();
  if (!pl) return fail(CA_EINVAL, "out of host memory");
  pl->p = p;
  pl->num_reqs = n;
  pl->hq = p.num_q_heads;
  pl->hkv = p.num_kv_heads;
  pl->group = p.num_q_heads / p.num_kv_heads;
  pl->d = p.head_dim;
  pl->ps = ps;
  pl->total_q = total_q;
  pl->max_q_len = max_q;
  pl->uniform_q = max_q;
  for (int32_t r = 0; r < n; ++r)
    if (qsl[r + 1] - qsl[r] != max_q) pl->uniform_q = 0;
  pl->max_seq_len = max_seq;
  pl->scale = p.softmax_scale > 0.f ? p.softmax_scale : 1.0f / std::sqrt((float)p.head_dim);
  pl->kv_fp8 = p.kv_dtype == CA_KV_FP8_E4M3 ? 1 : 0;
  pl->part_fp32 = p.partials_fp32;
  pl->k_scale = (pl->kv_fp8 && p.k_scale > 0.f) ? p.k_scale : 1.f;
  pl->v_scale = (pl->kv_fp8 && p.v_scale > 0.f) ? p.v_scale : 1.f;

  // Step 1: shared pages. Step 2: cap at min num_computed, floor to a page.
  pl->common_blocks = count_common_blocks(bt, n, stride, seq_lens, ps);
  int64_t min_computed = INT64_MAX;
  for (int32_t r = 0; r < n; ++r) min_computed = std::min<int64_t>(min_computed, seq_lens[r] - (qsl[r + 1] - qsl[r]));
  int64_t plen = (int64_t)pl->common_blocks * ps;
  plen = std::min(plen, min_computed);
  plen = (plen / ps) * ps;
  pl->prefix_len = (int32_t)plen;
  // [p2] section 3: shared prefix >= 256 tokens and >= 8 requests (reported).
  pl->gates_pass = (plen >= 256 && n >= 8) ? 1 : 0;
  // The gate AUTO applies, re-derived for these kernels on MI355X: the same
  // prefix length, but any batch of two or more requests; the cost model
  // decides the rest. Decode batches of 2 and 4 requests with prefixes of
  // 1024 tokens and more measured 1.2-1.6x faster on the cascade path.
  const bool auto_gate = plen >= 256 && n >= 2;

  int64_t sum_seq = 0;
  for (int32_t r = 0; r < n; ++r) sum_seq += seq_lens[r];
  pl->sum_seq = sum_seq;
  pl->kv_tokens_noncascade = sum_seq;
  pl->kv_tokens_cascade = plen + (sum_seq - plen * n);

  const CostModel cm;
  const double bpt = 2.0 * pl->kv_bytes() * pl->hkv * pl->d;

  // The prefix tree below the batch-wide prefix (requests of a batch larger
  // than the tree-order table get none): the nested levels of the cascade
  // path, and positions the non-cascade path reads several times.
  std::vector<TreeCand> all_groups;
  if (plen > 0 && n <= kOrderCapacity) {
    std::vector<int32_t> all(n);
    for (int32_t r = 0; r < n; ++r) all[r] = r;
    tree_visit(bt, stride, seq_lens, qsl, ps, all, (int32_t)plen, 0, -1, kMaxShared, all_groups);
  }
  pl->cand_groups = (int32_t)all_groups.size();   // part of the shape, whether used or not

  // Non-cascade estimate: every request streams its whole sequence; the
  // shared pages are fetched from HBM once and re-read from cache by the
  // other requests when they fit in it.
  pl->key_start = 0;
  pl->max_suffix_len = max_seq;
  PhaseTile nc = choose_suffix(*pl, cus, true);
  // merge of the non-cascade path's KV chunks: a launch, or inside the
  // attention launch by the last chunk of each (request, row tile, KV head)
  auto nc_merge = [&](const PhaseTile& t, bool* in_launch) {
    const double bytes = (double)t.splits * total_q * pl->hq * pl->part_row_bytes() + (double)total_q * pl->hq * pl->d * 2.0;
    const double ml = est_merge_launch_us(bytes, cm);
    const int64_t items = (int64_t)n * t.mtiles * pl->hkv * t.splits;
    const double mi =
        est_merge_in_launch_us(*pl, (int64_t)t.rows_per_wg() * (t.kernel == 1 ? pl->hkv : 1), t.splits, items, cus, cm);
    *in_launch = merges_in_launch(p, n, t.mtiles, pl->hkv, mi, ml);
    return *in_launch ? mi : ml;
  };
  bool nc_in_launch = false;
  {
    // Chunking a request's KV range fills the chip but adds the merge: keep
    // one chunk per request (the attention writes the output) when the
    // chunked plan does not save the merge's cost.
    const PhaseTile direct = choose_suffix(*pl, cus, false);
    if (direct.splits < nc.splits) {
      const double t_stage = nc.kernel == 1 ? cm.decode_stage_us : cm.rows_stage_us;
      const int64_t base = (int64_t)pl->num_reqs * nc.mtiles * pl->hkv;
      auto items_us = [&](const PhaseTile& t) {
        const double rounds = std::ceil((double)(base * t.splits) / (2.0 * cus));
        return rounds * (cm.item_latency_us + (double)(t.split_tokens / kTileKeys) * t_stage);
      };
      bool il = false;
      const double m_us = nc_merge(nc, &il);
      if (items_us(direct) <= items_us(nc) + m_us - cm.merge_floor_us + cm.merge_trip_us) nc = direct;
    }
    // positions shared by several requests (the prefix, the nested groups'
    // documents): one copy of each comes from HBM, the rest are re-reads.
    // The re-reads go at a rate of elements (the items' per-element work
    // bounds it), so fp8 caches count as bf16 there.
    int64_t shared_tokens = plen, reread_tokens = plen * (int64_t)(n - 1);
    for (const TreeCand& g : all_groups) {
      shared_tokens += g.len - g.parent_len;
      reread_tokens += (int64_t)(g.members.size() - 1) * (g.len - g.parent_len);
    }
    const double shared_bytes = bpt * shared_tokens;
    const double reread = (double)(2 * 2 * pl->hkv * pl->d) * reread_tokens;
    int64_t hbm_tokens = sum_seq - reread_tokens;
    double extra = 0.0;
    if (shared_bytes <= cm.mall_bytes) extra = reread;
    else hbm_tokens = sum_seq;
    // however few bytes, the launch takes its floor, its items' CU time, or
    // its longest item
    const double t_stage = nc.kernel == 1 ? cm.decode_stage_us : cm.rows_stage_us;
    const double t_longest = cm.item_latency_us + (double)(nc.split_tokens / kTileKeys) * t_stage;
    const double floor_us = nc.splits > 1 && nc.kernel == 1 ? cm.chunked_floor_us : cm.kernel_floor_us;
    const double t_items =
        std::max(std::max(floor_us, t_longest), items_cu_us(*pl, nc, qsl, seq_lens, nullptr, cm) / cus);
    const double m_us = nc.splits > 1 ? nc_merge(nc, &nc_in_launch) : 0.0;
    pl->est_us_noncascade = (float)est_suffix_us(*pl, hbm_tokens, suffix_padded_flops(*pl, qsl, seq_lens, nullptr),
                                                 nc.splits, nc.splits > 1, m_us, cus, cm, extra, t_items);
  }

  // Cascade estimate (only meaningful when something is shared): the
  // batch-wide prefix, the group level when there is one, each request's
  // remaining positions, and the merge.
  PhaseTile pre, suf;
  Tree tree;
  bool casc_in_launch = false;
  std::vector<int64_t> kstart(n, plen);   // first suffix position of each request
  int64_t group_items = 0, group_stages = 0;
  if (plen > 0) {
    pl->prefix_len = (int32_t)plen;
    double pre_us = 0.0;
    pre = choose_prefix(*pl, cus, cm, &pre_us);
    if (p.prefix_splits > 0) {   // explicit split count (e.g. from the autotuner)
      const int64_t ntiles = cdiv(plen, kTileKeys);
      const int64_t tiles_per = std::min<int64_t>(cdiv(ntiles, std::min<int64_t>(p.prefix_splits, ntiles)),
                                                  kMaxItemTokens / kTileKeys);
      pre.splits = (int32_t)cdiv(ntiles, tiles_per);
      pre.split_tokens = (int32_t)(tiles_per * kTileKeys);
    }
    // nested levels kept by the plan: at most max_levels - 1 below the
    // batch-wide prefix, at most kMaxTreeGroups groups
    const int32_t max_levels = p.max_levels == 0 ? kMaxShared : p.max_levels;
    std::vector<TreeCand> groups = all_groups;
    if (max_levels < kMaxShared) {   // keep the shallower levels (children follow their parents)
      std::vector<TreeCand> kept;
      std::vector<int32_t> remap(groups.size(), -1);
      for (size_t g = 0; g < groups.size(); ++g) {
        if (groups[g].level > max_levels - 1) continue;
        remap[g] = (int32_t)kept.size();
        kept.push_back(groups[g]);
        kept.back().parent = groups[g].parent >= 0 ? remap[groups[g].parent] : -1;
      }
      groups.swap(kept);
    }
    groups = limit_tree(std::move(groups));
    double t_grp = 0.0;
    int64_t group_tokens = 0;
    if (!groups.empty()) {
      const int32_t G = (int32_t)groups.size();
      tree.n = G;
      std::vector<int32_t> deep(n, -1);   // innermost group of each request
      for (int32_t g = 0; g < G; ++g)
        for (int32_t r : groups[g].members) deep[r] = g;   // children come after their parents
      // tree order: requests sorted by the chain of groups that hold them
      // (outermost first), so that every group's members are adjacent
      std::vector<std::vector<int32_t>> key(n);
      for (int32_t r = 0; r < n; ++r) {
        for (int32_t g = deep[r]; g >= 0; g = groups[g].parent) key[r].insert(key[r].begin(), g);
        key[r].resize(kMaxShared, INT32_MAX);
      }
      std::vector<int32_t> order(n);
      for (int32_t r = 0; r < n; ++r) order[r] = r;
      std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return key[a] < key[b]; });
      std::vector<int32_t> pos_of(n);
      tree.pos_cum[0] = 0;
      for (int32_t p2 = 0; p2 < n; ++p2) {
        pos_of[order[p2]] = p2;
        tree.pos_tok[p2] = qsl[order[p2]];
        tree.pos_cum[p2 + 1] = tree.pos_cum[p2] + (qsl[order[p2] + 1] - qsl[order[p2]]);
      }
      for (int32_t r = 0; r < n; ++r) tree.deepest[r] = deep[r] >= 0 ? (uint8_t)deep[r] : (uint8_t)0xff;
      tree.levels = 1;
      for (const auto& g : groups) tree.levels = std::max(tree.levels, g.level + 1);
      // Every group of a level gets the same number of KV splits (so its
      // rows fill that level's partial slots): about 512 keys per item for
      // the level's longest group, at most 8 splits unless the per-item cap
      // needs more.
      for (int32_t lev = 1; lev < tree.levels; ++lev) {
        int64_t max_tiles = 1;
        for (const auto& g : groups)
          if (g.level == lev) max_tiles = std::max(max_tiles, cdiv(g.len - g.parent_len, kTileKeys));
        tree.level_splits[lev] = (int32_t)std::max(std::min<int64_t>(cdiv(max_tiles, 8), 8),
                                                    cdiv(max_tiles, kMaxItemTokens / kTileKeys));
      }
      int32_t slot = pre.splits;
      for (int32_t lev = 1; lev < tree.levels; ++lev) {
        tree.level_slot_base[lev] = slot;
        slot += tree.level_splits[lev];
      }
      double flops = 0.0;
      for (int32_t j = 0; j < G; ++j) {
        const TreeCand& g = groups[j];
        int32_t pb = n, pe = 0;
        for (int32_t r : g.members) {
          pb = std::min(pb, pos_of[r]);
          pe = std::max(pe, pos_of[r] + 1);
        }
        tree.level[j] = g.level;
        tree.parent[j] = g.parent;
        tree.first_req[j] = g.members[0];
        tree.pos_begin[j] = pb;
        tree.pos_end[j] = pe;
        tree.key_begin[j] = g.parent_len;
        tree.key_end[j] = g.len;
        const int64_t splits = tree.level_splits[g.level];
        const int64_t tiles_per = cdiv(cdiv(g.len - g.parent_len, kTileKeys), splits);
        tree.split_tokens[j] = (int32_t)(tiles_per * kTileKeys);
        group_stages = std::max(group_stages, tiles_per);
        tree.rows[j] = (tree.pos_cum[pe] - tree.pos_cum[pb]) * pl->group;
        tree.item_begin[j] = (int32_t)group_items;
        const int64_t mtiles = cdiv(tree.rows[j], pre.rows_per_wg());
        group_items += mtiles * pl->hkv * splits;
        group_tokens += g.len - g.parent_len;
        flops += 4.0 * (double)(mtiles * pre.rows_per_wg()) * pl->hkv * pl->d * (double)(g.len - g.parent_len);
        for (int32_t r : g.members) kstart[r] = std::max<int64_t>(kstart[r], g.len);
      }
      tree.item_begin[G] = (int32_t)group_items;
      t_grp = std::max(flops / ((double)cus * cm.cu_mfma_rows), bpt * group_tokens / cm.hbm_bw) * 1e6 +
              cm.item_latency_us;
    }
    int64_t suffix_tokens = 0, max_suffix = 0;
    for (int32_t r = 0; r < n; ++r) {
      suffix_tokens += seq_lens[r] - kstart[r];
      max_suffix = std::max<int64_t>(max_suffix, seq_lens[r] - kstart[r]);
    }
    pl->key_start = (int32_t)plen;
    pl->max_suffix_len = (int32_t)max_suffix;
    suf = choose_suffix(*pl, cus, true);
    const double t_suf = est_suffix_us(*pl, suffix_tokens, suffix_padded_flops(*pl, qsl, seq_lens, kstart.data()),
                                       suf.splits, false, 0.0, cus, cm, 0.0, 0.0);
    const double merge_bytes = (double)(pre.splits + tree.slots() + suf.splits) * total_q * pl->hq * pl->part_row_bytes() +
                               (double)total_q * pl->hq * pl->d * 2.0;
    // The single launch also takes no less than its items' CU time (decode
    // items running several KV heads pay their start-up once).
    const double x_pre = pre.row_blocks > 1 ? cm.mfma_stage_cu_us : cm.rows_stage_cu_us;
    const int64_t pre_items = (int64_t)pre.mtiles * pl->hkv * pre.splits;
    const int32_t heads = pl->kv_fp8 ? 1
                                     : pick_heads_per_item(*pl, pre_items + group_items,
                                                           std::max<int64_t>(pre.split_tokens / kTileKeys, group_stages),
                                                           suf, cus);
    const double cu_us = (double)pre_items * (cm.item_cu_us + (double)(pre.split_tokens / kTileKeys) * x_pre) +
                         (double)group_items * (cm.item_cu_us + (double)group_stages * x_pre) +
                         items_cu_us(*pl, suf, qsl, seq_lens, kstart.data(), cm, heads);
    const double t_launch = std::max(cm.kernel_floor_us, cu_us / cus) + cm.launch_us;
    // one launch runs the phases (t_suf carries its launch cost), one the merge
    // merge: a launch, or inside the launch by the item completing each row
    // block (a prefix item completes a whole prefix tile's rows)
    const int32_t c_slots = pre.splits + tree.slots() + suf.splits;
    const double ml = est_merge_launch_us(merge_bytes, cm);
    const int64_t c_items = pre_items + group_items + (int64_t)n * suf.mtiles * (pl->hkv / std::max(1, heads)) * suf.splits;
    const double mi = est_merge_in_launch_us(*pl, std::min<int64_t>(pre.rows_per_wg(), total_q * pl->group), c_slots,
                                             c_items, cus, cm);
    // (not with nested levels: the merge units would need the tree's rows)
    casc_in_launch = tree.n == 0 && merges_in_launch(p, n, suf.mtiles, pl->hkv, mi, ml);
    pl->est_us_cascade = (float)(std::max(pre_us + t_grp + t_suf, t_launch) + (casc_in_launch ? mi : ml));
    pl->kv_tokens_cascade = plen + group_tokens + suffix_tokens;
  }

  // A sliding window that hides some position from some query rules the
  // packed non-causal prefix out ([p2] section 3); one that never binds is
  // plain causal attention and is dropped.
  const bool window_binds = p.sliding_window > 0 && max_seq > p.sliding_window;
  pl->window = window_binds ? p.sliding_window : 0;
  bool cascade = false;
  if (p.mode == CA_MODE_FORCE_ON) {
    if (window_binds && plen > 0) {
      delete pl;
      return fail(CA_EUNSUPPORTED, "cascade cannot run with a binding sliding window");
    }
    cascade = plen > 0;
  } else if (p.mode == CA_MODE_AUTO) {
    cascade = !window_binds && auto_gate && pl->est_us_cascade < pl->est_us_noncascade;
  }
  pl->use_cascade = cascade ? 1 : 0;

  if (cascade) {
    pl->key_start = (int32_t)plen;
    pl->prefix = pre;
    pl->suffix = suf;
    pl->tree = tree;
    // all phases share one launch (two work-groups per CU): 2 stages of
    // bf16 or 4 of fp8 in the same LDS; fp8 items run one KV head each
    pl->prefix.stages = pl->kv_fp8 ? 4 : 2;
    pl->suffix.stages = pl->kv_fp8 ? 4 : 2;
    pl->suffix.heads_per_item =
        pl->kv_fp8 ? 1
                   : pick_heads_per_item(*pl, (int64_t)pre.mtiles * pl->hkv * pre.splits + group_items,
                                         std::max<int64_t>(pre.split_tokens / kTileKeys, group_stages), suf, cus);
    pl->separate_phases = p.separate_phases;
    pl->num_slots = pre.splits + tree.slots() + suf.splits;
    pl->direct_out = false;
    order_requests(*pl, p, seq_lens, kstart.data());
  } else {
    pl->key_start = 0;
    pl->max_suffix_len = max_seq;
    pl->prefix = PhaseTile{};
    pl->suffix = nc;
    if (pl->kv_fp8) pl->suffix.stages = 4;
    pl->suffix.heads_per_item = (nc.kernel == 1 && p.heads_per_item > 0 && !pl->kv_fp8) ? p.heads_per_item : 1;
    pl->separate_phases = 0;
    pl->num_slots = nc.splits > 1 ? nc.splits : 0;
    pl->direct_out = nc.splits == 1;
    const std::vector<int64_t> zero(n, 0);
    order_requests(*pl, p, seq_lens, zero.data());
  }
  pl->slot_elems = total_q * pl->hq * pl->d;
  // Merge inside the attention launch (the estimate's choice above)
  pl->merge_in_launch = (pl->num_slots > 0 && (cascade ? casc_in_launch : nc_in_launch)) ? 1 : 0;
  if (pl->num_slots > 0) {
    const int64_t o_bytes = round_up((int64_t)pl->num_slots * pl->slot_elems * (pl->part_fp32 ? 4 : 2), 256);
    const int64_t l_bytes = round_up((int64_t)pl->num_slots * total_q * pl->hq * 4, 256);
    pl->ws_o_offset = kCounterBytes;
    pl->ws_lse_offset = kCounterBytes + o_bytes;
    pl->workspace_bytes = kCounterBytes + o_bytes + l_bytes;
  } else {
    pl->ws_o_offset = 0;
    pl->ws_lse_offset = 0;
    pl->workspace_bytes = 0;
  }
  // With use_tuned, a choice recorded for this shape replaces AUTO's, unless
  // the caller fixed one of the tuned settings. Without it (the default) the
  // plan depends on the batch and the params only.
  TunedChoice tc;
  if (p.use_tuned == 1 && p.mode == CA_MODE_AUTO && p.prefix_splits == 0 && p.heads_per_item == 0 &&
      p.max_levels == 0 && tune_lookup(*pl, &tc) && tc.mode != CA_MODE_AUTO &&
      !(tc.mode == CA_MODE_FORCE_ON && pl->window > 0)) {
    ca_params_t q2 = p;
    q2.mode = tc.mode;
    q2.prefix_splits = tc.prefix_splits;
    q2.heads_per_item = tc.heads_per_item;
    q2.max_levels = tc.max_levels;
    q2.num_cus = cus;
    delete pl;
    return cascade_attn_plan(&q2, bt, qsl, seq_lens, num_computed, out_plan);
  }
  *out_plan = pl;
  return CA_OK;
}

extern "C" ca_status_t cascade_attn_plan_info(ca_plan_t pl, ca_plan_info_t* out) {
  if (!pl || !out) return fail(CA_EINVAL, "null plan or output");
  std::memset(out, 0, sizeof(*out));
  out->use_cascade = pl->use_cascade;
  out->num_common_prefix_blocks = pl->common_blocks;
  out->common_prefix_len = pl->prefix_len;
  out->gates_pass = pl->gates_pass;
  out->prefix_splits = pl->use_cascade ? pl->prefix.splits : 0;
  out->prefix_row_tile = pl->use_cascade ? pl->prefix.rows_per_wg() : 0;
  out->suffix_chunks = pl->suffix.splits;
  out->suffix_chunk_tokens = pl->suffix.split_tokens;
  out->suffix_kernel = pl->suffix.kernel;
  out->num_partial_slots = pl->num_slots;
  out->prefix_stages = pl->use_cascade ? pl->prefix.stages : 0;
  out->suffix_stages = pl->suffix.stages;
  out->merge_in_launch = pl->merge_in_launch;
  out->suffix_heads_per_item = pl->suffix.heads_per_item;
  out->separate_phases = pl->separate_phases;
  out->num_level1_groups = pl->tree.n;
  out->level1_splits = pl->tree.n > 0 ? pl->tree.level_splits[1] : 0;
  out->shared_levels = pl->use_cascade ? pl->tree.levels : 0;
  out->kv_dtype = pl->kv_fp8 ? CA_KV_FP8_E4M3 : CA_KV_BF16;
  out->sliding_window = pl->window;
  out->suffix_longest_first = pl->order_n > 0 ? 1 : 0;
  out->partials_fp32 = pl->part_fp32;
  out->total_q = pl->total_q;
  out->workspace_bytes = pl->workspace_bytes;
  out->kv_tokens_cascade = pl->kv_tokens_cascade;
  out->kv_tokens_noncascade = pl->kv_tokens_noncascade;
  out->est_us_cascade = pl->est_us_cascade;
  out->est_us_noncascade = pl->est_us_noncascade;
  return CA_OK;
}

extern "C" ca_status_t cascade_attn_plan_groups(ca_plan_t pl, int32_t capacity, int32_t* groups_out,
                                                int32_t* deepest_out, int32_t* n_out) {
  if (!pl || !n_out || (capacity > 0 && !groups_out)) return fail(CA_EINVAL, "null plan or output");
  if (capacity < 0) return fail(CA_EINVAL, "capacity must be >= 0");
  const Tree& T = pl->tree;
  for (int32_t j = 0; j < T.n && j < capacity; ++j) {
    groups_out[4 * j] = T.level[j];
    groups_out[4 * j + 1] = T.parent[j];
    groups_out[4 * j + 2] = T.key_begin[j];
    groups_out[4 * j + 3] = T.key_end[j];
  }
  if (deepest_out)
    for (int32_t r = 0; r < pl->num_reqs; ++r) deepest_out[r] = (T.n > 0 && T.deepest[r] != 0xff) ? T.deepest[r] : -1;
  *n_out = T.n;
  return CA_OK;
}

extern "C" void cascade_attn_plan_destroy(ca_plan_t pl) { delete pl; }

extern "C" ca_status_t cascade_attn_autotune_record(const ca_params_t* params, const int32_t* bt, const int32_t* qsl,
                                                    const int32_t* seq_lens, const int32_t* num_computed,
                                                    int32_t mode, int32_t prefix_splits, int32_t heads_per_item,
                                                    int32_t max_levels) {
  if (!params) return fail(CA_EINVAL, "null pointer argument");
  if (mode != CA_MODE_FORCE_ON && mode != CA_MODE_FORCE_OFF) return fail(CA_EINVAL, "mode must be FORCE_ON or FORCE_OFF");
  if (prefix_splits < 0 || heads_per_item < 0 || max_levels < 0 || max_levels > kMaxShared)
    return fail(CA_EINVAL, "prefix_splits, heads_per_item must be >= 0 and max_levels in [0, 4]");
  // the shape key is that of the AUTO plan, made without the table
  ca_params_t p = *params;
  p.mode = CA_MODE_AUTO;
  p.use_tuned = 0;
  p.prefix_splits = 0;
  p.heads_per_item = 0;
  p.max_levels = 0;
  ca_plan_t base = nullptr;
  const ca_status_t st = cascade_attn_plan(&p, bt, qsl, seq_lens, num_computed, &base);
  if (st != CA_OK) return st;
  if (mode == CA_MODE_FORCE_ON && base->window > 0) {
    cascade_attn_plan_destroy(base);
    return fail(CA_EUNSUPPORTED, "cascade cannot run with a binding sliding window");
  }
  TunedChoice c;
  c.mode = mode;
  c.prefix_splits = prefix_splits;
  c.heads_per_item = heads_per_item;
  c.max_levels = max_levels;
  tune_record(*base, c);
  cascade_attn_plan_destroy(base);
  return CA_OK;
}
