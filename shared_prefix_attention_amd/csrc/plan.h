// Internal plan record shared by the host planner (plan.cpp) and the launcher
// (run.hip). Not part of the public ABI.
#pragma once

#include <cstdint>
#include <string>

#include "cascade_attn.h"

namespace ca {

// Keys staged per LDS tile by the tiled kernel (4 pages of 16 tokens).
constexpr int kTileKeys = 64;
// Threads per work-group of every attention kernel (4 wave64s).
constexpr int kThreads = 256;

struct PhaseTile {
  int32_t row_blocks = 1;      // 16-row MFMA blocks per wave
  int32_t row_waves = 4;       // waves splitting the rows (rows per WG = 16 * row_blocks * row_waves)
  int32_t key_groups = 1;      // waves splitting each 64-key stage
  int32_t mtiles = 0;          // row tiles (prefix: of the packed rows; suffix: max per request)
  int32_t splits = 1;          // KV splits (prefix) or chunks per request (suffix)
  int32_t split_tokens = 0;    // tokens per split / chunk (multiple of kTileKeys)
  int32_t kernel = 0;          // 0 = tiled rows, 1 = decode (rows <= 16, waves split the keys)
  int32_t stages = 2;          // LDS pipeline depth of the tiled kernel (2 or 4)
  int32_t heads_per_item = 1;  // per-request phase, decode shape: consecutive KV heads one item runs
  int32_t rows_per_wg() const { return 16 * row_blocks * row_waves; }
};

// Longest KV range one work item may cover (its page ids are held in LDS).
constexpr int kMaxItemTokens = 512 * 16;

// Nested shared levels: groups of requests (any requests, not only
// consecutive ones) that share pages beyond the batch-wide prefix, found on
// the prefix tree of the requests' page-id sequences, up to kMaxShared
// shared levels in all (the batch-wide prefix is level 0). At most
// kMaxTreeGroups groups; they travel to the kernels as launch arguments.
constexpr int kMaxTreeGroups = 64;
constexpr int kMaxShared = 4;
// Requests whose work-item order a plan can set (kernel-argument table).
constexpr int kOrderCapacity = 512;

// The first kCounterBytes of every workspace hold the arrival counters of
// the merge inside the attention launch (zero before a workspace's first
// run; every run leaves them zero). Fixed size and place, so one workspace
// serves any sequence of plans.
constexpr int64_t kCounterBytes = int64_t(256) << 10;
constexpr int64_t kMaxCounters = kCounterBytes / 4;

struct Tree {
  int32_t n = 0;                               // groups in use
  int32_t levels = 1;                          // shared levels in use (1: the batch-wide prefix only)
  int32_t level_splits[kMaxShared] = {};       // KV splits of every group of level l (l >= 1)
  int32_t level_slot_base[kMaxShared] = {};    // first partial slot of level l
  // per group, parents before children
  int32_t level[kMaxTreeGroups] = {};          // 1 .. levels - 1
  int32_t parent[kMaxTreeGroups] = {};         // enclosing group, -1: the batch-wide prefix
  int32_t first_req[kMaxTreeGroups] = {};      // a member (its block-table row holds the shared pages)
  int32_t pos_begin[kMaxTreeGroups] = {};      // members: tree-order positions [pos_begin, pos_end)
  int32_t pos_end[kMaxTreeGroups] = {};
  int32_t key_begin[kMaxTreeGroups] = {};      // positions shared beyond the enclosing level
  int32_t key_end[kMaxTreeGroups] = {};
  int32_t split_tokens[kMaxTreeGroups] = {};   // keys per split (multiple of kTileKeys)
  int32_t rows[kMaxTreeGroups] = {};           // packed query rows: member tokens x group size
  int32_t item_begin[kMaxTreeGroups + 1] = {};
  // tree order: requests sorted so that every group's members are adjacent
  int32_t pos_tok[kOrderCapacity] = {};        // first query token of the request at each position
  int32_t pos_cum[kOrderCapacity + 1] = {};    // query tokens before each position
  uint8_t deepest[kOrderCapacity] = {};        // innermost group of each request, 0xff: none
  int32_t slots() const {
    int32_t s = 0;
    for (int l = 1; l < levels; ++l) s += level_splits[l];
    return s;
  }
};

}  // namespace ca

struct ca_plan {
  ca_params_t p;
  int32_t num_reqs = 0, hq = 0, hkv = 0, group = 0, d = 0, ps = 0;
  int64_t total_q = 0;
  int32_t max_q_len = 0;
  int32_t uniform_q = 0;       // > 0: every request has this many query tokens
  int32_t max_seq_len = 0;
  float scale = 0.f;
  int32_t kv_fp8 = 0;          // K/V caches hold fp8 e4m3 (1 byte per element)
  float k_scale = 1.f;         // dequantisation factors of the caches (1 for bf16)
  float v_scale = 1.f;
  int32_t kv_bytes() const { return kv_fp8 ? 1 : 2; }
  int32_t part_fp32 = 0;       // partial outputs in fp32 (else bf16); partial LSEs are fp32
  // bytes of one (token, head) partial state: output and LSE
  double part_row_bytes() const { return part_fp32 ? (d + 1) * 4.0 : d * 2.0 + 4.0; }
  int32_t window = 0;          // sliding window of the non-cascade path (0: none)

  int32_t common_blocks = 0;
  int32_t prefix_len = 0;
  int32_t gates_pass = 0;
  int32_t use_cascade = 0;

  ca::PhaseTile prefix;       // used when use_cascade
  ca::PhaseTile suffix;       // suffix phase (cascade) or the only phase
  int32_t key_start = 0;      // first KV position of the suffix phase (prefix_len or 0)
  int32_t max_suffix_len = 0; // max over requests of seq_len - key_start
  int32_t num_slots = 0;      // partial states per (token, head)
  bool direct_out = false;    // the last attention launch writes the bf16 output directly
  int32_t separate_phases = 0;// cascade: prefix and suffix as two launches
  ca::Tree tree;              // cascade: nested shared levels (n = 0: none)
  int64_t slot_elems = 0;     // T * Hq * d
  int32_t merge_in_launch = 0;// partial states merged inside the attention launch (no merge launch)
  int64_t ws_o_offset = 0;    // byte offset of the partial outputs (after the counters)
  int64_t ws_lse_offset = 0;  // byte offset of the partial LSE array
  int64_t workspace_bytes = 0;

  int64_t sum_seq = 0;         // shape signature inputs (autotuning table)
  int32_t cand_groups = 0;     // nested groups the detector found (taken or not)
  // dispatch order of the per-request work items: the j-th request slot runs
  // request order[j] (order_n = 0: batch order; else order_n = num_reqs)
  int32_t order_n = 0;
  uint16_t order[ca::kOrderCapacity] = {};
  int64_t kv_tokens_cascade = 0;
  int64_t kv_tokens_noncascade = 0;
  float est_us_cascade = 0.f, est_us_noncascade = 0.f;
};

namespace ca {
void set_error(const std::string& msg);

// Choice recorded by the autotuner for a batch shape (ca_params_t fields).
struct TunedChoice {
  int32_t mode = CA_MODE_AUTO;
  int32_t prefix_splits = 0;
  int32_t heads_per_item = 0;
  int32_t max_levels = 0;
};
void tune_record(const ca_plan& pl, const TunedChoice& c);
}
