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

// Second shared level: groups of consecutive requests that share pages
// beyond the batch-wide prefix. At most kMaxLevel1Groups (they travel to the
// kernels as launch arguments).
constexpr int kMaxLevel1Groups = 64;
// Requests whose work-item order a plan can set (kernel-argument table).
constexpr int kOrderCapacity = 512;

// The first kCounterBytes of every workspace hold the arrival counters of
// the merge inside the attention launch (zero before a workspace's first
// run; every run leaves them zero). Fixed size and place, so one workspace
// serves any sequence of plans.
constexpr int64_t kCounterBytes = int64_t(256) << 10;
constexpr int64_t kMaxCounters = kCounterBytes / 4;

struct Level1 {
  int32_t n = 0;                               // groups in use
  int32_t splits = 0;                          // KV splits of every group
  int32_t req_begin[kMaxLevel1Groups] = {};    // requests [req_begin, req_end), ascending
  int32_t req_end[kMaxLevel1Groups] = {};
  int32_t key_end[kMaxLevel1Groups] = {};      // group shares positions [prefix_len, key_end)
  int32_t split_tokens[kMaxLevel1Groups] = {}; // keys per split (multiple of kTileKeys)
  int32_t item_begin[kMaxLevel1Groups + 1] = {};
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
  ca::Level1 lvl1;            // cascade: second shared level (n = 0: none)
  int64_t slot_elems = 0;     // T * Hq * d
  int32_t merge_in_launch = 0;// partial states merged inside the attention launch (no merge launch)
  int64_t ws_o_offset = 0;    // byte offset of the partial outputs (after the counters)
  int64_t ws_lse_offset = 0;  // byte offset of the partial LSE array
  int64_t workspace_bytes = 0;

  int64_t sum_seq = 0;         // shape signature inputs (autotuning table)
  int32_t cand_groups = 0;     // second-level groups the detector found (taken or not)
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
