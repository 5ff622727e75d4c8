// Host-only driver for the planner (csrc/plan.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer. It walks random and nested block tables, the
// 64-group and 512-request-order limits and every validation error path
// through the C ABI, and checks the plans against rules written out here
// independently of the planner:
//   * the shared-page count is the longest run of leading block-table columns
//     equal in every row, inside every row's own pages ("vLLM Cascade
//     Attention：用法、场景与原理解析", beaiera.top, section 8 Step 1);
//   * the shared prefix is that count in tokens, capped at the smallest
//     num_computed_tokens and floored to a page (same page, Step 2);
//   * a cascade plan's second-level groups are disjoint runs of requests
//     whose shared length lies past the batch-wide prefix.
// Exit status 0 when every check passes; the sanitizers abort on the first
// memory or undefined-behaviour error.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "cascade_attn.h"

// The planner queries the device's compute-unit count only when
// params.num_cus == 0; this host-only build answers for a 256-CU device.
extern "C" int ca_query_num_cus(int32_t* out) {
  *out = 256;
  return 0;
}

static int g_fail = 0;
static int g_cascade = 0, g_grouped = 0, g_deep = 0, g_ordered = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      std::fprintf(stderr, "check failed: %s: ", #cond); \
      std::fprintf(stderr, __VA_ARGS__);                  \
      std::fprintf(stderr, "\n");                         \
      ++g_fail;                                           \
    }                                                     \
  } while (0)

struct Batch {
  int n = 0, stride = 0, pages = 0;
  std::vector<int32_t> bt, qsl, sl, nc;
};

// Random batch: a shared prefix, optional runs of requests that share a
// document, some of whose members share a chapter of it, and so on (up to 3
// nested levels), then each request's own pages; the requests in random
// order half of the time; some block-table padding.
static Batch make_batch(std::mt19937& rng, int n, int prefix_pages, int max_groups, int max_own, int max_q) {
  auto U = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  Batch b;
  b.n = n;
  std::vector<std::vector<int32_t>> rows(n);
  int next = 0;
  std::vector<int32_t> shared;
  for (int j = 0; j < prefix_pages; ++j) shared.push_back(next++);
  int r = 0;
  int groups = max_groups > 0 ? U(0, max_groups) : 0;
  std::vector<int> doc(n, 0);
  std::vector<std::vector<int32_t>> doc_pages(n);
  for (int gi = 0; gi < groups && r < n; ++gi) {
    const int m = std::min(n - r, U(1, 6));
    for (int lvl = 0, lo = r, hi = r + m; lvl < 3 && hi - lo >= 1; ++lvl) {
      const int dp = U(1, 40);
      for (int j = 0; j < dp; ++j)
        for (int k = lo; k < hi; ++k) doc_pages[k].push_back(next + j);
      next += dp;
      // a sub-run of the members goes one level deeper
      const int a = U(lo, hi - 1), e = U(a + 1, hi);
      lo = a;
      hi = e;
      if (U(0, 2) == 0) break;
    }
    r += m + U(0, 2);
  }
  if (U(0, 1)) std::shuffle(doc_pages.begin(), doc_pages.end(), rng);
  int maxp = 0;
  for (int i = 0; i < n; ++i) {
    rows[i] = shared;
    for (int32_t p : doc_pages[i]) rows[i].push_back(p);
    const int own = U(1, max_own);
    for (int j = 0; j < own; ++j) rows[i].push_back(next++);
    maxp = std::max<int>(maxp, rows[i].size());
  }
  b.pages = next + 3;
  b.stride = maxp + U(0, 3);
  b.bt.assign((size_t)n * b.stride, 0);
  b.qsl.assign(n + 1, 0);
  b.sl.assign(n, 0);
  b.nc.assign(n, 0);
  for (int i = 0; i < n; ++i) {
    for (int j = 0; j < b.stride; ++j)
      b.bt[(size_t)i * b.stride + j] = j < (int)rows[i].size() ? rows[i][j] : U(0, b.pages - 1);
    const int used = (int)rows[i].size();
    // the last page holds 1..16 tokens
    b.sl[i] = (used - 1) * 16 + U(1, 16);
    const int q = std::min(b.sl[i], U(1, max_q));
    b.qsl[i + 1] = b.qsl[i] + q;
    b.nc[i] = b.sl[i] - q;
  }
  return b;
}

static int brute_common(const Batch& b) {
  int limit = b.stride;
  for (int i = 0; i < b.n; ++i) limit = std::min(limit, (b.sl[i] + 15) / 16);
  int c = 0;
  while (c < limit) {
    bool same = true;
    for (int i = 1; i < b.n; ++i) same = same && b.bt[(size_t)i * b.stride + c] == b.bt[c];
    if (!same) break;
    ++c;
  }
  return c;
}

static ca_params_t base_params(const Batch& b, int hq, int hkv, int d) {
  ca_params_t p;
  std::memset(&p, 0, sizeof(p));
  p.num_reqs = b.n;
  p.num_q_heads = hq;
  p.num_kv_heads = hkv;
  p.head_dim = d;
  p.page_size = 16;
  p.block_table_stride = b.stride;
  p.num_pages = b.pages;
  p.kv_stride_page = (int64_t)16 * hkv * d;
  p.kv_stride_token = (int64_t)hkv * d;
  p.kv_stride_head = d;
  p.num_cus = 256;
  return p;
}

static void check_plan(const Batch& b, const ca_params_t& p, ca_plan_t pl) {
  ca_plan_info_t info;
  CHECK(cascade_attn_plan_info(pl, &info) == CA_OK, "plan_info");
  const int common = brute_common(b);
  CHECK(info.num_common_prefix_blocks == common, "common %d vs %d", info.num_common_prefix_blocks, common);
  int min_nc = b.nc[0];
  for (int i = 0; i < b.n; ++i) min_nc = std::min(min_nc, b.nc[i]);
  const int plen = std::min(common * 16, min_nc) / 16 * 16;
  CHECK(info.common_prefix_len == plen, "prefix %d vs %d", info.common_prefix_len, plen);
  CHECK(info.gates_pass == (plen >= 256 && b.n >= 8), "gates");
  if (p.mode == CA_MODE_FORCE_OFF) CHECK(info.use_cascade == 0, "forced off");
  if (p.mode == CA_MODE_FORCE_ON && p.sliding_window == 0) CHECK(info.use_cascade == (plen > 0), "forced on");
  CHECK(info.total_q == b.qsl[b.n], "total_q");
  g_cascade += info.use_cascade;
  g_grouped += info.num_level1_groups > 0;
  g_deep += info.shared_levels >= 3;
  g_ordered += info.suffix_longest_first;
  CHECK(info.workspace_bytes >= 0 && (info.num_partial_slots == 0) == (info.workspace_bytes == 0), "workspace");
  // groups: a tree under the batch prefix (parents first), each group
  // sharing >= 256 more tokens than its parent, capped at its members'
  // num_computed; >= 2 members, which share the group's pages
  int32_t n_groups = -1;
  CHECK(cascade_attn_plan_groups(pl, 0, nullptr, nullptr, &n_groups) == CA_OK, "groups count");
  CHECK(n_groups == info.num_level1_groups && n_groups <= 64, "groups %d", n_groups);
  if (!info.use_cascade) CHECK(info.shared_levels == 0 && n_groups == 0, "non-cascade levels");
  else if (n_groups == 0) CHECK(info.shared_levels == 1, "one level");
  CHECK(info.shared_levels <= (p.max_levels == 0 ? 4 : p.max_levels), "shared levels %d", info.shared_levels);
  if (n_groups > 0) {
    std::vector<int32_t> g((size_t)4 * n_groups), deep(b.n, -7);
    int32_t n2 = 0;
    CHECK(cascade_attn_plan_groups(pl, n_groups, g.data(), deep.data(), &n2) == CA_OK && n2 == n_groups, "groups");
    std::vector<int> members(n_groups, 0);
    int max_level = 0;
    for (int j = 0; j < n_groups; ++j) {
      const int lev = g[4 * j], par = g[4 * j + 1], kb = g[4 * j + 2], ke = g[4 * j + 3];
      max_level = std::max(max_level, lev);
      CHECK(par >= -1 && par < j, "parent order %d %d", j, par);
      CHECK(lev == (par < 0 ? 1 : g[4 * par] + 1), "level %d", lev);
      CHECK(kb == (par < 0 ? plen : g[4 * par + 3]), "key_begin %d", kb);
      CHECK(ke % 16 == 0 && ke - kb >= 256, "group length %d %d", kb, ke);
    }
    CHECK(info.shared_levels == max_level + 1, "levels %d %d", info.shared_levels, max_level);
    for (int r = 0; r < b.n; ++r) {
      CHECK(deep[r] >= -1 && deep[r] < n_groups, "deepest %d", deep[r]);
      for (int j = deep[r]; j >= 0; j = g[4 * j + 1]) {
        ++members[j];
        CHECK(g[4 * j + 3] <= b.nc[r], "group cap");
        // the member holds the group's pages: those of the group's first
        // member found so far (page ids equal on every shared column)
        for (int c = 0; c < g[4 * j + 3] / 16; ++c) {
          int first = -1;
          for (int r2 = 0; r2 < b.n && first < 0; ++r2)
            for (int k = deep[r2]; k >= 0; k = g[4 * k + 1])
              if (k == j) { first = r2; break; }
          CHECK(first >= 0 && b.bt[(size_t)r * b.stride + c] == b.bt[(size_t)first * b.stride + c], "group pages");
        }
      }
    }
    for (int j = 0; j < n_groups; ++j) CHECK(members[j] >= 2, "group members %d", members[j]);
    // a short buffer: only cap rows are written
    std::vector<int32_t> s((size_t)4 * n_groups + 4, -9);
    CHECK(cascade_attn_plan_groups(pl, n_groups - 1, s.data(), nullptr, &n2) == CA_OK && n2 == n_groups, "short");
    CHECK(s[(size_t)4 * (n_groups - 1)] == -9, "wrote past capacity");
  }
}

static void fuzz(std::mt19937& rng, int iters) {
  auto U = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int heads[][2] = {{4, 4}, {32, 8}, {64, 8}, {8, 2}, {1, 1}, {16, 4}};
  for (int it = 0; it < iters; ++it) {
    const int n = U(1, it % 50 == 0 ? 700 : 40);
    Batch b = make_batch(rng, n, U(0, 70), U(0, 6), U(1, 40), U(1, it % 3 == 0 ? 80 : 2));
    int32_t blocks = -1;
    CHECK(cascade_attn_num_common_prefix_blocks(b.bt.data(), b.n, b.stride, b.sl.data(), 16, &blocks) == CA_OK,
          "detector");
    CHECK(blocks == brute_common(b), "detector %d vs %d", blocks, brute_common(b));
    const int* hh = heads[U(0, 5)];
    const int d = U(0, 1) ? 128 : 64;
    ca_params_t p = base_params(b, hh[0], hh[1], d);
    p.mode = U(0, 2);
    p.max_levels = U(0, 4);
    p.separate_phases = U(0, 1);
    p.suffix_order = U(0, 1);
    p.partials_fp32 = U(0, 1);
    p.use_tuned = U(0, 1);
    p.merge_mode = U(0, 2);
    if (U(0, 3) == 0) p.prefix_splits = U(1, 70);
    if (U(0, 3) == 0) {
      const int h = U(1, hh[1]);
      if (hh[1] % h == 0) p.heads_per_item = h;
    }
    if (U(0, 5) == 0) p.sliding_window = U(1, 600);
    if (d == 128 && U(0, 4) == 0) {
      p.kv_dtype = CA_KV_FP8_E4M3;
      p.k_scale = 0.125f;
      p.v_scale = 0.0625f;
    }
    if (U(0, 7) == 0) p.num_cus = 0;   // the stub answers
    if (U(0, 9) == 0) {
      const int mode = U(1, 2);
      const ca_status_t rs =
          cascade_attn_autotune_record(&p, b.bt.data(), b.qsl.data(), b.sl.data(), b.nc.data(), mode, U(0, 8), 0,
                                       U(0, 4));
      // a cascade choice is refused where a sliding window rules cascade out
      CHECK(rs == CA_OK || (rs == CA_EUNSUPPORTED && mode == CA_MODE_FORCE_ON && p.sliding_window > 0),
            "record %d: %s", rs, cascade_attn_last_error());
    }
    ca_plan_t pl = nullptr;
    const ca_status_t st =
        cascade_attn_plan(&p, b.bt.data(), b.qsl.data(), b.sl.data(), U(0, 1) ? b.nc.data() : nullptr, &pl);
    if (st != CA_OK) {
      // the one refusal valid metadata may meet: FORCE_ON with a binding window
      CHECK(st == CA_EUNSUPPORTED && p.mode == CA_MODE_FORCE_ON && p.sliding_window > 0, "plan failed %d: %s", st,
            cascade_attn_last_error());
      CHECK(pl == nullptr, "no plan on error");
      continue;
    }
    check_plan(b, p, pl);
    cascade_attn_plan_destroy(pl);
  }
  cascade_attn_autotune_reset();
}

// More than 64 second-level groups: 150 pairs of requests, each pair sharing
// a 320-token document after a 256-token prefix. The plan keeps 64 groups.
static void many_groups() {
  Batch b;
  b.n = 300;
  const int prefix_pages = 16, doc_pages = 20, own = 2;
  b.stride = prefix_pages + doc_pages + own;
  b.bt.assign((size_t)b.n * b.stride, 0);
  int next = prefix_pages;
  for (int pr = 0; pr < 150; ++pr) {
    const int doc0 = next;
    next += doc_pages;
    for (int k = 0; k < 2; ++k) {
      const int i = 2 * pr + k;
      for (int j = 0; j < prefix_pages; ++j) b.bt[(size_t)i * b.stride + j] = j;
      for (int j = 0; j < doc_pages; ++j) b.bt[(size_t)i * b.stride + prefix_pages + j] = doc0 + j;
      for (int j = 0; j < own; ++j) b.bt[(size_t)i * b.stride + prefix_pages + doc_pages + j] = next++;
    }
  }
  b.pages = next;
  b.qsl.assign(b.n + 1, 0);
  b.sl.assign(b.n, b.stride * 16);
  b.nc.assign(b.n, b.stride * 16 - 1);
  for (int i = 0; i < b.n; ++i) b.qsl[i + 1] = i + 1;
  ca_params_t p = base_params(b, 8, 2, 128);
  p.mode = CA_MODE_FORCE_ON;
  ca_plan_t pl = nullptr;
  CHECK(cascade_attn_plan(&p, b.bt.data(), b.qsl.data(), b.sl.data(), b.nc.data(), &pl) == CA_OK, "many groups: %s",
        cascade_attn_last_error());
  if (pl) {
    ca_plan_info_t info;
    cascade_attn_plan_info(pl, &info);
    CHECK(info.num_level1_groups == 64, "kept %d groups", info.num_level1_groups);
    check_plan(b, p, pl);
    cascade_attn_plan_destroy(pl);
  }
}

// Every validation error path returns its status, a message and no plan.
static void error_paths() {
  std::mt19937 rng(5);
  Batch b = make_batch(rng, 6, 20, 1, 5, 3);
  const ca_params_t good = base_params(b, 8, 2, 128);
  auto expect = [&](const ca_params_t& p, const int32_t* bt, const int32_t* qsl, const int32_t* sl,
                    const int32_t* nc, ca_status_t want, const char* what) {
    ca_plan_t pl = reinterpret_cast<ca_plan_t>(&b);   // must be reset to null on error
    const ca_status_t st = cascade_attn_plan(&p, bt, qsl, sl, nc, &pl);
    CHECK(st == want, "%s: status %d, want %d", what, st, want);
    if (st != CA_OK) CHECK(pl == nullptr && std::strlen(cascade_attn_last_error()) > 0, "%s: message", what);
    else cascade_attn_plan_destroy(pl);
  };
  const int32_t *bt = b.bt.data(), *qsl = b.qsl.data(), *sl = b.sl.data(), *nc = b.nc.data();
  expect(good, bt, qsl, sl, nc, CA_OK, "good");
  CHECK(cascade_attn_plan(nullptr, bt, qsl, sl, nc, nullptr) == CA_EINVAL, "null params");
  expect(good, nullptr, qsl, sl, nc, CA_EINVAL, "null bt");
  expect(good, bt, nullptr, sl, nc, CA_EINVAL, "null qsl");
  expect(good, bt, qsl, nullptr, nc, CA_EINVAL, "null seq_lens");
  struct Mut {
    void (*f)(ca_params_t&);
    ca_status_t want;
    const char* what;
  };
  const Mut muts[] = {
      {[](ca_params_t& p) { p.num_reqs = 0; }, CA_EINVAL, "num_reqs"},
      {[](ca_params_t& p) { p.num_q_heads = 0; }, CA_EINVAL, "heads"},
      {[](ca_params_t& p) { p.num_q_heads = 7; }, CA_EUNSUPPORTED, "head ratio"},
      {[](ca_params_t& p) { p.head_dim = 96; }, CA_EUNSUPPORTED, "head_dim"},
      {[](ca_params_t& p) { p.page_size = 32; }, CA_EUNSUPPORTED, "page_size"},
      {[](ca_params_t& p) { p.block_table_stride = 0; }, CA_EINVAL, "stride"},
      {[](ca_params_t& p) { p.num_pages = 0; }, CA_EINVAL, "num_pages"},
      {[](ca_params_t& p) { p.kv_stride_token = 12; }, CA_EUNSUPPORTED, "kv stride"},
      {[](ca_params_t& p) { p.kv_stride_token = (int64_t)1 << 27; }, CA_EUNSUPPORTED, "kv stride range"},
      {[](ca_params_t& p) { p.mode = 3; }, CA_EINVAL, "mode"},
      {[](ca_params_t& p) { p.heads_per_item = 3; }, CA_EINVAL, "heads_per_item"},
      {[](ca_params_t& p) { p.separate_phases = 2; }, CA_EINVAL, "separate_phases"},
      {[](ca_params_t& p) { p.max_levels = 5; }, CA_EINVAL, "max_levels"},
      {[](ca_params_t& p) { p.kv_dtype = 2; }, CA_EINVAL, "kv_dtype"},
      {[](ca_params_t& p) { p.sliding_window = -1; }, CA_EINVAL, "window"},
      {[](ca_params_t& p) { p.prefix_splits = -1; }, CA_EINVAL, "prefix_splits"},
      {[](ca_params_t& p) { p.suffix_order = 2; }, CA_EINVAL, "suffix_order"},
      {[](ca_params_t& p) { p.partials_fp32 = 2; }, CA_EINVAL, "partials_fp32"},
      {[](ca_params_t& p) { p.use_tuned = 2; }, CA_EINVAL, "use_tuned"},
      {[](ca_params_t& p) { p.merge_mode = 3; }, CA_EINVAL, "merge_mode"},
      {[](ca_params_t& p) { p.k_scale = 1.0f / 0.0f; }, CA_EINVAL, "k_scale"},
      {[](ca_params_t& p) { p.kv_dtype = CA_KV_FP8_E4M3; p.head_dim = 64; p.kv_stride_page = 16 * 2 * 64;
                            p.kv_stride_token = 128; p.kv_stride_head = 64; }, CA_EUNSUPPORTED, "fp8 head_dim"},
      {[](ca_params_t& p) { p.kv_dtype = CA_KV_FP8_E4M3; p.kv_stride_head = 136; }, CA_EUNSUPPORTED, "fp8 strides"},
  };
  for (const Mut& m : muts) {
    ca_params_t p = good;
    m.f(p);
    expect(p, bt, qsl, sl, nc, m.want, m.what);
  }
  // metadata errors
  {
    std::vector<int32_t> q2 = b.qsl;
    q2[0] = 1;
    expect(good, bt, q2.data(), sl, nc, CA_EMETA, "qsl[0]");
    q2 = b.qsl;
    q2[2] = q2[1];   // request 1 without a query token
    expect(good, bt, q2.data(), sl, nullptr, CA_EMETA, "empty query");
    std::vector<int32_t> n2 = b.nc;
    n2[3] += 1;
    expect(good, bt, qsl, sl, n2.data(), CA_EMETA, "num_computed");
    std::vector<int32_t> s2 = b.sl;
    s2[1] = b.stride * 16 + 1;
    expect(good, bt, qsl, s2.data(), nullptr, CA_EMETA, "too many pages");
    s2 = b.sl;
    s2[0] = 0;
    expect(good, bt, qsl, s2.data(), nullptr, CA_EMETA, "seq_len below q_len");
    std::vector<int32_t> b2 = b.bt;
    b2[(size_t)2 * b.stride] = b.pages;
    expect(good, b2.data(), qsl, sl, nc, CA_EMETA, "page id range");
    b2 = b.bt;
    b2[(size_t)4 * b.stride + 1] = -1;
    expect(good, b2.data(), qsl, sl, nc, CA_EMETA, "negative page id");
  }
  // detector errors
  int32_t out = 0;
  CHECK(cascade_attn_num_common_prefix_blocks(nullptr, 1, 1, sl, 16, &out) == CA_EINVAL, "detector null");
  CHECK(cascade_attn_num_common_prefix_blocks(bt, 0, b.stride, sl, 16, &out) == CA_EINVAL, "detector n");
  CHECK(cascade_attn_num_common_prefix_blocks(bt, b.n, 1, sl, 16, &out) == CA_EMETA, "detector stride");
  // getters and record
  CHECK(cascade_attn_plan_info(nullptr, nullptr) == CA_EINVAL, "info null");
  int32_t n_out = 0;
  CHECK(cascade_attn_plan_groups(nullptr, 0, nullptr, nullptr, &n_out) == CA_EINVAL, "groups null");
  CHECK(cascade_attn_autotune_record(&good, bt, qsl, sl, nc, CA_MODE_AUTO, 0, 0, 0) == CA_EINVAL, "record mode");
  CHECK(cascade_attn_autotune_record(nullptr, bt, qsl, sl, nc, CA_MODE_FORCE_ON, 0, 0, 0) == CA_EINVAL,
        "record null");
  cascade_attn_plan_destroy(nullptr);
  cascade_attn_autotune_reset();
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 2000;
  std::mt19937 rng(20261202);
  error_paths();
  many_groups();
  fuzz(rng, iters);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  if (g_grouped < iters / 20 || g_deep < iters / 200) {
    std::fprintf(stderr, "too few plans with groups (%d) or with >= 3 levels (%d)\n", g_grouped, g_deep);
    return 1;
  }
  std::printf("plan_fuzz: %d random batches (%d cascade plans, %d with groups, %d with >= 3 levels, %d "
              "longest-first), error paths and the group limit: all checks passed\n",
              iters, g_cascade, g_grouped, g_deep, g_ordered);
  return 0;
}
