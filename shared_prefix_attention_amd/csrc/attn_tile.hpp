// Tiled paged attention on bf16 MFMA (gfx950), producing partial softmax
// states. One kernel serves three roles:
//   * the prefix phase: every query row of the batch (all requests' tokens
//     packed as one sequence, times the query heads of one KV head) attends
//     non-causally to the shared-prefix pages (block-table row 0);
//   * the suffix phase: each request's rows attend causally to its own KV
//     range [key_start, seq_len) through its block-table row;
//   * a second shared level: the rows of each group of consecutive requests
//     that share more pages than the whole batch attend non-causally to
//     those extra pages (block-table row of the group's first request);
//   * the non-cascade path: the suffix phase with key_start = 0, writing the
//     final bf16 output directly when its KV range is one work item.
// The cascade phases run in one launch (cascade_phases_kernel); their
// partial states are combined by the merge kernel.
// ("vLLM Cascade Attention：用法、场景与原理解析", beaiera.top, section 8
// Step 5: prefix phase, suffix phase, LSE merge; section 4 for which keys
// each query sees.)
//
// Work-group: RW * KG wave64s owning one (KV head, row tile, KV range) item.
// K/V are streamed SK keys (SK/16 pages) per stage straight from HBM into
// LDS with global_load_lds_dwordx4 (no register staging), NS stage buffers.
// Shapes with several row waves share each stage (one barrier per stage);
// the decode shape (one row wave, KG key groups) runs one pipeline per wave,
// since each wave reads only the keys its own DMA wrote.
// Each LDS row (one key, d contiguous) has its 16-byte chunks XOR-swizzled
// by the key index so the MFMA operand reads are bank-conflict free.
// Wave (rw, kg) owns query rows [rw*16*RB, +16*RB) of the tile and keys
// [kg*SK/KG, +SK/KG) of every stage, with its own online-softmax state; the
// KG states of a row block are merged through LDS at the end. Per wave and
// stage:
//   S^T[key][row] = K Q^T   (v_mfma_f32_16x16x32_bf16: A = K from LDS,
//                            B = Q^T kept in registers)
//   online softmax on S^T (exp2 domain, fp32; the per-row reference max
//                          moves only past a slack, so rescales are rare),
//                          P^T rounded to bf16
//   O^T[d][row] += V^T P^T (A = V^T read with the LDS transpose load
//                            ds_read_b64_tr_b16, B = P^T taken straight from
//                            the S^T accumulators; 16x16x32 MFMA for 32-key
//                            groups, 16x16x16 for 16-key groups)
// Computing the transposed products leaves P in the lane layout the second
// product needs, so P never moves between lanes.
//
// Partial states (normalised o, bf16 or fp32, and the natural-log LSE) go
// to the workspace for the merge kernel; an item covering a request's whole
// range on the non-cascade path writes the final bf16 output instead.
// Per-request items run in the plan's order (longest key range first).
//
// Masking: positions past the item's range are loaded from the item's last
// valid position (so no unused page or NaN tail slot is ever read) and their
// scores are set to -inf; causally hidden positions likewise. Stages that
// need no mask skip it.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "merge.hpp"

namespace ca {

struct TileArgs {
  const uint16_t* q;            // [T][hq][D] bf16 bits
  const uint16_t* k;            // paged cache, element strides below
  const uint16_t* v;
  int64_t sp, st, sh;           // page, token-slot, head strides (elements)
  const int32_t* bt;            // [num_reqs][bt_stride]
  const int32_t* qsl;           // [num_reqs + 1]
  const int32_t* seq_lens;      // [num_reqs]
  int32_t bt_stride;
  int32_t hq, hkv, group;
  float scale_log2;             // softmax_scale * log2(e)
  int32_t prefix_mode;          // 1: prefix phase, 2: nested group levels, 0: per-request phase
  int32_t total_rows;           // prefix: T * group
  int32_t key_start;            // per-request phase: first KV position
  int32_t prefix_len;           // prefix phase: number of shared KV positions
  int32_t num_reqs;
  int32_t mtiles;               // row tiles (prefix) / max row tiles per request
  int32_t splits;               // KV splits (prefix) / chunks per request
  int32_t heads_per_item;       // per-request phase: consecutive KV heads one item runs (divides hkv)
  int32_t split_tokens;         // multiple of 64, <= kMaxItemPages * 16
  void* part_o;                 // [slots][T][hq][D] bf16 or fp32 (partial mode)
  int32_t part_fp32;            // partial outputs in fp32 (else bf16)
  float* part_lse;              // [slots][T][hq] fp32, natural log
  int32_t slot_base;
  int64_t slot_elems;           // T * hq * D
  int64_t slot_rows;            // T * hq
  uint16_t* out;                // [T][hq][D] bf16 (direct / merge mode)
  float* lse_out;               // [T][hq] (may be null)
  int32_t direct;               // write the final output (no partial)
  float v_scale;                // dequantisation factor of V (1 for bf16 caches)
  int32_t window;               // per-request phase: sliding window W (> 0: keys p - W < t <= p)
  const float* sinks;           // [hq] attention-sink logits (natural log) or null; direct mode only
  int32_t coherent;             // partial states are merged inside this launch: device-scope stores
};

// Merge inside the attention launch (counters null: a separate merge
// launch). A merge unit is (request r, per-request row tile m, KV head g):
// the rows [m * m_suf_rows, +m_suf_rows) of r under the query heads of g.
// Every work item that writes partial states of a unit's rows counts itself
// at the unit once; the item that brings the count to the unit's number of
// such items merges the unit and resets the counter to 0. A kernel argument
// of its own, read only at an item's end, so that none of its fields stays
// in registers through the stage loop.
struct MergeTailArgs {
  int32_t* counters;            // [num_reqs][m_suf_mtiles][hkv] int32, zero between launches
  const int32_t* qsl;           // [num_reqs + 1]
  const void* part_o;           // partial states, as in TileArgs
  const float* part_lse;
  uint16_t* out;
  float* lse_out;
  const float* sinks;
  int64_t slot_elems, slot_rows;
  int32_t part_fp32;
  int32_t merge_slots;          // partial states per row
  int32_t hq, hkv, group, num_reqs;
  int32_t m_pre_splits;         // prefix items per prefix row tile (0: no prefix phase)
  int32_t m_pre_rows;           // rows per prefix tile
  int32_t m_suf_splits;         // per-request items per (request, row tile, KV head)
  int32_t m_suf_rows;           // rows per per-request tile
  int32_t m_suf_mtiles;         // per-request row tiles of the longest query (counter stride)
  int32_t uniform_q;            // > 0: every request has this many query tokens (request r's tokens
                                // are [r * uniform_q, (r + 1) * uniform_q): no lookup needed)
};

// What an item wrote, for its merge tail: role (prefix_mode as in
// TileArgs), request (or the group's first request), group, rows in the
// role's own numbering, KV heads g0 .. g0 + H - 1. wrote = 0: nothing.
struct ItemEnd {
  int32_t wrote, mode, req, grp, row_begin, row_end, g0, H;
};

// Nested shared levels: groups of requests that share KV positions
// [key_begin, key_end) beyond the level that encloses them (the batch-wide
// prefix, or another group). Members are any requests: in the tree order
// (requests sorted so that every group's members are adjacent) group j holds
// positions [pos_begin[j], pos_end[j]). Its packed query rows are its
// members' tokens in that order, times the query heads of a KV head; pos_tok
// and pos_cum give the first token of the request at each position and the
// tokens before it. Group j's work items are [item_begin[j], item_begin[j +
// 1]) of the group-level launch, (row tile, KV head, split) with its level's
// split count; the levels' partial slots follow one another. Passed by value
// (kernel arguments), so the plan needs no device copy.
constexpr int kMaxGroups = 64;
constexpr int kMaxLevels = 4;              // shared levels, the batch-wide prefix included
constexpr int kMaxTreeOrder = 512;
struct GroupTable {
  int32_t n;                               // groups (0: one shared level)
  int32_t levels;                          // shared levels in use
  int32_t level_splits[kMaxLevels];        // [l]: KV splits of every group of level l >= 1
  int32_t level_slot_base[kMaxLevels];     // [l]: first partial slot of level l
  int32_t uniform_q;                       // > 0: every request has this many query tokens
  int32_t item_begin[kMaxGroups + 1];
  int32_t level[kMaxGroups];
  int32_t first_req[kMaxGroups];           // a member: its block-table row holds the shared pages
  int32_t pos_begin[kMaxGroups];
  int32_t pos_end[kMaxGroups];
  int32_t key_begin[kMaxGroups];
  int32_t key_end[kMaxGroups];
  int32_t split_tokens[kMaxGroups];        // multiple of 64
  int32_t rows[kMaxGroups];                // packed query rows of the group
  int32_t pos_tok[kMaxTreeOrder];
  int32_t pos_cum[kMaxTreeOrder + 1];
  uint8_t deepest[kMaxTreeOrder];          // [request]: innermost group, 0xff: none
};

// Kernels of plans without nested levels take an empty struct in place of
// the group table: every launch copies its argument block, so a smaller one
// costs less host time per launch.
struct NoGroupTable {};
template <bool TREE>
using GroupTableArg = std::conditional_t<TREE, GroupTable, NoGroupTable>;

// Group-table fields used by the per-request and nested-level items; the
// empty table of plans without nested levels answers as a table with no
// groups (its values are never used).
__device__ __forceinline__ int gt_deepest(const GroupTable& gt, int r) {
  return (gt.n > 0 && gt.deepest[r] != 0xff) ? gt.deepest[r] : -1;
}
__device__ __forceinline__ int gt_deepest(const NoGroupTable&, int) { return -1; }
__device__ __forceinline__ int gt_key_end(const GroupTable& gt, int j) { return gt.key_end[j]; }
__device__ __forceinline__ int gt_key_end(const NoGroupTable&, int) { return 0; }
__device__ __forceinline__ int gt_rows(const GroupTable& gt, int j) { return gt.rows[j]; }
__device__ __forceinline__ int gt_rows(const NoGroupTable&, int) { return 0; }
__device__ __forceinline__ int gt_slot_base(const GroupTable& gt, int j) { return gt.level_slot_base[gt.level[j]]; }
__device__ __forceinline__ int gt_slot_base(const NoGroupTable&, int) { return 0; }

// Query token of group-local token t of group j (its members' tokens in tree
// order): the position p holding it, then the token within p's request.
__device__ __forceinline__ int group_token(const GroupTable& gt, int j, int t) {
  const int tg = gt.pos_cum[gt.pos_begin[j]] + t;
  int p;
  if (gt.uniform_q > 0) {
    p = gt.pos_begin[j] + t / gt.uniform_q;
  } else {   // the last position in [pos_begin, pos_end) with pos_cum <= tg
    int lo = gt.pos_begin[j], hi = gt.pos_end[j] - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gt.pos_cum[mid] <= tg) lo = mid;
      else hi = mid - 1;
    }
    p = lo;
  }
  return gt.pos_tok[p] + (tg - gt.pos_cum[p]);
}

// Dispatch order of the per-request work items: request slot j runs request
// req[j] (n = 0: batch order, else n = num_reqs). The planner starts the
// longest key ranges first, so a launch ends on short items. Kernel argument.
constexpr int kMaxOrderedReqs = 512;
struct ReqOrder {
  int32_t n;
  uint16_t req[kMaxOrderedReqs];
};

constexpr int kMaxItemPages = 512;

// Online softmax: the per-row reference max (log2 domain) is raised only when
// a stage's max exceeds it by more than this many units, so the exponentials
// taken against it lie in (0, 2^kRescaleSlack].
constexpr float kRescaleSlack = 8.f;

// ESZ: bytes per cache element, 2 (bf16) or 1 (fp8).
template <int D, int NS, int SK, int ESZ = 2>
struct TileSmem {
  static constexpr int TILE_BYTES = SK * D * ESZ;          // one of K or V, one stage
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int NS_STAGE_BYTES = NS * STAGE_BYTES;  // the page table follows
  // After the page table has been read into registers, the same bytes hold
  // each wave's 16 rows of Q (bf16), requested by DMA (one-row-block shapes)
  static constexpr int Q_BYTES = 4 * 16 * D * 2;
  static constexpr int BYTES = NS_STAGE_BYTES + (kMaxItemPages * 4 > Q_BYTES ? kMaxItemPages * 4 : Q_BYTES);
};

// 16-byte chunk swizzles of a key row (rows are D*2 bytes apart), chosen
// from LDS bank-conflict counts measured on gfx950. K rows are read one
// 16-byte chunk column across 16 consecutive keys (MFMA A operand); V rows
// by the transpose load, 8 bytes from each of 4 consecutive keys per group of
// 4 lanes. Both depend on key mod 16 only, so they repeat every 16 keys.
template <int D>
__device__ __forceinline__ int chunk_swz(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int chunk_swz_v(int key) {
  return D == 128 ? ((2 * key) & 15) : ((key >> 1) & 7);
}

// fp8 caches (head_dim 128: key rows of 128 bytes, 8 chunks of 16 bytes).
// K is read one 16-byte chunk column across 16 consecutive keys; XOR with key
// mod 8, bit 0 flipped for keys 8..15, puts those reads in 16 distinct (row
// parity, chunk) bank groups of a 256-byte LDS cycle. V is read with the
// 8-bit transpose load, 8 key rows x 2 halves per 16-lane group (see
// read_v8 in attn_item); bits 1, 2 and 4 of the key pick the XOR so that a
// group's 16 reads are distinct and the two groups of a cycle complementary.
__device__ __forceinline__ int chunk_swz_k8(int key) { return (key & 7) ^ ((key >> 3) & 1); }
__device__ __forceinline__ int chunk_swz_v8(int key) {
  return ((key >> 1) & 1) | ((((key >> 4) ^ (key >> 2)) & 1) << 1) | (((key >> 2) & 1) << 2);
}

// Two fp8 (OCP e4m3) values, bytes 0-1 (high: 2-3) of w, as two bf16 in one
// v_cvt_scalef32_pk_bf16_fp8 with scale 1. Every e4m3 value, subnormals
// included, is a bf16 value, so the conversion is exact (checked on the device
// against v_cvt_pk_f32_fp8 + v_cvt_pk_bf16_f32 for all 256 codes in both
// halves of both words).
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}
// Eight fp8 values, bytes 0..7 of (w0, w1), as eight bf16 in element order.
__device__ __forceinline__ u32x4_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return u32x4_t{fp8x2_to_bf16<false>(w0), fp8x2_to_bf16<true>(w0), fp8x2_to_bf16<false>(w1),
                 fp8x2_to_bf16<true>(w1)};
}
// Four fp8 values (bytes 0..3 of w) as four bf16.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16(uint32_t w) {
  return u32x2_t{fp8x2_to_bf16<false>(w), fp8x2_to_bf16<true>(w)};
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds_block + 16 l (the block address must be wave-uniform).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_block) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(uintptr_t)lds_block, 16, 0, 0);
}

// Waits until at most N vector-memory ops of this wave are outstanding
// (expcnt / lgkmcnt left unconstrained). gfx9 s_waitcnt encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// LDS reads through inline asm: the compiler does not track them, so it
// neither inserts waits of its own (the builtin transpose read would make it
// wait for every in-flight LDS DMA, vmcnt 0) nor interleaves them with their
// consumers. Their results must pass through lds_wait_regs() before use.
template <int OFF>
__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// 16-key block kb of a K tile (key rows STRIDE bytes apart), kb a constant
// after unrolling
template <int STRIDE>
__device__ __forceinline__ u32x4_t lds_read_b128_kb(uint32_t addr, int kb) {
  switch (kb) {
    case 0: return lds_read_b128<0>(addr);
    case 1: return lds_read_b128<16 * STRIDE>(addr);
    case 2: return lds_read_b128<32 * STRIDE>(addr);
    default: return lds_read_b128<48 * STRIDE>(addr);
  }
}

// ds_read_b64_tr_b16: within each 16-lane group, lane 4*j + c supplies the
// address of row j, columns [4c, 4c+4) of a 4 x 16 block of 16-bit values;
// lane i receives column i of the four rows.
template <int OFF = 0>
__device__ __forceinline__ u32x2_t lds_read_tr16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}

// ds_read_b64_tr_b8: within each 16-lane group, lane 2*j + c supplies the
// address of row j, bytes [8c, 8c+8) of an 8 x 16 block of bytes; lane i
// receives column i of the eight rows (byte j = row j). Measured on the
// device with an in-bounds probe.
template <int OFF = 0>
__device__ __forceinline__ u32x2_t lds_read_tr8(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}

// Pins a value in program order: code that produces it stays above, code
// that consumes it stays below (inline asm statements keep their order).
template <typename T>
__device__ __forceinline__ void reg_fence(T& x) {
  asm volatile("" : "+v"(x));
}
template <typename T, int N>
__device__ __forceinline__ void reg_fence(T (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) reg_fence(x[i]);
}

// Waits for this wave's LDS reads and makes the registers that received them
// outputs of the wait, so no consumer can be scheduled above it.
template <typename T, int N>
__device__ __forceinline__ void lds_wait_regs(T (&r)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  reg_fence(r);
}

// Work-group barrier without the memory fences of __syncthreads() (which
// would wait for every in-flight LDS DMA): this wave's LDS reads are retired
// first (lgkmcnt 0); DMA completion is waited for explicitly by the caller.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4_t mfma16x16x16(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}

// Token range [q0, q1) of request r.
__device__ __forceinline__ void req_tokens(const MergeTailArgs& a, int r, int& q0, int& q1) {
  if (a.uniform_q > 0) {
    q0 = r * a.uniform_q;
    q1 = q0 + a.uniform_q;
  } else {
    q0 = a.qsl[r];
    q1 = a.qsl[r + 1];
  }
}

// Items that write partial states of unit (r, m): the prefix tiles that
// overlap its rows (times the prefix splits) and its own per-request items
// (one per KV chunk). Plans with nested shared levels merge in a launch of
// their own. q0 / q1: r's token range.
__device__ __forceinline__ int unit_item_count(const MergeTailArgs& a, int m, int q0, int q1) {
  const int rows_r = (q1 - q0) * a.group;
  const int lo = m * a.m_suf_rows, hi = min(lo + a.m_suf_rows, rows_r);   // request-local rows
  int e = a.m_suf_splits;
  if (a.m_pre_splits > 0) {
    const int base = q0 * a.group;   // packed row of the request's first row
    e += a.m_pre_splits * ((base + hi - 1) / a.m_pre_rows - (base + lo) / a.m_pre_rows + 1);
  }
  return e;
}

// Work list of a merge tail in LDS: [0] = entries; entry k at 4 + 4k:
// counter index, first token of the request, first row of the unit inside
// the request, rows of the unit.
constexpr int kTailEntryInts = 4;

// Wave 0, one lane: counts this item's arrival at unit (r, m, g) and, if it
// completes the unit, appends the unit to the work-group's list.
__device__ __forceinline__ void arrive(const MergeTailArgs& a, int r, int m, int g, int q0, int q1,
                                       int32_t* s_list) {
  const int u = (r * a.m_suf_mtiles + m) * a.hkv + g;
  const int expect = unit_item_count(a, m, q0, q1);
  const int old = __hip_atomic_fetch_add(a.counters + u, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1 == expect) {
    const int k = __hip_atomic_fetch_add(s_list, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    int32_t* ent = s_list + 4 + kTailEntryInts * k;
    const int lo = m * a.m_suf_rows;
    ent[0] = u;
    ent[1] = q0;
    ent[2] = lo;
    ent[3] = min(lo + a.m_suf_rows, (q1 - q0) * a.group) - lo;
  }
}

// Wave 0: the last request r in [r_lo, r_end) with qsl[r] <= tok, searched
// 64 candidates per memory round trip.
__device__ __forceinline__ int request_of_token(const MergeTailArgs& a, int r_lo, int r_end, int tok) {
  if (a.uniform_q > 0) return min(max(tok / a.uniform_q, r_lo), r_end - 1);
  const int lane = threadIdx.x & 63;
  int lo = r_lo, n = r_end - r_lo;   // answer in [lo, lo + n)
  while (n > 1) {
    const int step = (n + 63) / 64;
    const int c = lo + lane * step;   // candidate starts
    const bool le = c < lo + n && a.qsl[c] <= tok;
    const uint64_t mask = __builtin_amdgcn_ballot_w64(le);
    const int j = mask ? 63 - __builtin_clzll(mask) : 0;   // last candidate with qsl <= tok
    lo = lo + j * step;
    n = min(step, r_end - lo);
  }
  return lo;
}

// End of a work item when the merge runs inside the launch. The item's
// partial states were written with device-scope stores; every thread waits
// until its stores are complete, then wave 0 counts the item at every unit
// whose rows it wrote (device-scope atomic add). Units it completes are
// merged here, by the whole work-group, reading the partial states with
// device-scope loads issued after the counts came back: every row part in
// the canonical slot order of the merge kernel, so the result does not
// depend on which item came last. No L2-wide write-back or invalidation is
// needed (the partial states never sit dirty, or stale, in an XCD's L2).
// The counters go back to 0 for the next launch.
// s_list: LDS the item no longer uses (its stage buffers), >= 4 KB.
template <int D, int NT>
__device__ __forceinline__ void merge_tail(const MergeTailArgs& a, const ItemEnd& e, int32_t* s_list) {
  if (!e.wrote) return;
  const int tid = threadIdx.x;
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) expcnt(0) lgkmcnt(0): this thread's stores are done
  __syncthreads();                 // (and every wave is done with the stage buffers)
  if (tid == 0) s_list[0] = 0;
  __syncthreads();
  if (tid < 64) {
    const int G = a.group, RS = a.m_suf_rows;
    if (e.mode == 0) {
      const int m = e.row_begin / RS;
      int q0, q1;
      req_tokens(a, e.req, q0, q1);
      for (int h = tid; h < e.H; h += 64) arrive(a, e.req, m, e.g0 + h, q0, q1, s_list);
    } else {
      // packed rows [p_lo, p_hi) and the requests they may belong to
      const int p_lo = e.row_begin, p_hi = e.row_end, r_lo = 0, r_end = a.num_reqs;
      const int tok_lo = p_lo / G, tok_hi = (p_hi - 1) / G;
      const int first = request_of_token(a, r_lo, r_end, tok_lo);
      for (int r = first + tid; r < r_end; r += 64) {
        int q0, q1;
        req_tokens(a, r, q0, q1);
        if (q0 > tok_hi) break;
        const int base = q0 * G, rows_r = (q1 - q0) * G;
        const int l0 = max(p_lo, base) - base, l1 = min(p_hi, base + rows_r) - base;
        if (l0 >= l1) continue;
        for (int m = l0 / RS; m <= (l1 - 1) / RS; ++m) arrive(a, r, m, e.g0, q0, q1, s_list);
      }
    }
  }
  __syncthreads();
  const int n_won = s_list[0];
  if (n_won == 0) return;
  // each thread merges NCH 16-byte chunks of a row (16 chunks in flight per
  // batch of slots); unit k owns flat work items [cum_k, cum_k + rows_k * tpr)
  constexpr int NCH = 2;
  constexpr int TPR_BF16 = D / 8 / NCH, TPR_F32 = D / 4 / NCH;
  const int tpr = a.part_fp32 ? TPR_F32 : TPR_BF16;
  MergeArgs ma;
  ma.part_o = a.part_o;
  ma.part_lse = a.part_lse;
  ma.slots = a.merge_slots;
  ma.rows = a.slot_rows;
  ma.slot_elems = a.slot_elems;
  ma.out = a.out;
  ma.lse_out = a.lse_out;
  ma.sinks = a.sinks;
  ma.hq = a.hq;
  int k = 0, cum = 0;   // the unit holding this thread's first work item (scan kept across passes)
  for (int w = tid;; w += NT) {
    while (k < n_won && cum + s_list[4 + kTailEntryInts * k + 3] * tpr <= w) {
      cum += s_list[4 + kTailEntryInts * k + 3] * tpr;
      ++k;
    }
    if (k >= n_won) break;
    const int32_t* ent = s_list + 4 + kTailEntryInts * k;
    const int g = ent[0] % a.hkv;
    const int i = ent[2] + (w - cum) / tpr;   // request-local row
    const int part = (w - cum) % tpr;
    const int64_t row = (int64_t)(ent[1] + i / a.group) * a.hq + g * a.group + i % a.group;
    if (a.part_fp32) merge_row_part<D, true, true, NCH>(ma, row, part);
    else merge_row_part<D, false, true, NCH>(ma, row, part);
  }
  if (tid < n_won)
    __hip_atomic_store(a.counters + s_list[4 + kTailEntryInts * tid], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// MH: the item may cover several consecutive KV heads of one request (same
// pages and key range), run as one continuous stage pipeline.
// WIN: the item may apply a sliding window and attention sinks (the
// stand-alone kernel; the cascade launch has neither).
// PM: the role (prefix_mode) when fixed at compile time, -1: a.prefix_mode.
// smem: the work-group's LDS array (its size is checked against the shape's).
// GT: GroupTable, or NoGroupTable for plans without nested levels.
template <int D, int RB, int RW, int KG, int NS, int SK, bool MH, bool F8, bool WIN, int PM = -1, size_t NB = 0,
          typename GT = GroupTable>
__device__ __forceinline__ void attn_item(const TileArgs& a, const GT& gt, const ReqOrder& ro, const int bid,
                                          uint8_t (&smem)[NB], ItemEnd& end) {
  constexpr bool TREE = std::is_same<GT, GroupTable>::value;
  end.wrote = 0;
  const int pmode = PM >= 0 ? PM : a.prefix_mode;
  constexpr int W = RW * KG;              // waves per work-group
  constexpr int NT = 64 * W;              // threads
  constexpr int ROWS = 16 * RB * RW;      // query rows per work-group
  constexpr int KC = D / 32;              // 32-wide d chunks per QK^T MFMA chain
  constexpr int DB = D / 16;              // 16-wide d blocks of the output
  constexpr int ESZ = F8 ? 1 : 2;         // bytes per cache element
  constexpr int CPR = D * ESZ / 16;       // 16-byte chunks per K/V row
  constexpr int KPB = 64 / CPR;           // keys per 1 KB DMA block
  constexpr int BLK = SK / KPB;           // 1 KB DMA blocks per tile (K or V)
  static_assert(BLK % W == 0, "DMA blocks must divide among the waves");
  constexpr int BLK_PER_WAVE = BLK / W;
  constexpr int OPS = 2 * BLK_PER_WAVE;   // vector-memory ops per wave per stage
  constexpr int NKB = SK / 16 / KG;       // 16-key blocks per wave per stage
  static_assert((NKB == 1 || NKB == 2 || NKB == 4) && SK % (16 * KG) == 0, "each wave needs 1, 2 or 4 16-key blocks");
  // Decode shape (one row wave, the stage's keys split over the W waves):
  // wave w reads exactly the 16 keys of each stage that its own DMA writes,
  // so its pipeline needs no work-group barrier, and it refills a buffer as
  // soon as it holds that stage's K and V fragments in registers (one more
  // stage in flight than a shared buffer allows).
  constexpr bool PRIV = RW == 1;
  static_assert(!PRIV || (KG == W && NKB == 1 && SK / W == 16), "per-wave pipelines need one 16-key block per wave");
  constexpr int ROWB = D * ESZ;           // LDS bytes per key row
  using SM = TileSmem<D, NS, SK, ESZ>;
  static_assert(NB >= (size_t)SM::BYTES, "LDS array smaller than the shape's layout");
  // The key-group states are combined in the stage buffer just consumed
  // (bf16); fp8 stages are too small for that, so fp8 items run one head
  // and combine at the item's end, when no DMA is in flight, from LDS 0.
  static_assert(!F8 || (D == 128 && !MH), "fp8 caches: head_dim 128, one head per item");
  static_assert(KG == 1 || (DB % KG == 0 && KG * RW * 16 * RB * ((KG - 1) * (DB / KG) * 16 + 4) * 4 <=
                                           (F8 ? NS : 1) * SM::STAGE_BYTES), "key-group combine scratch");
  int32_t* s_pages = reinterpret_cast<int32_t*>(smem + NS * SM::STAGE_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
  const int rw = wave % RW;
  const int kg = wave / RW;
  const int lr = lane & 15;
  const int lq = lane >> 4;

  // ---------------------------------------------------------- item decode
  // Everything that needs no memory comes from the block index. The page ids
  // of the item's KV range are fetched speculatively (the block-table row is
  // known before the lengths are) in the same round trip as the per-request
  // lengths; entries past the request's pages are read but never used.
  int g0, row_begin, row_end, key_begin, key_end, slot;
  int tok_base = 0, q_pos_base = 0;      // token of row 0, causal position of row 0's token
  bool causal;
  const int32_t* bt_row;
  int req = 0, c = 0, mt = 0, grp = -1;
  int split_tokens = a.split_tokens;
  int win_lo_max = 0x80000000;          // window start of the item's last row (no window: none)
  int page_skip = 0;                    // pages of the item skipped below a sliding window
  const int H = MH ? a.heads_per_item : 1;   // KV heads g0 .. g0 + H - 1, one after another
  if (pmode) {
    int local = bid, splits = a.splits;
    key_begin = a.key_start;
    if constexpr (TREE) {
      if (pmode == 2) {
        // nested level: find the group whose items contain bid
        int lo = 0, hi = gt.n - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (gt.item_begin[mid] <= bid) lo = mid;
          else hi = mid - 1;
        }
        grp = lo;
        local = bid - gt.item_begin[grp];
        split_tokens = gt.split_tokens[grp];
        splits = gt.level_splits[gt.level[grp]];
        req = gt.first_req[grp];
        key_begin = gt.key_begin[grp];
      }
    }
    // The KV head is the fastest-varying index: work-groups are dealt to the
    // XCDs in turn, so with 8 KV heads all items of one head (every row tile
    // and split: they share its K/V tiles and its Q rows) run on one XCD and
    // meet in its L2.
    g0 = local % a.hkv;
    const int rest = local / a.hkv;
    c = rest % splits;
    mt = rest / splits;
    key_begin += c * split_tokens;
    causal = false;
    bt_row = a.bt + (int64_t)req * a.bt_stride;
  } else {
    c = bid % a.splits;
    int rest = bid / a.splits;
    mt = rest % a.mtiles;
    rest /= a.mtiles;
    const int groups = a.hkv / H;
    g0 = (rest % groups) * H;
    req = ro.n > 0 ? ro.req[rest / groups] : rest / groups;
    // a request in a group starts after its innermost group's shared positions
    grp = gt_deepest(gt, req);
    key_begin = (grp >= 0 ? gt_key_end(gt, grp) : a.key_start) + c * split_tokens;
    causal = true;
    bt_row = a.bt + (int64_t)req * a.bt_stride;
  }
  const int first_page = key_begin >> 4;
  constexpr int PG_PER_THREAD = (kMaxItemPages + NT - 1) / NT;
  int pg_reg[PG_PER_THREAD];
  const int item_pages = split_tokens >> 4;
#pragma unroll
  for (int k = 0; k < PG_PER_THREAD; ++k) {
    const int i = tid + k * NT;
    pg_reg[k] = i < item_pages ? bt_row[min(first_page + i, a.bt_stride - 1)] : 0;
  }
  row_begin = mt * ROWS;
  slot = (pmode == 2 ? gt_slot_base(gt, grp) : a.slot_base) + c;
  if (pmode == 1) {
    row_end = min(row_begin + ROWS, a.total_rows);
    key_end = min(key_begin + split_tokens, a.prefix_len);
  } else if (pmode == 2) {   // (only with a group table)
    row_end = min(row_begin + ROWS, gt_rows(gt, grp));
    if (row_begin >= row_end) return;   // uniform across the work-group
    key_end = max(key_begin, min(key_begin + split_tokens, gt_key_end(gt, grp)));
  } else {
    const int q0 = a.qsl[req];
    const int q_len = a.qsl[req + 1] - q0;
    const int seq_len = a.seq_lens[req];
    row_end = min(row_begin + ROWS, q_len * a.group);
    if (row_begin >= row_end) return;   // uniform across the work-group
    key_end = max(key_begin, min(key_begin + split_tokens, seq_len));
    tok_base = q0;
    q_pos_base = seq_len - q_len;        // num_computed_tokens
    if (WIN && a.window > 0) {
      // sliding window: stages wholly below the first row's window are
      // skipped (the page table stays indexed from the item's first page)
      win_lo_max = q_pos_base + (row_end - 1) / a.group - a.window + 1;
      const int lo_min = q_pos_base + row_begin / a.group - a.window + 1;
      const int skip = min(max(0, (lo_min - key_begin) / SK), (key_end - key_begin + SK - 1) / SK);
      key_begin += skip * SK;
      page_skip = skip * SK / 16;
    }
    // levels deeper than the request's innermost group hold no state for
    // its rows: mark those partial slots (contiguous, the last levels')
    // empty, weight 0 in the merge
    int e_lo = 0, n_empty = 0;
    if constexpr (TREE) {
      const int lv = grp >= 0 ? gt.level[grp] + 1 : 1;
      if (lv < gt.levels) {
        e_lo = gt.level_slot_base[lv];
        n_empty = gt.level_slot_base[gt.levels - 1] + gt.level_splits[gt.levels - 1] - e_lo;
      }
    }
    if (c == 0 && n_empty > 0) {
      const int nrows = row_end - row_begin;
      for (int e = tid; e < nrows * H * n_empty; e += NT) {
        const int s = e / (nrows * H);
        const int rh = e - s * (nrows * H);
        const int hh = rh / nrows;
        const int m = row_begin + (rh - hh * nrows);
        const int64_t row = (int64_t)(tok_base + m / a.group) * a.hq + (g0 + hh) * a.group + m % a.group;
        float* lp = a.part_lse + (int64_t)(e_lo + s) * a.slot_rows + row;
        if (a.coherent) store_dev_f32(lp, -INFINITY);
        else *lp = -INFINITY;
      }
    }
  }
  const int n_tiles = max(0, (key_end - key_begin + SK - 1) / SK);
  // keys at or below this position are visible to every row of the item
  const int all_visible_to = causal ? q_pos_base + row_begin / a.group : 0x7fffffff;
#pragma unroll
  for (int k = 0; k < PG_PER_THREAD; ++k) {
    const int i = tid + k * NT;
    if (i < item_pages) s_pages[i] = pg_reg[k];
  }
  __syncthreads();

  // ------------------------------------------------- per-lane query rows
  // Row m of the tile is (token m / G, head-in-group m % G); the query head
  // of KV head g is g*G + m % G. Q of the first head is loaded before the
  // K/V stages are issued, so waiting for the first stage also waits for it.
  const int wrow0 = row_begin + rw * 16 * RB;
  const bool wave_active = wrow0 < row_end;
  int row_tok[RB], row_j[RB], row_qpos[RB];
  bool row_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int m = wrow0 + rb * 16 + lr;
    row_ok[rb] = m < row_end;
    const int t_in = m / a.group;
    row_j[rb] = m - t_in * a.group;
    row_tok[rb] = tok_base + t_in;
    // nested level: packed rows are the group members' tokens in tree order
    if constexpr (TREE)
      if (pmode == 2) row_tok[rb] = row_ok[rb] ? group_token(gt, grp, t_in) : 0;
    row_qpos[rb] = q_pos_base + t_in;
  }
  auto load_q = [&](int g, u32x4_t (&q)[RB][KC]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (row_ok[rb]) {
          // k-slot (lq, j) of chunk kc is d = kc*32 + 8*lq + j (bf16), or,
          // matching the fp8 K fragments, d = 16*(lq + 4*(kc/2)) + 8*(kc%2) + j
          const int d0 = F8 ? 16 * (lq + 4 * (kc >> 1)) + 8 * (kc & 1) : kc * 32 + lq * 8;
          q[rb][kc] = load16(a.q + ((int64_t)row_tok[rb] * a.hq + g * a.group + row_j[rb]) * D + d0);
        } else {
          q[rb][kc] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
  };
  // One row block per wave: the first head's Q goes through LDS by DMA, like
  // K and V, requested after the page table has been read (its bytes hold Q)
  // and waited for by hand once the first stages are requested, so that the
  // first stage is not held back: a register load would make the compiler
  // wait for every LDS-DMA request issued after it (vmcnt 0) before Q's first
  // use. Two row blocks: Q in registers.
  constexpr bool QLDS = RB == 1;
  static_assert(!QLDS || W == 4, "Q tiles: four waves");
  u32x4_t qf[RB][KC];
  if constexpr (!QLDS) load_q(g0, qf);

  f32x4_t o[DB][RB];
  float m_run[RB], l_run[RB];
  auto reset_state = [&]() {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[db][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m_run[rb] = -INFINITY;
      l_run[rb] = 0.f;
    }
  };
  reset_state();

  // Lane-constant parts of the LDS operand addresses (the XOR swizzle
  // depends on key mod 16 only, so 16-key blocks differ by a constant).
  const uint32_t smem_base = lds_addr(smem);
  auto swz_k = [](int key) { return F8 ? chunk_swz_k8(key) : chunk_swz<D>(key); };
  auto swz_v = [](int key) { return F8 ? chunk_swz_v8(key) : chunk_swz_v<D>(key); };
  uint32_t k_off[KC];
  uint32_t v_off[DB];
  if constexpr (!F8) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) k_off[kc] = lr * ROWB + (((kc * 4 + lq) ^ swz_k(lr)) * 16);
    const int tr_row = 4 * lq + (lr >> 2);   // key within a 16-key block for the transpose read
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = db * 16 + 4 * (lr & 3);
      v_off[db] = tr_row * ROWB + (((d0 >> 3) ^ swz_v(tr_row)) * 16) + (d0 & 7) * 2;
    }
  } else {
    // K: lane (lr, lq) reads chunks lq and lq + 4 (d = 16*chunk ..) of key lr
#pragma unroll
    for (int p = 0; p < KC / 2; ++p) k_off[p] = lr * ROWB + (((lq + 4 * p) ^ swz_k(lr)) * 16);
    // V, 8-bit transpose read: lane 2j + c of group lq supplies row j, half
    // c of a 16-byte d block. 32-key MFMA: row j is key (j < 4 ? 4*lq + j :
    // 16 + 4*lq + j - 4) of a 32-key group (the S^T accumulators' k-slot
    // map). 16-key MFMA: row j is key 4*lq + j%4 at d block m + 4*(j/4), so
    // one read gives d blocks m and m + 4.
    const int j = lr >> 1, c = lr & 1;
    if constexpr (NKB >= 2) {
      const int key = j < 4 ? 4 * lq + j : 16 + 4 * lq + j - 4;
#pragma unroll
      for (int db = 0; db < DB; ++db) v_off[db] = key * ROWB + ((db ^ swz_v(key)) * 16) + 8 * c;
    } else {
      const int key = 4 * lq + (j & 3);
#pragma unroll
      for (int m = 0; m < DB / 2; ++m)
        v_off[m] = key * ROWB + (((m + 4 * (j >> 2)) ^ swz_v(kg * 16 + key)) * 16) + 8 * c;
    }
  }

  // ---------------------------------------------------- K/V DMA sources
  // The KPW keys a wave moves per stage lie inside one 16-token page (every
  // stage starts on a page boundary), so the page id, the source base and the
  // LDS destinations are wave-uniform (scalar registers); per lane only a
  // 32-bit byte offset within the page remains, the same every stage. Lane l
  // of DMA block i writes LDS bytes [16 l, 16 l + 16) = (key, chunk column)
  // of the swizzled layout and loads the matching source chunk.
  // Page table: lane j of register r holds this wave's page id for stage
  // 64 r + j, read once from LDS; a stage takes its entry with v_readlane.
  constexpr int KPW = SK / W;                                   // keys per wave per stage
  static_assert(16 % KPW == 0, "a wave's keys of a stage must lie in one page");
  constexpr int NPR = (kMaxItemPages * 16 / SK + 63) / 64;      // page-table registers
  int ptab[NPR];
#pragma unroll
  for (int r = 0; r < NPR; ++r) {
    const int st_i = lane + 64 * r;
    ptab[r] = st_i < n_tiles ? s_pages[page_skip + ((st_i * SK + wave * KPW) >> 4)] : 0;
  }
  // page of the item's last position: the source of every clamped lane
  const int last_pid = n_tiles > 0 ? s_pages[((key_end - 1) >> 4) - first_page] : 0;
  auto stage_pid = [&](int t) {
    int v = ptab[0];
#pragma unroll
    for (int r = 1; r < NPR; ++r) v = (t >> 6) == r ? ptab[r] : v;
    return __builtin_amdgcn_readlane(v, t & 63);
  };
  const int col = lane % CPR;
  uint32_t dma_koff[BLK_PER_WAVE], dma_voff[BLK_PER_WAVE];
#pragma unroll
  for (int i = 0; i < BLK_PER_WAVE; ++i) {
    const int key = wave * KPW + i * KPB + lane / CPR;          // key within the stage
    dma_koff[i] = (uint32_t)((key & 15) * a.st * ESZ + (col ^ swz_k(key)) * 16);
    dma_voff[i] = (uint32_t)((key & 15) * a.st * ESZ + (col ^ swz_v(key)) * 16);
  }
  // Stage u of the item is tile t of head h (u = h * n_tiles + t); stages are
  // issued in order, so the issue position advances one (h, t) at a time.
  int iss_u = 0, iss_h = 0, iss_t = 0;
  auto issue_next = [&]() {
    const int t = iss_t;
    const int64_t head_bytes = (int64_t)(g0 + iss_h) * a.sh * ESZ;
    const uint32_t lds_k = smem_base + (iss_u % NS) * SM::STAGE_BYTES + wave * BLK_PER_WAVE * 1024;
    const uint32_t lds_v = lds_k + SM::TILE_BYTES;
    const int kt0 = key_begin + t * SK;
    const int wpos = kt0 + wave * KPW;
    // positions past the item re-read its last position, which lies in this
    // wave's page or, if the whole range is past it, in last_pid
    const int pid = wpos < key_end ? stage_pid(t) : last_pid;
    const int64_t pg = (int64_t)pid * a.sp * ESZ + head_bytes;
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.k) + pg;
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.v) + pg;
    if (wpos + KPW <= key_end) {
      // fresh 32-bit offsets, all live at once: each address is (scalar base
      // + its own lane offset), so no VGPR is rewritten while an earlier DMA
      // may still be waiting to read it
      uint32_t ko[BLK_PER_WAVE], vo[BLK_PER_WAVE];
#pragma unroll
      for (int i = 0; i < BLK_PER_WAVE; ++i) {
        ko[i] = dma_koff[i];
        vo[i] = dma_voff[i];
      }
      reg_fence(ko);
      reg_fence(vo);
#pragma unroll
      for (int i = 0; i < BLK_PER_WAVE; ++i) {
        lds_dma16(kb + ko[i], lds_k + i * 1024);
        lds_dma16(vb + vo[i], lds_v + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < BLK_PER_WAVE; ++i) {
        const int key = wave * KPW + i * KPB + lane / CPR;
        const int slot_t = min(kt0 + key, key_end - 1) & 15;
        const uint32_t ko = (uint32_t)(slot_t * a.st * ESZ + (col ^ swz_k(key)) * 16);
        const uint32_t vo = (uint32_t)(slot_t * a.st * ESZ + (col ^ swz_v(key)) * 16);
        lds_dma16(kb + ko, lds_k + i * 1024);
        lds_dma16(vb + vo, lds_v + i * 1024);
      }
    }
    ++iss_u;
    if (++iss_t == n_tiles) {
      iss_t = 0;
      ++iss_h;
    }
  };
  auto wait_stage = [&](int after) {   // `after` stages were issued after the one needed
    if (NS >= 4 && after >= 3) wait_vmcnt<3 * OPS>();
    else if (NS >= 3 && after >= 2) wait_vmcnt<2 * OPS>();
    else if (after >= 1) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
  };

  // All NS buffers are filled up front. Afterwards, with shared buffers, stage
  // u + NS - 1 goes into the buffer that stage u - 1 used, once every wave is
  // past stage u's barrier; per-wave pipelines refill a buffer themselves (in
  // the stage loop).
  const int U = H * n_tiles;
  const int pro = min(NS, U);
  // Q tile of this wave: its 16 rows, row r at r * QROWB bytes, 16-byte chunk
  // c at position c ^ swz(r) (the swizzle of the K tiles, read in the same
  // pattern by the MFMA operand reads)
  constexpr int QROWB = D * 2;
  const uint32_t q_lds = smem_base + NS * SM::STAGE_BYTES + wave * 16 * QROWB;
  if constexpr (QLDS) {
    block_barrier();   // every wave has read the page table, whose bytes the Q tiles reuse
    if (wave_active) {
      constexpr int QCH = QROWB / 16;          // 16-byte chunks per row
      constexpr int QRPB = 64 / QCH;           // rows per 1 KB DMA block
#pragma unroll
      for (int i = 0; i < 16 / QRPB; ++i) {
        const int r = i * QRPB + lane / QCH;   // row of the tile this lane's chunk belongs to
        const int c = lane % QCH;              // its chunk position in LDS
        // lane r holds row r's token and head-in-group; rows past the item's
        // last take the wave's first row (never used)
        const int src = wrow0 + r < row_end ? r : 0;
        const int tok = __shfl(row_tok[0], src);
        const int j = __shfl(row_j[0], src);
        lds_dma16(a.q + ((int64_t)tok * a.hq + g0 * a.group + j) * D + (c ^ chunk_swz<D>(r)) * 8,
                  q_lds + i * 1024);
      }
    }
  }
  for (int p = 0; p < pro; ++p) issue_next();
  if constexpr (QLDS) {
    if (wave_active) {
      // Q's requests precede the stages': they are done once at most the
      // stages' requests are outstanding
      if (pro >= 4) wait_vmcnt<4 * OPS>();
      else if (pro == 3) wait_vmcnt<3 * OPS>();
      else if (pro == 2) wait_vmcnt<2 * OPS>();
      else if (pro == 1) wait_vmcnt<OPS>();
      else wait_vmcnt<0>();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        // the k-slot order of load_q
        const int ch = F8 ? 2 * (lq + 4 * (kc >> 1)) + (kc & 1) : kc * 4 + lq;
        qf[0][kc] = lds_read_b128<0>(q_lds + lr * QROWB + ((ch ^ chunk_swz<D>(lr)) * 16));
      }
      lds_wait_regs(qf[0]);
    }
  } else {
    // Q was requested before these stages, so it lands before the first of
    // them. Passing it through an asm operand here makes the compiler put its
    // wait for Q at this point: left to itself, it waits for Q at the products
    // inside the stage loop, i.e. for every DMA in flight, at every stage.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) reg_fence(qf[rb]);
  }

  // ------------------------------------------------- end of one KV head
  // Per wave and row: m (scaled, log2 domain), l and o (unnormalised). With
  // key groups (KG > 1) every wave publishes, in the stage buffer all waves
  // have just finished with (the DMA in flight targets the other buffers),
  // its m, l and the o blocks outside its own share of d; then each wave folds
  // its share of d (DB / KG blocks) of the KG states, in key-group order, and
  // writes it: the fold and the stores are spread over the waves.
  auto finish_head = [&](int g, int buf) {
    constexpr int QD = DB / KG;                  // d blocks a wave folds and writes
    constexpr int XP = (KG - 1) * QD * 16 + 4;   // floats per published row: other shares, m, l
    constexpr int SLOT_F = 16 * RB * XP;         // floats per published wave state
    // position of share q among the shares wave w publishes (all but its own)
    auto share_pos = [](int q, int w) { return q < w ? q : q - 1; };
    float* xs = reinterpret_cast<float*>(smem + (F8 ? 0 : buf * SM::STAGE_BYTES));
    if constexpr (KG > 1) {
      block_barrier();                           // every wave is done with this buffer
      if (wave_active) {
        float* my = xs + (kg * RW + rw) * SLOT_F;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float* r = my + (rb * 16 + lr) * XP;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int q = db / QD;
            if (q != kg)
              *reinterpret_cast<f32x4_t*>(r + (share_pos(q, kg) * QD + db % QD) * 16 + lq * 4) = o[db][rb];
          }
          const float l_tot = wave_sum_across_quads(l_run[rb]);
          if (lq == 0) {
            r[XP - 4] = m_run[rb];
            r[XP - 3] = l_tot;
          }
        }
      }
      block_barrier();                           // states published
    }
    if (!wave_active) return;
    // The rest with this wave's share Q known at compile time, so that every
    // o block is named by a constant index (a register array indexed at run
    // time would be placed in scratch memory).
    auto fold_and_write = [&](auto share_c) {
      constexpr int Q = decltype(share_c)::value;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float m_fin = m_run[rb];
        float l_tot;
        if constexpr (KG > 1) {
          // key group 0's state first, then groups 1 .. KG - 1 folded in order
          const float* r0 = xs + (0 * RW + rw) * SLOT_F + (rb * 16 + lr) * XP;
          float m = r0[XP - 4], l = r0[XP - 3];
          f32x4_t acc[QD];
#pragma unroll
          for (int i = 0; i < QD; ++i)
            acc[i] = Q == 0 ? o[i][rb]
                            : *reinterpret_cast<const f32x4_t*>(r0 + (share_pos(Q, 0) * QD + i) * 16 + lq * 4);
#pragma unroll
          for (int k2 = 1; k2 < KG; ++k2) {
            const float* r = xs + (k2 * RW + rw) * SLOT_F + (rb * 16 + lr) * XP;
            const float m2 = r[XP - 4], l2 = r[XP - 3];
            const float mn = vmax(m, m2);
            const float mu = (mn == -INFINITY) ? 0.f : mn;
            const float a1 = __builtin_amdgcn_exp2f(m - mu), a2 = __builtin_amdgcn_exp2f(m2 - mu);
#pragma unroll
            for (int i = 0; i < QD; ++i) {
              const f32x4_t o2 =
                  k2 == Q ? o[Q * QD + i][rb]
                          : *reinterpret_cast<const f32x4_t*>(r + (share_pos(Q, k2) * QD + i) * 16 + lq * 4);
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(o2[j], a2, acc[i][j] * a1);
            }
            l = __builtin_fmaf(l2, a2, l * a1);
            m = mn;
          }
#pragma unroll
          for (int i = 0; i < QD; ++i) o[Q * QD + i][rb] = acc[i];
          m_fin = m;
          l_tot = l;
        } else {
          l_tot = wave_sum_across_quads(l_run[rb]);
        }
        float o_fac = 1.f;
        if (WIN && a.direct && a.sinks && row_ok[rb]) {
          // attention sink: one more term exp(z) of the normaliser, no value
          const float z = a.sinks[g * a.group + row_j[rb]] * kLog2e;
          const float mn = vmax(m_fin, z);
          if (mn != -INFINITY) {
            o_fac = (m_fin == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_fin - mn);
            l_tot = l_tot * o_fac + __builtin_amdgcn_exp2f(z - mn);
            m_fin = mn;
          }
        }
        const bool live = l_tot > 0.f;
        const float inv = live ? a.v_scale * o_fac / l_tot : 0.f;
        const float lse = live ? (m_fin + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
        if (!row_ok[rb]) continue;
        const int64_t row = (int64_t)row_tok[rb] * a.hq + g * a.group + row_j[rb];
        // one wave (share 0) writes each row's LSE
        if (a.direct) {
#pragma unroll
          for (int i = 0; i < QD; ++i) {
            constexpr int db0 = Q * QD;
            const f32x4_t acc = o[db0 + i][rb] * inv;
            *reinterpret_cast<u32x2_t*>(a.out + row * D + (db0 + i) * 16 + lq * 4) =
                u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
          }
          if (Q == 0 && lq == 0 && a.lse_out) a.lse_out[row] = lse;
        } else {
          const int64_t e0 = (int64_t)slot * a.slot_elems + row * D;
          if (a.part_fp32) {
            float* dst = static_cast<float*>(a.part_o) + e0;
#pragma unroll
            for (int i = 0; i < QD; ++i) {
              constexpr int db0 = Q * QD;
              const f32x4_t r = o[db0 + i][rb] * inv;
              float* d = dst + (db0 + i) * 16 + lq * 4;
              if (a.coherent) {
                const u32x4_t w = __builtin_bit_cast(u32x4_t, r);
                store_dev_u64(d, (uint64_t)w[0] | ((uint64_t)w[1] << 32));
                store_dev_u64(d + 2, (uint64_t)w[2] | ((uint64_t)w[3] << 32));
              } else {
                *reinterpret_cast<f32x4_t*>(d) = r;
              }
            }
          } else {
            uint16_t* dst = static_cast<uint16_t*>(a.part_o) + e0;
#pragma unroll
            for (int i = 0; i < QD; ++i) {
              constexpr int db0 = Q * QD;
              const f32x4_t r = o[db0 + i][rb] * inv;
              const uint32_t lo = pack_bf16x2(r[0], r[1]), hi = pack_bf16x2(r[2], r[3]);
              uint16_t* d = dst + (db0 + i) * 16 + lq * 4;
              if (a.coherent) store_dev_u64(d, (uint64_t)lo | ((uint64_t)hi << 32));
              else *reinterpret_cast<u32x2_t*>(d) = u32x2_t{lo, hi};
            }
          }
          if (Q == 0 && lq == 0) {
            float* lp = a.part_lse + (int64_t)slot * a.slot_rows + row;
            if (a.coherent) store_dev_f32(lp, lse);
            else *lp = lse;
          }
        }
      }
    };
    if constexpr (KG == 1) {
      fold_and_write(std::integral_constant<int, 0>{});
    } else {
      static_assert(KG == 4, "key-group shares: four waves");
      switch (kg) {
        case 0: fold_and_write(std::integral_constant<int, 0>{}); break;
        case 1: fold_and_write(std::integral_constant<int, 1>{}); break;
        case 2: fold_and_write(std::integral_constant<int, 2>{}); break;
        default: fold_and_write(std::integral_constant<int, 3>{}); break;
      }
    }
  };

  // An empty KV range (a chunk past a short request's end) still writes its
  // rows: o = 0, lse = -inf, which the merge ignores.
  end = ItemEnd{1, pmode, req, grp, row_begin, row_end, g0, H};
  if (U == 0) {
    for (int hh = 0; hh < H; ++hh) finish_head(g0 + hh, 0);
    return;
  }

  // Stage u of the item is tile t of head h (u = h * n_tiles + t): an inner
  // loop over a head's tiles, and each head's end (the key-group combine,
  // the next head's Q) outside it.
  int u = 0;
  for (int h = 0; h < H; ++h) {
  for (int t = 0; t < n_tiles; ++t, ++u) {
    // Shared buffers: the prologue filled NS buffers and iteration i >= 1
    // issued stage i + NS - 1, so stage u is followed by min(NS - 2, ...)
    // issued stages here (NS - 1 at u = 0).
    // Per-wave pipelines: stages u .. u + NS - 1 are in flight here, and
    // stage u + NS goes into stage u's buffer once its fragments are read,
    // except after a head's last tile, whose buffer holds the key-group
    // combine (then it is issued after the combine).
    const bool refill = PRIV && u + NS < U;
    const bool refill_now = refill && t != n_tiles - 1;
    if constexpr (PRIV) {
      wait_stage(min(NS - 1, U - 1 - u));
      if (refill_now && !wave_active) issue_next();
    } else {
      wait_stage(u == 0 ? min(NS - 1, U - 1) : min(NS - 2, U - 1 - u));
      block_barrier();
      // the next stage goes into the buffer every wave finished with before
      // this barrier
      if (u >= 1 && u + NS - 1 < U) issue_next();
    }
    const uint32_t stage = smem_base + (u % NS) * SM::STAGE_BYTES;
    if (wave_active) {
      const uint32_t sK = stage + kg * NKB * 16 * ROWB;
      const uint32_t sV = stage + SM::TILE_BYTES + kg * NKB * 16 * ROWB;
      const int kt0 = key_begin + t * SK + kg * NKB * 16;   // first key of this wave's group
      constexpr int NKK = NKB >= 2 ? NKB / 2 : 1;
      constexpr int VH = (RB >= 2 && NKB >= 2) ? 2 : 1;   // d halves
      constexpr int DBV = DB / VH;                          // d blocks per half
      u32x4_t vf[NKB >= 2 ? DBV * NKK : 1];
      u32x2_t vh[NKB == 1 ? DB : 1];
      // fp8: raw transpose reads (8 keys of one d column per lane), converted
      // after the softmax
      u32x2_t vr8[F8 && NKB >= 2 ? DBV * NKK : 1];
      u32x2_t vr1[F8 && NKB == 1 ? DB / 2 : 1];
      // one 16-key block: V^T of the block with the transpose load
      auto read_v1 = [&]() {
        if constexpr (F8) {
#pragma unroll
          for (int m = 0; m < DB / 2; ++m) vr1[m] = lds_read_tr8(sV + v_off[m]);
        } else {
#pragma unroll
          for (int db = 0; db < DB; ++db) vh[db] = lds_read_tr16(sV + v_off[db]);
        }
      };
      // per-wave pipelines: with K and V in registers the buffer is free
      auto release = [&]() {
        if constexpr (PRIV) {
          if constexpr (F8) reg_fence(vr1);
          else reg_fence(vh);
          if (refill_now) issue_next();
        }
      };
      // S^T = K Q^T for NKB blocks of 16 keys. All K fragments of the stage
      // are read before one wait; the MFMA chains of the blocks interleave.
      u32x4_t kf[NKB * KC];
      if constexpr (!F8) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) kf[kb * KC + kc] = lds_read_b128_kb<ROWB>(sK + k_off[kc], kb);
        if constexpr (PRIV) read_v1();
        lds_wait_regs(kf);
        release();
      } else {
        // 16 fp8 of chunk lq + 4p are k-slots of chunks kc = 2p (bytes 0-7)
        // and 2p + 1 (bytes 8-15), the order load_q gives Q
        u32x4_t kr[NKB * KC / 2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int p = 0; p < KC / 2; ++p) kr[kb * (KC / 2) + p] = lds_read_b128_kb<ROWB>(sK + k_off[p], kb);
        if constexpr (PRIV) read_v1();
        lds_wait_regs(kr);
        release();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int p = 0; p < KC / 2; ++p) {
            const u32x4_t r = kr[kb * (KC / 2) + p];
            kf[kb * KC + 2 * p] = fp8x8_to_bf16(r[0], r[1]);
            kf[kb * KC + 2 * p + 1] = fp8x8_to_bf16(r[2], r[3]);
          }
      }
      f32x4_t s[NKB][RB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[kb][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s[kb][rb] = mfma16x16x32(kf[kb * KC + kc], qf[rb][kc], s[kb][rb]);
      // V^T fragments do not depend on the softmax: read them now so that
      // their latency overlaps it. The transpose load gives lane lr of group
      // lq, for keys kb*16 + 4*lq + (0..3), the values at d = db*16 + lr.
      // For 32-key MFMAs, k-slot (lq, j) <-> key kk*32 + (j < 4 ? 4*lq + j :
      // 16 + 4*lq + j - 4), the map the S^T accumulators give P^T.
      // With two row blocks the fragments are read in two halves of d (the
      // second after the first is consumed) to stay within 256 VGPRs.
      auto read_v = [&](int half) {
#pragma unroll
        for (int i = 0; i < DBV; ++i) {
          const uint32_t va = sV + v_off[half * DBV + i];
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            if constexpr (F8) {
              vr8[i * NKK + kk] = kk == 0 ? lds_read_tr8<0>(va) : lds_read_tr8<32 * ROWB>(va);
            } else {
              const u32x2_t h0 = kk == 0 ? lds_read_tr16<0>(va) : lds_read_tr16<32 * ROWB>(va);
              const u32x2_t h1 = kk == 0 ? lds_read_tr16<16 * ROWB>(va) : lds_read_tr16<48 * ROWB>(va);
              vf[i * NKK + kk] = u32x4_t{h0[0], h0[1], h1[0], h1[1]};
            }
          }
        }
      };
      auto wait_v = [&]() {
        if constexpr (F8) {
          lds_wait_regs(vr8);
#pragma unroll
          for (int i = 0; i < DBV * NKK; ++i) vf[i] = fp8x8_to_bf16(vr8[i][0], vr8[i][1]);
        } else {
          lds_wait_regs(vf);
        }
      };
      if constexpr (NKB == 1) {
        if constexpr (!PRIV) read_v1();
      } else {
        read_v(0);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) reg_fence(s[kb]);   // softmax below the V reads
      // online softmax over this wave's keys of the stage, per row (lane lr)
      const bool need_mask =
          (kt0 + NKB * 16 > key_end) || (kt0 + NKB * 16 - 1 > all_visible_to) || (WIN && kt0 < win_lo_max);
      u32x2_t pb[RB][NKB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (need_mask) {
          // key kt0 + kb*16 + lq*4 + i is visible iff it is below both the
          // item end and (causal) the row's position + 1
          const int lim = causal ? min(key_end, row_qpos[rb] + 1) : key_end;
          const int rem = lim - (kt0 + lq * 4);
          // and, with a sliding window, at or above the row's window start
          const int lo = (WIN && a.window > 0) ? row_qpos[rb] - a.window + 1 - (kt0 + lq * 4) : -0x40000000;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              s[kb][rb][i] = (kb * 16 + i < rem && kb * 16 + i >= lo) ? s[kb][rb][i] : -INFINITY;
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          tmax = vmax(tmax, vmax(vmax(s[kb][rb][0], s[kb][rb][1]), vmax(s[kb][rb][2], s[kb][rb][3])));
        tmax = wave_max_across_quads(tmax) * a.scale_log2;
        // The reference max m_run only moves when the stage's max passes it
        // by more than kRescaleSlack (so exponentials stay <= 2^slack, exact
        // in fp32 and bf16 alike): o and l need rescaling on few stages. The
        // choice is per row; a skipped rescale is a product with 1.
        const bool bump = tmax > m_run[rb] + kRescaleSlack;   // also -inf -> finite
        const float m_new = bump ? tmax : m_run[rb];
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = bump ? __builtin_amdgcn_exp2f(m_run[rb] - m_use) : 1.f;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][rb][i], a.scale_log2, -m_use));
            psum += p[i];
          }
          pb[rb][kb] = u32x2_t{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        }
        l_run[rb] = l_run[rb] * alpha + psum;
        m_run[rb] = m_new;
        // most stages move no row's reference max: the wave skips the product
        if (__builtin_amdgcn_ballot_w64(bump) != 0) {
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db][rb] *= alpha;
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) reg_fence(pb[rb]);   // softmax done before the V wait
      // O^T += V^T P^T
      if constexpr (NKB == 1) {
        if constexpr (F8) {
          lds_wait_regs(vr1);
#pragma unroll
          for (int m = 0; m < DB / 2; ++m) {
            vh[m] = fp8x4_to_bf16(vr1[m][0]);
            vh[m + DB / 2] = fp8x4_to_bf16(vr1[m][1]);
          }
        } else {
          lds_wait_regs(vh);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[db][rb] = mfma16x16x16(vh[db], pb[rb][0], o[db][rb]);
      } else {
#pragma unroll
        for (int half = 0; half < VH; ++half) {
          if (half > 0) read_v(half);
          wait_v();
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int i = 0; i < DBV; ++i)
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) {
                const u32x4_t pk = u32x4_t{pb[rb][2 * kk][0], pb[rb][2 * kk][1], pb[rb][2 * kk + 1][0],
                                           pb[rb][2 * kk + 1][1]};
                o[half * DBV + i][rb] = mfma16x16x32(vf[i * NKK + kk], pk, o[half * DBV + i][rb]);
              }
        }
      }
    }
  }
  // end of head g0 + h, whose last tile was stage u - 1: the next head's Q
  // is requested first so that its latency overlaps the combine
  {
    const int ul = u - 1;
    const bool refill = PRIV && ul + NS < U;
    u32x4_t qn[RB][KC];
    const bool more = MH && h + 1 < H;
    if (more) load_q(g0 + h + 1, qn);
    finish_head(g0 + h, ul % NS);
    if (more) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) qf[rb][kc] = qn[rb][kc];
      reset_state();
      // the next head's Q has landed here (its wait is placed here, not in
      // the stage loop)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) reg_fence(qf[rb]);
    }
    if (refill) {
      block_barrier();   // every wave is past the combine in this buffer
      issue_next();
    }
  }
  }
}

// 128-row items ask for two work-groups per CU explicitly: left alone, the
// compiler gives them a few more registers than two allow.
template <int D, int RB, int RW, int KG, int NS, int SK, bool MH, bool F8, bool TREE, bool WIN = true, int PM = -1>
__global__ __launch_bounds__(64 * RW * KG, RB == 2 ? 2 : 1) void attn_tile_kernel(const TileArgs a,
                                                                                  const GroupTableArg<TREE> gt,
                                                                                  const ReqOrder ro,
                                                                                  const MergeTailArgs mt) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[TileSmem<D, NS, SK, F8 ? 1 : 2>::BYTES];
  ItemEnd end;
  attn_item<D, RB, RW, KG, NS, SK, MH, F8, WIN, PM>(a, gt, ro, blockIdx.x, smem, end);
  if (mt.counters) merge_tail<D, 64 * RW * KG>(mt, end, reinterpret_cast<int32_t*>(smem));
}

// One launch for all cascade phases: work-groups [0, n_prefix) run prefix
// items, the next n_group run nested-level items (same shape as the
// prefix), the rest run suffix items, so the MFMA-heavy shared levels and the
// bandwidth-heavy suffix share the CUs. All write partial states. Each role
// has its own pipeline shape (stages x keys per stage) inside one LDS
// allocation, sized so that two work-groups fit on a CU.
template <int D, int PRB, int PRW, int PKG, int PNS, int PSK, int SRB, int SRW, int SKG, int SNS, int SSK, bool F8,
          bool TREE>
__global__ __launch_bounds__(256) void cascade_phases_kernel(const TileArgs pa, const TileArgs ga, const TileArgs sa,
                                                             const int n_prefix, const int n_group,
                                                             const GroupTableArg<TREE> gt, const ReqOrder ro,
                                                             const MergeTailArgs mt) {
  static_assert(PRW * PKG == 4 && SRW * SKG == 4, "both roles use 4 waves");
  constexpr int ESZ = F8 ? 1 : 2;
  constexpr int PB = TileSmem<D, PNS, PSK, ESZ>::BYTES, SB = TileSmem<D, SNS, SSK, ESZ>::BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[PB > SB ? PB : SB];
  const int bid = blockIdx.x;
  ItemEnd end;
  if (bid < n_prefix) attn_item<D, PRB, PRW, PKG, PNS, PSK, false, F8, false, 1>(pa, gt, ro, bid, smem, end);
  else if (TREE && bid < n_prefix + n_group)
    attn_item<D, PRB, PRW, PKG, PNS, PSK, false, F8, false, 2>(ga, gt, ro, bid - n_prefix, smem, end);
  else
    attn_item<D, SRB, SRW, SKG, SNS, SSK, (SKG > 1) && !F8, F8, false, 0>(sa, gt, ro, bid - n_prefix - n_group,
                                                                             smem, end);
  if (mt.counters) merge_tail<D, 256>(mt, end, reinterpret_cast<int32_t*>(smem));
}

}  // namespace ca
