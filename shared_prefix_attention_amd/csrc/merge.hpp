// LSE merge of partial attention states ("vLLM Cascade Attention：用法、场景与
// 原理解析", beaiera.top, section 1 step 3 and section 8 Step 5: the partial
// outputs are combined by log-sum-exp rescaling; section 5: an element-wise
// weighted sum). n-way: it combines the prefix splits and the suffix chunks
// of every (token, head) row in one pass:
//   M = max_s lse_s, w_s = exp(lse_s - M), out = sum_s w_s o_s / sum_s w_s,
//   lse = M + log(sum_s w_s).
// Partials with lse = -inf have weight 0 and their o is not read. An
// attention sink (one logit per query head) enters as one more state with
// lse = sink and o = 0.
//
// One canonical order of operations, used by the stand-alone merge kernel
// and by the merge inside the attention launch alike, so both give the same
// bits: the slots are cut into SG contiguous groups (SG = 4 above 16 slots,
// else 1); each group is folded in slot order (online form, group 0 starting
// from the sink); then groups 1 .. SG-1 are folded into group 0 in order.
#pragma once

#include "device_common.hpp"

namespace ca {

struct MergeArgs {
  const void* part_o;      // [slots][rows][D] bf16 or fp32
  const float* part_lse;   // [slots][rows]
  int32_t slots;
  int64_t rows;            // T * hq
  int64_t slot_elems;      // rows * D
  uint16_t* out;           // [rows][D] bf16
  float* lse_out;          // [rows] (may be null)
  const float* sinks;      // [hq] attention-sink logits or null: a state lse = sink, o = 0
  int32_t hq;
};

constexpr int kMergeBatch = 16;   // slots whose loads are issued together
__host__ __device__ constexpr int merge_groups(int slots) { return slots > kMergeBatch ? 4 : 1; }

// Folds an unnormalised state (m2, w2, acc2) into (m, w, acc): acc / w is
// the merged output and m + log(w) its LSE. Products are fused explicitly so
// that every inlined copy rounds the same way.
template <int N>
__device__ __forceinline__ void fold_state(float& m, float& w, f32x4_t (&acc)[N], float m2, float w2,
                                           const f32x4_t (&acc2)[N]) {
  if (m2 == -INFINITY) return;
  const float mn = fmaxf(m, m2);
  const float a1 = (m == -INFINITY) ? 0.f : exp2f((m - mn) * kLog2e);
  const float a2 = exp2f((m2 - mn) * kLog2e);
  w = __builtin_fmaf(w2, a2, w * a1);
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(acc2[i][j], a2, acc[i][j] * a1);
  m = mn;
}

// Two bf16 (one 32-bit word, element 0 in the low half) widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// One slot group of one row part: NCH x V consecutive d values (V = 8 bf16
// or 4 fp32 per 16-byte chunk) of flat row `row`, starting at chunk
// part * NCH; slots [s_begin, s_end) folded in order onto (m, wsum, acc). The
// loads of a batch of slots (LSE and o, only for slots that exist) are issued
// before their first use, so a batch costs one memory round trip.
template <int D, bool F32, bool COH = false, int NCH = 1>
__device__ __forceinline__ void merge_slot_range(const MergeArgs& a, int64_t row, int part, int s_begin, int s_end,
                                                 float& m, float& wsum, f32x4_t (&acc)[NCH * (F32 ? 1 : 2)]) {
  constexpr int V = F32 ? 4 : 8;
  constexpr int NV = NCH * (V / 4);
  constexpr int B = kMergeBatch / NCH;   // slots per batch: 16 chunks in flight per thread
  for (int s0 = s_begin; s0 < s_end; s0 += B) {
    float l[B];
    u32x4_t w[B][NCH];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      l[k] = -INFINITY;
#pragma unroll
      for (int c = 0; c < NCH; ++c) w[k][c] = u32x4_t{0u, 0u, 0u, 0u};
      if (s0 + k < s_end) {
        const int sl = s0 + k;
        const float* lp = a.part_lse + (int64_t)sl * a.rows + row;
        const int64_t e = (int64_t)sl * a.slot_elems + row * D + part * NCH * V;
        const uint8_t* src = static_cast<const uint8_t*>(a.part_o) + e * (F32 ? 4 : 2);
        if constexpr (COH) {
          l[k] = load_dev_f32(lp);
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            const uint64_t w0 = load_dev_u64(src + 16 * c), w1 = load_dev_u64(src + 16 * c + 8);
            w[k][c] = u32x4_t{(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32)};
          }
        } else {
          l[k] = *lp;
#pragma unroll
          for (int c = 0; c < NCH; ++c) w[k][c] = *reinterpret_cast<const u32x4_t*>(src + 16 * c);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      // bf16 partials widened exactly once every load of the batch is out
      f32x4_t x[NV];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if constexpr (F32) {
          x[c] = __builtin_bit_cast(f32x4_t, w[k][c]);
        } else {
          x[2 * c] = f32x4_t{bf16_lo(w[k][c][0]), bf16_hi(w[k][c][0]), bf16_lo(w[k][c][1]), bf16_hi(w[k][c][1])};
          x[2 * c + 1] = f32x4_t{bf16_lo(w[k][c][2]), bf16_hi(w[k][c][2]), bf16_lo(w[k][c][3]), bf16_hi(w[k][c][3])};
        }
      }
      // partial states are normalised (o_s = acc_s / w_s): one state of weight
      // 1; slots past the range have lse = -inf and are skipped
      fold_state(m, wsum, acc, l[k], 1.f, x);
    }
  }
}

// Start of slot group g: the sink (if any) joins group 0 as a state with no value.
__device__ __forceinline__ void merge_seed(const MergeArgs& a, int64_t row, int g, float& m, float& wsum) {
  m = -INFINITY;
  wsum = 0.f;
  if (a.sinks && g == 0) {
    m = a.sinks[row % a.hq];
    wsum = m == -INFINITY ? 0.f : 1.f;
  }
}

// Normalises a merged state and writes the row part's bf16 output (RNE) and,
// from part 0, the natural-log LSE.
template <int D, bool F32, int NCH = 1>
__device__ __forceinline__ void merge_store(const MergeArgs& a, int64_t row, int part, float m, float wsum,
                                            const f32x4_t (&acc)[NCH * (F32 ? 1 : 2)]) {
  constexpr int V = F32 ? 4 : 8;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* dst = a.out + row * D + part * NCH * V;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if constexpr (F32) {
      const f32x4_t r = acc[c] * inv;
      *reinterpret_cast<u32x2_t*>(dst + c * V) = u32x2_t{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    } else {
      const f32x4_t r0 = acc[2 * c] * inv, r1 = acc[2 * c + 1] * inv;
      *reinterpret_cast<u32x4_t*>(dst + c * V) = u32x4_t{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]),
                                                         pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
    }
  }
  if (part == 0 && a.lse_out) a.lse_out[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

// The canonical merge of one row part by one thread (all slot groups in
// turn, then the fold of groups 1.. into group 0).
template <int D, bool F32, bool COH, int NCH>
__device__ __forceinline__ void merge_row_part(const MergeArgs& a, int64_t row, int part) {
  constexpr int NV = NCH * (F32 ? 1 : 2);
  const int sg = merge_groups(a.slots);
  const int per = (a.slots + sg - 1) / sg;
  float m, wsum;
  f32x4_t acc[NV];
  merge_seed(a, row, 0, m, wsum);
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  merge_slot_range<D, F32, COH, NCH>(a, row, part, 0, min(a.slots, per), m, wsum, acc);
  for (int g = 1; g < sg; ++g) {
    float m2, w2;
    f32x4_t acc2[NV];
    merge_seed(a, row, g, m2, w2);
#pragma unroll
    for (int i = 0; i < NV; ++i) acc2[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    merge_slot_range<D, F32, COH, NCH>(a, row, part, g * per, min(a.slots, (g + 1) * per), m2, w2, acc2);
    fold_state(m, wsum, acc, m2, w2, acc2);
  }
  merge_store<D, F32, NCH>(a, row, part, m, wsum, acc);
}

// Stand-alone merge launch. Each thread owns V consecutive d values of a row
// (16-byte loads: 4 fp32 or 8 bf16), so D/V threads cover a row. F32:
// partial outputs in fp32, else bf16 (widened exactly). SG slot groups
// (merge_groups) run in parallel thread groups, and group 0 folds the
// others in, in group order, through LDS: the canonical order above.
template <int D, bool F32, int SG>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  constexpr int V = F32 ? 4 : 8;
  constexpr int NV = V / 4;                // f32x4 pieces per thread
  constexpr int TPR = D / V;
  constexpr int RPB = 256 / (TPR * SG);
  const int part = threadIdx.x % TPR;
  const int rl = (threadIdx.x / TPR) % RPB;
  const int g = threadIdx.x / (TPR * RPB);
  const int64_t row = (int64_t)blockIdx.x * RPB + rl;
  const bool live = row < a.rows;
  if (SG == 1 && !live) return;
  const int per = (a.slots + SG - 1) / SG;
  float m = -INFINITY, wsum = 0.f;
  f32x4_t acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (live) {
    merge_seed(a, row, g, m, wsum);
    merge_slot_range<D, F32>(a, row, part, g * per, min(a.slots, (g + 1) * per), m, wsum, acc);
  }
  if constexpr (SG > 1) {
    constexpr int F = V + 2;   // floats a thread publishes: acc, m, wsum
    __shared__ float xs[SG - 1][RPB][TPR][F];
    if (g > 0) {
      float* r = xs[g - 1][rl][part];
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) r[4 * i + j] = acc[i][j];
      r[V] = m;
      r[V + 1] = wsum;
    }
    __syncthreads();
    if (g > 0 || !live) return;
#pragma unroll
    for (int g2 = 1; g2 < SG; ++g2) {
      const float* r = xs[g2 - 1][rl][part];
      f32x4_t o2[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) o2[i] = f32x4_t{r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]};
      fold_state(m, wsum, acc, r[V], r[V + 1], o2);
    }
  }
  merge_store<D, F32>(a, row, part, m, wsum, acc);
}

}  // namespace ca
