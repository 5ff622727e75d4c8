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

// D/4 threads per row, each owning 4 consecutive d values. F32: partial
// outputs in fp32, else bf16 (widened exactly).
template <int D, bool F32>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= a.rows) return;
  // Online merge over slots in batches whose loads (LSE and o, the latter
  // unconditionally: every slot is in bounds) are all issued before the first
  // use, so a row costs one memory round trip per batch.
  constexpr int B = 16;
  float m = -INFINITY, wsum = 0.f;
  if (a.sinks) {   // the sink joins the normaliser as one more state with no value
    m = a.sinks[row % a.hq];
    wsum = m == -INFINITY ? 0.f : 1.f;
  }
  f32x4_t acc[1] = {f32x4_t{0.f, 0.f, 0.f, 0.f}};
  for (int s0 = 0; s0 < a.slots; s0 += B) {
    float l[B];
    f32x4_t x[B][1];
    u32x2_t w[F32 ? 1 : B];   // bf16 partials: raw words, widened once all loads are out
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int sl = min(s0 + k, a.slots - 1);
      l[k] = (s0 + k < a.slots) ? a.part_lse[(int64_t)sl * a.rows + row] : -INFINITY;
      const int64_t e = (int64_t)sl * a.slot_elems + row * D + part * 4;
      if constexpr (F32) x[k][0] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.part_o) + e);
      else w[k] = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(a.part_o) + e);
    }
    if constexpr (!F32) {
#pragma unroll
      for (int k = 0; k < B; ++k)
        x[k][0] = f32x4_t{__builtin_bit_cast(float, w[k][0] << 16), __builtin_bit_cast(float, w[k][0] & 0xffff0000u),
                          __builtin_bit_cast(float, w[k][1] << 16), __builtin_bit_cast(float, w[k][1] & 0xffff0000u)};
    }
#pragma unroll
    for (int k = 0; k < B; ++k) merge_step(m, wsum, acc, l[k], x[k]);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const f32x4_t r = acc[0] * inv;
  *reinterpret_cast<u32x2_t*>(a.out + row * D + part * 4) = u32x2_t{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
  if (part == 0 && a.lse_out) a.lse_out[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

}  // namespace ca
