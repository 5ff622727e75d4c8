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

// Folds an unnormalised state (m2, w2, acc2) into (m, w, acc): acc / w is
// the merged output and m + log(w) its LSE.
template <int N>
__device__ __forceinline__ void fold_state(float& m, float& w, f32x4_t (&acc)[N], float m2, float w2,
                                           const f32x4_t (&acc2)[N]) {
  if (m2 == -INFINITY) return;
  const float mn = fmaxf(m, m2);
  const float a1 = (m == -INFINITY) ? 0.f : exp2f((m - mn) * kLog2e);
  const float a2 = exp2f((m2 - mn) * kLog2e);
  w = w * a1 + w2 * a2;
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = acc[i] * a1 + acc2[i] * a2;
  m = mn;
}

// Two bf16 (one 32-bit word, element 0 in the low half) widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Each thread owns V consecutive d values of a row (16-byte loads: 4 fp32
// or 8 bf16), so D/V threads cover a row. F32: partial outputs in fp32, else
// bf16 (widened exactly). SG slot groups share a row's slots (contiguous
// ranges) when there are many slots and few rows: each group merges its
// range, and group 0 folds the others in, in group order, through LDS (so
// the result is fixed by the slot count).
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
  const int s_begin = g * per, s_end = min(a.slots, s_begin + per);
  // Online merge over the group's slots in batches whose loads (LSE and o,
  // the latter unconditionally: every slot is in bounds) are all issued
  // before the first use, so a row costs one memory round trip per batch.
  constexpr int B = 16;
  float m = -INFINITY, wsum = 0.f;
  if (a.sinks && g == 0 && live) {   // the sink joins the normaliser as one more state with no value
    m = a.sinks[row % a.hq];
    wsum = m == -INFINITY ? 0.f : 1.f;
  }
  f32x4_t acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_begin; live && s0 < s_end; s0 += B) {
    float l[B];
    f32x4_t x[B][NV];
    u32x4_t w[F32 ? 1 : B];   // bf16 partials: raw words, widened once all loads are out
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int sl = min(s0 + k, s_end - 1);
      l[k] = (s0 + k < s_end) ? a.part_lse[(int64_t)sl * a.rows + row] : -INFINITY;
      const int64_t e = (int64_t)sl * a.slot_elems + row * D + part * V;
      if constexpr (F32) x[k][0] = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(a.part_o) + e);
      else w[k] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.part_o) + e);
    }
    if constexpr (!F32) {
#pragma unroll
      for (int k = 0; k < B; ++k) {
        x[k][0] = f32x4_t{bf16_lo(w[k][0]), bf16_hi(w[k][0]), bf16_lo(w[k][1]), bf16_hi(w[k][1])};
        x[k][1] = f32x4_t{bf16_lo(w[k][2]), bf16_hi(w[k][2]), bf16_lo(w[k][3]), bf16_hi(w[k][3])};
      }
    }
#pragma unroll
    for (int k = 0; k < B; ++k) merge_step(m, wsum, acc, l[k], x[k]);
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
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* dst = a.out + row * D + part * V;
  if constexpr (NV == 1) {
    const f32x4_t r = acc[0] * inv;
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
  } else {
    const f32x4_t r0 = acc[0] * inv, r1 = acc[1] * inv;
    *reinterpret_cast<u32x4_t*>(dst) =
        u32x4_t{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]), pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
  }
  if (part == 0 && a.lse_out) a.lse_out[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

}  // namespace ca
