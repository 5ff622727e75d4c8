// Device-side helpers shared by the attention and merge kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ca {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 bits.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ float wave_max_across_quads(float x) {
  // lanes l, l^16, l^32, l^48 hold the same MFMA row
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float wave_sum_across_quads(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Online LSE merge step: folds one partial state (lse_s natural log, o_s
// normalised) into a running (m, wsum, acc) where acc / wsum is the merged
// output and m + log(wsum) the merged LSE. A partial with lse_s = -inf has
// weight 0 and its o_s (which may be garbage) is not used.
template <int N>
__device__ __forceinline__ void merge_step(float& m, float& wsum, f32x4_t (&acc)[N], float lse_s,
                                           const f32x4_t (&o_s)[N]) {
  if (lse_s == -INFINITY) return;
  const float m_new = fmaxf(m, lse_s);
  const float a_old = (m == -INFINITY) ? 0.f : exp2f((m - m_new) * kLog2e);
  const float a_new = exp2f((lse_s - m_new) * kLog2e);
  wsum = wsum * a_old + a_new;
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = acc[i] * a_old + o_s[i] * a_new;
  m = m_new;
}

}  // namespace ca
