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
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

// Two fp32 -> bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// max without the NaN-quieting operand copies fmaxf needs in IEEE mode
// (v_maximum3_f32; NaN-propagating, which no finite or -inf input sees).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48 hold the same MFMA row). v_permlane32_swap of x with itself leaves the
// low rows' values in one register and the high rows' in the other (XOR 32);
// v_permlane16_swap does the same for even / odd rows (XOR 16). No LDS; every
// lane ends with the same, bitwise identical, result.
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  a = __builtin_bit_cast(float, (uint32_t)r[0]);
  b = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  a = __builtin_bit_cast(float, (uint32_t)r[0]);
  b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float wave_max_across_quads(float x) {
  float a, b;
  swap32(x, a, b);
  x = vmax(a, b);
  swap16(x, a, b);
  return vmax(a, b);
}

__device__ __forceinline__ float wave_sum_across_quads(float x) {
  float a, b;
  swap32(x, a, b);
  x = a + b;
  swap16(x, a, b);
  return a + b;
}

// Device-scope (agent) coherent accesses for data one work-group writes and
// another reads inside the same launch: relaxed atomic stores and loads at
// agent scope (gfx950: global_store / global_load with sc1), written through
// to, and read from, the device's point of coherence rather than an XCD's
// own L2. Ordering against the arrival counter comes from waiting for the
// stores to complete (vmcnt 0) before the counter is bumped, and from issuing
// the loads only after the counter's value has come back.
__device__ __forceinline__ void store_dev_u64(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_dev_u64(const void* p) {
  return __hip_atomic_load(static_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev_f32(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace ca
