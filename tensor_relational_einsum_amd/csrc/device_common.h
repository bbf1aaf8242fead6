// device_common.h -- small device helpers shared by the HIP kernels.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace jagg {

// bfloat16 <-> float on raw 16-bit patterns.  float -> bf16 uses the
// hardware convert (round to nearest, ties to even; NaN stays a quiet NaN).
typedef float jagg_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 jagg_bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two floats -> two bf16 in one 32-bit word, the first in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const jagg_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, jagg_bf16x2));
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T *p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

__device__ __forceinline__ float load_dt(const void *base, int64_t off, int dt) {
  return dt ? bf16_to_f32(reinterpret_cast<const uint16_t *>(base)[off]) : reinterpret_cast<const float *>(base)[off];
}

__device__ __forceinline__ void store_dt(void *base, int64_t off, int dt, float v) {
  if (dt)
    reinterpret_cast<uint16_t *>(base)[off] = f32_to_bf16(v);
  else
    reinterpret_cast<float *>(base)[off] = v;
}

// g with its kind fixed at compile time.  Missing operands of MUL / ADD are
// filled with the operation's identity by the callers, so both always take
// three operands.  Divisions use the hardware reciprocal (1 ulp).
template <int G>
__device__ __forceinline__ float g_fn(float x0, float x1, float x2, float beta, float eps) {
  if constexpr (G == 0) return x0 * x1 * x2;
  else if constexpr (G == 1) return x0;
  else if constexpr (G == 2) return x0 * x0;
  else if constexpr (G == 3) return __expf(x0 - x1);
  else if constexpr (G == 4) return __expf(x0 - x1) * __builtin_amdgcn_rcpf(x2);
  else if constexpr (G == 5) return x0 * rsqrtf(x1 * beta + eps) * x2;
  else if constexpr (G == 6) return x0 * __builtin_amdgcn_rcpf(1.0f + __expf(-x0)) * x1;
  else return x0 + x1 + x2;
}

template <int G>
constexpr float g_fill() { return G == 0 ? 1.0f : 0.0f; }

}  // namespace jagg
