// device_common.h -- small device helpers shared by the HIP kernels.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace jagg {

// bfloat16 <-> float on raw 16-bit patterns.  float -> bf16 rounds to nearest,
// ties to even: add 0x7fff plus the lowest kept bit, then truncate; NaN maps
// to a quiet NaN.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
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

}  // namespace jagg
