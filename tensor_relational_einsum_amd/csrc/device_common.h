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

typedef __attribute__((address_space(3))) void *lds_dma_ptr;
typedef int i32x4_rsrc __attribute__((ext_vector_type(4)));

// Buffer resource as four scalar words: base, stride 0, byte count, and the
// gfx950 word-3 flags (raw buffer, 32-bit data format); lanes whose offset
// lies at or past `bytes` read zeros.
__device__ __forceinline__ i32x4_rsrc dma_rsrc(const void *base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_rsrc r;
  r.x = int(uint32_t(a));
  r.y = int(uint32_t(a >> 32) & 0xffffu);
  r.z = int(bytes);
  r.w = 0x00020000;
  return r;
}

// One 16-byte buffer load per lane into LDS: the wavefront's 64 vectors land
// contiguously at `lds` (lane l at lds + 16 l).  Written as inline assembly
// so that the compiler's wait-count pass does not track it: its per-object
// tracking of LDS-writing loads loses precision across the loop back edge
// and would wait for every stage on the first step of each unrolled pass.
// The kernel waits for these loads itself (vmcnt, in issue order).
__device__ __forceinline__ void dma16(i32x4_rsrc rs, uint32_t voff, const char *lds) {
  const uint32_t m0 = uint32_t(reinterpret_cast<uintptr_t>((lds_dma_ptr)(lds)));
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(m0)
               : "memory", "m0");
}

// dma16 with the LDS destination given as an SGPR base plus a constant: the
// add happens in the asm block, so the compiler keeps one base register live
// instead of one register per destination.  The add writes SCC, which the
// clobber list declares (the compiler may otherwise hold a carry or a branch
// condition in SCC across the block).
template <uint32_t OFF>
__device__ __forceinline__ void dma16_at(i32x4_rsrc rs, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(lds_base),
               "i"(OFF)
               : "memory", "m0", "scc");
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
