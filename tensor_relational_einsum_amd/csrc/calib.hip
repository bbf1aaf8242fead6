// calib.hip -- the matrix-core probes of include/jagg_calib.h: register-only
// loops of v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2f32 on operands
// loaded once from memory.
#include <hip/hip_runtime.h>

#include "../../include/jagg_calib.h"

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

__global__ __launch_bounds__(256) void mfma_loop_kernel(const bf16x8 *__restrict__ ops, float *__restrict__ sink,
                                                        int iters) {
  const int lane = threadIdx.x & 63;
  // eight fragments per lane: 8 x 64 lanes x 8 values = 4096 bf16
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[i * 64 + lane];
    b[i] = ops[(4 + i) * 64 + lane];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  // one element of every accumulator keeps every MFMA chain live
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][(i * 4 + j) & 15];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(256) void mfma_f32_loop_kernel(const float *__restrict__ ops, float *__restrict__ sink,
                                                            int iters) {
  const int lane = threadIdx.x & 63;
  float a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[i * 64 + lane];
    b[i] = ops[(4 + i) * 64 + lane];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][(i * 4 + j) & 15];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" int jagg_calib_mfma_f32(void *hip_stream, const float *operands, float *sink, int n_blocks, int iters) {
  if (!operands || !sink || n_blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mfma_f32_loop_kernel, dim3(n_blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(hip_stream),
                     operands, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int jagg_calib_mfma_bf16(void *hip_stream, const void *operands, float *sink, int n_blocks, int iters) {
  if (!operands || !sink || n_blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(hip_stream),
                     static_cast<const bf16x8 *>(operands), sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
