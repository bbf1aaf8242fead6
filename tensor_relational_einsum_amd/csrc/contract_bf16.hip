// contract_bf16.hip -- bf16-input instantiations of the block contraction
// (see contract_impl.h and contract_dma.h).
#include "contract_dma.h"

namespace jagg {
namespace {
typedef float sum_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int sum_u32x2 __attribute__((ext_vector_type(2)));

// The parts of a split walk added in part order, scaled by alpha and
// written as C: four consecutive elements per thread (every element of the
// output relation, padding included, is one of some tile's).
__global__ __launch_bounds__(256) void split_sum_kernel(const float *__restrict__ part, int S, int64_t stride,
                                                        void *__restrict__ out, int out_bf16, float alpha,
                                                        int64_t n) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    sum_f32x4 s = *reinterpret_cast<const sum_f32x4 *>(part + i);
    for (int q = 1; q < S; ++q) s += *reinterpret_cast<const sum_f32x4 *>(part + q * stride + i);
    s *= alpha;
    if (out_bf16)
      *reinterpret_cast<sum_u32x2 *>(static_cast<uint16_t *>(out) + i) =
          sum_u32x2{pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w)};
    else
      *reinterpret_cast<sum_f32x4 *>(static_cast<float *>(out) + i) = s;
    return;
  }
  for (int64_t j = i; j < n; ++j) {
    float s = part[j];
    for (int q = 1; q < S; ++q) s += part[q * stride + j];
    s *= alpha;
    if (out_bf16) static_cast<uint16_t *>(out)[j] = f32_to_bf16(s);
    else static_cast<float *>(out)[j] = s;
  }
}
}  // namespace

hipError_t launch_split_sum(const ContractArgs &a, int out_bf16, int64_t n_out, hipStream_t st) {
  if (a.split <= 1 || !a.part || n_out > a.part_stride) return hipErrorInvalidValue;
  const int64_t blocks = (n_out + 1023) / 1024;
  hipLaunchKernelGGL(split_sum_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, a.part, int(a.split), a.part_stride,
                     a.C, out_bf16, a.alpha, n_out);
  return hipGetLastError();
}

hipError_t launch_contract_bf16(const ContractArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                                hipStream_t st, const char **which) {
  // 256x256 tiles over 16-byte vectors without a causal mask on the reduced
  // letter: the LDS-DMA pipeline
  if (a.epi == 2) {
    // SwiGLU recompose: the LDS-pipelined kernel only (A contiguous along K)
    if (!(big && va == 8 && vb == 8 && !a.causal_red && a_kc)) return hipErrorInvalidValue;
    *which = "bf16 256x128 lds pipeline, swiglu";
    if (out_bf16) return b_kc ? launch_dma<1, true, true, 3>(a, st) : launch_dma<1, true, false, 3>(a, st);
    return b_kc ? launch_dma<0, true, true, 3>(a, st) : launch_dma<0, true, false, 3>(a, st);
  }
  if (a.epi == 1 && big && va == 8 && vb == 8 && !a.causal_red && a_kc) {
    // MUL_PLUS on the LDS pipeline (A contiguous along K; other layouts take
    // the general kernel, whose epilogue adds the addend as well)
    *which = "bf16 256x256 lds pipeline, plus addend";
#define JAGG_DMA_X(OB, E) return b_kc ? launch_dma<OB, true, true, E>(a, st) : launch_dma<OB, true, false, E>(a, st);
    if (out_bf16) {
      if (a.x_bf16) { JAGG_DMA_X(1, 2) }
      JAGG_DMA_X(1, 1)
    }
    if (a.x_bf16) { JAGG_DMA_X(0, 2) }
    JAGG_DMA_X(0, 1)
#undef JAGG_DMA_X
  }
  if (big && va == 8 && vb == 8 && !a.causal_red && a.epi == 0) {
    *which = "bf16 256x256 lds pipeline";
#define JAGG_DMA(OB)                                                  \
  if (a_kc && b_kc) return launch_dma<OB, true, true>(a, st);        \
  if (a_kc && !b_kc) return launch_dma<OB, true, false>(a, st);      \
  if (!a_kc && b_kc) return launch_dma<OB, false, true>(a, st);      \
  return launch_dma<OB, false, false>(a, st);
    if (out_bf16) {
      JAGG_DMA(1)
    } else {
      JAGG_DMA(0)
    }
#undef JAGG_DMA
  }
  *which = big ? "bf16 256x256"
                : (a.N + 63) / 64 * 64 < (a.N + 127) / 128 * 128 ? "bf16 128x64"
                : (!out_bf16 && va == 8 && vb == 8 && !a.causal_red && short_walk<uint16_t>(a)) ? "bf16 128x128 one stage"
                : "bf16 128x128";
  return launch_typed<uint16_t>(a, out_bf16, a_kc, b_kc, va, vb, big, st);
}
bool launch_contract_bf16_group(const DmaGroupArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                                hipStream_t st, hipError_t *err) {
  if (!(big && va == 8 && vb == 8 && !a.common.causal_red)) return false;
  if (a.common.epi != 0) {
    // grouped recompose forms: A contiguous along K, as for one launch
    if (!a_kc) return false;
    const int E = a.common.epi == 2 ? 3 : (a.common.x_bf16 ? 2 : 1);
#define JAGG_DMA_GX(OB, EE) \
  *err = b_kc ? launch_dma_group<OB, true, true, EE>(a, st) : launch_dma_group<OB, true, false, EE>(a, st);
    if (out_bf16) {
      if (E == 3) { JAGG_DMA_GX(1, 3) } else if (E == 2) { JAGG_DMA_GX(1, 2) } else { JAGG_DMA_GX(1, 1) }
    } else {
      if (E == 3) { JAGG_DMA_GX(0, 3) } else if (E == 2) { JAGG_DMA_GX(0, 2) } else { JAGG_DMA_GX(0, 1) }
    }
#undef JAGG_DMA_GX
    return true;
  }
#define JAGG_DMA_G(OB)                                                         \
  if (a_kc && b_kc) *err = launch_dma_group<OB, true, true>(a, st);           \
  else if (a_kc && !b_kc) *err = launch_dma_group<OB, true, false>(a, st);    \
  else if (!a_kc && b_kc) *err = launch_dma_group<OB, false, true>(a, st);    \
  else *err = launch_dma_group<OB, false, false>(a, st);
  if (out_bf16) {
    JAGG_DMA_G(1)
  } else {
    JAGG_DMA_G(0)
  }
#undef JAGG_DMA_G
  return true;
}
}  // namespace jagg
