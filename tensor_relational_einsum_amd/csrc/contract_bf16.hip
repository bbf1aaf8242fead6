// contract_bf16.hip -- bf16-input instantiations of the block contraction
// (see contract_impl.h and contract_dma.h).
#include "contract_dma.h"

namespace jagg {
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
