// contract_bf16.hip -- bf16-input instantiations of the block contraction
// (see contract_impl.h and contract_dma.h).
#include "contract_dma.h"

namespace jagg {
hipError_t launch_contract_bf16(const ContractArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                                hipStream_t st, const char **which) {
  // 256x256 tiles over 16-byte vectors without a causal mask on the reduced
  // letter: the LDS-DMA pipeline
  if (big && va == 8 && vb == 8 && !a.causal_red) {
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
