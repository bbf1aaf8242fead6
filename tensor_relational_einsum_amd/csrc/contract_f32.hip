// contract_f32.hip -- fp32-input instantiations of the block contraction
// (see contract_impl.h).
#include "contract_impl.h"

namespace jagg {
hipError_t launch_contract_f32(const ContractArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                               hipStream_t st, const char **which) {
  *which = big ? "f32 256x256"
                : (a.N + 63) / 64 * 64 < (a.N + 127) / 128 * 128 ? "f32 128x64"
                : (!out_bf16 && va == 4 && vb == 4 && !a.causal_red && short_walk<float>(a)) ? "f32 128x128 one stage"
                : "f32 128x128";
  return launch_typed<float>(a, out_bf16, a_kc, b_kc, va, vb, big, st);
}
}  // namespace jagg
