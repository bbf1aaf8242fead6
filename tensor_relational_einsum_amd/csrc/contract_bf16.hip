// contract_bf16.hip -- bf16-input instantiations of the block contraction
// (see contract_impl.h).
#include "contract_impl.h"

namespace jagg {
hipError_t launch_contract_bf16(const ContractArgs &a, int out_bf16, bool a_kc, bool b_kc, int va, int vb, bool big,
                                hipStream_t st) {
  return launch_typed<uint16_t>(a, out_bf16, a_kc, b_kc, va, vb, big, st);
}
}  // namespace jagg
