// gdn2_prefill_inst.hip -- instantiates the prefill kernel for one key-head
// dimension and one input dtype. Built several times with
//   -DGDN2_INST_DK=<16|32|64|128> -DGDN2_INST_BF16=<0|1> -DGDN2_INST_FN=<name>
// so that the instantiations compile in parallel.
#include "gdn2_prefill.hpp"

#if !defined(GDN2_INST_DK) || !defined(GDN2_INST_BF16) || !defined(GDN2_INST_FN)
#error "GDN2_INST_DK, GDN2_INST_BF16 and GDN2_INST_FN must be defined"
#endif

namespace gdn2 {

// Largest chunk whose LDS working set fits one workgroup (fp32 operands
// are twice as wide as bf16 ones).
template <int DK, bool BF16>
constexpr int max_chunk() {
  return (!BF16 && DK >= 64) ? 32 : 64;
}

hipError_t GDN2_INST_FN(const PrefillArgs &a, hipStream_t st) {
  constexpr int DK = GDN2_INST_DK;
  constexpr bool BF16 = GDN2_INST_BF16 != 0;
  switch (a.chunk) {
    case 16: return dispatch_prefill_nct<DK, 16, BF16>(a, st);
    case 32: return dispatch_prefill_nct<DK, 32, BF16>(a, st);
    case 64:
      if constexpr (max_chunk<DK, BF16>() >= 64) return dispatch_prefill_nct<DK, 64, BF16>(a, st);
      else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn2
