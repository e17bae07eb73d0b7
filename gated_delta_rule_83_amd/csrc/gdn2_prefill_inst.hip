// gdn2_prefill_inst.hip -- instantiates the prefill kernel for one key-head
// dimension and one input dtype. Built several times with
//   -DGDN2_INST_DK=<16|32|64|128> -DGDN2_INST_BF16=<0|1> -DGDN2_INST_FN=<name>
// so that the instantiations compile in parallel.
#include "gdn2_prefill.hpp"

#if !defined(GDN2_INST_DK) || !defined(GDN2_INST_BF16) || !defined(GDN2_INST_FN)
#error "GDN2_INST_DK, GDN2_INST_BF16 and GDN2_INST_FN must be defined"
#endif

namespace gdn2 {

hipError_t GDN2_INST_FN(const PrefillArgs &a, hipStream_t st, PrefillPlan *plan_only) {
  return dispatch_prefill<GDN2_INST_DK, GDN2_INST_BF16 != 0>(a, st, plan_only);
}

}  // namespace gdn2

#ifdef GDN2_PHASE_TIMING
extern "C" int gdn2_phase_cycles_read(unsigned long long *host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn2::gdn2_phase_cycles), sizeof(gdn2::gdn2_phase_cycles));
}
#endif
