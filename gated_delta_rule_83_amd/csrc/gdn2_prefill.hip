// gdn2_prefill.hip -- picks the prefill kernel instance for a problem.
#include <stdlib.h>

#include "gdn2_internal.hpp"

namespace gdn2 {

hipError_t launch_prefill_bf16_dk16(const PrefillArgs &, hipStream_t);
hipError_t launch_prefill_bf16_dk32(const PrefillArgs &, hipStream_t);
hipError_t launch_prefill_bf16_dk64(const PrefillArgs &, hipStream_t);
hipError_t launch_prefill_bf16_dk128(const PrefillArgs &, hipStream_t);
hipError_t launch_prefill_f32_dk16(const PrefillArgs &, hipStream_t);
hipError_t launch_prefill_f32_dk32(const PrefillArgs &, hipStream_t);
hipError_t launch_prefill_f32_dk64(const PrefillArgs &, hipStream_t);
hipError_t launch_prefill_f32_dk128(const PrefillArgs &, hipStream_t);

// Value columns per workgroup = 16 * nct (nct = 1, 2 or 4), one wave per 16
// columns plus helper waves up to four. Wider workgroups share the chunk's
// Gram matrices and triangular solve across more columns (less
// recomputation, fewer reads of q, k, a, b).
int prefill_pick_nct(int B, int H_v, int d_v) {
  (void)B;
  (void)H_v;
  const char *env = getenv("GDN2_PREFILL_NCT");
  if (env) {
    const int v = atoi(env);
    if ((v == 1 || v == 2 || v == 4) && d_v % (16 * v) == 0) return v;
  }
  if (d_v % 64 == 0) return 4;
  if (d_v % 32 == 0) return 2;
  return 1;
}

hipError_t launch_prefill(const PrefillArgs &in, hipStream_t st) {
  PrefillArgs a = in;
  if (a.B == 0 || a.H_v == 0) return hipSuccess;
  if (a.bf16) {
    switch (a.d_k) {
      case 16: return launch_prefill_bf16_dk16(a, st);
      case 32: return launch_prefill_bf16_dk32(a, st);
      case 64: return launch_prefill_bf16_dk64(a, st);
      case 128: return launch_prefill_bf16_dk128(a, st);
    }
  } else {
    switch (a.d_k) {
      case 16: return launch_prefill_f32_dk16(a, st);
      case 32: return launch_prefill_f32_dk32(a, st);
      case 64: return launch_prefill_f32_dk64(a, st);
      case 128: return launch_prefill_f32_dk128(a, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn2
