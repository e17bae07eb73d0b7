// gdn2_prefill.hip -- picks the prefill kernel instance for a problem, and
// the hand-off kernel of split sequences.
#include <stdlib.h>

#include "gdn2_internal.hpp"

namespace gdn2 {

hipError_t launch_prefill_bf16_dk16(const PrefillArgs &, hipStream_t, PrefillPlan *);
hipError_t launch_prefill_bf16_dk32(const PrefillArgs &, hipStream_t, PrefillPlan *);
hipError_t launch_prefill_bf16_dk64(const PrefillArgs &, hipStream_t, PrefillPlan *);
hipError_t launch_prefill_bf16_dk128(const PrefillArgs &, hipStream_t, PrefillPlan *);
hipError_t launch_prefill_f32_dk16(const PrefillArgs &, hipStream_t, PrefillPlan *);
hipError_t launch_prefill_f32_dk32(const PrefillArgs &, hipStream_t, PrefillPlan *);
hipError_t launch_prefill_f32_dk64(const PrefillArgs &, hipStream_t, PrefillPlan *);
hipError_t launch_prefill_f32_dk128(const PrefillArgs &, hipStream_t, PrefillPlan *);

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

namespace {

hipError_t dispatch(const PrefillArgs &a, hipStream_t st, PrefillPlan *plan_only) {
  if (a.bf16) {
    switch (a.d_k) {
      case 16: return launch_prefill_bf16_dk16(a, st, plan_only);
      case 32: return launch_prefill_bf16_dk32(a, st, plan_only);
      case 64: return launch_prefill_bf16_dk64(a, st, plan_only);
      case 128: return launch_prefill_bf16_dk128(a, st, plan_only);
    }
  } else {
    switch (a.d_k) {
      case 16: return launch_prefill_f32_dk16(a, st, plan_only);
      case 32: return launch_prefill_f32_dk32(a, st, plan_only);
      case 64: return launch_prefill_f32_dk64(a, st, plan_only);
      case 128: return launch_prefill_f32_dk128(a, st, plan_only);
    }
  }
  return hipErrorInvalidValue;
}

// One workgroup per (sequence-head, block of CB state columns); thread
// (row i = tid / 2, half = tid % 2) owns columns half * CB/2 .. +CB/2 of row i.
// The running state block stays in LDS; the transition rows are read from
// memory (each row by two threads).
template <int CB>
__global__ __launch_bounds__(256) void split_combine_kernel(float *state, const float *trans, int nseg,
                                                             int BH, int d_k, int d_v) {
  constexpr int CH = CB / 2;
  __shared__ __attribute__((aligned(16))) float X[128][CB + 4];  // 16-byte rows, 4 banks apart
  const int nblk = d_v / CB;
  const int bh = blockIdx.x / nblk, c0 = (blockIdx.x % nblk) * CB;
  const int i = threadIdx.x >> 1, half = threadIdx.x & 1;
  const bool row = i < d_k;
  const size_t sstate = (size_t)BH * d_k * d_v, strans = (size_t)BH * d_k * d_k;
  const size_t s_row = ((size_t)bh * d_k + i) * d_v + c0 + half * CH;
  if (row)
    for (int c = 0; c < CH; ++c) X[i][half * CH + c] = state[s_row + c];
  for (int j = 1; j + 1 < nseg; ++j) {
    __syncthreads();
    float acc[CH];
    const float *m = trans + j * strans + ((size_t)bh * d_k + i) * d_k;
    if (row) {
      for (int c = 0; c < CH; ++c) acc[c] = state[j * sstate + s_row + c];
      for (int k = 0; k < d_k; ++k) {
        const float mk = m[k];
        for (int c = 0; c < CH; ++c) acc[c] = fmaf(mk, X[k][half * CH + c], acc[c]);
      }
    }
    __syncthreads();
    if (row)
      for (int c = 0; c < CH; ++c) {
        X[i][half * CH + c] = acc[c];
        state[j * sstate + s_row + c] = acc[c];
      }
  }
}

}  // namespace

hipError_t launch_split_combine(float *state, const float *trans, int nseg, int BH, int d_k, int d_v,
                                hipStream_t st) {
  if (nseg < 3 || BH == 0) return hipSuccess;
  if (d_k > 128) return hipErrorInvalidValue;
  if (d_v % 32 == 0)
    hipLaunchKernelGGL((split_combine_kernel<32>), dim3(BH * (d_v / 32)), dim3(256), 0, st, state, trans, nseg,
                       BH, d_k, d_v);
  else
    hipLaunchKernelGGL((split_combine_kernel<16>), dim3(BH * (d_v / 16)), dim3(256), 0, st, state, trans, nseg,
                       BH, d_k, d_v);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
  if (a.B == 0 || a.H_v == 0) return hipSuccess;
  return dispatch(a, st, nullptr);
}

PrefillPlan prefill_plan(const PrefillArgs &a) {
  PrefillPlan pl{a.chunk, 1, a.T, 0};
  if (a.B == 0 || a.H_v == 0) return pl;
  if (dispatch(a, nullptr, &pl) != hipSuccess) pl = PrefillPlan{a.chunk, 1, a.T, 0};
  return pl;
}

}  // namespace gdn2
