// gdn2_prefill.hip -- picks the prefill kernel instance for a problem, and
// the hand-off kernel of split sequences.
#include <stdlib.h>

#include "gdn2_device.hpp"
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
// The running state block stays in LDS; each thread holds its row of the
// next transition matrix in registers, requested one step ahead (16-byte
// loads), so the sequential steps wait on arithmetic, not on memory.
template <int CB>
__global__ __launch_bounds__(256) void split_combine_kernel(float *state, const float *trans, int jlast,
                                                             int BH, int d_k, int d_v, float *S_T) {
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
  const int nk4 = d_k / 4;  // d_k is a multiple of 16
  floatx4 m[32];
  auto load_row = [&](int j) {
    const floatx4 *src = reinterpret_cast<const floatx4 *>(trans + j * strans + ((size_t)bh * d_k + (row ? i : 0)) * d_k);
#pragma unroll
    for (int k4 = 0; k4 < 32; ++k4) m[k4] = k4 < nk4 ? src[k4] : zero4();
  };
  if (jlast >= 1) load_row(1);
  for (int j = 1; j <= jlast; ++j) {
    __syncthreads();
    float acc[CH];
    if (row)
      for (int c = 0; c < CH; ++c) acc[c] = state[j * sstate + s_row + c];
#pragma unroll
    for (int k4 = 0; k4 < 32; ++k4) {
      if (k4 < nk4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float mk = m[k4][e];
          const float *xr = &X[4 * k4 + e][half * CH];
#pragma unroll
          for (int c = 0; c < CH; ++c) acc[c] = fmaf(mk, xr[c], acc[c]);
        }
      }
    }
    if (j < jlast) load_row(j + 1);
    __syncthreads();
    if (row)
      for (int c = 0; c < CH; ++c) {
        X[i][half * CH + c] = acc[c];
        state[j * sstate + s_row + c] = acc[c];
      }
  }
  __syncthreads();
  // the state after segment jlast, [BH][d_k][d_v]
  if (S_T && row)
    for (int c = 0; c < CH; ++c) S_T[s_row + c] = X[i][half * CH + c];
}

// Output correction of split sequences: a segment run from a zero entering
// state wrote o_zero_t = (S^0_t)^T q_t, and its identity columns the
// transition's query reads oI_t = (Phi_t)^T q_t; with the segment's exact
// entering state S_in the output is o_t = o_zero_t + S_in^T oI_t, because
// the state after t is Phi_t S_in + S^0_t (the recurrence is linear in the
// state, column by column). Per (segment s >= 1, sequence, value head, slab
// of tokens), four waves of 16-token tiles: out^T = S_in^T oI^T as MFMA
// tiles (rows = output columns, columns = tokens), S_in^T held in registers
// as A fragments, oI rows read as B fragments; then o += out.
// K slots: slot j of lane group g in K32 step p is key channel 32p + 8g + j
// for both operands. Output rows: row 4g + j of tile 2q + h is column
// 32q + 8g + 4h + j, so that lane (token c, g) holds columns 32q + 8g .. +7
// of its token for q = 0 .. DV/32 - 1 (16 contiguous bytes in bf16) and the
// four lanes of a token cover 64 contiguous bytes per access.
template <int DK, int DV, bool BF16>
__global__ __launch_bounds__(256) void split_correct_kernel(void *o_, const void *oI_, const float *state, int B,
                                                             int T, int H_v, int seg_len, int nseg, int slab) {
  using E = Elem<BF16>;
  using O = Op<BF16>;
  using ET = typename E::T;
  typedef typename O::T OT;
  constexpr int NCT = DV / 16, NKP = (DK + 31) / 32;
  const int nslab = (seg_len + slab - 1) / slab;
  int idx = blockIdx.x;
  const int sl = idx % nslab;
  idx /= nslab;
  const int h = idx % H_v;
  idx /= H_v;
  const int n = idx % B;
  const int s = 1 + idx / B;  // segment (>= 1)
  const int t_beg = s * seg_len + sl * slab;
  const int t_end = min(min(t_beg + slab, (s + 1) * seg_len), T);
  if (s >= nseg || t_beg >= t_end) return;
  const float *Sin = state + (((size_t)(s - 1) * B + n) * H_v + h) * (size_t)(DK * DV);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  // S_in^T in the operand type, staged through LDS: read as whole rows of
  // S_in (16-byte loads), written transposed ([column][key channel], rows
  // padded against bank conflicts), then each lane's fragments are runs of 8
  // key channels of one column.
  constexpr int SP = DK + (BF16 ? 8 : 4);
  __shared__ OT sT[DV * SP];
  for (int e = 4 * (int)threadIdx.x; e < DK * DV; e += 4 * 256) {
    const int k = e / DV, col = e % DV;
    const floatx4 v = *reinterpret_cast<const floatx4 *>(Sin + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) sT[(col + i) * SP + k] = O::cvt(v[i]);
  }
  __syncthreads();
  // output column of row r of tile ct
  auto ocol = [](int ct, int r) { return DV >= 32 ? 32 * (ct >> 1) + 8 * (r >> 2) + 4 * (ct & 1) + (r & 3) : r; };
  Pair<BF16> sa[NCT][NKP];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int p = 0; p < NKP; ++p) {
      const int k0 = 32 * p + 8 * g;  // a multiple of 8: the run is wholly inside d_k or wholly past it
      if (k0 < DK) {
        const OT *src = sT + ocol(ct, c) * SP + k0;
        sa[ct][p] = Pair<BF16>{*reinterpret_cast<const typename O::Frag *>(src),
                               *reinterpret_cast<const typename O::Frag *>(src + 4)};
      } else {
        sa[ct][p] = Pair<BF16>{O::zero(), O::zero()};
      }
    }
  const size_t row0 = (size_t)n * T;  // token index of the sequence's first token
  const ET *oIh = static_cast<const ET *>(oI_) + (size_t)h * DK;
  ET *oh = static_cast<ET *>(o_) + (size_t)h * DV;
  // One 16-token tile of this wave per step: its oI rows (B fragments: 8
  // consecutive key channels of token t per K32 step, one 16-byte load in
  // bf16, two in fp32) and the o pieces it updates are requested together,
  // one step ahead (the next step's requests are issued before this step's
  // products), so a step waits on one memory round trip at most. Tokens
  // past the slab's end read the slab's first row and store nothing.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int NQ = DV >= 32 ? DV / 32 : 1;  // 8-column groups of a lane
  struct Step {
    Pair<BF16> b[NKP];
    floatx4 od[NQ][BF16 ? 1 : 2];  // the o pieces (bf16: raw 16-byte words)
  };
  auto request = [&](int t0, Step &L) {
    const int t = t0 + c;
    const bool ok = t < t_end;
    const ET *src = oIh + (row0 + (ok ? t : t_beg)) * (size_t)H_v * DK;
#pragma unroll
    for (int p = 0; p < NKP; ++p) {
      const int k0 = 32 * p + 8 * g;
      const bool in = k0 < DK;  // compile-time per p and lane group's run
      if constexpr (BF16) {
        const u32x4 raw = in ? *reinterpret_cast<const u32x4 *>(src + k0) : u32x4{0u, 0u, 0u, 0u};
        L.b[p].lo = __builtin_bit_cast(typename O::Frag, uint2{raw.x, raw.y});
        L.b[p].hi = __builtin_bit_cast(typename O::Frag, uint2{raw.z, raw.w});
      } else {
        L.b[p].lo = in ? *reinterpret_cast<const floatx4 *>(src + k0) : zero4();
        L.b[p].hi = in ? *reinterpret_cast<const floatx4 *>(src + k0 + 4) : zero4();
      }
    }
    if constexpr (DV >= 32) {
      const ET *d = oh + (row0 + (ok ? t : t_beg)) * (size_t)H_v * DV + 8 * g;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if constexpr (BF16) {
          L.od[q][0] = __builtin_bit_cast(floatx4, *reinterpret_cast<const u32x4 *>(d + 32 * q));
        } else {
          L.od[q][0] = *reinterpret_cast<const floatx4 *>(d + 32 * q);
          L.od[q][1] = *reinterpret_cast<const floatx4 *>(d + 32 * q + 4);
        }
      }
    }
  };
  auto tile = [&](const Step &L, int ct) {
    floatx4 acc = zero4();
#pragma unroll
    for (int p = 0; p < NKP; ++p) acc = O::mma32(acc, sa[ct][p].lo, sa[ct][p].hi, L.b[p].lo, L.b[p].hi);
    return acc;
  };
  auto finish = [&](int t0, const Step &L) {
    const int t = t0 + c;
    const bool ok = t < t_end;
    ET *dst = oh + (row0 + (ok ? t : t_beg)) * (size_t)H_v * DV;
    if constexpr (DV >= 32) {
      // columns 32 q + 8 g .. +7: tiles 2q (first four) and 2q + 1
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const floatx4 a0 = tile(L, 2 * q), a1 = tile(L, 2 * q + 1);
        if (ok) {
          ET *d = dst + 32 * q + 8 * g;
          if constexpr (BF16) {
            const u32x4 u = __builtin_bit_cast(u32x4, L.od[q][0]);
            const floatx4 lo = {__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
            const floatx4 hi = {__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u),
                                __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u)};
            const uint2 x = __builtin_bit_cast(uint2, __builtin_convertvector(lo + a0, bf16x4));
            const uint2 y = __builtin_bit_cast(uint2, __builtin_convertvector(hi + a1, bf16x4));
            *reinterpret_cast<u32x4 *>(d) = u32x4{x.x, x.y, y.x, y.y};
          } else {
            floatx4 *df = reinterpret_cast<floatx4 *>(d);
            df[0] = L.od[q][0] + a0;
            df[1] = L.od[q][1] + a1;
          }
        }
      }
    } else {  // DV = 16: rows are the columns
      const floatx4 acc = tile(L, 0);
      if (ok) {
        ET *d = dst + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) E::st(d + j, E::ld(d + j) + acc[j]);
      }
    }
  };
  // two register sets in turn (no copies between them)
  Step s0, s1;
  int t0 = t_beg + 16 * wave;
  if (t0 < t_end) request(t0, s0);
  for (; t0 < t_end; t0 += 128) {
    request(t0 + 64, s1);
    finish(t0, s0);
    if (t0 + 64 >= t_end) break;
    request(t0 + 128, s0);
    finish(t0 + 64, s1);
  }
  (void)sizeof(OT);
}

template <int DK, bool BF16>
hipError_t launch_correct_dv(void *o, const void *oI, const float *state, int B, int T, int H_v, int d_v,
                             int seg_len, int nseg, hipStream_t st) {
  // tokens per workgroup: each stages its segment's entering state once, so
  // shorter slabs repeat that; longer ones leave few workgroups per compute
  // unit (2048 and 4096 tokens measured 25% and 12% slower at B1 T65536 H16,
  // 256 tokens 12%)
  const int slab = 512;
  const int nslab = (seg_len + slab - 1) / slab;
  const dim3 grid((unsigned)((nseg - 1) * B * H_v * nslab));
  switch (d_v) {
    case 16: hipLaunchKernelGGL((split_correct_kernel<DK, 16, BF16>), grid, dim3(256), 0, st, o, oI, state, B, T, H_v, seg_len, nseg, slab); break;
    case 32: hipLaunchKernelGGL((split_correct_kernel<DK, 32, BF16>), grid, dim3(256), 0, st, o, oI, state, B, T, H_v, seg_len, nseg, slab); break;
    case 64: hipLaunchKernelGGL((split_correct_kernel<DK, 64, BF16>), grid, dim3(256), 0, st, o, oI, state, B, T, H_v, seg_len, nseg, slab); break;
    case 128: hipLaunchKernelGGL((split_correct_kernel<DK, 128, BF16>), grid, dim3(256), 0, st, o, oI, state, B, T, H_v, seg_len, nseg, slab); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_correct_dk(void *o, const void *oI, const float *state, int B, int T, int H_v, int d_k, int d_v,
                             int seg_len, int nseg, hipStream_t st) {
  switch (d_k) {
    case 16: return launch_correct_dv<16, BF16>(o, oI, state, B, T, H_v, d_v, seg_len, nseg, st);
    case 32: return launch_correct_dv<32, BF16>(o, oI, state, B, T, H_v, d_v, seg_len, nseg, st);
    case 64: return launch_correct_dv<64, BF16>(o, oI, state, B, T, H_v, d_v, seg_len, nseg, st);
    case 128: return launch_correct_dv<128, BF16>(o, oI, state, B, T, H_v, d_v, seg_len, nseg, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_split_combine(float *state, const float *trans, int jlast, int BH, int d_k, int d_v,
                                float *S_T, hipStream_t st) {
  if ((jlast < 1 && !S_T) || BH == 0) return hipSuccess;
  if (d_k > 128) return hipErrorInvalidValue;
  // narrow column blocks: many workgroups, each step short (the steps are
  // sequential, the column blocks independent)
  hipLaunchKernelGGL((split_combine_kernel<8>), dim3(BH * (d_v / 8)), dim3(256), 0, st, state, trans, jlast, BH,
                     d_k, d_v, S_T);
  return hipGetLastError();
}

hipError_t launch_split_correct(void *o, const void *oI, const float *state, int B, int T, int H_v, int d_k,
                                int d_v, int seg_len, int nseg, bool bf16, hipStream_t st) {
  if (nseg < 2 || B == 0 || H_v == 0) return hipSuccess;
  return bf16 ? launch_correct_dk<true>(o, oI, state, B, T, H_v, d_k, d_v, seg_len, nseg, st)
              : launch_correct_dk<false>(o, oI, state, B, T, H_v, d_k, d_v, seg_len, nseg, st);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
  if (a.B == 0 || a.H_v == 0) return hipSuccess;
  return dispatch(a, st, nullptr);
}

PrefillPlan prefill_plan(const PrefillArgs &a) {
  PrefillPlan pl{a.chunk, 1, a.T, 0, false};
  if (a.B == 0 || a.H_v == 0) return pl;
  if (dispatch(a, nullptr, &pl) != hipSuccess) pl = PrefillPlan{a.chunk, 1, a.T, 0, false};
  return pl;
}

}  // namespace gdn2
