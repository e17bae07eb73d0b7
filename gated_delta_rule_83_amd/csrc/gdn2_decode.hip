// gdn2_decode.hip -- single-token decode step of the Gated DeltaNet-2
// recurrence: one streaming pass over the fp32 state.
//
// Gate forms as for the prefill: per-channel gates, their pre-activations,
// the coupled erase/write gate beta, and the scalar decay alpha with it.
//
// Per (sequence n, value head h) the step is (Gated DeltaNet-2 post on
// tilnote.io, GDN-2 design section; delta-rule tutorial on
// ai-systems-engineering.com, "record the difference" and key-versus-query
// sections):
//   S~ = diag(a) S;  r = S~^T k;  S' = S~ - (b*k) r^T + k (w*v)^T;  o = S'^T q.
//
// Bandwidth design: the state (64 KiB per head at d_k = d_v = 128) is the
// only large operand. Each workgroup owns one head's state. A thread owns 4
// adjacent value columns (one 16-byte load per row) on RPT rows; the wave's
// lanes walk a row contiguously, so every load and store is a coalesced
// 128-bit access. The state is held in registers between the two column
// reductions (key read r, query read o): each is a sum over rows, done
// first within the thread, then across lanes with butterfly shuffles, then
// across waves through LDS. S is read exactly once and written exactly once;
// the stores are marked nontemporal (the loads are not: measured, nontemporal
// loads made the step about 8% slower).
#include "gdn2_device.hpp"
#include "gdn2_internal.hpp"

namespace gdn2 {

template <int DK, int DV>
struct DecodeCfg {
  static constexpr int NT = (DK * DV / 4) < 256 ? (DK * DV / 4) : 256;  // threads
  static constexpr int TPR = DV / 4;       // threads covering one row (4 columns each)
  static constexpr int RG = NT / TPR;      // row groups
  static constexpr int RPT = DK / RG;      // rows per thread
  static constexpr int NW = NT / 64;       // waves
  static_assert(NT % 64 == 0, "at least one full wave");
  static_assert(TPR <= 64 && 64 % TPR == 0, "a row fits in one wave");
  static_assert(RPT >= 1 && RG * RPT == DK, "rows split evenly");
};

// Sum x over the threads that share this thread's 4 columns (all row groups).
template <int DK, int DV>
__device__ __forceinline__ floatx4 column_sum(floatx4 x, float (*red)[DV], int tid) {
  using Cf = DecodeCfg<DK, DV>;
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = Cf::TPR; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] += __shfl_xor(x[c], off, 64);
  }
  if (Cf::NW == 1) return x;
  const int c4 = tid % Cf::TPR;
  if (lane < Cf::TPR) *reinterpret_cast<floatx4 *>(&red[wave][4 * c4]) = x;
  __syncthreads();
  floatx4 s = zero4();
#pragma unroll
  for (int w = 0; w < Cf::NW; ++w) s += *reinterpret_cast<const floatx4 *>(&red[w][4 * c4]);
  return s;
}

template <int DK, int DV, bool BF16, int GF>
__global__ __launch_bounds__((DecodeCfg<DK, DV>::NT)) void decode_step_kernel(
    const typename Elem<BF16>::T *__restrict__ q, const typename Elem<BF16>::T *__restrict__ k,
    const typename Elem<BF16>::T *__restrict__ v, const void *__restrict__ a,
    const void *__restrict__ b, const void *__restrict__ w, float *__restrict__ S,
    typename Elem<BF16>::T *__restrict__ o, int H_qk, int H_v) {
  using Cf = DecodeCfg<DK, DV>;
  using E = Elem<BF16>;
  using ET = typename E::T;
  __shared__ float s_a[DK], s_bk[DK], s_k[DK], s_q[DK], s_u[DV];
  __shared__ float s_red1[Cf::NW][DV], s_red2[Cf::NW][DV];

  const int unit = blockIdx.x;  // n * H_v + h
  const int n = unit / H_v, h = unit - n * H_v;
  const int g = h / (H_v / H_qk);
  const int tid = threadIdx.x;
  const int c4 = tid % Cf::TPR, rg = tid / Cf::TPR;

  float *Sh = S + (size_t)unit * (DK * DV);
  // Issue every state load first: RPT independent 16-byte loads per thread.
  floatx4 s[Cf::RPT];
#pragma unroll
  for (int r = 0; r < Cf::RPT; ++r) {
    const int row = r * Cf::RG + rg;
    s[r] = *reinterpret_cast<const floatx4 *>(Sh + row * DV + 4 * c4);
  }
  // Per-row gates and per-column values through LDS (tiny), in the gate form
  // GF: per-channel fp32; per-channel pre-activations in the input dtype,
  // activated here; coupled beta (b = w, one fp32 per head); scalar alpha
  // and beta.
  const size_t qk_off = ((size_t)n * H_qk + g) * DK;
  const size_t ab_off = (size_t)unit * DK;
  const size_t vw_off = (size_t)unit * DV;
  const float *af = static_cast<const float *>(a), *bf = static_cast<const float *>(b);
  const float *wf = static_cast<const float *>(w);
  for (int i = tid; i < DK; i += Cf::NT) {
    const float kk = E::ld(k + qk_off + i);
    s_k[i] = kk;
    s_q[i] = E::ld(q + qk_off + i);
    float ai, bi;
    if constexpr (GF == kGatePre) {
      ai = decay_from_pre(E::ld(static_cast<const ET *>(a) + ab_off + i));
      bi = gate_from_pre(E::ld(static_cast<const ET *>(b) + ab_off + i));
    } else {
      ai = GF == kGateScalar ? af[unit] : af[ab_off + i];
      bi = GF >= kGateCoupled ? bf[unit] : bf[ab_off + i];
    }
    s_a[i] = ai;
    s_bk[i] = bi * kk;
  }
  for (int j = tid; j < DV; j += Cf::NT) {
    float wj;
    if constexpr (GF == kGatePre)
      wj = gate_from_pre(E::ld(static_cast<const ET *>(w) + vw_off + j));
    else
      wj = GF >= kGateCoupled ? bf[unit] : wf[vw_off + j];
    s_u[j] = wj * E::ld(v + vw_off + j);
  }
  __syncthreads();

  // Decay the key-axis rows, then the key read of the decayed state.
  floatx4 part = zero4();
#pragma unroll
  for (int r = 0; r < Cf::RPT; ++r) {
    const int row = r * Cf::RG + rg;
    s[r] *= s_a[row];
    part += s[r] * s_k[row];
  }
  const floatx4 rk = column_sum<DK, DV>(part, s_red1, tid);

  // Erase the key-side component (gate b on the key axis), write the
  // value-side component (gate w on the value axis), then the query read.
  const floatx4 u = *reinterpret_cast<const floatx4 *>(&s_u[4 * c4]);
  floatx4 po = zero4();
#pragma unroll
  for (int r = 0; r < Cf::RPT; ++r) {
    const int row = r * Cf::RG + rg;
    s[r] = s[r] - s_bk[row] * rk + s_k[row] * u;
    po += s[r] * s_q[row];
    __builtin_nontemporal_store(s[r], reinterpret_cast<floatx4 *>(Sh + row * DV + 4 * c4));
  }
  const floatx4 oo = column_sum<DK, DV>(po, s_red2, tid);
  if (tid < Cf::TPR) {
#pragma unroll
    for (int c = 0; c < 4; ++c) E::st(o + vw_off + 4 * c4 + c, oo[c]);
  }
}

template <int DK, int DV, bool BF16, int GF>
static void launch_decode_form(const DecodeArgs &p, hipStream_t st) {
  using T = typename Elem<BF16>::T;
  hipLaunchKernelGGL((decode_step_kernel<DK, DV, BF16, GF>), dim3(p.B * p.H_v), dim3(DecodeCfg<DK, DV>::NT), 0,
                     st, (const T *)p.q, (const T *)p.k, (const T *)p.v, p.a, p.b, p.w, p.S, (T *)p.o, p.H_qk,
                     p.H_v);
}

template <int DK, int DV, bool BF16>
static hipError_t launch_decode_t(const DecodeArgs &p, hipStream_t st) {
  if (p.B * p.H_v == 0) return hipSuccess;
  switch (p.gate_form) {
    case kGatePre: launch_decode_form<DK, DV, BF16, kGatePre>(p, st); break;
    case kGateCoupled: launch_decode_form<DK, DV, BF16, kGateCoupled>(p, st); break;
    case kGateScalar: launch_decode_form<DK, DV, BF16, kGateScalar>(p, st); break;
    default: launch_decode_form<DK, DV, BF16, kGateGeneral>(p, st); break;
  }
  return hipGetLastError();
}

template <int DK, bool BF16>
static hipError_t dispatch_dv(const DecodeArgs &p, hipStream_t st) {
  switch (p.d_v) {
    case 16: return launch_decode_t<DK, 16, BF16>(p, st);
    case 32: return launch_decode_t<DK, 32, BF16>(p, st);
    case 64: return launch_decode_t<DK, 64, BF16>(p, st);
    case 128: return launch_decode_t<DK, 128, BF16>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
static hipError_t dispatch_dk(const DecodeArgs &p, hipStream_t st) {
  switch (p.d_k) {
    case 16: return dispatch_dv<16, BF16>(p, st);
    case 32: return dispatch_dv<32, BF16>(p, st);
    case 64: return dispatch_dv<64, BF16>(p, st);
    case 128: return dispatch_dv<128, BF16>(p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs &p, hipStream_t st) {
  return p.bf16 ? dispatch_dk<true>(p, st) : dispatch_dk<false>(p, st);
}

}  // namespace gdn2
