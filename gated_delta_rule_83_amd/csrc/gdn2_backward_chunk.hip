// gdn2_backward_chunk.hip -- the backward pass in chunk form, on the matrix
// cores (bf16 inputs, d_k = d_v = 128, per-channel fp32 gates).
//
// The forward step of one chunk of C tokens from its entering state S0
// (Gated DeltaNet-2 post on tilnote.io, GDN-2 design section; the chunk form
// of the delta rule's WY representation), with cumulative decays
// gamma_t = a_1 ... a_t per key channel, an anchor A per channel (1, or the
// decay at the chunk's middle when the chunk decays too far) and
// lambda_t = gamma_t / A, mu_s = A / gamma_s:
//   Ql = lambda q, Kl = lambda k, Km = mu k, Bm = mu b k, U = w v,
//   S0a = diag(A) S0, Akk = stril(Kl Km^T), Akb = stril(Kl Bm^T),
//   Mqk = tril(Ql Km^T), Mqb = tril(Ql Bm^T), L = I + Akb,
//   R = L^-1 (Kl S0a + Akk U)            (the erase reads r_t)
//   O = Ql S0a + Mqk U - Mqb R            (the outputs)
//   S_C = diag(gamma_C / A) (S0a + Km^T U - Bm^T R).
// Its adjoint, given dO and dS_C (the gradient of the chunk's exiting
// state), with dSs = diag(gamma_C / A) dS_C:
//   dR = -Bm dSs - Mqb^T dO,  dZ = L^-T dR,
//   dU = Km dSs + Mqk^T dO + Akk^T dZ     (-> dv = w dU, dw = v dU)
//   dMqk = tril(dO U^T), dMqb = -tril(dO R^T), dAkk = stril(dZ U^T),
//   dAkb = -stril(dZ R^T),
//   dQl = dO S0a^T + dMqk Km + dMqb Bm,  dKl = dZ S0a^T + dAkk Km + dAkb Bm,
//   dKm = U dSs^T + dMqk^T Ql + dAkk^T Kl, dBm = -R dSs^T + dMqb^T Ql + dAkb^T Kl,
//   dq = lambda dQl, dk = lambda dKl + mu dKm + mu b dBm, db = mu k dBm,
// the log-decay gradient per token and channel
//   dg_t = Ql dQl + Kl dKl - Km dKm - Bm dBm  (+ rowsum(dS_C * S_C) at t = C),
// da_t = (sum over t' >= t of dg_t') / a_t, and the adjoint entering the chunk
//   dS_prev = diag(gamma_C) dS_C + Kd^T dZ + Qd^T dO  (Kd = gamma k, Qd = gamma q).
// The anchor cancels in every product; the operands only carry factors up
// to e^60 (the prefill's chunk classes). Chunks that decay faster than the
// middle anchor can carry (the prefill steps them token by token) are not
// handled here: the host then runs the per-token backward instead.
//
// Four launches:
//   1. the prefill, storing the state entering every chunk (bf16);
//   2. bwd_prep_kernel, per chunk: the operands of the chunk's adjoint step
//      dS_prev = diag(gamma_C) dS_C - Kd^T (Wt dS_C) + Qe^T dO, with
//      Wt = L^-T Bc, Qe = Qd - (L^-T Mqb^T)^T Kd, Bc = (gamma_C / gamma) b k,
//      stored in the order of the MFMA fragments that read them;
//   3. bwd_dstate_kernel, per (sequence, head, 64 value columns): the
//      adjoint of the state from the last chunk to the first (three MFMA
//      products per chunk), storing dS_C of every chunk (bf16) and dS0;
//   4. bwd_grad_kernel, per (sequence, query/key head, chunk): every
//      gradient of the chunk from its stored state and adjoint, summing the
//      value heads that share the query/key head.
#include <hip/hip_runtime.h>

#include "gdn2_device.hpp"
#include "gdn2_internal.hpp"

namespace gdn2 {
namespace {

constexpr int kC = 32;  // chunk length
using OB = Op<true>;
using BF = __bf16;
using Fr = OB::Frag;
using P2 = Pair<true>;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes (a plain vector: kept in registers)

// e^-60: the smallest decay over a chunk (anchor at its start) or over each
// half of it (anchor at its middle) whose inverse the operands may carry
constexpr float kMinDecay = 8.75651076e-27f;

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------- LDS fragments
// Lane l: c = l & 15, g = l >> 4. Conventions of gdn2_device.hpp.

// bf16 arrays in LDS hold rows of W elements (W = 128, 64 or 32) as 8-byte
// chunks of 4 elements; chunk q of row r sits at q ^ swz<W>(r). The
// permutations keep the two read patterns below free of bank conflicts (64
// banks; 16 lanes per pass): a fragment read (16 lanes on 16 consecutive
// rows, one chunk each) and a transposing read (16 lanes on 4 consecutive
// rows x 4 consecutive chunks), and row writes of 16 lanes on consecutive
// chunks.
template <int W>
__device__ __forceinline__ int swz(int r) {
  static_assert(W == 128 || W == 64 || W == 32, "row width");
  if constexpr (W == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else if constexpr (W == 64) return ((r >> 1) & 1) << 2;
  else return (r >> 2) & 7;
}
// index of element (r, col)
template <int W>
__device__ __forceinline__ int sx(int r, int col) {
  return r * W + (((col >> 2) ^ swz<W>(r)) << 2) + (col & 3);
}

// lane gets X[k0 + 4g + j][m0 + c], j = 0..3: a transposing LDS read (lane
// 4a + b of a 16-lane group receives element b of the 8-byte chunks
// addressed by lanes a, a + 4, a + 8, a + 12)
template <int W>
__device__ __forceinline__ Fr tr_frag(const BF *X, int k0, int m0, int c, int g) {
  const BF *p = X + sx<W>(k0 + 4 * g + (c >> 2), m0 + 4 * (c & 3));
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(__attribute__((address_space(3))) const char *)p);
  return __builtin_bit_cast(Fr, r);
}
// K32 operand whose 16 rows (A: rows m, or B: columns n) are rows of X and
// whose k runs along X's rows: X[m0 + c][k0 + ...]
template <int W>
__device__ __forceinline__ P2 op_rows(const BF *X, int m0, int k0, int c, int g) {
  const int r = m0 + c;
  return P2{OB::ld(X + sx<W>(r, k0 + 4 * g)), OB::ld(X + sx<W>(r, k0 + 16 + 4 * g))};
}
// K32 operand whose k runs down X's columns: X[k0 + ...][m0 + c]
template <int W>
__device__ __forceinline__ P2 op_cols(const BF *X, int m0, int k0, int c, int g) {
  return P2{tr_frag<W>(X, k0, m0, c, g), tr_frag<W>(X, k0 + 16, m0, c, g)};
}
__device__ __forceinline__ floatx4 mma(floatx4 acc, const P2 &a, const P2 &b) {
  return OB::mma32(acc, a.lo, a.hi, b.lo, b.hi);
}
// two accumulator tiles (k rows 0-15 and 16-31 of a K32 block) as an operand
__device__ __forceinline__ P2 acc_pair(floatx4 x0, floatx4 x1) { return P2{OB::from_acc(x0), OB::from_acc(x1)}; }
__device__ __forceinline__ floatx4 fr_f32(Fr x) { return __builtin_convertvector(x, floatx4); }
// reciprocals (v_rcp_f32, 1 ulp): of lambda and of the decays, within [e^-60, e^60]
__device__ __forceinline__ floatx4 rcp4(floatx4 x) {
  return floatx4{__builtin_amdgcn_rcpf(x[0]), __builtin_amdgcn_rcpf(x[1]), __builtin_amdgcn_rcpf(x[2]),
                 __builtin_amdgcn_rcpf(x[3])};
}

// Per-channel factors of one chunk. mode: 0 = anchor at the chunk start
// (A = 1), 1 = at the middle token (A = gamma_{C/2-1}), 2 = neither keeps
// the factors below e^60. h1, h2: the decay over each half.
__device__ __forceinline__ int chan_mode(const float (&a)[kC], float &h1, float &h2) {
  h1 = 1.f;
  h2 = 1.f;
#pragma unroll
  for (int t = 0; t < kC / 2; ++t) h1 *= a[t];
#pragma unroll
  for (int t = kC / 2; t < kC; ++t) h2 *= a[t];
  return (h1 * h2 >= kMinDecay) ? 0 : (h1 >= kMinDecay && h2 >= kMinDecay) ? 1 : 2;
}
// x: the decays a_t in, lambda_t = gamma_t / A out; the anchor A, gamma_C
// (may underflow to 0 in mode 1) and gamma_C / A
__device__ __forceinline__ void chan_lambda(float (&x)[kC], int mode, float h1, float h2, float &A, float &gC,
                                            float &gCA) {
  if (mode == 0) {
    float gm = 1.f;
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      gm *= x[t];
      x[t] = gm;
    }
    A = 1.f;
    gC = gm;
    gCA = gm;
  } else {
    // prod_{C/2 <= s <= t} a_s from the middle on, 1 / prod_{t < s < C/2} a_s before it
    float m = 1.f;
#pragma unroll
    for (int t = kC / 2; t < kC; ++t) {
      m *= x[t];
      x[t] = m;
    }
    float y = 1.f;
#pragma unroll
    for (int t = kC / 2 - 1; t >= 0; --t) {
      const float at = x[t];
      x[t] = 1.f / y;
      y *= at;
    }
    A = h1;
    gC = h1 * h2;
    gCA = h2;
  }
}

// lambda_t per channel from the chunk's decays staged in LDS (stage: [C][D]
// fp32, 1 past the end, written and synchronised by the caller) into lam
// (may be the same array); the anchor, gamma_C and gamma_C / A per channel.
// Returns the chunk's mode (the same in every thread; mode 2 writes
// nothing). Every thread of the workgroup calls it; it ends with a barrier.
template <int D>
__device__ int lambda_scan(const float *stage, float *lam, float *Ach, float *gCch, float *gCAch, int tid) {
  float x[kC], h1 = 1.f, h2 = 1.f;
  int m = 0;
  if (tid < D) {
#pragma unroll
    for (int t = 0; t < kC; ++t) x[t] = stage[t * D + tid];
    m = chan_mode(x, h1, h2);
  }
  const bool any2 = __syncthreads_or(m == 2) != 0;
  const bool any1 = __syncthreads_or(m == 1) != 0;
  const int mode = any2 ? 2 : any1 ? 1 : 0;
  if (mode != 2 && tid < D) {
    float A, gC, gCA;
    chan_lambda(x, mode, h1, h2, A, gC, gCA);
#pragma unroll
    for (int t = 0; t < kC; ++t) lam[t * D + tid] = x[t];
    Ach[tid] = A;
    gCch[tid] = gC;
    gCAch[tid] = gCA;
  }
  __syncthreads();
  return mode;
}

// The e-th quad (4 channels) of a chunk's [C][D] rows: token and channel.
template <int D>
__device__ __forceinline__ int quad_t(int e) { return e / (D / 4); }
template <int D>
__device__ __forceinline__ int quad_i(int e) { return 4 * (e % (D / 4)); }

// (I + N)^-1 for N strictly lower triangular (fp32 [C][C], LDS), written
// as bf16 into Li ([C][C] row-major), by blocks of 16. The diagonal blocks'
// inverses by substitution (lane j of lanes 0..31 one column, zero above
// the diagonal without branches: every x_u with u below the column is
// zero) go into N's diagonal blocks; then X = N10 L00^-1 (into N's upper
// block) and the lower block -L11^-1 X, one entry per thread of the first
// 256. Every thread of the workgroup calls it (three barriers).
__device__ __forceinline__ void unit_lower_inverse(float (*N)[kC], BF *Li, int tid) {
  constexpr int H = kC / 2;
  if (tid < kC) {
    int j = tid & (H - 1);
    asm volatile("" : "+v"(j));  // keeps the delta_tj selects here (hoisted, they were spilled)
    const int o = tid < H ? 0 : H;  // the block
    float x[H];
#pragma unroll
    for (int t = 0; t < H; ++t) {
      float s0 = t == j ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
      for (int u = 0; u < t; ++u) {
        if (u & 1)
          s1 -= N[o + t][o + u] * x[u];
        else
          s0 -= N[o + t][o + u] * x[u];
      }
      x[t] = s0 + s1;
    }
#pragma unroll
    for (int t = 0; t < H; ++t) {
      N[o + t][o + j] = x[t];
      Li[sx<kC>(o + t, o + j)] = (BF)x[t];
      Li[sx<kC>(t, H + j)] = (BF)0.f;  // the upper block
    }
  }
  __syncthreads();
  const int t = tid >> 4, j = tid & (H - 1);
  if (tid < H * H) {  // X[t][j] = sum_u N10[t][u] L00^-1[u][j]
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int u = 0; u < H; u += 2) {
      s0 += N[H + t][u] * N[u][j];
      s1 += N[H + t][u + 1] * N[u + 1][j];
    }
    N[t][H + j] = s0 + s1;
  }
  __syncthreads();
  if (tid < H * H) {  // -sum_u L11^-1[t][u] X[u][j]
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int u = 0; u < H; u += 2) {
      s0 += N[H + t][H + u] * N[u][H + j];
      s1 += N[H + t][H + u + 1] * N[u + 1][H + j];
    }
    Li[sx<kC>(H + t, j)] = (BF)(-(s0 + s1));
  }
  __syncthreads();
}

__device__ __forceinline__ void st_bf4(BF *p, floatx4 v) { *reinterpret_cast<Fr *>(p) = __builtin_convertvector(v, Fr); }

// The gates in each stored form (GF, kGate*): per-channel fp32 values;
// pre-activations in bf16, activated here (decay 1 / (1 + e^x), erase and
// write gates sigmoid(x)); coupled: b = w = beta, one fp32 value per token
// and value head; scalar: also a = alpha per token and value head. th is
// the (token, value head) index, i4 / i a channel (or value column).
template <int GF, int D>
__device__ __forceinline__ floatx4 gate_a4(const void *a, size_t th, int i4) {
  if constexpr (GF == kGateScalar) {
    const float x = static_cast<const float *>(a)[th];
    return floatx4{x, x, x, x};
  } else if constexpr (GF == kGatePre) {
    const floatx4 x = fr_f32(*reinterpret_cast<const Fr *>(static_cast<const BF *>(a) + th * D + i4));
    return floatx4{decay_from_pre(x[0]), decay_from_pre(x[1]), decay_from_pre(x[2]), decay_from_pre(x[3])};
  } else {
    return *reinterpret_cast<const floatx4 *>(static_cast<const float *>(a) + th * D + i4);
  }
}
// erase gate (b) or write gate (w, from `w`; the coupled forms read beta from `b`)
template <int GF, int D>
__device__ __forceinline__ floatx4 gate_bw4(const void *bw, const void *b, size_t th, int i4) {
  if constexpr (GF == kGateCoupled || GF == kGateScalar) {
    const float x = static_cast<const float *>(b)[th];
    return floatx4{x, x, x, x};
  } else if constexpr (GF == kGatePre) {
    const floatx4 x = fr_f32(*reinterpret_cast<const Fr *>(static_cast<const BF *>(bw) + th * D + i4));
    return floatx4{gate_from_pre(x[0]), gate_from_pre(x[1]), gate_from_pre(x[2]), gate_from_pre(x[3])};
  } else {
    return *reinterpret_cast<const floatx4 *>(static_cast<const float *>(bw) + th * D + i4);
  }
}
template <int GF, int D>
__device__ __forceinline__ float gate_bw1(const void *bw, const void *b, size_t th, int i) {
  if constexpr (GF == kGateCoupled || GF == kGateScalar) {
    return static_cast<const float *>(b)[th];
  } else if constexpr (GF == kGatePre) {
    return gate_from_pre(bf16_to_f32(static_cast<const uint16_t *>(bw)[th * D + i]));
  } else {
    return static_cast<const float *>(bw)[th * D + i];
  }
}
// a gate gradient dx of a per-channel gate x (activated value) in the stored
// form: fp32 as is, or for pre-activations dx dx/dpre in bf16 (dpre = dx *
// (-x (1 - x)) for the decay, dx * x (1 - x) for the erase and write gates)
template <int GF>
__device__ __forceinline__ void put_gate_grad(void *out, size_t idx, float dx, float x, bool decay) {
  if constexpr (GF == kGatePre) {
    const float s = x * (1.f - x);
    static_cast<uint16_t *>(out)[idx] = f32_to_bf16(dx * (decay ? -s : s));
  } else {
    static_cast<float *>(out)[idx] = dx;
  }
}

// ---------------------------------------------------------------- layouts
// The chunk-boundary states of few long sequences come from segments run in
// parallel (PrefillArgs::cst_segs) when the prefill's own split plan would cut
// the sequences into segments of equal length: its first two passes give the
// state entering every segment (seg_states), then one launch runs all
// segments from those states, storing the states at their chunk boundaries.
// seg.nseg = 1: one launch over whole sequences.
struct CstSplit {
  int nseg, seg_len, req;  // req: the force_nseg that yields this plan
};

PrefillArgs cst_prefill_args(int B, int T, int H_qk, int H_v) {
  PrefillArgs fa{};
  fa.B = B; fa.T = T; fa.H_qk = H_qk; fa.H_v = H_v; fa.d_k = 128; fa.d_v = 128;
  fa.chunk = 64;
  fa.bf16 = true;
  fa.nct = prefill_pick_nct(B, H_v, 128);
  // up to two rounds of the compute units in the split's first pass: the
  // segments' state launch (no identity blocks) then fills one round
  fa.split_wgs = 2 * kNumCU;
  return fa;
}

CstSplit cst_split_plan(int B, int T, int H_qk, int H_v) {
  const CstSplit none{1, T, 1};
  PrefillArgs fa = cst_prefill_args(B, T, H_qk, H_v);
  const PrefillPlan def = prefill_plan(fa);  // the prefill's own choice
  if (def.nseg < 2) return none;
  fa.force_nseg = def.nseg;
  const PrefillPlan pl = prefill_plan(fa);
  if (pl.nseg < 2 || pl.chunk != kC || (long)pl.nseg * pl.seg_len != T || pl.seg_len % kC != 0) return none;
  return CstSplit{pl.nseg, pl.seg_len, def.nseg};
}

struct ChunkLayout {
  int B, T, H_qk, H_v, nch;
  CstSplit seg;
  size_t cst, dst, prep, gc, flag, trans, segst, sin, total;  // byte offsets of the workspace regions
};

template <int D>
ChunkLayout chunk_layout(int B, int T, int H_qk, int H_v) {
  ChunkLayout l;
  l.B = B; l.T = T; l.H_qk = H_qk; l.H_v = H_v;
  l.nch = (T + kC - 1) / kC;
  l.seg = cst_split_plan(B, T, H_qk, H_v);
  const size_t units = (size_t)B * H_v, mat = (size_t)D * D * 2;
  l.cst = 0;
  l.dst = align256(units * (l.nch + 1) * mat);
  l.prep = l.dst + align256(units * l.nch * mat);
  l.gc = l.prep + align256(units * l.nch * 3 * kC * D * 2);
  l.flag = l.gc + align256(units * l.nch * D * 4);
  // segments: transitions, exiting states, entering states (fp32)
  const size_t segm = l.seg.nseg > 1 ? align256((size_t)l.seg.nseg * units * D * D * 4) : 0;
  l.trans = l.flag + 256;
  l.segst = l.trans + segm;
  l.sin = l.segst + segm;
  l.total = l.sin + segm;
  return l;
}

// ---------------------------------------------------------------- 2. chunk operands
// Per (unit = n * H_v + h, chunk): Wt as A fragments [tb][ib][lane][4]
// (lane (c, g) of tile (tb, ib): Wt[16tb + c][16ib + 4g + j]), then Kd and
// Qe as transposed A fragments [ib][tb][lane][4] (Kd[16tb + 4g + j][16ib + c]),
// and gamma_C per channel. Wt = L^-T Bc and Qe = Qd - Mqb (L^-1 Kd).
template <int D>
struct PrepSmem {
  alignas(16) float lam[kC * D];
  alignas(16) BF Ql[kC * D], Kl[kC * D], Bm[kC * D], Kd[kC * D], Qd[kC * D], Bc[kC * D];
  alignas(16) float Akb[kC][kC];
  alignas(16) BF Mqb[kC * kC], Lb[kC * kC];
  alignas(16) float A[D], gC[D], gCA[D];
};

struct PrepParams {
  const uint16_t *q, *k;
  const void *a, *b;  // in the gate form's layout
  BF *prep;
  float *gc;
  int *flag;
  int T, H_qk, H_v, nch;
};

template <int D, int GF>
__global__ __launch_bounds__(256) void bwd_prep_kernel(PrepParams p) {
  static_assert(D == 128, "d_k = 128");
  constexpr int NT = 256;
  __shared__ PrepSmem<D> sm;
  const int chunk = blockIdx.x % p.nch, unit = blockIdx.x / p.nch;
  const int n = unit / p.H_v, h = unit - n * p.H_v, gq = h / (p.H_v / p.H_qk);
  const int t0 = chunk * kC, Tc = min(kC, p.T - t0);
  const size_t tok0 = (size_t)n * p.T + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;

  // every request of the chunk first: decays, q, k, b (zero past the end)
  constexpr int NQ = kC * D / 4 / NT;
  floatx4 av[NQ], bv[NQ];
  Fr qv[NQ], kv[NQ];
#pragma unroll
  for (int it = 0; it < NQ; ++it) {
    const int e = tid + NT * it, t = quad_t<D>(e), i4 = quad_i<D>(e);
    av[it] = floatx4{1.f, 1.f, 1.f, 1.f};
    bv[it] = zero4();
    qv[it] = kv[it] = OB::zero();
    if (t < Tc) {
      const size_t row = tok0 + t;
      av[it] = gate_a4<GF, D>(p.a, row * p.H_v + h, i4);
      bv[it] = gate_bw4<GF, D>(p.b, p.b, row * p.H_v + h, i4);
      qv[it] = *reinterpret_cast<const Fr *>(p.q + (row * p.H_qk + gq) * D + i4);
      kv[it] = *reinterpret_cast<const Fr *>(p.k + (row * p.H_qk + gq) * D + i4);
    }
  }
#pragma unroll
  for (int it = 0; it < NQ; ++it) {
    const int e = tid + NT * it;
    *reinterpret_cast<floatx4 *>(&sm.lam[quad_t<D>(e) * D + quad_i<D>(e)]) = av[it];
  }
  __syncthreads();
  const int mode = lambda_scan<D>(sm.lam, sm.lam, sm.A, sm.gC, sm.gCA, tid);
  if (mode == 2) {  // uniform: some channel decays too far for either anchor
    if (tid == 0) atomicOr(p.flag, 1);
    return;
  }
  if (tid < D) p.gc[((size_t)unit * p.nch + chunk) * D + tid] = sm.gC[tid];
  // operands: lambda-scaled q, k; mu-scaled b k; gamma-scaled k, q; the
  // carry's (gamma_C / gamma) b k
#pragma unroll
  for (int it = 0; it < NQ; ++it) {
    const int e = tid + NT * it, t = quad_t<D>(e), i4 = quad_i<D>(e);
    const floatx4 q4 = fr_f32(qv[it]), k4 = fr_f32(kv[it]);
    const floatx4 lam = *reinterpret_cast<const floatx4 *>(&sm.lam[t * D + i4]);
    const floatx4 A = *reinterpret_cast<const floatx4 *>(&sm.A[i4]);
    const floatx4 gCA = *reinterpret_cast<const floatx4 *>(&sm.gCA[i4]);
    const floatx4 mu = rcp4(lam), bk = bv[it] * k4;
    st_bf4(&sm.Ql[sx<D>(t, i4)], lam * q4);
    st_bf4(&sm.Kl[sx<D>(t, i4)], lam * k4);
    st_bf4(&sm.Bm[sx<D>(t, i4)], mu * bk);
    st_bf4(&sm.Kd[sx<D>(t, i4)], A * lam * k4);
    st_bf4(&sm.Qd[sx<D>(t, i4)], A * lam * q4);
    st_bf4(&sm.Bc[sx<D>(t, i4)], gCA * mu * bk);
  }
  __syncthreads();
  // Gram tiles: Akb = stril(Kl Bm^T) (fp32), Mqb = tril(Ql Bm^T) (bf16);
  // lower tiles (0,0), (1,0), (1,1) of each
  for (int tile = wave; tile < 6; tile += NT / 64) {
    const int mat = tile / 3, tt = tile % 3;
    const int tb = tt == 0 ? 0 : 1, sb = tt == 2 ? 1 : 0;
    const BF *L = mat == 0 ? sm.Kl : sm.Ql;
    floatx4 acc = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32)
      acc = mma(acc, op_rows<D>(L, 16 * tb, k0, c, g), op_rows<D>(sm.Bm, 16 * sb, k0, c, g));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 16 * tb + 4 * g + j, s = 16 * sb + c;
      if (mat == 0) {
        sm.Akb[t][s] = s < t ? acc[j] : 0.f;
      } else {
        sm.Mqb[sx<kC>(t, s)] = (BF)(s <= t ? acc[j] : 0.f);
        sm.Mqb[sx<kC>(t & 15, 16 + (s & 15))] = (BF)0.f;  // the upper tile
      }
    }
  }
  __syncthreads();
  unit_lower_inverse(sm.Akb, sm.Lb, tid);

  BF *out = p.prep + ((size_t)unit * p.nch + chunk) * 3 * kC * D;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int ib = 2 * wave + x;
    // Wt^T = Bc^T L^-1: the accumulator of tile (ib, tb) is Wt's A fragment
    // Wk = L^-1 Kd, Qe = Qd - Mqb Wk
    floatx4 Wk[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const floatx4 wt = mma(zero4(), op_cols<D>(sm.Bc, 16 * ib, 0, c, g), op_cols<kC>(sm.Lb, 16 * tb, 0, c, g));
      *reinterpret_cast<Fr *>(out + ((tb * (D / 16) + ib) * 64 + lane) * 4) = OB::from_acc(wt);
      Wk[tb] = mma(zero4(), op_rows<kC>(sm.Lb, 16 * tb, 0, c, g), op_cols<D>(sm.Kd, 16 * ib, 0, c, g));
    }
    const P2 Wkn = acc_pair(-Wk[0], -Wk[1]);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const Fr kd = tr_frag<D>(sm.Kd, 16 * tb, 16 * ib, c, g);
      *reinterpret_cast<Fr *>(out + kC * D + ((ib * 2 + tb) * 64 + lane) * 4) = kd;
      floatx4 qe = fr_f32(tr_frag<D>(sm.Qd, 16 * tb, 16 * ib, c, g));
      qe = mma(qe, op_rows<kC>(sm.Mqb, 16 * tb, 0, c, g), Wkn);
      *reinterpret_cast<Fr *>(out + 2 * kC * D + ((ib * 2 + tb) * 64 + lane) * 4) = OB::from_acc(qe);
    }
  }
}

// ---------------------------------------------------------------- 3. adjoint of the state
// One workgroup per (unit, 64 value columns), four waves of 16 columns;
// lane (c, g) holds dS[16 mt + 4g + j][col] in dS[mt][j]. From the last
// chunk to the first: dS (the adjoint of chunk c's exiting state) is stored
// (bf16, [unit][chunk][column][channel]), then
// dS <- diag(gamma_C) dS - Kd^T (Wt dS) + Qe^T dO.
// A chunk's operands are requested two chunks ahead into one of two
// register sets (plain vector types: arrays of HIP's uint4 struct were kept
// in scratch), and staged in LDS one chunk ahead.
template <int D>
struct DstSmem {
  alignas(16) BF ops[2][3 * kC * D];
  alignas(16) BF dO[2][kC * 64];
  alignas(16) float gc[2][D];
};

// The sweep over segments of seg_chunks chunks (the last may be shorter),
// segments seg_first .. seg_first + nseg - 1 in one launch, per (segment,
// unit) NCB value column blocks and ncb_id identity column blocks. A value
// block starts from dS_in[in_base - s] (null: dS_T for the sequence's last
// segment, zero for the others) and ends in L_out[out_base - s] (null: dS0
// for segment 0); it stores the chunks' exiting adjoints when dst_all or its
// segment is the sequence's last. An identity block runs the homogeneous
// part (no dO term) on the columns of the identity and ends in
// M_out[out_base - s], the segment's map of its exiting adjoint to its
// entering one; none for the last segment. Per (slot, unit) d x d fp32.
struct DstParams {
  const BF *prep;
  const float *gc;
  const uint16_t *dO;
  const float *dST;
  float *dS0;
  BF *dst;
  int T, H_v, nch, units;
  int seg_chunks, seg_first, ncb_id, in_base, out_base;
  bool dst_all;
  const float *dS_in;
  float *L_out, *M_out;
};

template <int D>
__global__ __launch_bounds__(256) void bwd_dstate_kernel(DstParams p) {
  static_assert(D == 128, "d = 128");
  constexpr int NCB = D / 64, NMT = D / 16;
  constexpr int OPS16 = 3 * kC * D / 8;  // 16-byte pieces of a chunk's operands
  static_assert(OPS16 % 256 == 0, "whole pieces per thread");
  __shared__ DstSmem<D> sm;
  const int ncbt = NCB + p.ncb_id;
  const int cbt = blockIdx.x % ncbt, su = blockIdx.x / ncbt;  // su = (s - seg_first) * units + unit
  const int unit = su % p.units, s = p.seg_first + su / p.units;
  const int c_lo = s * p.seg_chunks, c_hi = min(c_lo + p.seg_chunks, p.nch), nloc = c_hi - c_lo;
  const bool last = c_hi == p.nch, ident = cbt >= NCB;
  if (nloc <= 0 || (ident && last)) return;
  const int cb = ident ? cbt - NCB : cbt;
  const int n = unit / p.H_v, h = unit - n * p.H_v;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int col = cb * 64 + 16 * wave + c;

  floatx4 dS[NMT];
  const float *din = p.dS_in ? p.dS_in + ((size_t)(p.in_base - s) * p.units + unit) * D * D
                     : (last && p.dST) ? p.dST + (size_t)unit * D * D
                                       : nullptr;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * mt + 4 * g + j;
      dS[mt][j] = ident ? (row == col ? 1.f : 0.f) : din ? din[(size_t)row * D + col] : 0.f;
    }
  const bool store = !ident && (p.dst_all || last);

  struct Raw {
    u32x4 o[OPS16 / 256];
    u32x4 d;
    floatx4 gcv;
  };
  // chunk ch's operands into registers; every request is issued on every
  // call (past the end: a clamped row, zeroed), so that the number of
  // requests between a request and its use never varies
  auto fetch = [&](int ch, Raw &r) __attribute__((always_inline)) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(p.prep + ((size_t)unit * p.nch + ch) * 3 * kC * D);
#pragma unroll
    for (int it = 0; it < OPS16 / 256; ++it) r.o[it] = src[tid + 256 * it];
    const int t = tid >> 3, q8 = tid & 7;  // 32 tokens x 8 pieces of 8 columns
    const int tok = ch * kC + t;
    const u32x4 d = *reinterpret_cast<const u32x4 *>(p.dO + ((size_t)n * p.T + min(tok, p.T - 1)) * p.H_v * D +
                                                    (size_t)h * D + cb * 64 + 8 * q8);
    r.d = tok < p.T && !ident ? d : u32x4{0u, 0u, 0u, 0u};
    r.gcv = *reinterpret_cast<const floatx4 *>(p.gc + ((size_t)unit * p.nch + ch) * D + 4 * (tid % (D / 4)));
  };
  auto stash = [&](int buf, const Raw &r) __attribute__((always_inline)) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(sm.ops[buf]);
#pragma unroll
    for (int it = 0; it < OPS16 / 256; ++it) dst[tid + 256 * it] = r.o[it];
    *reinterpret_cast<u32x4 *>(&sm.dO[buf][sx<64>(tid >> 3, 8 * (tid & 7))]) = r.d;
    if (tid < D / 4) reinterpret_cast<floatx4 *>(sm.gc[buf])[tid] = r.gcv;
  };

  Raw r0, r1;  // chunk k (from the segment's last) is requested into set k % 2, two chunks ahead
  auto body = [&](Raw &cur, Raw &nxt, int k) __attribute__((always_inline)) {
    const int ch = c_hi - 1 - k, buf = k & 1;
    fetch(max(ch - 2, c_lo), cur);  // cur held chunk ch, staged in the previous step (c_lo again at the end)
    // the adjoint of this chunk's exiting state
    if (store) {
      BF *dsto = p.dst + (((size_t)unit * p.nch + ch) * D + col) * D + 4 * g;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) *reinterpret_cast<Fr *>(dsto + 16 * mt) = OB::from_acc(dS[mt]);
    }
    const BF *Wt = sm.ops[buf], *Kd = sm.ops[buf] + kC * D, *Qe = sm.ops[buf] + 2 * kC * D;
    auto frag = [&](const BF *base, int idx) { return OB::ld(base + (idx * 64 + lane) * 4); };
    // Y = -Wt dS (tokens x this wave's columns)
    floatx4 Y[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      floatx4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < NMT / 2; ++kk)
        acc = mma(acc, P2{frag(Wt, tb * NMT + 2 * kk), frag(Wt, tb * NMT + 2 * kk + 1)},
                  acc_pair(dS[2 * kk], dS[2 * kk + 1]));
      Y[tb] = -acc;
    }
    const P2 dOf{tr_frag<64>(sm.dO[buf], 0, 16 * wave, c, g), tr_frag<64>(sm.dO[buf], 16, 16 * wave, c, g)};
    const P2 Yf = acc_pair(Y[0], Y[1]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const floatx4 gcv = *reinterpret_cast<const floatx4 *>(&sm.gc[buf][16 * mt + 4 * g]);
      floatx4 acc = dS[mt] * gcv;
      acc = mma(acc, P2{frag(Qe, mt * 2), frag(Qe, mt * 2 + 1)}, dOf);
      acc = mma(acc, P2{frag(Kd, mt * 2), frag(Kd, mt * 2 + 1)}, Yf);
      dS[mt] = acc;
    }
    // the next chunk (requested a step ago) into the other buffer, last
    // read in the previous step, before its barrier
    if (k + 1 < nloc) stash(buf ^ 1, nxt);
    __syncthreads();
  };
  fetch(c_hi - 1, r0);
  fetch(max(c_hi - 2, c_lo), r1);
  stash(0, r0);
  __syncthreads();
  for (int k = 0; k < nloc; k += 2) {
    body(r0, r1, k);
    if (k + 1 < nloc) body(r1, r0, k + 1);
  }
  float *out = ident ? p.M_out + ((size_t)(p.out_base - s) * p.units + unit) * D * D
               : p.L_out ? p.L_out + ((size_t)(p.out_base - s) * p.units + unit) * D * D
               : s == 0 && p.dS0 ? p.dS0 + (size_t)unit * D * D
                                 : nullptr;
  if (out) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[(size_t)(16 * mt + 4 * g + j) * D + col] = dS[mt][j];
  }
}

// Optional per-phase cycle counters of bwd_grad_kernel for kernel
// development, compiled only with -DGDN2_BWD_TIMING: 8 workgroups from
// GDN2_BWD_TIMER_BLOCK0 on store s_memtime deltas per wave and phase into
// gdn2_bwd_cycles[block][wave][phase] (read by gdn2_bwd_cycles_read).
#ifdef GDN2_BWD_TIMING
#ifndef GDN2_BWD_TIMER_BLOCK0
#define GDN2_BWD_TIMER_BLOCK0 4096
#endif
__device__ unsigned long long gdn2_bwd_cycles[8][8][16];
#define BWD_TIMER_INIT unsigned long long bt_acc[16] = {}, bt_prev = __builtin_amdgcn_s_memtime();
#define BWD_MARK(i)                                                 \
  do {                                                              \
    const unsigned long long bt_now = __builtin_amdgcn_s_memtime(); \
    bt_acc[i] += bt_now - bt_prev;                                  \
    bt_prev = bt_now;                                               \
  } while (0)
#define BWD_TIMER_STORE                                                                                   \
  if (blockIdx.x >= GDN2_BWD_TIMER_BLOCK0 && blockIdx.x < GDN2_BWD_TIMER_BLOCK0 + 8 && lane == 0)         \
    for (int i = 0; i < 16; ++i) gdn2_bwd_cycles[blockIdx.x - GDN2_BWD_TIMER_BLOCK0][wave][i] = bt_acc[i];
#else
#define BWD_TIMER_INIT
#define BWD_MARK(i) ((void)0)
#define BWD_TIMER_STORE
#endif

// ---------------------------------------------------------------- 4. gradients of a chunk
// One workgroup of eight waves per (sequence, query/key head, chunk); wave
// w owns value columns 16w.. and key channels 16w.. of every product.
template <int D>
struct GradSmem {
  alignas(16) BF Ql[kC * D], Kl[kC * D], Km[kC * D], Bm[kC * D];
  alignas(16) BF U[kC * D], dO[kC * D], R[kC * D], dZ[kC * D];
  // S0a^T and dSs^T ([column][channel]); after the key-side products the
  // log-decay gradients and the carry terms (S0a region) and the decays
  // (dSs region). R and dZ hold lambda (fp32 [C][D]) while the operands are
  // built.
  alignas(16) BF S0a[D * D], dSs[D * D];
  alignas(16) BF Akk[kC * kC], Mqk[kC * kC], Mqb[kC * kC], Lb[kC * kC];
  alignas(16) BF dMqk[kC * kC], dMqb[kC * kC], dAkk[kC * kC], dAkb[kC * kC];
  alignas(16) float Akb[kC][kC];
  alignas(16) float A[D], gCA[D], gC[D], rs[8][D];
  float beta8[8][kC];  // coupled forms: d(beta) per wave and token
};

struct GradParams {
  const uint16_t *q, *k, *v, *dO;
  const void *a, *b, *w;  // in the gate form's layout
  const BF *cst, *dst;
  uint16_t *dq, *dk, *dv;
  void *da, *db, *dw;  // likewise (coupled forms: db is d(beta); scalar: da is d(alpha))
  int T, H_qk, H_v, nch;
};

// GRP: several value heads per query/key head (G = H_v / H_qk > 1, looped
// over); the G = 1 instance has no loop, so nothing is kept across heads.
// GF: the gate form (kGate*).
template <int D, bool GRP, int GF>
__global__ __launch_bounds__(512) void bwd_grad_kernel(GradParams p) {
  static_assert(D == 128, "d = 128");
  constexpr bool CPL = GF == kGateCoupled || GF == kGateScalar, SCA = GF == kGateScalar;
  constexpr int NT = 512;
  static_assert(NT / 64 == D / 16, "one wave per 16 columns");
  __shared__ GradSmem<D> sm;
  static_assert(sizeof(GradSmem<D>::R) + sizeof(GradSmem<D>::dZ) == kC * D * 4, "R, dZ hold lambda");
  float *const lam0 = reinterpret_cast<float *>(sm.R);            // [C][D], over R and dZ
  float *const dgF = reinterpret_cast<float *>(sm.S0a);           // [C][D]
  float *const crF = reinterpret_cast<float *>(sm.S0a) + kC * D;  // [C][D]
  float *const aE = reinterpret_cast<float *>(sm.dSs);            // [C][D]
  float *const daS = reinterpret_cast<float *>(sm.dSs) + kC * D;  // [C][D], scalar decay: da per channel
  const int chunk = blockIdx.x % p.nch, ug = blockIdx.x / p.nch;  // ug = n * H_qk + gq
  const int n = ug / p.H_qk, gq = ug - n * p.H_qk;
  const int G = GRP ? p.H_v / p.H_qk : 1;
  const int t0 = chunk * kC, Tc = min(kC, p.T - t0);
  const size_t tok0 = (size_t)n * p.T + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const size_t qk_row = (size_t)p.H_qk * D, v_row = (size_t)p.H_v * D;
  const int nb = wave, ib = wave;  // this wave's 16-column blocks

  // dq, dk summed over the group's value heads; tiles (tb, ib)
  floatx4 dq[2] = {zero4(), zero4()}, dk[2] = {zero4(), zero4()};
  BWD_TIMER_INIT

  // One value head: a lambda so that, with several heads, the thread's
  // indices can be made opaque per head (otherwise the addresses derived
  // from them are hoisted out of the loop and held across it, in scratch).
  auto head = [&](const int hv, const int tid, const int c, const int g) __attribute__((always_inline)) {
    const int lane = tid & 63, wave = tid >> 6;
    const int nb = wave, ib = wave;
    const int h = gq * G + hv;
    const size_t unit = (size_t)n * p.H_v + h;
    // ---- every request of the chunk first, the decays first of all (the
    // first wait is for them only): decays, q, k, b, v, w, dO (rows past
    // the end read the last row and are replaced), then the entering state
    // and the exiting adjoint
    constexpr int NQ = kC * D / 4 / NT, NS = D * D / 4 / NT;
    floatx4 av[NQ], bv[NQ], wv[NQ];
    Fr qv[NQ], kv[NQ], vv[NQ], ov[NQ], s0v[NS], dsv[NS];
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + NT * it, t = quad_t<D>(e), i4 = quad_i<D>(e);
      av[it] = gate_a4<GF, D>(p.a, (tok0 + min(t, Tc - 1)) * p.H_v + h, i4);
    }
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + NT * it, t = quad_t<D>(e), i4 = quad_i<D>(e);
      const size_t row = tok0 + min(t, Tc - 1), off = row * v_row + (size_t)h * D + i4;
      bv[it] = gate_bw4<GF, D>(p.b, p.b, row * p.H_v + h, i4);
      wv[it] = gate_bw4<GF, D>(p.w, p.b, row * p.H_v + h, i4);
      qv[it] = *reinterpret_cast<const Fr *>(p.q + row * qk_row + (size_t)gq * D + i4);
      kv[it] = *reinterpret_cast<const Fr *>(p.k + row * qk_row + (size_t)gq * D + i4);
      vv[it] = *reinterpret_cast<const Fr *>(p.v + off);
      ov[it] = *reinterpret_cast<const Fr *>(p.dO + off);
    }
    {
      const BF *s0 = p.cst + (unit * (p.nch + 1) + chunk) * D * D;
      const BF *ds = p.dst + (unit * p.nch + chunk) * D * D;
#pragma unroll
      for (int it = 0; it < NS; ++it) {
        const int e = tid + NT * it;
        s0v[it] = *reinterpret_cast<const Fr *>(s0 + 4 * e);
        dsv[it] = *reinterpret_cast<const Fr *>(ds + 4 * e);
      }
    }
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      if (quad_t<D>(tid + NT * it) >= Tc) {
        av[it] = floatx4{1.f, 1.f, 1.f, 1.f};
        bv[it] = wv[it] = zero4();
        qv[it] = kv[it] = vv[it] = ov[it] = OB::zero();
      }
    }
    // ---- lambda (the chunk's anchor: at its start or its middle; chunks
    // that need neither do not reach this kernel), then the operands
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + NT * it;
      *reinterpret_cast<floatx4 *>(&lam0[quad_t<D>(e) * D + quad_i<D>(e)]) = av[it];
    }
    __syncthreads();
    BWD_MARK(0);
    lambda_scan<D>(lam0, lam0, sm.A, sm.gC, sm.gCA, tid);
    BWD_MARK(1);
    // lambda at this lane's positions of the key-side tiles (for dq, dk, db)
    float lq[2][4];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) lq[tb][j] = lam0[(16 * tb + 4 * g + j) * D + 16 * ib + c];
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + NT * it, t = quad_t<D>(e), i4 = quad_i<D>(e);
      const floatx4 lam = *reinterpret_cast<const floatx4 *>(&lam0[t * D + i4]), mu = rcp4(lam);
      const floatx4 q4 = fr_f32(qv[it]), k4 = fr_f32(kv[it]);
      st_bf4(&sm.Ql[sx<D>(t, i4)], lam * q4);
      st_bf4(&sm.Kl[sx<D>(t, i4)], lam * k4);
      st_bf4(&sm.Km[sx<D>(t, i4)], mu * k4);
      st_bf4(&sm.Bm[sx<D>(t, i4)], mu * bv[it] * k4);
      st_bf4(&sm.U[sx<D>(t, i4)], fr_f32(vv[it]) * wv[it]);
      *reinterpret_cast<Fr *>(&sm.dO[sx<D>(t, i4)]) = ov[it];
    }
    // S0a = diag(A) S0 and dSs = diag(gamma_C / A) dS_C, both [column][channel];
    // rs[i] = sum_j dS_C S0 over this thread's columns (then over the lane
    // pair 32 apart, whose quads are the same channels)
    {
      const int i4 = 4 * (tid % (D / 4));
      const floatx4 Av = *reinterpret_cast<const floatx4 *>(&sm.A[i4]);
      const floatx4 Gv = *reinterpret_cast<const floatx4 *>(&sm.gCA[i4]);
      floatx4 rsum = zero4();
#pragma unroll
      for (int it = 0; it < NS; ++it) {
        const int e = tid + NT * it;
        const floatx4 sv = fr_f32(s0v[it]), dv = fr_f32(dsv[it]);
        rsum += sv * dv;
        st_bf4(&sm.S0a[sx<D>(quad_t<D>(e), i4)], sv * Av);
        st_bf4(&sm.dSs[sx<D>(quad_t<D>(e), i4)], dv * Gv);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) rsum[j] += __shfl_xor(rsum[j], 32);
      if ((lane & 32) == 0) *reinterpret_cast<floatx4 *>(&sm.rs[tid / (D / 2)][i4]) = rsum;
    }
    __syncthreads();
    BWD_MARK(2);
    // ---- Gram tiles (three lower 16x16 tiles of each; the upper one is zero)
    for (int tile = wave; tile < 12; tile += NT / 64) {
      const int mat = tile / 3, tt = tile % 3;
      const int tb = tt == 0 ? 0 : 1, sb = tt == 2 ? 1 : 0;
      const BF *L = mat < 2 ? sm.Kl : sm.Ql;  // Akk, Akb | Mqk, Mqb
      const BF *Rt = (mat & 1) ? sm.Bm : sm.Km;
      floatx4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32)
        acc = mma(acc, op_rows<D>(L, 16 * tb, k0, c, g), op_rows<D>(Rt, 16 * sb, k0, c, g));
      const bool strict = mat < 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * tb + 4 * g + j, s = 16 * sb + c;
        const float x = (strict ? s < t : s <= t) ? acc[j] : 0.f;
        if (mat == 1) {
          sm.Akb[t][s] = x;
        } else {
          BF *M = mat == 0 ? sm.Akk : mat == 2 ? sm.Mqk : sm.Mqb;
          M[sx<kC>(t, s)] = (BF)x;
          M[sx<kC>(t & 15, 16 + (s & 15))] = (BF)0.f;
        }
      }
    }
    __syncthreads();
    BWD_MARK(3);
    unit_lower_inverse(sm.Akb, sm.Lb, tid);
    BWD_MARK(4);

    // coupled forms: this lane's part of d(beta) for its 8 tokens
    float bsum[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // ---- value side (columns 16 nb ..)
    {
      const int jc = 16 * nb + c;
      float wq[2][4], vq[2][4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * tb + 4 * g + j;
          const size_t row = tok0 + min(t, Tc - 1);
          wq[tb][j] = gate_bw1<GF, D>(p.w, p.b, row * p.H_v + h, jc);
          vq[tb][j] = bf16_to_f32(p.v[row * v_row + (size_t)h * D + jc]);
        }
      floatx4 Z[2], dR[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        floatx4 z = zero4(), r = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32) {
          z = mma(z, op_rows<D>(sm.Kl, 16 * tb, k0, c, g), op_rows<D>(sm.S0a, 16 * nb, k0, c, g));
          r = mma(r, op_rows<D>(sm.Bm, 16 * tb, k0, c, g), op_rows<D>(sm.dSs, 16 * nb, k0, c, g));
        }
        z = mma(z, op_rows<kC>(sm.Akk, 16 * tb, 0, c, g), op_cols<D>(sm.U, 16 * nb, 0, c, g));
        r = mma(r, op_cols<kC>(sm.Mqb, 16 * tb, 0, c, g), op_cols<D>(sm.dO, 16 * nb, 0, c, g));
        Z[tb] = z;
        dR[tb] = -r;
      }
      const P2 Zf = acc_pair(Z[0], Z[1]), dRf = acc_pair(dR[0], dR[1]);
      floatx4 Rr[2], dZr[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        Rr[tb] = mma(zero4(), op_rows<kC>(sm.Lb, 16 * tb, 0, c, g), Zf);
        dZr[tb] = mma(zero4(), op_cols<kC>(sm.Lb, 16 * tb, 0, c, g), dRf);
      }
      const P2 dZf = acc_pair(dZr[0], dZr[1]);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        floatx4 u = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 32)
          u = mma(u, op_rows<D>(sm.Km, 16 * tb, k0, c, g), op_rows<D>(sm.dSs, 16 * nb, k0, c, g));
        u = mma(u, op_cols<kC>(sm.Mqk, 16 * tb, 0, c, g), op_cols<D>(sm.dO, 16 * nb, 0, c, g));
        u = mma(u, op_cols<kC>(sm.Akk, 16 * tb, 0, c, g), dZf);
        // dv = w dU, dw = v dU
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * tb + 4 * g + j;
          if (t < Tc) {
            const size_t off = (tok0 + t) * v_row + (size_t)h * D + jc;
            p.dv[off] = f32_to_bf16(wq[tb][j] * u[j]);
            if constexpr (CPL)
              bsum[tb][j] = vq[tb][j] * u[j];
            else
              put_gate_grad<GF>(p.dw, off, vq[tb][j] * u[j], wq[tb][j], false);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * tb + 4 * g + j;
          sm.R[sx<D>(t, jc)] = (BF)Rr[tb][j];
          sm.dZ[sx<D>(t, jc)] = (BF)dZr[tb][j];
        }
      }
    }
    __syncthreads();
    BWD_MARK(5);

    // ---- key side (channels 16 ib ..). Requested first: the decays again
    // (for lambda and da at the end), b and k at this lane's positions
    floatx4 av2[NQ];
    float bq[2][4], kq[2][4];
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + NT * it, t = quad_t<D>(e), i4 = quad_i<D>(e);
      av2[it] = floatx4{1.f, 1.f, 1.f, 1.f};
      if (t < Tc) av2[it] = gate_a4<GF, D>(p.a, (tok0 + t) * p.H_v + h, i4);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * tb + 4 * g + j, i = 16 * ib + c;
        const size_t row = tok0 + min(t, Tc - 1);
        bq[tb][j] = t < Tc ? gate_bw1<GF, D>(p.b, p.b, row * p.H_v + h, i) : 0.f;
        kq[tb][j] = t < Tc ? bf16_to_f32(p.k[row * qk_row + (size_t)gq * D + i]) : 0.f;
      }
    floatx4 dQl[2], dKl[2], dKm[2], dBm[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      floatx4 a0 = zero4(), a1 = zero4(), a2 = zero4(), a3 = zero4();
#pragma unroll 2
      for (int k0 = 0; k0 < D; k0 += 32) {
        const P2 s0 = op_cols<D>(sm.S0a, 16 * ib, k0, c, g), ds = op_cols<D>(sm.dSs, 16 * ib, k0, c, g);
        a0 = mma(a0, op_rows<D>(sm.dO, 16 * tb, k0, c, g), s0);
        a1 = mma(a1, op_rows<D>(sm.dZ, 16 * tb, k0, c, g), s0);
        a2 = mma(a2, op_rows<D>(sm.U, 16 * tb, k0, c, g), ds);
        a3 = mma(a3, op_rows<D>(sm.R, 16 * tb, k0, c, g), ds);
      }
      dQl[tb] = a0;
      dKl[tb] = a1;
      dKm[tb] = a2;
      dBm[tb] = -a3;
    }
    // adjoints of the Gram matrices (lower tiles)
    for (int tile = wave; tile < 12; tile += NT / 64) {
      const int mat = tile / 3, tt = tile % 3;
      const int tb = tt == 0 ? 0 : 1, sb = tt == 2 ? 1 : 0;
      const BF *L = mat < 2 ? sm.dO : sm.dZ;  // dMqk, dMqb | dAkk, dAkb
      const BF *Rt = (mat & 1) ? sm.R : sm.U;
      floatx4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32)
        acc = mma(acc, op_rows<D>(L, 16 * tb, k0, c, g), op_rows<D>(Rt, 16 * sb, k0, c, g));
      const bool strict = mat >= 2;
      const float sg = (mat & 1) ? -1.f : 1.f;
      BF *M = mat == 0 ? sm.dMqk : mat == 1 ? sm.dMqb : mat == 2 ? sm.dAkk : sm.dAkb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * tb + 4 * g + j, s = 16 * sb + c;
        M[sx<kC>(t, s)] = (BF)((strict ? s < t : s <= t) ? sg * acc[j] : 0.f);
        M[sx<kC>(t & 15, 16 + (s & 15))] = (BF)0.f;
      }
    }
    __syncthreads();
    BWD_MARK(6);
    // carry terms of the log-decay gradient (before the Gram parts are
    // added), the Gram parts, then the log-decay gradient per token with
    // the same bf16 operands as the products
    {
      const P2 km0 = op_cols<D>(sm.Km, 16 * ib, 0, c, g), bm0 = op_cols<D>(sm.Bm, 16 * ib, 0, c, g);
      const P2 ql0 = op_cols<D>(sm.Ql, 16 * ib, 0, c, g), kl0 = op_cols<D>(sm.Kl, 16 * ib, 0, c, g);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const floatx4 ql = fr_f32(tr_frag<D>(sm.Ql, 16 * tb, 16 * ib, c, g));
        const floatx4 kl = fr_f32(tr_frag<D>(sm.Kl, 16 * tb, 16 * ib, c, g));
        const floatx4 km = fr_f32(tr_frag<D>(sm.Km, 16 * tb, 16 * ib, c, g));
        const floatx4 bm = fr_f32(tr_frag<D>(sm.Bm, 16 * tb, 16 * ib, c, g));
        const floatx4 cr = km * dKm[tb] + bm * dBm[tb];
        dQl[tb] = mma(mma(dQl[tb], op_rows<kC>(sm.dMqk, 16 * tb, 0, c, g), km0),
                      op_rows<kC>(sm.dMqb, 16 * tb, 0, c, g), bm0);
        dKl[tb] = mma(mma(dKl[tb], op_rows<kC>(sm.dAkk, 16 * tb, 0, c, g), km0),
                      op_rows<kC>(sm.dAkb, 16 * tb, 0, c, g), bm0);
        dKm[tb] = mma(mma(dKm[tb], op_cols<kC>(sm.dMqk, 16 * tb, 0, c, g), ql0),
                      op_cols<kC>(sm.dAkk, 16 * tb, 0, c, g), kl0);
        dBm[tb] = mma(mma(dBm[tb], op_cols<kC>(sm.dMqb, 16 * tb, 0, c, g), ql0),
                      op_cols<kC>(sm.dAkb, 16 * tb, 0, c, g), kl0);
        const floatx4 dg = ql * dQl[tb] + kl * dKl[tb] - km * dKm[tb] - bm * dBm[tb];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int o = (16 * tb + 4 * g + j) * D + 16 * ib + c;
          crF[o] = cr[j];
          dgF[o] = dg[j];
        }
      }
    }
    // the decays (for da; the dSs region is free)
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + NT * it;
      *reinterpret_cast<floatx4 *>(&aE[quad_t<D>(e) * D + quad_i<D>(e)]) = av2[it];
    }
    __syncthreads();
    BWD_MARK(7);
    // dq, dk (summed over the group), db
    {
      const int i = 16 * ib + c;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * tb + 4 * g + j;
          const float lam = lq[tb][j], mu = __builtin_amdgcn_rcpf(lam);
          dq[tb][j] += lam * dQl[tb][j];
          dk[tb][j] += lam * dKl[tb][j] + mu * (dKm[tb][j] + bq[tb][j] * dBm[tb][j]);
          if (t < Tc) {
            const float dbv = mu * kq[tb][j] * dBm[tb][j];
            if constexpr (CPL)
              bsum[tb][j] += dbv;
            else
              put_gate_grad<GF>(p.db, (tok0 + t) * v_row + (size_t)h * D + i, dbv, bq[tb][j], false);
          }
        }
      }
    }
    // da: reverse sums of the log-decay gradient over the chunk; the chunk's
    // end carries the exiting state's term and the carry terms
    if (tid < D) {
      const int i = tid;
      float acc = 0.f;
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) acc += sm.rs[r8][i];
      acc *= sm.gC[i];
      // in blocks of 8 tokens: the reads of a block are issued together
#pragma unroll 1
      for (int t0 = 0; t0 < kC; t0 += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = crF[(t0 + k) * D + i];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc += v[k];
      }
#pragma unroll 1
      for (int t0 = kC - 8; t0 >= 0; t0 -= 8) {
        float dg8[8], a8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          dg8[k] = dgF[(t0 + k) * D + i];
          a8[k] = aE[(t0 + k) * D + i];
        }
#pragma unroll
        for (int k = 7; k >= 0; --k) {
          acc += dg8[k];
          const int t = t0 + k;
          if (t < Tc) {
            const float dav = acc * __builtin_amdgcn_rcpf(a8[k]);
            if constexpr (SCA)
              daS[t * D + i] = dav;  // summed over the channels below
            else
              put_gate_grad<GF>(p.da, (tok0 + t) * v_row + (size_t)h * D + i, dav, a8[k], true);
          }
        }
      }
    }
    // coupled forms: d(beta) of this lane's tokens summed over the wave's 16
    // columns (write side) and 16 channels (erase side), then over the waves
    if constexpr (CPL) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = bsum[tb][j];
          x += __shfl_xor(x, 8, 16);
          x += __shfl_xor(x, 4, 16);
          x += __shfl_xor(x, 2, 16);
          x += __shfl_xor(x, 1, 16);
          if (c == 0) sm.beta8[wave][16 * tb + 4 * g + j] = x;
        }
    }
    __syncthreads();
    if constexpr (CPL) {
      if (tid < Tc) {
        float sb = 0.f;
#pragma unroll
        for (int w8 = 0; w8 < 8; ++w8) sb += sm.beta8[w8][tid];
        static_cast<float *>(p.db)[(tok0 + tid) * p.H_v + h] = sb;
      }
    }
    if constexpr (SCA) {  // d(alpha): da summed over the channels
      if (tid < Tc) {
        float sa = 0.f;
        for (int i = 0; i < D; ++i) sa += daS[tid * D + i];
        static_cast<float *>(p.da)[(tok0 + tid) * p.H_v + h] = sa;
      }
    }
    BWD_MARK(9);
    if (hv == G - 1) {  // dq, dk
      const int i = 16 * ib + c;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * tb + 4 * g + j;
          if (t < Tc) {
            const size_t off = (tok0 + t) * qk_row + (size_t)gq * D + i;
            p.dq[off] = f32_to_bf16(dq[tb][j]);
            p.dk[off] = f32_to_bf16(dk[tb][j]);
          }
        }
    }
  };
  if constexpr (GRP) {
    for (int hv = 0; hv < G; ++hv) {
      int tid_h = tid, c_h = c, g_h = g;
      asm volatile("" : "+v"(tid_h), "+v"(c_h), "+v"(g_h));
      head(hv, tid_h, c_h, g_h);
    }
  } else {
    head(0, tid, c, g);
  }
  BWD_MARK(10);
  BWD_TIMER_STORE
}

}  // namespace

// ---------------------------------------------------------------- host
bool backward_chunked_eligible(const BackwardArgs &a) {
  if (a.cu_seqlens || !a.bf16 || a.d_k != 128 || a.d_v != 128) return false;
  if (a.B <= 0 || a.T <= 0 || a.H_v % a.H_qk != 0) return false;
  PrefillArgs fa{};
  fa.B = a.B; fa.T = a.T; fa.H_qk = a.H_qk; fa.H_v = a.H_v; fa.d_k = a.d_k; fa.d_v = a.d_v;
  fa.chunk = 64;
  fa.bf16 = true;
  fa.nct = prefill_pick_nct(a.B, a.H_v, a.d_v);
  fa.force_nseg = 1;
  return prefill_plan(fa).chunk == kC;
}

size_t backward_chunked_workspace_bytes(int B, int T, int H_qk, int H_v) {
  return chunk_layout<128>(B, T, H_qk, H_v).total;
}

// Runs the chunk-form backward. *ran = false (and nothing written but the
// workspace) when some chunk decays too fast for its anchors: the caller
// then runs the per-token backward. Synchronises the stream once (after the
// chunk operands) to read that flag.
hipError_t launch_backward_chunked(const BackwardArgs &a, hipStream_t st, bool *ran) {
  constexpr int D = 128;
  *ran = false;
  const ChunkLayout l = chunk_layout<D>(a.B, a.T, a.H_qk, a.H_v);
  char *w = static_cast<char *>(a.workspace);
  BF *cst = reinterpret_cast<BF *>(w + l.cst);
  BF *dst = reinterpret_cast<BF *>(w + l.dst);
  BF *prep = reinterpret_cast<BF *>(w + l.prep);
  float *gc = reinterpret_cast<float *>(w + l.gc);
  int *flag = reinterpret_cast<int *>(w + l.flag);
  const int units = a.B * a.H_v;

  hipError_t e = hipMemsetAsync(flag, 0, sizeof(int), st);
  if (e != hipSuccess) return e;
  // 1. the states entering every chunk
  PrefillArgs fa = cst_prefill_args(a.B, a.T, a.H_qk, a.H_v);
  const bool coupled = a.gate_form == kGateCoupled || a.gate_form == kGateScalar;
  fa.q = a.q; fa.k = a.k; fa.v = a.v; fa.a = a.a; fa.b = a.b; fa.w = coupled ? a.b : a.w; fa.S0 = a.S0;
  fa.coupled = coupled;
  fa.scalar_decay = a.gate_form == kGateScalar;
  fa.preact = a.gate_form == kGatePre;
  if (l.seg.nseg > 1) {
    // the state entering every segment (the prefill split's first two passes)
    float *trans = reinterpret_cast<float *>(w + l.trans);
    float *segst = reinterpret_cast<float *>(w + l.segst);
    float *sin = reinterpret_cast<float *>(w + l.sin);
    fa.force_nseg = l.seg.req;
    fa.seg_states = segst;
    fa.workspace = trans;
    fa.workspace_bytes = l.segst - l.trans;
    const PrefillPlan pl = prefill_plan(fa);
    if (pl.nseg != l.seg.nseg || pl.seg_len != l.seg.seg_len) return hipErrorInvalidValue;
    if ((e = launch_prefill(fa, st)) != hipSuccess) return e;
    if ((e = launch_split_states(sin, a.S0, segst, a.B, a.H_v, l.seg.nseg, D * D, st)) != hipSuccess) return e;
    // every segment from its entering state, as B * nseg sequences
    fa.B = a.B * l.seg.nseg;
    fa.T = l.seg.seg_len;
    fa.nct = prefill_pick_nct(fa.B, a.H_v, a.d_v);
    fa.S0 = sin;
    fa.seg_states = nullptr;
    fa.workspace = nullptr;
    fa.workspace_bytes = 0;
    fa.cst_segs = l.seg.nseg;
  }
  fa.force_nseg = 1;
  fa.chunk_states = cst;
  e = launch_prefill(fa, st);
  if (e != hipSuccess) return e;
  // 2. chunk operands of the state's adjoint
  PrepParams pp{};
  pp.q = static_cast<const uint16_t *>(a.q); pp.k = static_cast<const uint16_t *>(a.k);
  pp.a = a.a; pp.b = a.b;
  pp.prep = prep; pp.gc = gc; pp.flag = flag;
  pp.T = a.T; pp.H_qk = a.H_qk; pp.H_v = a.H_v; pp.nch = l.nch;
  switch (a.gate_form) {
    case kGatePre: hipLaunchKernelGGL((bwd_prep_kernel<D, kGatePre>), dim3(units * l.nch), dim3(256), 0, st, pp); break;
    case kGateCoupled:
      hipLaunchKernelGGL((bwd_prep_kernel<D, kGateCoupled>), dim3(units * l.nch), dim3(256), 0, st, pp);
      break;
    case kGateScalar:
      hipLaunchKernelGGL((bwd_prep_kernel<D, kGateScalar>), dim3(units * l.nch), dim3(256), 0, st, pp);
      break;
    default: hipLaunchKernelGGL((bwd_prep_kernel<D, kGateGeneral>), dim3(units * l.nch), dim3(256), 0, st, pp);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int hflag = 0;
  if ((e = hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
  if (hflag) return hipSuccess;
  // 3. the state's adjoint at every chunk boundary, and dS0
  DstParams dp{};
  dp.prep = prep; dp.gc = gc;
  dp.dO = static_cast<const uint16_t *>(a.dO);
  dp.dST = a.dST; dp.dS0 = a.dS0; dp.dst = dst;
  dp.T = a.T; dp.H_v = a.H_v; dp.nch = l.nch; dp.units = units;
  dp.seg_chunks = l.nch;
  dp.dst_all = true;
  constexpr int NCB = D / 64;
  if (l.seg.nseg > 1) {
    // segments swept at once in reverse (the states' regions are free now):
    // 1. segments 1 .. nseg - 1 from a zero exiting adjoint (the last from
    //    dS_T, storing its chunks' adjoints), ending in L[nseg - 1 - s], and
    //    the maps M[nseg - 1 - s] of segments 1 .. nseg - 2;
    // 2. L[j] = M[j] L[j - 1] + L[j] for j = 1 .. nseg - 2: L[nseg - 2 - s]
    //    is then the exact adjoint leaving segment s;
    // 3. segments 0 .. nseg - 2 from those, storing their chunks' adjoints
    //    (segment 0 also dS0).
    const int ns = l.seg.nseg;
    float *M = reinterpret_cast<float *>(w + l.trans), *L = reinterpret_cast<float *>(w + l.segst);
    dp.seg_chunks = l.seg.seg_len / kC;
    dp.seg_first = 1;
    dp.ncb_id = NCB;
    dp.out_base = ns - 1;
    dp.dst_all = false;
    dp.L_out = L; dp.M_out = M;
    hipLaunchKernelGGL(bwd_dstate_kernel<D>, dim3((ns - 1) * units * 2 * NCB), dim3(256), 0, st, dp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ns > 2 && (e = launch_split_combine(L, M, ns - 2, units, D, D, nullptr, st)) != hipSuccess) return e;
    dp.seg_first = 0;
    dp.ncb_id = 0;
    dp.dS_in = L; dp.in_base = ns - 2;
    dp.dst_all = true;
    dp.L_out = nullptr; dp.M_out = nullptr;
    hipLaunchKernelGGL(bwd_dstate_kernel<D>, dim3((ns - 1) * units * NCB), dim3(256), 0, st, dp);
  } else {
    hipLaunchKernelGGL(bwd_dstate_kernel<D>, dim3(units * NCB), dim3(256), 0, st, dp);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 4. the gradients
  GradParams gp{};
  gp.q = static_cast<const uint16_t *>(a.q); gp.k = static_cast<const uint16_t *>(a.k);
  gp.v = static_cast<const uint16_t *>(a.v); gp.dO = static_cast<const uint16_t *>(a.dO);
  gp.a = a.a; gp.b = a.b; gp.w = a.w;
  gp.cst = cst; gp.dst = dst;
  gp.dq = static_cast<uint16_t *>(a.dq); gp.dk = static_cast<uint16_t *>(a.dk);
  gp.dv = static_cast<uint16_t *>(a.dv);
  gp.da = a.da; gp.db = a.db; gp.dw = a.dw;
  gp.T = a.T; gp.H_qk = a.H_qk; gp.H_v = a.H_v; gp.nch = l.nch;
  const dim3 ggrid(a.B * a.H_qk * l.nch), gblock(512);
  const bool grp = a.H_v != a.H_qk;
  switch (a.gate_form) {
    case kGatePre:
      if (grp) hipLaunchKernelGGL((bwd_grad_kernel<D, true, kGatePre>), ggrid, gblock, 0, st, gp);
      else hipLaunchKernelGGL((bwd_grad_kernel<D, false, kGatePre>), ggrid, gblock, 0, st, gp);
      break;
    case kGateCoupled:
      if (grp) hipLaunchKernelGGL((bwd_grad_kernel<D, true, kGateCoupled>), ggrid, gblock, 0, st, gp);
      else hipLaunchKernelGGL((bwd_grad_kernel<D, false, kGateCoupled>), ggrid, gblock, 0, st, gp);
      break;
    case kGateScalar:
      if (grp) hipLaunchKernelGGL((bwd_grad_kernel<D, true, kGateScalar>), ggrid, gblock, 0, st, gp);
      else hipLaunchKernelGGL((bwd_grad_kernel<D, false, kGateScalar>), ggrid, gblock, 0, st, gp);
      break;
    default:
      if (grp) hipLaunchKernelGGL((bwd_grad_kernel<D, true, kGateGeneral>), ggrid, gblock, 0, st, gp);
      else hipLaunchKernelGGL((bwd_grad_kernel<D, false, kGateGeneral>), ggrid, gblock, 0, st, gp);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  *ran = true;
  return hipSuccess;
}

#ifdef GDN2_BWD_TIMING
extern "C" int gdn2_bwd_cycles_read(unsigned long long *host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn2_bwd_cycles), sizeof(gdn2_bwd_cycles));
}
#endif

}  // namespace gdn2
