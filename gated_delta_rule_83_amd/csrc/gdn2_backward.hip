// gdn2_backward.hip -- gradients of the Gated DeltaNet-2 recurrence (the
// backward pass of gdn2_chunk_forward, for training).
//
// Forward step per (sequence n, value head h), for every value column j
// (Gated DeltaNet-2 post on tilnote.io, GDN-2 design section; delta-rule
// tutorial on ai-systems-engineering.com, "record the difference" and
// key-versus-query sections):
//   Sd = diag(a_t) S_{t-1};  r_j = k_t . Sd[:, j];
//   S_t[:, j] = Sd[:, j] - r_j e_t + u_j k_t   (e = b*k, u = w*v);
//   o_t[j] = q_t . S_t[:, j].
// Value columns never mix, so each column's d_k-vector state, and its
// adjoint L = dLoss/dS[:, j], can be run alone; key-side gradients (dq, dk,
// da, db) sum over the columns. Reverse mode, from the last token to the
// first (L starts at dS_T):
//   dq_t += S_t[:, j] dO_t[j];                L += q_t dO_t[j]
//   du_j = k_t . L  -> dv = du w, dw = du v;  dr_j = -(e_t . L)
//   de -= L r_j  -> db = de*k, dk += de*b;    dk += u_j L + dr_j Sd[:, j]
//   L += dr_j k_t;  da_t += L * S_{t-1}[:, j];  L = a_t * L
// and dS0[:, j] = L at the end.
//
// MI355X design: this is a per-token recurrence with two 16-lane key
// reductions per token and column, so it runs on the vector ALUs, not the
// matrix cores. One workgroup per (n, h, block of CB value columns, 64
// when d_v allows): one wave per 8 columns; lane = (column pair c4,
// key group kg) holds columns 2*c4, 2*c4+1 of its wave on the key channels
// kg*KPL .. +KPL. Key sums (k-read, du, dr) are DPP rotations within a
// 16-lane row; key-side gradient sums over the wave's columns are a
// two-step reduce-scatter across the four column pairs, then a fixed-order
// sum over the waves in LDS (deterministic, no atomics).
//
// Memory: phase 1 runs the recurrence forward in 16-token stages and stores
// the state at the start of every kSub-token sub-segment and every token's
// k-read (fp32, in the workspace); phase 2 walks the sub-segments backward,
// rebuilds a sub-segment's kSub + 1 states into registers from its
// checkpoint and the stored k-reads (no key sums), and runs the adjoint over
// it. Inputs of a stage or sub-segment are staged in LDS (one set of loads
// per workgroup, requested one stage or sub-segment ahead). Key-side sums go to the
// workspace per column block and are added up by backward_reduce_kernel,
// which also sums the value heads that share a query/key head.
#include "gdn2_device.hpp"
#include "gdn2_internal.hpp"

#ifndef GDN2_BWD_BF16
#error "build with -DGDN2_BWD_BF16=0 or 1"
#endif

namespace gdn2 {

hipError_t launch_backward_bf16(const BackwardParams &p, int d_k, hipStream_t st);

// Adjoint-only sweep of a split backward (see adjoint_sweep_kernel).
struct SweepParams {
  const void *q, *k, *a, *b, *dO;
  const float *dST;  // [B][H_v][d_k][d_v] or null (zero)
  float *Lout;       // [B * nseg][H_v][d_k][d_v]: exiting adjoint of segment j of sequence n at n * nseg + j
  int B, T, H_qk, H_v, d_v, nseg, seg_len;
};
hipError_t launch_sweep_bf16(const SweepParams &p, int d_k, int form, hipStream_t st);

namespace {

constexpr int kSub = 4;  // tokens per sub-segment (the register history)

// Value columns per workgroup (one wave per 8): 64 when d_v allows.
__host__ __device__ constexpr int bwd_cb(int d_v) { return d_v >= 64 ? 64 : d_v >= 32 ? 32 : 16; }

template <int DK, int CB>
struct BwdCfg {
  static constexpr int NWV = CB / 8;   // waves, 8 value columns each
  static constexpr int NT = 64 * NWV;  // threads
  static constexpr int KPL = DK / 16;  // key channels per lane
  static constexpr int L = kSub;
  static constexpr int L1 = 16;                           // tokens per forward-phase stage
  static constexpr int NKS = L * DK / 4;                  // key quads staged per sub-segment
  static constexpr int KIT = (NKS + NT - 1) / NT;         // ... per thread
  static constexpr int NCS = L * CB / 4;                  // column quads staged per sub-segment
  static constexpr int NKS1 = L1 * DK / 4;                // ... per forward-phase stage
  static constexpr int KIT1 = (NKS1 + NT - 1) / NT;
  static constexpr int NCS1 = L1 * CB / 4;
  static_assert(NCS <= NT && NCS1 <= NT, "one column quad per thread at most");
  static_assert(L1 % L == 0, "checkpoints at sub-segment starts");
  static_assert(CB == 16 || CB == 32 || CB == 64, "column block");
};

template <int DK, int CB>
struct BwdSmem {
  using Cf = BwdCfg<DK, CB>;
  union {
    struct {  // forward phase: one L1-token stage
      alignas(16) float kae[Cf::L1][3][DK];         // k, a, e = b*k
      alignas(16) float u[Cf::L1][CB];              // u = w*v of the workgroup's columns
      alignas(16) float r[Cf::L1][CB];              // k-reads of the stage, written out as rows
    } f;
    struct {  // backward phase: one sub-segment
      alignas(16) float kqae[Cf::L][4][DK];         // k, q, a, e = b*k of the sub-segment's tokens
      alignas(16) float col[Cf::L][5][CB];          // u = w*v, v, w, dO, k-read r of the block's columns
      alignas(16) float red[Cf::NWV][Cf::L][4][DK]; // per-wave key-side sums (dq, dk part, e part, da)
      alignas(16) float du[Cf::L][CB];              // du per token and column
    } b;
  };
};

// Sums over the 16 lanes of the row, of two or four independent values at
// once: x += (x from lane (l + R) mod 16) for R = 8, 4, 2, 1 (DPP row_ror),
// every lane ending with the same value (each step adds two values that are
// equal in both lanes of a rotation pair). One asm block interleaves the
// chains, so that the wait a DPP read needs after the VALU write of its
// source is filled by the other chains (four chains: three instructions
// apart; two chains: one s_nop per round); the leading s_nop covers the
// writes before the block, which the compiler does not see through it.
__device__ __forceinline__ void row_sum16x4(float &x0, float &x1, float &x2, float &x3) {
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %3, %3, %3 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %2, %2 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %3, %3, %3 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %2, %2 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %3, %3, %3 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %2, %2 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %3, %3, %3 row_ror:1 row_mask:0xf bank_mask:0xf"
      : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
}
__device__ __forceinline__ void row_sum16x2(float &x0, float &x1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 0\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %1, %1 row_ror:1 row_mask:0xf bank_mask:0xf"
      : "+v"(x0), "+v"(x1));
}
// One value: the same rotations, two wait states before each (s_nop 1).
__device__ __forceinline__ void row_sum16x1(float &x) {
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf"
      : "+v"(x));
}

// Lane exchange of the column reduce-scatter (gfx950 v_permlane32_swap /
// v_permlane16_swap), N pairs at once: after swap32(A, B), A holds
// [A lanes 0-31, B lanes 0-31] and B [A lanes 32-63, B lanes 32-63] (swap16
// likewise between rows 0/1 and 2/3), so A + B is, in the lower half, A plus
// the upper half's A, and in the upper half B plus the lower half's B.
// Written as asm with both registers read and written: with the compiler
// builtins, the second result was taken from the first register (the sum
// came out as twice the first). One leading s_nop per block covers the wait
// after a VALU write of the operands.
template <int W>
__device__ __forceinline__ void swap1(float &a, float &b) {
  if constexpr (W == 32)
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  else
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
template <int W>
__device__ __forceinline__ void swap4(float &a0, float &b0, float &a1, float &b1, float &a2, float &b2, float &a3,
                                      float &b3) {
  if constexpr (W == 32)
    asm volatile(
        "s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\t"
        "v_permlane32_swap_b32 %4, %5\n\tv_permlane32_swap_b32 %6, %7"
        : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "+v"(a2), "+v"(b2), "+v"(a3), "+v"(b3));
  else
    asm volatile(
        "s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\t"
        "v_permlane16_swap_b32 %4, %5\n\tv_permlane16_swap_b32 %6, %7"
        : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "+v"(a2), "+v"(b2), "+v"(a3), "+v"(b3));
}
// a[i] <- a[i] + b[i] summed across the exchange above, for N values.
template <int W, int N>
__device__ __forceinline__ void swap_sum_n(float (&a)[N], float (&b)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) swap4<W>(a[i], b[i], a[i + 1], b[i + 1], a[i + 2], b[i + 2], a[i + 3], b[i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) swap1<W>(a[i], b[i]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] += b[i];
}

// Raw inputs of one sub-segment, held by a thread between its request and
// its LDS store.
template <int DK, int CB>
struct Stage1 {
  floatx4 k[BwdCfg<DK, CB>::KIT1], a[BwdCfg<DK, CB>::KIT1], b[BwdCfg<DK, CB>::KIT1];
  floatx4 v, w;
};
template <int DK, int CB>
struct Stage {
  floatx4 k[BwdCfg<DK, CB>::KIT], q[BwdCfg<DK, CB>::KIT], a[BwdCfg<DK, CB>::KIT], b[BwdCfg<DK, CB>::KIT];
  floatx4 v, w, d, r;
};

}  // namespace

// Gate forms (GF): kGateGeneral, fp32 per-channel gates; kGatePre, the
// per-channel gates as pre-activations in the input dtype (decay
// a = exp(-softplus(x)), b, w = sigmoid(x)), activated as they are staged,
// dw being then the gradient of the write gate's pre-activation; kGateCoupled,
// b = w = beta one scalar per token and value head ([.., T, H_v]), the value
// side of d(beta) summed per column block into p.wsum; kGateScalar, also the
// decay a = alpha one scalar per token and value head.
template <int DK, int CB, bool BF16, int GF>
__global__ __launch_bounds__((BwdCfg<DK, CB>::NT)) void backward_kernel(BackwardParams p) {
  constexpr bool PRE = GF == kGatePre, CPL = GF == kGateCoupled || GF == kGateScalar, SCA = GF == kGateScalar;
  using Cf = BwdCfg<DK, CB>;
  using E = Elem<BF16>;
  using ET = typename E::T;
  constexpr int KPL = Cf::KPL, L = Cf::L;
  __shared__ BwdSmem<DK, CB> sm;

  const int ncb = p.d_v / CB;
  const int cb = blockIdx.x % ncb, unit = blockIdx.x / ncb;  // unit = n * H_v + h
  const int n = unit / p.H_v, h = unit - n * p.H_v;
  const int g = h / (p.H_v / p.H_qk);
  const int d_v = p.d_v;
  // the sequence's tokens: packed sequences take theirs from cu (offsets
  // clamped to [0, p.T]); otherwise sequence n is tokens n*T .. n*T + T-1
  size_t tok0;  // first token of the sequence in the token axis
  int T;        // its length
  if (p.cu) {
    const int t0 = min(max(p.cu[n], 0), p.T), t1 = min(max(p.cu[n + 1], t0), p.T);
    tok0 = (size_t)t0;
    T = t1 - t0;
  } else {
    tok0 = (size_t)n * p.T;
    T = p.T;
  }
  const size_t BT = p.cu ? (size_t)p.T : (size_t)p.B * p.T;  // tokens in all
  const int nsub = (T + L - 1) / L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c4 = lane >> 4, kg = lane & 15;
  const int lcol = wave * 8 + 2 * c4;  // the lane's first column within the block
  const int col = cb * CB + lcol;      // ... within the head
  // the lane's key channels: quads 4kg .. 4kg+3 of every 64 keys, so that a
  // row read or write of 16 lanes covers the 64 banks once (contiguous
  // 32-byte pieces per lane would put lanes kg and kg+8 on the same banks);
  // kg*KPL .. for KPL < 4
  auto key = [&](int e) { return KPL >= 4 ? (e >> 2) * 64 + 4 * kg + (e & 3) : kg * KPL + e; };

  const ET *qh = (const ET *)p.q + tok0 * p.H_qk * DK + (size_t)g * DK;
  const ET *kh = (const ET *)p.k + tok0 * p.H_qk * DK + (size_t)g * DK;
  using GT = typename std::conditional<PRE, ET, float>::type;  // stored gate type
  const GT *ah = (const GT *)p.a + tok0 * p.H_v * DK + (size_t)h * DK;
  const GT *bh = (const GT *)p.b + tok0 * p.H_v * DK + (size_t)h * DK;
  const ET *vh = (const ET *)p.v + tok0 * p.H_v * d_v + (size_t)h * d_v + cb * CB;
  const GT *wh = (const GT *)p.w + tok0 * p.H_v * d_v + (size_t)h * d_v + cb * CB;
  // scalar gates: one value per token and value head (token stride H_v)
  const float *alpha_h = p.a + tok0 * p.H_v + h, *beta_h = p.b + tok0 * p.H_v + h;
  auto bcast = [](float x) { return floatx4{x, x, x, x}; };
  // four gates (activated) from their stored form
  auto decay_q = [&](const GT *x) -> floatx4 {
    if constexpr (PRE) {
      const floatx4 y = E::ld4(x);
      return floatx4{decay_from_pre(y[0]), decay_from_pre(y[1]), decay_from_pre(y[2]), decay_from_pre(y[3])};
    } else {
      return *reinterpret_cast<const floatx4 *>(x);
    }
  };
  auto gate_q = [&](const GT *x) -> floatx4 {
    if constexpr (PRE) {
      const floatx4 y = E::ld4(x);
      return floatx4{gate_from_pre(y[0]), gate_from_pre(y[1]), gate_from_pre(y[2]), gate_from_pre(y[3])};
    } else {
      return *reinterpret_cast<const floatx4 *>(x);
    }
  };
  const ET *dOh = (const ET *)p.dO + tok0 * p.H_v * d_v + (size_t)h * d_v + cb * CB;
  const size_t qk_t = (size_t)p.H_qk * DK, ab_t = (size_t)p.H_v * DK, vw_t = (size_t)p.H_v * d_v;
  const size_t s_off = (size_t)unit * DK * d_v;
  // checkpoints: per (n, h, column block, sub-segment) DK * CB floats; the
  // thread's 2 * KPL values s[e][c] (flat 2e + c) in pieces of CW floats,
  // piece q of every thread contiguous (each store instruction writes one
  // contiguous range)
  constexpr int CW = 2 * KPL < 4 ? 2 * KPL : 4;
  // a sequence's checkpoints start at slot tok0 / L + n of its (head, column
  // block) range of BT / L + B slots: room for its ceil(T / L) sub-segments
  const size_t nslot = BT / L + p.B;
  float *ckp = p.ck + (((size_t)h * ncb + cb) * nslot + tok0 / L + n) * (DK * CB) + (size_t)tid * CW;
  auto store_ck = [&](float *ck, const float (&x)[KPL][2]) {
#pragma unroll
    for (int q = 0; q < 2 * KPL / CW; ++q) {
      if constexpr (CW == 4)
        *reinterpret_cast<floatx4 *>(ck + q * (Cf::NT * CW)) =
            floatx4{x[2 * q][0], x[2 * q][1], x[2 * q + 1][0], x[2 * q + 1][1]};
      else
        *reinterpret_cast<floatx2 *>(ck + q * (Cf::NT * CW)) = floatx2{x[q][0], x[q][1]};
    }
  };
  // k-reads of the block's columns ([token][H_v][d_v], like v)
  float *rh = p.rk + tok0 * vw_t + (size_t)h * d_v + cb * CB;

  // Request sub-segment `sub`'s inputs into registers; tokens past the end
  // are identity steps (a = 1, everything else 0).
  auto request = [&](int sub, Stage<DK, CB> &st) {
#pragma unroll
    for (int it = 0; it < Cf::KIT; ++it) {
      const int idx = tid + it * Cf::NT;
      const int tt = idx / (DK / 4), kq = idx % (DK / 4);
      const int t = sub * L + tt;
      const bool ok = idx < Cf::NKS && t < T;
      st.k[it] = ok ? E::ld4(kh + t * qk_t + 4 * kq) : zero4();
      st.q[it] = ok ? E::ld4(qh + t * qk_t + 4 * kq) : zero4();
      if constexpr (SCA)
        st.a[it] = ok ? bcast(alpha_h[(size_t)t * p.H_v]) : floatx4{1.f, 1.f, 1.f, 1.f};
      else
        st.a[it] = ok ? decay_q(ah + t * ab_t + 4 * kq) : floatx4{1.f, 1.f, 1.f, 1.f};
      if constexpr (CPL)
        st.b[it] = ok ? bcast(beta_h[(size_t)t * p.H_v]) : zero4();
      else
        st.b[it] = ok ? gate_q(bh + t * ab_t + 4 * kq) : zero4();
    }
    {
      const int tt = tid / (CB / 4), cq = tid % (CB / 4);
      const int t = sub * L + tt;
      const bool ok = tid < Cf::NCS && t < T;
      st.v = ok ? E::ld4(vh + t * vw_t + 4 * cq) : zero4();
      if constexpr (CPL)
        st.w = ok ? bcast(beta_h[(size_t)t * p.H_v]) : zero4();
      else
        st.w = ok ? gate_q(wh + t * vw_t + 4 * cq) : zero4();
      st.d = ok ? E::ld4(dOh + t * vw_t + 4 * cq) : zero4();
      st.r = ok ? *reinterpret_cast<const floatx4 *>(rh + (size_t)t * vw_t + 4 * cq) : zero4();
    }
  };
  auto stash = [&](const Stage<DK, CB> &st) {
#pragma unroll
    for (int it = 0; it < Cf::KIT; ++it) {
      const int idx = tid + it * Cf::NT;
      if (idx < Cf::NKS) {
        const int tt = idx / (DK / 4), kq = idx % (DK / 4);
        *reinterpret_cast<floatx4 *>(&sm.b.kqae[tt][0][4 * kq]) = st.k[it];
        *reinterpret_cast<floatx4 *>(&sm.b.kqae[tt][1][4 * kq]) = st.q[it];
        *reinterpret_cast<floatx4 *>(&sm.b.kqae[tt][2][4 * kq]) = st.a[it];
        *reinterpret_cast<floatx4 *>(&sm.b.kqae[tt][3][4 * kq]) = st.b[it] * st.k[it];
      }
    }
    if (tid < Cf::NCS) {
      const int tt = tid / (CB / 4), cq = tid % (CB / 4);
      *reinterpret_cast<floatx4 *>(&sm.b.col[tt][0][4 * cq]) = st.w * st.v;
      *reinterpret_cast<floatx4 *>(&sm.b.col[tt][1][4 * cq]) = st.v;
      *reinterpret_cast<floatx4 *>(&sm.b.col[tt][2][4 * cq]) = st.w;
      *reinterpret_cast<floatx4 *>(&sm.b.col[tt][3][4 * cq]) = st.d;
      *reinterpret_cast<floatx4 *>(&sm.b.col[tt][4][4 * cq]) = st.r;
    }
  };
  // x[e] = row[key(e)]: the lane's key channels of one staged row
  auto lds_row = [&](const float *row, float (&x)[KPL]) {
#pragma unroll
    for (int e = 0; e < KPL; e += (KPL >= 4 ? 4 : KPL)) {
      if constexpr (KPL >= 4) {
        const floatx4 y = *reinterpret_cast<const floatx4 *>(row + key(e));
        x[e] = y[0]; x[e + 1] = y[1]; x[e + 2] = y[2]; x[e + 3] = y[3];
      } else if constexpr (KPL == 2) {
        const floatx2 y = *reinterpret_cast<const floatx2 *>(row + key(e));
        x[e] = y[0]; x[e + 1] = y[1];
      } else {
        x[e] = row[key(e)];
      }
    }
  };
  auto lds_keys = [&](int tt, int which, float (&x)[KPL]) { lds_row(sm.b.kqae[tt][which], x); };
  // Forward phase: request stage sb's inputs (k, a, b of every key channel,
  // v, w of the block's columns; tokens past the end are identity steps),
  // stage them in LDS, and run one token on the lane's two columns.
  auto request1 = [&](int sb, Stage1<DK, CB> &st) {
#pragma unroll
    for (int it = 0; it < Cf::KIT1; ++it) {
      const int idx = tid + it * Cf::NT;
      const int tt = idx / (DK / 4), kq = idx % (DK / 4);
      const int t = sb * Cf::L1 + tt;
      const bool ok = idx < Cf::NKS1 && t < T;
      st.k[it] = ok ? E::ld4(kh + t * qk_t + 4 * kq) : zero4();
      if constexpr (SCA)
        st.a[it] = ok ? bcast(alpha_h[(size_t)t * p.H_v]) : floatx4{1.f, 1.f, 1.f, 1.f};
      else
        st.a[it] = ok ? decay_q(ah + t * ab_t + 4 * kq) : floatx4{1.f, 1.f, 1.f, 1.f};
      if constexpr (CPL)
        st.b[it] = ok ? bcast(beta_h[(size_t)t * p.H_v]) : zero4();
      else
        st.b[it] = ok ? gate_q(bh + t * ab_t + 4 * kq) : zero4();
    }
    const int tt = tid / (CB / 4), cq = tid % (CB / 4);
    const int t = sb * Cf::L1 + tt;
    const bool ok = tid < Cf::NCS1 && t < T;
    st.v = ok ? E::ld4(vh + t * vw_t + 4 * cq) : zero4();
    if constexpr (CPL)
      st.w = ok ? bcast(beta_h[(size_t)t * p.H_v]) : zero4();
    else
      st.w = ok ? gate_q(wh + t * vw_t + 4 * cq) : zero4();
  };
  auto stash1 = [&](const Stage1<DK, CB> &st) {
#pragma unroll
    for (int it = 0; it < Cf::KIT1; ++it) {
      const int idx = tid + it * Cf::NT;
      if (idx < Cf::NKS1) {
        const int tt = idx / (DK / 4), kq = idx % (DK / 4);
        *reinterpret_cast<floatx4 *>(&sm.f.kae[tt][0][4 * kq]) = st.k[it];
        *reinterpret_cast<floatx4 *>(&sm.f.kae[tt][1][4 * kq]) = st.a[it];
        *reinterpret_cast<floatx4 *>(&sm.f.kae[tt][2][4 * kq]) = st.b[it] * st.k[it];
      }
    }
    if (tid < Cf::NCS1) {
      const int tt = tid / (CB / 4), cq = tid % (CB / 4);
      *reinterpret_cast<floatx4 *>(&sm.f.u[tt][4 * cq]) = st.w * st.v;
    }
  };
  auto fwd_step = [&](int tt, float (&s)[KPL][2], float &r0, float &r1) {
    float kk[KPL], aa[KPL], ee[KPL];
    lds_row(sm.f.kae[tt][0], kk);
    lds_row(sm.f.kae[tt][1], aa);
    lds_row(sm.f.kae[tt][2], ee);
    float x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
      s[e][0] *= aa[e];
      s[e][1] *= aa[e];
      x0 = fmaf(kk[e], s[e][0], x0);
      x1 = fmaf(kk[e], s[e][1], x1);
    }
    row_sum16x2(x0, x1);
    r0 = x0;
    r1 = x1;
    const float u0 = sm.f.u[tt][lcol], u1 = sm.f.u[tt][lcol + 1];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
      s[e][0] = fmaf(kk[e], u0, fmaf(-ee[e], r0, s[e][0]));
      s[e][1] = fmaf(kk[e], u1, fmaf(-ee[e], r1, s[e][1]));
    }
  };

  // ---------------------------------------------------------------- phase 1: forward, checkpoints
  float s[KPL][2];
#pragma unroll
  for (int e = 0; e < KPL; ++e) {
    if (p.S0) {
      const floatx2 x = *reinterpret_cast<const floatx2 *>(p.S0 + s_off + (size_t)key(e) * d_v + col);
      s[e][0] = x[0];
      s[e][1] = x[1];
    } else {
      s[e][0] = s[e][1] = 0.f;
    }
  }
  // (stages of L1 tokens: each request covers enough work to hide its latency)
  {
    const int nst = (T + Cf::L1 - 1) / Cf::L1;
    Stage1<DK, CB> st1;
    if (nst > 0) request1(0, st1);
    for (int sb = 0; sb < nst; ++sb) {
      __syncthreads();  // the previous stage's readers are done
      stash1(st1);
      __syncthreads();
      if (sb + 1 < nst) request1(sb + 1, st1);
#pragma unroll
      for (int tt = 0; tt < Cf::L1; ++tt) {
        const int t = sb * Cf::L1 + tt;
        if (tt % L == 0 && t < T)  // checkpoint: the state before sub-segment t / L
          store_ck(ckp + (size_t)(t / L) * (DK * CB), s);
        float r0, r1;
        fwd_step(tt, s, r0, r1);
        if (kg == 0) *reinterpret_cast<floatx2 *>(&sm.f.r[tt][lcol]) = floatx2{r0, r1};
      }
      __syncthreads();
      // the stage's k-reads as whole rows of the block's columns
      if (tid < Cf::NCS1) {
        const int tt = tid / (CB / 4), cq = tid % (CB / 4);
        const int t = sb * Cf::L1 + tt;
        if (t < T)
          *reinterpret_cast<floatx4 *>(rh + (size_t)t * vw_t + 4 * cq) =
              *reinterpret_cast<const floatx4 *>(&sm.f.r[tt][4 * cq]);
      }
    }
  }

  // ---------------------------------------------------------------- phase 2: backward
  float lam[KPL][2];
#pragma unroll
  for (int e = 0; e < KPL; ++e) {
    if (p.dST) {
      const floatx2 x = *reinterpret_cast<const floatx2 *>(p.dST + s_off + (size_t)key(e) * d_v + col);
      lam[e][0] = x[0];
      lam[e][1] = x[1];
    } else {
      lam[e][0] = lam[e][1] = 0.f;
    }
  }
  // the checkpoint of the next sub-segment to process, requested one ahead
  floatx2 ckn[KPL];
  auto request_ck = [&](int sub) {
    const float *ck = ckp + (size_t)sub * (DK * CB);
#pragma unroll
    for (int q = 0; q < 2 * KPL / CW; ++q) {
      if constexpr (CW == 4) {
        const floatx4 x = *reinterpret_cast<const floatx4 *>(ck + q * (Cf::NT * CW));
        ckn[2 * q] = floatx2{x[0], x[1]};
        ckn[2 * q + 1] = floatx2{x[2], x[3]};
      } else {
        ckn[q] = *reinterpret_cast<const floatx2 *>(ck + q * (Cf::NT * CW));
      }
    }
  };
  // the k-reads of phase 1 were stored by other waves of the workgroup: the
  // barrier (workgroup-scope release and acquire) makes them visible
  __syncthreads();
  Stage<DK, CB> st;
  if (nsub > 0) {
    request(nsub - 1, st);
    request_ck(nsub - 1);
  }
  for (int sub = nsub - 1; sub >= 0; --sub) {
    __syncthreads();  // the previous sub-segment's readers (and the sums below) are done
    stash(st);
    __syncthreads();
    // the sub-segment's states: hs[tt] = S before token tt, hs[L] = S after the last
    float hs[L + 1][KPL][2];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
      hs[0][e][0] = ckn[e][0];
      hs[0][e][1] = ckn[e][1];
    }
    if (sub > 0) {
      request(sub - 1, st);
      request_ck(sub - 1);
    }
    // (the k-reads come from phase 1: no key sums here)
#pragma unroll
    for (int tt = 0; tt < L; ++tt) {
      float kk[KPL], aa[KPL], ee[KPL];
      lds_keys(tt, 0, kk);
      lds_keys(tt, 2, aa);
      lds_keys(tt, 3, ee);
      const float u0 = sm.b.col[tt][0][lcol], u1 = sm.b.col[tt][0][lcol + 1];
      const float r0 = sm.b.col[tt][4][lcol], r1 = sm.b.col[tt][4][lcol + 1];
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        hs[tt + 1][e][0] = fmaf(kk[e], u0, fmaf(-ee[e], r0, hs[tt][e][0] * aa[e]));
        hs[tt + 1][e][1] = fmaf(kk[e], u1, fmaf(-ee[e], r1, hs[tt][e][1] * aa[e]));
      }
    }

#pragma unroll
    for (int tt = L - 1; tt >= 0; --tt) {
      float kk[KPL], qq[KPL], aa[KPL], ee[KPL];
      lds_keys(tt, 0, kk);
      lds_keys(tt, 1, qq);
      lds_keys(tt, 2, aa);
      lds_keys(tt, 3, ee);
      const float u0 = sm.b.col[tt][0][lcol], u1 = sm.b.col[tt][0][lcol + 1];
      const float d0 = sm.b.col[tt][3][lcol], d1 = sm.b.col[tt][3][lcol + 1];
      const float r0 = sm.b.col[tt][4][lcol], r1 = sm.b.col[tt][4][lcol + 1];
      // x[0] dq part, x[1] dk part (u L + a * dr S_{t-1}), x[2] sum_j r_j L (de = -x[2]), x[3] da
      float x[4][KPL];
      float pu0 = 0.f, pu1 = 0.f, pe0 = 0.f, pe1 = 0.f;
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        x[0][e] = fmaf(hs[tt + 1][e][0], d0, hs[tt + 1][e][1] * d1);
        lam[e][0] = fmaf(qq[e], d0, lam[e][0]);
        lam[e][1] = fmaf(qq[e], d1, lam[e][1]);
        pu0 = fmaf(lam[e][0], kk[e], pu0);
        pu1 = fmaf(lam[e][1], kk[e], pu1);
        pe0 = fmaf(lam[e][0], ee[e], pe0);
        pe1 = fmaf(lam[e][1], ee[e], pe1);
      }
      row_sum16x4(pu0, pu1, pe0, pe1);
      const float du0 = pu0, du1 = pu1, dr0 = -pe0, dr1 = -pe1;
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        x[2][e] = fmaf(lam[e][0], r0, lam[e][1] * r1);
        const float p2 = fmaf(lam[e][0], u0, lam[e][1] * u1);
        lam[e][0] = fmaf(kk[e], dr0, lam[e][0]);
        lam[e][1] = fmaf(kk[e], dr1, lam[e][1]);
        const float p4 = fmaf(hs[tt][e][0], dr0, hs[tt][e][1] * dr1);
        x[3][e] = fmaf(lam[e][0], hs[tt][e][0], lam[e][1] * hs[tt][e][1]);
        x[1][e] = fmaf(aa[e], p4, p2);
        lam[e][0] *= aa[e];
        lam[e][1] *= aa[e];
      }
      // reduce-scatter over the four column pairs: lane group c4 ends with
      // sum x[c4][.] of the wave's 8 columns. swap32(A, B) gives
      // [A lanes 0-31, B lanes 0-31] and [A lanes 32-63, B lanes 32-63], so
      // their sum is, in the lower half, A plus the upper half's A, and in
      // the upper half, B plus the lower half's B; swap16 does the same
      // between rows 0/1 and 2/3.
      swap_sum_n<32, KPL>(x[0], x[2]);
      swap_sum_n<32, KPL>(x[1], x[3]);
      swap_sum_n<16, KPL>(x[0], x[1]);
      // x[0] now holds the lane group's vector c4 on the lane's keys
      float *dst = &sm.b.red[wave][tt][c4][0];
      if constexpr (KPL >= 4) {
#pragma unroll
        for (int e = 0; e < KPL; e += 4)
          *reinterpret_cast<floatx4 *>(dst + key(e)) = floatx4{x[0][e], x[0][e + 1], x[0][e + 2], x[0][e + 3]};
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) dst[key(e)] = x[0][e];
      }
      if (kg == 0) {
        sm.b.du[tt][lcol] = du0;
        sm.b.du[tt][lcol + 1] = du1;
      }
    }
    __syncthreads();

    // key-side sums of the block (fixed wave order) -> workspace
    constexpr int NQ = L * 4 * DK / 4;
    for (int idx = tid; idx < NQ; idx += Cf::NT) {
      const int tt = idx / DK, rem = idx % DK;  // rem = vector * (DK / 4) + key quad
      const int vec = rem / (DK / 4), kq = rem % (DK / 4);
      const int t = sub * L + tt;
      if (t < T) {
        floatx4 acc = *reinterpret_cast<const floatx4 *>(&sm.b.red[0][tt][vec][4 * kq]);
#pragma unroll
        for (int w2 = 1; w2 < Cf::NWV; ++w2) acc += *reinterpret_cast<const floatx4 *>(&sm.b.red[w2][tt][vec][4 * kq]);
        float *dst = p.part + (((size_t)cb * BT + tok0 + t) * p.H_v + h) * (4 * DK) + vec * DK + 4 * kq;
        *reinterpret_cast<floatx4 *>(dst) = acc;
      }
    }
    // dv = du * w, dw = du * v
    for (int idx = tid; idx < L * CB; idx += Cf::NT) {
      const int tt = idx / CB, c = idx % CB;
      const int t = sub * L + tt;
      if (t < T) {
        const float du = sm.b.du[tt][c];
        const size_t o = (tok0 + t) * vw_t + (size_t)h * d_v + cb * CB + c;
        E::st((ET *)p.dv + o, du * sm.b.col[tt][2][c]);
        if constexpr (PRE) {  // through w = sigmoid(x): dw/dx = w (1 - w)
          const float wg = sm.b.col[tt][2][c];
          E::st((ET *)p.dw + o, du * sm.b.col[tt][1][c] * (wg * (1.f - wg)));
        } else if constexpr (!CPL) {
          p.dw[o] = du * sm.b.col[tt][1][c];
        }
      }
    }
    if constexpr (CPL) {  // value side of d(beta): sum over the block's columns of du * v
      if (tid < L) {
        const int t = sub * L + tid;
        if (t < T) {
          float acc = 0.f;
          for (int c = 0; c < CB; ++c) acc = fmaf(sm.b.du[tid][c], sm.b.col[tid][1][c], acc);
          p.wsum[((size_t)cb * BT + tok0 + t) * p.H_v + h] = acc;
        }
      }
    }
  }
  if (p.dS0) {
#pragma unroll
    for (int e = 0; e < KPL; ++e)
      *reinterpret_cast<floatx2 *>(p.dS0 + s_off + (size_t)key(e) * d_v + col) = floatx2{lam[e][0], lam[e][1]};
  }
}

// Key-side gradients: per (token, query/key head g), sum the column blocks'
// partial sums of every value head h that shares g:
//   dq = sum x0;  dk = sum (x1 - b*x2);  per h: da = x3, db = -k*x2.
template <int DK, bool BF16, int GF>
__global__ __launch_bounds__(256) void backward_reduce_kernel(BackwardParams p) {
  constexpr bool PRE = GF == kGatePre, CPL = GF == kGateCoupled || GF == kGateScalar, SCA = GF == kGateScalar;
  using E = Elem<BF16>;
  using ET = typename E::T;
  constexpr int TPR = DK / 4;  // threads per (token, g) row, 4 keys each
  const int ncb = p.d_v / bwd_cb(p.d_v);
  const size_t BT = p.cu ? (size_t)p.T : (size_t)p.B * p.T;
  const size_t row = (size_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= BT * p.H_qk) return;
  const int kq = threadIdx.x % TPR;
  const size_t tok = row / p.H_qk;
  const int g = (int)(row % p.H_qk), G = p.H_v / p.H_qk;
  const floatx4 kk = E::ld4((const ET *)p.k + row * DK + 4 * kq);
  floatx4 dq = zero4(), dk = zero4();
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    floatx4 x[4] = {zero4(), zero4(), zero4(), zero4()};
    for (int c = 0; c < ncb; ++c) {
      const float *src = p.part + (((size_t)c * BT + tok) * p.H_v + h) * (4 * DK) + 4 * kq;
#pragma unroll
      for (int vec = 0; vec < 4; ++vec) x[vec] += *reinterpret_cast<const floatx4 *>(src + vec * DK);
    }
    const size_t o = (tok * p.H_v + h) * DK + 4 * kq;
    floatx4 bb;
    if constexpr (CPL) {  // scalar beta (and alpha): sums over the key channels of the row
      const size_t so = tok * p.H_v + h;
      const float beta = p.b[so];
      bb = floatx4{beta, beta, beta, beta};
      const floatx4 dbk = -(kk * x[2]);
      float sdb = dbk[0] + dbk[1] + dbk[2] + dbk[3];
      float sda = x[3][0] + x[3][1] + x[3][2] + x[3][3];
#pragma unroll
      for (int m = TPR / 2; m >= 1; m /= 2) {
        sdb += __shfl_xor(sdb, m, 64);
        if constexpr (SCA) sda += __shfl_xor(sda, m, 64);
      }
      if constexpr (!SCA) *reinterpret_cast<floatx4 *>(p.da + o) = x[3];
      if (kq == 0) {
        for (int c = 0; c < ncb; ++c) sdb += p.wsum[((size_t)c * BT + tok) * p.H_v + h];
        p.db[so] = sdb;
        if constexpr (SCA) p.da[so] = sda;
      }
    } else if constexpr (PRE) {  // gradients of the pre-activations: da/dx = -a (1 - a), db/dx = b (1 - b)
      const floatx4 xa = E::ld4((const ET *)p.a + o), xb = E::ld4((const ET *)p.b + o);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float aa = decay_from_pre(xa[e]);
        bb[e] = gate_from_pre(xb[e]);
        E::st((ET *)p.da + o + e, x[3][e] * (-aa * (1.f - aa)));
        E::st((ET *)p.db + o + e, -(kk[e] * x[2][e]) * (bb[e] * (1.f - bb[e])));
      }
    } else {
      bb = *reinterpret_cast<const floatx4 *>(p.b + o);
      *reinterpret_cast<floatx4 *>(p.da + o) = x[3];
      *reinterpret_cast<floatx4 *>(p.db + o) = -(kk * x[2]);
    }
    dq += x[0];
    dk += x[1] - bb * x[2];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    E::st((ET *)p.dq + row * DK + 4 * kq + e, dq[e]);
    E::st((ET *)p.dk + row * DK + 4 * kq + e, dk[e]);
  }
}

namespace {

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }


template <int DK, int CB, bool BF16, int GF>
hipError_t launch_t(const BackwardParams &p, hipStream_t st) {
  const int ncb = p.d_v / CB;
  hipLaunchKernelGGL((backward_kernel<DK, CB, BF16, GF>), dim3(p.B * p.H_v * ncb), dim3(BwdCfg<DK, CB>::NT), 0, st,
                     p);
  hipError_t e = hipGetLastError();
  const size_t BT = p.cu ? (size_t)p.T : (size_t)p.B * p.T;
  if (e != hipSuccess || BT == 0) return e;
  const size_t rows = BT * p.H_qk;
  const size_t rpb = 256 / (DK / 4);
  hipLaunchKernelGGL((backward_reduce_kernel<DK, BF16, GF>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, st,
                     p);
  return hipGetLastError();
}

template <int DK, bool BF16, int GF>
hipError_t launch_cb(const BackwardParams &p, hipStream_t st) {
  switch (bwd_cb(p.d_v)) {
    case 64: return launch_t<DK, 64, BF16, GF>(p, st);
    case 32: return launch_t<DK, 32, BF16, GF>(p, st);
  }
  return launch_t<DK, 16, BF16, GF>(p, st);
}

template <int DK, bool BF16>
hipError_t launch_dk(const BackwardParams &p, hipStream_t st) {
  switch (p.gate_form) {
    case kGatePre: return launch_cb<DK, BF16, kGatePre>(p, st);
    case kGateCoupled: return launch_cb<DK, BF16, kGateCoupled>(p, st);
    case kGateScalar: return launch_cb<DK, BF16, kGateScalar>(p, st);
  }
  return launch_cb<DK, BF16, kGateGeneral>(p, st);
}

// ---------------------------------------------------------------- split sequences
// Few long sequences run as segments in parallel: the packed-sequence
// backward over the segments, each from its exact entering state and with
// its exact exiting adjoint. The entering states come from the prefill's
// split passes; the exiting adjoints from one sequential adjoint-only sweep
// per sequence. The adjoint of the state does not depend on the state:
// L_{t-1} = diag(a_t) (I - k_t e_t^T) (L_t + q_t dO_t^T), e = b * k, so the
// sweep needs no forward states and four operations per state element and
// token (the full backward needs about twenty).

constexpr int kSweepL = 16;  // tokens per staged block of the sweep

template <int DK, int CB>
struct SweepSmem {
  alignas(16) float kqae[2][kSweepL][4][DK];  // k, q, a, e = b*k per token (double-buffered)
  alignas(16) float dO[2][kSweepL][CB];
};

// One workgroup per (sequence, value head, CB columns); a lane holds one
// column x DK/16 keys (backward_kernel's lanes hold two columns: one halves
// the instructions per token and wave), key sums over 16-lane rows, four
// columns per wave, keys interleaved as in backward_kernel. From
// the last token to the first; after each block that starts a segment j > 0
// the adjoint of the state entering it, i.e. the exiting adjoint of segment
// j - 1, goes to Lout[n * nseg + j - 1]; Lout[n * nseg + nseg - 1] gets dS_T
// (or zero).
template <int CB>
constexpr int sweep_threads() { return 16 * CB; }  // CB / 4 waves

template <int DK, int CB, bool BF16, int GF>
__global__ __launch_bounds__(sweep_threads<CB>()) void adjoint_sweep_kernel(SweepParams p) {
  constexpr bool PRE = GF == kGatePre, CPL = GF == kGateCoupled || GF == kGateScalar, SCA = GF == kGateScalar;
  using E = Elem<BF16>;
  using ET = typename E::T;
  constexpr int KPL = DK / 16, NT = sweep_threads<CB>(), LS = kSweepL;
  static_assert(CB % 4 == 0 && CB <= 64, "four columns per wave");
  constexpr int NKQ = LS * DK / 4;  // key quads per block and array
  constexpr int KIT = (NKQ + NT - 1) / NT;
  constexpr int NCQ = LS * CB / 4;  // dO quads per block
  static_assert(NCQ <= NT, "one dO quad per thread at most");
  __shared__ SweepSmem<DK, CB> sm;

  const int ncb = p.d_v / CB;
  const int cb = blockIdx.x % ncb, unit = blockIdx.x / ncb;  // unit = n * H_v + h
  const int n = unit / p.H_v, h = unit - n * p.H_v;
  const int g = h / (p.H_v / p.H_qk);
  const int d_v = p.d_v, T = p.T;
  const size_t tok0 = (size_t)n * T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c4 = lane >> 4, kg = lane & 15;
  const int lcol = wave * 4 + c4;  // the lane's column within the block
  const int col = cb * CB + lcol;  // ... within the head
  // the lane's keys: quads 4kg .. 4kg+3 of every 64 keys (a row read of 16
  // lanes then covers 64 banks once), or 2kg, 2kg+1 / kg for DK < 64
  auto key = [&](int e) { return KPL >= 4 ? (e >> 2) * 64 + 4 * kg + (e & 3) : kg * KPL + e; };
  using GT = typename std::conditional<PRE, ET, float>::type;
  const ET *qh = (const ET *)p.q + tok0 * p.H_qk * DK + (size_t)g * DK;
  const ET *kh = (const ET *)p.k + tok0 * p.H_qk * DK + (size_t)g * DK;
  // per-channel gates [token][H_v][DK]; scalar ones [token][H_v]
  const size_t a_t = (size_t)p.H_v * (SCA ? 1 : DK), b_t = (size_t)p.H_v * (CPL ? 1 : DK);
  const GT *ah = (const GT *)p.a + tok0 * a_t + (size_t)h * (SCA ? 1 : DK);
  const GT *bh = (const GT *)p.b + tok0 * b_t + (size_t)h * (CPL ? 1 : DK);
  const ET *dOh = (const ET *)p.dO + tok0 * p.H_v * d_v + (size_t)h * d_v + cb * CB;
  const size_t qk_t = (size_t)p.H_qk * DK, vw_t = (size_t)p.H_v * d_v;

  struct Raw {
    floatx4 k[KIT], q[KIT], a[KIT], e[KIT], d;
  };
  // block bi's inputs into registers (tokens past the end are never read)
  auto request = [&](int bi, Raw &r) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int idx = tid + it * NT;
      const int tt = idx / (DK / 4), kq = idx % (DK / 4);
      const int t = bi * LS + tt;
      const bool ok = idx < NKQ && t < T;
      floatx4 kv = zero4(), qv = zero4(), av = floatx4{1.f, 1.f, 1.f, 1.f}, bv = zero4();
      if (ok) {
        kv = E::ld4(kh + (size_t)t * qk_t + 4 * kq);
        qv = E::ld4(qh + (size_t)t * qk_t + 4 * kq);
        if constexpr (SCA) {
          const float x = ah[(size_t)t * a_t];
          av = floatx4{x, x, x, x};
        } else if constexpr (PRE) {
          const floatx4 x = E::ld4(ah + (size_t)t * a_t + 4 * kq);
          av = floatx4{decay_from_pre(x[0]), decay_from_pre(x[1]), decay_from_pre(x[2]), decay_from_pre(x[3])};
        } else {
          av = *reinterpret_cast<const floatx4 *>(ah + (size_t)t * a_t + 4 * kq);
        }
        if constexpr (CPL) {
          const float x = bh[(size_t)t * b_t];
          bv = floatx4{x, x, x, x};
        } else if constexpr (PRE) {
          const floatx4 x = E::ld4(bh + (size_t)t * b_t + 4 * kq);
          bv = floatx4{gate_from_pre(x[0]), gate_from_pre(x[1]), gate_from_pre(x[2]), gate_from_pre(x[3])};
        } else {
          bv = *reinterpret_cast<const floatx4 *>(bh + (size_t)t * b_t + 4 * kq);
        }
      }
      r.k[it] = kv;
      r.q[it] = qv;
      r.a[it] = av;
      r.e[it] = bv * kv;
    }
    const int tt = tid / (CB / 4), cq = tid % (CB / 4);
    const int t = bi * LS + tt;
    r.d = (tid < NCQ && t < T) ? E::ld4(dOh + (size_t)t * vw_t + 4 * cq) : zero4();
  };
  auto stash = [&](int buf, const Raw &r) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int idx = tid + it * NT;
      if (idx < NKQ) {
        const int tt = idx / (DK / 4), kq = idx % (DK / 4);
        *reinterpret_cast<floatx4 *>(&sm.kqae[buf][tt][0][4 * kq]) = r.k[it];
        *reinterpret_cast<floatx4 *>(&sm.kqae[buf][tt][1][4 * kq]) = r.q[it];
        *reinterpret_cast<floatx4 *>(&sm.kqae[buf][tt][2][4 * kq]) = r.a[it];
        *reinterpret_cast<floatx4 *>(&sm.kqae[buf][tt][3][4 * kq]) = r.e[it];
      }
    }
    if (tid < NCQ) {
      const int tt = tid / (CB / 4), cq = tid % (CB / 4);
      *reinterpret_cast<floatx4 *>(&sm.dO[buf][tt][4 * cq]) = r.d;
    }
  };
  auto lds_row = [&](const float *row, float (&x)[KPL]) {
#pragma unroll
    for (int e = 0; e < KPL; e += (KPL >= 4 ? 4 : KPL)) {
      if constexpr (KPL >= 4) {
        const floatx4 y = *reinterpret_cast<const floatx4 *>(row + key(e));
        x[e] = y[0]; x[e + 1] = y[1]; x[e + 2] = y[2]; x[e + 3] = y[3];
      } else if constexpr (KPL == 2) {
        const floatx2 y = *reinterpret_cast<const floatx2 *>(row + key(e));
        x[e] = y[0]; x[e + 1] = y[1];
      } else {
        x[e] = row[key(e)];
      }
    }
  };
  auto store_L = [&](int j, const float (&L)[KPL]) {
    float *dst = p.Lout + ((size_t)(n * p.nseg + j) * p.H_v + h) * DK * d_v + col;
#pragma unroll
    for (int e = 0; e < KPL; ++e) dst[(size_t)key(e) * d_v] = L[e];
  };

  float L[KPL];
#pragma unroll
  for (int e = 0; e < KPL; ++e) L[e] = p.dST ? p.dST[((size_t)unit * DK + key(e)) * d_v + col] : 0.f;
  store_L(p.nseg - 1, L);
  const int nb = (T + LS - 1) / LS;
  Raw r;
  if (nb > 0) {
    request(nb - 1, r);
    stash((nb - 1) & 1, r);
  }
  __syncthreads();
  for (int bi = nb - 1; bi >= 0; --bi) {
    const int buf = bi & 1;
    if (bi > 0) request(bi - 1, r);  // in flight during this block
    const int ntok = min(LS, T - bi * LS);
    // one token: its rows x (k, q, a, e) and dO of the lane's column
    struct Tok {
      float k[KPL], q[KPL], a[KPL], e[KPL];
      float d;
    };
    auto read_tok = [&](int tt, Tok &x) {
      lds_row(sm.kqae[buf][tt][0], x.k);
      lds_row(sm.kqae[buf][tt][1], x.q);
      lds_row(sm.kqae[buf][tt][2], x.a);
      lds_row(sm.kqae[buf][tt][3], x.e);
      x.d = sm.dO[buf][tt][lcol];
    };
    auto step = [&](const Tok &x) __attribute__((always_inline)) {
      // the output read's adjoint, then the key read e^T L (two partial
      // sums: a shorter dependent chain)
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        L[e] = fmaf(x.q[e], x.d, L[e]);
        if (e & 1)
          s1 = fmaf(x.e[e], L[e], s1);
        else
          s0 = fmaf(x.e[e], L[e], s0);
      }
      float s = s0 + s1;
      row_sum16x1(s);
#pragma unroll
      for (int e = 0; e < KPL; ++e) L[e] = x.a[e] * fmaf(-x.k[e], s, L[e]);  // erase along k, then the decay
    };
    // each token's rows are read while the token after it (in time) computes,
    // into two register sets in turn; the reads are unconditional (the last
    // one repeats token 0) so that the wait before a step covers only the
    // reads issued before it
    Tok xa, xb;
    read_tok(ntok - 1, xa);
    int tt = ntok - 1;
    for (; tt >= 1; tt -= 2) {
      read_tok(tt - 1, xb);
      step(xa);
      read_tok(max(tt - 2, 0), xa);
      step(xb);
    }
    if (tt == 0) step(xa);
    if (bi > 0 && (bi * LS) % p.seg_len == 0) store_L(bi * LS / p.seg_len - 1, L);
    __syncthreads();
    if (bi > 0) stash(buf ^ 1, r);
    __syncthreads();
  }
}

template <int DK, int CB, bool BF16>
hipError_t launch_sweep_cb(const SweepParams &p, int form, hipStream_t st) {
  const dim3 grid(p.B * p.H_v * (p.d_v / CB)), block(sweep_threads<CB>());
  switch (form) {
    case kGatePre: hipLaunchKernelGGL((adjoint_sweep_kernel<DK, CB, BF16, kGatePre>), grid, block, 0, st, p); break;
    case kGateCoupled:
      hipLaunchKernelGGL((adjoint_sweep_kernel<DK, CB, BF16, kGateCoupled>), grid, block, 0, st, p);
      break;
    case kGateScalar:
      hipLaunchKernelGGL((adjoint_sweep_kernel<DK, CB, BF16, kGateScalar>), grid, block, 0, st, p);
      break;
    default: hipLaunchKernelGGL((adjoint_sweep_kernel<DK, CB, BF16, kGateGeneral>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

// 16-column workgroups (4 waves). Every wave reads each token's rows from
// LDS, so a CU's LDS bandwidth bounds a token's step: fewer waves per CU
// (16 columns) measured faster than 32 or 64, and fewer still (8, 4) slower
// again (each workgroup stages every token's rows).
template <int DK, bool BF16>
hipError_t launch_sweep_dk(const SweepParams &p, int form, hipStream_t st) {
  return launch_sweep_cb<DK, 16, BF16>(p, form, st);
}

}  // namespace

// This translation unit holds the instances of one dtype (GDN2_BWD_BF16).
#if GDN2_BWD_BF16
hipError_t launch_backward_bf16(const BackwardParams &p, int d_k, hipStream_t st) {
  constexpr bool BF16 = true;
#else
hipError_t launch_backward_f32(const BackwardParams &p, int d_k, hipStream_t st) {
  constexpr bool BF16 = false;
#endif
  switch (d_k) {
    case 16: return launch_dk<16, BF16>(p, st);
    case 32: return launch_dk<32, BF16>(p, st);
    case 64: return launch_dk<64, BF16>(p, st);
    case 128: return launch_dk<128, BF16>(p, st);
  }
  return hipErrorInvalidValue;
}

#if GDN2_BWD_BF16
hipError_t launch_sweep_bf16(const SweepParams &p, int d_k, int form, hipStream_t st) {
  constexpr bool BF16 = true;
#else
hipError_t launch_sweep_f32(const SweepParams &p, int d_k, int form, hipStream_t st) {
  constexpr bool BF16 = false;
#endif
  switch (d_k) {
    case 16: return launch_sweep_dk<16, BF16>(p, form, st);
    case 32: return launch_sweep_dk<32, BF16>(p, form, st);
    case 64: return launch_sweep_dk<64, BF16>(p, form, st);
    case 128: return launch_sweep_dk<128, BF16>(p, form, st);
  }
  return hipErrorInvalidValue;
}

#if GDN2_BWD_BF16
hipError_t launch_backward_f32(const BackwardParams &p, int d_k, hipStream_t st);
hipError_t launch_sweep_f32(const SweepParams &p, int d_k, int form, hipStream_t st);

namespace {

// Segment offsets of the split: packed sequence i = n * nseg + j is tokens
// n * T + j * seg_len .. (clamped to the sequence).
__global__ __launch_bounds__(256) void split_cu_kernel(int32_t *cu, int B, int T, int nseg, int seg_len) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int ns = B * nseg;
  if (i > ns) return;
  const int n = i / nseg, j = i - n * nseg;
  cu[i] = i == ns ? B * T : n * T + min(j * seg_len, T);
}

// Entering state of packed sequence (n, j): S0 of sequence n (zero if null)
// for j = 0, else the state after segment j - 1 (seg_states, [nseg][B][H_v]).
__global__ __launch_bounds__(256) void split_states_kernel(float *S_in, const float *S0, const float *seg_states,
                                                            int B, int H_v, int nseg, int dkdv) {
  const int blk = blockIdx.x;  // (n * nseg + j) * H_v + h
  const int h = blk % H_v, i = blk / H_v;
  const int n = i / nseg, j = i - n * nseg;
  const size_t unit = (size_t)n * H_v + h;
  const float *src = j == 0 ? (S0 ? S0 + unit * dkdv : nullptr)
                            : seg_states + ((size_t)(j - 1) * B * H_v + unit) * dkdv;
  float *dst = S_in + (size_t)blk * dkdv;
  for (int x = 4 * threadIdx.x; x < dkdv; x += 4 * 256)
    *reinterpret_cast<floatx4 *>(dst + x) = src ? *reinterpret_cast<const floatx4 *>(src + x) : zero4();
}

// dS0 of sequence n is that of its first segment.
__global__ __launch_bounds__(256) void split_ds0_kernel(float *dS0, const float *dS0_seg, int H_v, int nseg,
                                                         int dkdv) {
  const int blk = blockIdx.x;  // n * H_v + h
  const int n = blk / H_v, h = blk - n * H_v;
  const float *src = dS0_seg + ((size_t)n * nseg * H_v + h) * dkdv;
  float *dst = dS0 + (size_t)blk * dkdv;
  for (int x = 4 * threadIdx.x; x < dkdv; x += 4 * 256)
    *reinterpret_cast<floatx4 *>(dst + x) = *reinterpret_cast<const floatx4 *>(src + x);
}

// nseg segments of seg_len tokens, from the prefill plan asked for req
// segments (asking again for nseg can give other segments: 16 chunks asked
// for 2 give 3 of 8 chunks, asked for 3 give 3 of 6)
struct BwdSplit {
  int nseg, seg_len, req;
};

// Split plan: with fewer than 128 workgroups (sequences x value heads x
// column blocks) and long sequences, segments of at least 2048 tokens and
// up to about 512 workgroups in all; the segments are those the prefill's
// split would use for the same count (whole chunks). GDN2_BACKWARD_SPLIT=<n>,
// read at each call, asks for n segments (1: never split).
BwdSplit backward_split_plan(int B, int T, int H_qk, int H_v, int d_k, int d_v, bool bf16) {
  const BwdSplit none{1, T, 1};
  if (B <= 0 || T <= 0 || (long)B * T > 0x7fffffffL) return none;
  const long wg = (long)B * H_v * (d_v / bwd_cb(d_v));
  long P = 1;
  if (const char *env = getenv("GDN2_BACKWARD_SPLIT")) {
    P = atol(env);
  } else if (wg < 128) {
    while (wg * P * 2 <= 512 && T / (P * 2) >= 2048) P *= 2;
  }
  if (P < 2) return none;
  PrefillArgs fa{};
  fa.B = B; fa.T = T; fa.H_qk = H_qk; fa.H_v = H_v; fa.d_k = d_k; fa.d_v = d_v;
  fa.chunk = 64;
  fa.bf16 = bf16;
  fa.nct = prefill_pick_nct(B, H_v, d_v);
  fa.force_nseg = (int)(P < 65536 ? P : 65536);
  const PrefillPlan pl = prefill_plan(fa);
  if (pl.nseg < 2 || pl.seg_len % kSweepL != 0) return none;
  return BwdSplit{pl.nseg, pl.seg_len, fa.force_nseg};
}

struct SplitLayout {
  size_t inner, states, segst, trans, cu, total;
};

SplitLayout split_layout(int B, int T, int H_v, int d_k, int d_v, const BwdSplit &sp) {
  SplitLayout l;
  const size_t ns = (size_t)B * sp.nseg;
  l.inner = align256(backward_workspace_bytes((int)ns, (size_t)B * T, H_v, d_k, d_v));
  l.states = align256(ns * H_v * d_k * d_v * 4);  // entering states, exiting adjoints, dS0 per segment
  l.segst = align256((size_t)sp.nseg * B * H_v * d_k * d_v * 4);
  l.trans = align256((size_t)sp.nseg * B * H_v * d_k * d_k * 4);
  l.cu = align256((ns + 1) * 4);
  l.total = l.inner + 3 * l.states + l.segst + l.trans + l.cu;
  return l;
}

hipError_t launch_backward_per_token(const BackwardArgs &a, hipStream_t st);

hipError_t launch_backward_split(const BackwardArgs &a, const BwdSplit &sp, hipStream_t st) {
  const SplitLayout l = split_layout(a.B, a.T, a.H_v, a.d_k, a.d_v, sp);
  const int ns = a.B * sp.nseg;
  const int dkdv = a.d_k * a.d_v;
  char *w = static_cast<char *>(a.workspace);
  void *inner = w;
  float *S_in = reinterpret_cast<float *>(w + l.inner);
  float *Lout = reinterpret_cast<float *>(w + l.inner + l.states);
  float *dS0_seg = reinterpret_cast<float *>(w + l.inner + 2 * l.states);
  float *segst = reinterpret_cast<float *>(w + l.inner + 3 * l.states);
  float *trans = reinterpret_cast<float *>(w + l.inner + 3 * l.states + l.segst);
  int32_t *cu = reinterpret_cast<int32_t *>(w + l.inner + 3 * l.states + l.segst + l.trans);
  const bool coupled = a.gate_form == kGateCoupled || a.gate_form == kGateScalar;

  hipLaunchKernelGGL(split_cu_kernel, dim3((ns + 256) / 256), dim3(256), 0, st, cu, a.B, a.T, sp.nseg, sp.seg_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // entering states: the prefill's split passes
  PrefillArgs fa{};
  fa.B = a.B; fa.T = a.T; fa.H_qk = a.H_qk; fa.H_v = a.H_v; fa.d_k = a.d_k; fa.d_v = a.d_v;
  fa.chunk = 64;
  fa.bf16 = a.bf16;
  fa.nct = prefill_pick_nct(a.B, a.H_v, a.d_v);
  fa.q = a.q; fa.k = a.k; fa.v = a.v;
  fa.a = a.a; fa.b = a.b; fa.w = coupled ? a.b : a.w;
  fa.S0 = a.S0;
  fa.coupled = coupled;
  fa.scalar_decay = a.gate_form == kGateScalar;
  fa.preact = a.gate_form == kGatePre;
  fa.workspace = trans;
  fa.workspace_bytes = l.trans;
  fa.force_nseg = sp.req;
  fa.seg_states = segst;
  const PrefillPlan fpl = prefill_plan(fa);
  if (fpl.nseg != sp.nseg || fpl.seg_len != sp.seg_len) return hipErrorInvalidValue;
  e = launch_prefill(fa, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(split_states_kernel, dim3(ns * a.H_v), dim3(256), 0, st, S_in, a.S0, segst, a.B, a.H_v,
                     sp.nseg, dkdv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // exiting adjoints: the adjoint-only sweep
  SweepParams sw{};
  sw.q = a.q; sw.k = a.k; sw.a = a.a; sw.b = a.b; sw.dO = a.dO; sw.dST = a.dST;
  sw.Lout = Lout;
  sw.B = a.B; sw.T = a.T; sw.H_qk = a.H_qk; sw.H_v = a.H_v; sw.d_v = a.d_v;
  sw.nseg = sp.nseg; sw.seg_len = sp.seg_len;
  e = a.bf16 ? launch_sweep_bf16(sw, a.d_k, a.gate_form, st) : launch_sweep_f32(sw, a.d_k, a.gate_form, st);
  if (e != hipSuccess) return e;
  // the segments as packed sequences
  BackwardArgs c = a;
  c.B = ns;
  c.T = a.B * a.T;
  c.cu_seqlens = cu;
  c.S0 = S_in;
  c.dST = Lout;
  c.dS0 = a.dS0 ? dS0_seg : nullptr;
  c.workspace = inner;
  e = launch_backward_per_token(c, st);
  if (e != hipSuccess || !a.dS0) return e;
  hipLaunchKernelGGL(split_ds0_kernel, dim3(a.B * a.H_v), dim3(256), 0, st, a.dS0, dS0_seg, a.H_v, sp.nseg, dkdv);
  return hipGetLastError();
}

hipError_t launch_backward_per_token(const BackwardArgs &a, hipStream_t st) {
  BackwardParams p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.a = a.a; p.b = a.b; p.w = a.w; p.S0 = a.S0;
  p.dO = a.dO; p.dST = a.dST;
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.da = a.da; p.db = a.db; p.dw = a.dw; p.dS0 = a.dS0;
  p.B = a.B; p.T = a.T; p.H_qk = a.H_qk; p.H_v = a.H_v; p.d_v = a.d_v;
  p.cu = a.cu_seqlens;
  p.gate_form = a.gate_form;
  const size_t BT = a.cu_seqlens ? (size_t)a.T : (size_t)a.B * a.T;
  const size_t ck = (BT / kSub + a.B) * (size_t)a.H_v * a.d_k * a.d_v * 4;
  const size_t part = ((size_t)a.d_v / bwd_cb(a.d_v)) * BT * a.H_v * 4 * a.d_k * 4;
  p.ck = reinterpret_cast<float *>(a.workspace);
  p.part = reinterpret_cast<float *>(reinterpret_cast<char *>(a.workspace) + align256(ck));
  p.rk = reinterpret_cast<float *>(reinterpret_cast<char *>(a.workspace) + align256(ck) + align256(part));
  p.wsum = reinterpret_cast<float *>(reinterpret_cast<char *>(p.rk) + align256(BT * a.H_v * a.d_v * 4));
  return a.bf16 ? launch_backward_bf16(p, a.d_k, st) : launch_backward_f32(p, a.d_k, st);
}

// ---------------------------------------------------------------- bounded workspace
// The per-token backward in rounds, for a workspace smaller than it needs at
// once: sequences cut into segments of about kRoundSeg tokens (whole chunks
// of the prefill's split), each segment's entering state and exiting
// adjoint as in launch_backward_split, then the packed-sequence backward over
// runs of one sequence's consecutive segments, as many per run as the rest of
// the workspace holds (whole sequences per run when a sequence is one
// segment). The runs go one after another on the stream.
constexpr int kRoundSeg = 512;

struct Rounds {
  int nseg, seg_len, req;  // as BwdSplit
  size_t trans, segst, states, cu, fixed;  // region bytes; fixed: their sum
};

Rounds rounds_plan(int B, int T, int H_qk, int H_v, int d_k, int d_v, bool bf16) {
  Rounds r{};
  r.nseg = 1;
  r.seg_len = T;
  r.req = 1;
  if (T > kRoundSeg) {
    PrefillArgs fa{};
    fa.B = B; fa.T = T; fa.H_qk = H_qk; fa.H_v = H_v; fa.d_k = d_k; fa.d_v = d_v;
    fa.chunk = 64;
    fa.bf16 = bf16;
    fa.nct = prefill_pick_nct(B, H_v, d_v);
    fa.force_nseg = (T + kRoundSeg - 1) / kRoundSeg;
    const PrefillPlan pl = prefill_plan(fa);
    if (pl.nseg >= 2 && pl.seg_len % kSweepL == 0) {
      r.nseg = pl.nseg;
      r.seg_len = pl.seg_len;
      r.req = fa.force_nseg;
    }
  }
  if (r.nseg >= 2) {
    const size_t mat = (size_t)H_v * d_k * d_v * 4;
    r.trans = align256((size_t)r.nseg * B * H_v * d_k * d_k * 4);
    r.segst = align256((size_t)r.nseg * B * mat);
    r.states = align256((size_t)B * r.nseg * mat);
    r.cu = align256((size_t)(r.nseg + 1) * 4);
  }
  r.fixed = r.trans + r.segst + 3 * r.states + r.cu;
  return r;
}

// workspace of one run: k segments of `tokens` tokens in all, or k whole sequences
size_t run_bytes(const Rounds &, int k, size_t tokens, int H_v, int d_k, int d_v) {
  return backward_workspace_bytes(k, tokens, H_v, d_k, d_v);
}

// Bytes per token of each token-major array: q, k (and dq, dk); v, dO (dv);
// a (da), b (db), w (dw) in the gate form's layout.
struct TokStrides {
  size_t qk, v, a, b, w;
};
TokStrides tok_strides(const BackwardArgs &a) {
  const size_t es = a.bf16 ? 2 : 4, gs = a.gate_form == kGatePre ? es : 4;
  const bool cpl = a.gate_form == kGateCoupled || a.gate_form == kGateScalar, sca = a.gate_form == kGateScalar;
  TokStrides t;
  t.qk = (size_t)a.H_qk * a.d_k * es;
  t.v = (size_t)a.H_v * a.d_v * es;
  t.a = sca ? (size_t)a.H_v * 4 : (size_t)a.H_v * a.d_k * gs;
  t.b = cpl ? (size_t)a.H_v * 4 : (size_t)a.H_v * a.d_k * gs;
  t.w = cpl ? 0 : (size_t)a.H_v * a.d_v * gs;
  return t;
}

// a's token arrays moved on by `tok` tokens
BackwardArgs at_token(const BackwardArgs &a, size_t tok) {
  const TokStrides t = tok_strides(a);
  auto in = [&](const void *p, size_t s) -> const void * { return p ? (const char *)p + tok * s : nullptr; };
  auto out = [&](void *p, size_t s) -> void * { return p ? (char *)p + tok * s : nullptr; };
  BackwardArgs c = a;
  c.q = in(a.q, t.qk); c.k = in(a.k, t.qk); c.v = in(a.v, t.v); c.dO = in(a.dO, t.v);
  c.a = (const float *)in(a.a, t.a); c.b = (const float *)in(a.b, t.b); c.w = (const float *)in(a.w, t.w);
  c.dq = out(a.dq, t.qk); c.dk = out(a.dk, t.qk); c.dv = out(a.dv, t.v);
  c.da = (float *)out(a.da, t.a); c.db = (float *)out(a.db, t.b); c.dw = (float *)out(a.dw, t.w);
  return c;
}

// Token offsets of a run of k segments of L tokens, the last ending at T_rem.
__global__ __launch_bounds__(256) void run_cu_kernel(int32_t *cu, int k, int L, int T_rem) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i <= k) cu[i] = min(i * L, T_rem);
}

hipError_t launch_backward_rounds(const BackwardArgs &a, hipStream_t st) {
  const Rounds r = rounds_plan(a.B, a.T, a.H_qk, a.H_v, a.d_k, a.d_v, a.bf16);
  if (a.workspace_bytes < r.fixed) return hipErrorInvalidValue;
  char *w = static_cast<char *>(a.workspace);
  char *inner = w + r.fixed;
  const size_t inner_bytes = a.workspace_bytes - r.fixed;
  const size_t mat = (size_t)a.H_v * a.d_k * a.d_v;  // floats of one state per sequence
  hipError_t e = hipSuccess;
  if (r.nseg < 2) {  // runs of whole sequences
    for (int n = 0; n < a.B;) {
      int m = 1;
      while (n + m < a.B && run_bytes(r, m + 1, (size_t)(m + 1) * a.T, a.H_v, a.d_k, a.d_v) <= inner_bytes) ++m;
      if (run_bytes(r, m, (size_t)m * a.T, a.H_v, a.d_k, a.d_v) > inner_bytes) return hipErrorInvalidValue;
      BackwardArgs c = at_token(a, (size_t)n * a.T);
      c.B = m;
      c.S0 = a.S0 ? a.S0 + (size_t)n * mat : nullptr;
      c.dST = a.dST ? a.dST + (size_t)n * mat : nullptr;
      c.dS0 = a.dS0 ? a.dS0 + (size_t)n * mat : nullptr;
      c.workspace = inner;
      c.workspace_bytes = inner_bytes;
      if ((e = launch_backward_per_token(c, st)) != hipSuccess) return e;
      n += m;
    }
    return hipSuccess;
  }
  float *trans = reinterpret_cast<float *>(w);
  float *segst = reinterpret_cast<float *>(w + r.trans);
  float *S_in = reinterpret_cast<float *>(w + r.trans + r.segst);
  float *Lout = reinterpret_cast<float *>(w + r.trans + r.segst + r.states);
  float *dS0_seg = reinterpret_cast<float *>(w + r.trans + r.segst + 2 * r.states);
  int32_t *cu = reinterpret_cast<int32_t *>(w + r.trans + r.segst + 3 * r.states);
  const bool coupled = a.gate_form == kGateCoupled || a.gate_form == kGateScalar;
  // entering states: the prefill's split passes (states only)
  PrefillArgs fa{};
  fa.B = a.B; fa.T = a.T; fa.H_qk = a.H_qk; fa.H_v = a.H_v; fa.d_k = a.d_k; fa.d_v = a.d_v;
  fa.chunk = 64;
  fa.bf16 = a.bf16;
  fa.nct = prefill_pick_nct(a.B, a.H_v, a.d_v);
  fa.q = a.q; fa.k = a.k; fa.v = a.v;
  fa.a = a.a; fa.b = a.b; fa.w = coupled ? a.b : a.w;
  fa.S0 = a.S0;
  fa.coupled = coupled;
  fa.scalar_decay = a.gate_form == kGateScalar;
  fa.preact = a.gate_form == kGatePre;
  fa.workspace = trans;
  fa.workspace_bytes = r.trans;
  fa.force_nseg = r.req;
  fa.seg_states = segst;
  const PrefillPlan fpl = prefill_plan(fa);
  if (fpl.nseg != r.nseg || fpl.seg_len != r.seg_len) return hipErrorInvalidValue;
  if ((e = launch_prefill(fa, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(split_states_kernel, dim3(a.B * r.nseg * a.H_v), dim3(256), 0, st, S_in, a.S0, segst, a.B,
                     a.H_v, r.nseg, a.d_k * a.d_v);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // exiting adjoints: the adjoint-only sweep
  SweepParams sw{};
  sw.q = a.q; sw.k = a.k; sw.a = a.a; sw.b = a.b; sw.dO = a.dO; sw.dST = a.dST;
  sw.Lout = Lout;
  sw.B = a.B; sw.T = a.T; sw.H_qk = a.H_qk; sw.H_v = a.H_v; sw.d_v = a.d_v;
  sw.nseg = r.nseg; sw.seg_len = r.seg_len;
  e = a.bf16 ? launch_sweep_bf16(sw, a.d_k, a.gate_form, st) : launch_sweep_f32(sw, a.d_k, a.gate_form, st);
  if (e != hipSuccess) return e;
  // runs of consecutive segments of one sequence
  const int L = r.seg_len;
  auto seg_tokens = [&](int j0, int j1) { return (size_t)(min(j1 * L, a.T) - j0 * L); };
  for (int n = 0; n < a.B; ++n) {
    for (int j = 0; j < r.nseg;) {
      int j1 = j + 1;
      while (j1 < r.nseg && run_bytes(r, j1 + 1 - j, seg_tokens(j, j1 + 1), a.H_v, a.d_k, a.d_v) <= inner_bytes) ++j1;
      if (run_bytes(r, j1 - j, seg_tokens(j, j1), a.H_v, a.d_k, a.d_v) > inner_bytes) return hipErrorInvalidValue;
      hipLaunchKernelGGL(run_cu_kernel, dim3((j1 - j + 256) / 256), dim3(256), 0, st, cu, j1 - j, L, a.T - j * L);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      BackwardArgs c = at_token(a, (size_t)n * a.T + (size_t)j * L);
      c.B = j1 - j;
      c.T = (int)seg_tokens(j, j1);
      c.cu_seqlens = cu;
      const size_t s0 = (size_t)n * r.nseg + j;
      c.S0 = S_in + s0 * mat;
      c.dST = Lout + s0 * mat;
      c.dS0 = a.dS0 ? dS0_seg + s0 * mat : nullptr;
      c.workspace = inner;
      c.workspace_bytes = inner_bytes;
      if ((e = launch_backward_per_token(c, st)) != hipSuccess) return e;
      j = j1;
    }
  }
  if (!a.dS0) return hipSuccess;
  hipLaunchKernelGGL(split_ds0_kernel, dim3(a.B * a.H_v), dim3(256), 0, st, a.dS0, dS0_seg, a.H_v, r.nseg,
                     a.d_k * a.d_v);
  return hipGetLastError();
}

size_t backward_rounds_min_bytes(int B, int T, int H_qk, int H_v, int d_k, int d_v, bool bf16) {
  const Rounds r = rounds_plan(B, T, H_qk, H_v, d_k, d_v, bf16);
  return r.fixed + (r.nseg >= 2 ? run_bytes(r, 1, (size_t)min(r.seg_len, T), H_v, d_k, d_v)
                                : run_bytes(r, 1, (size_t)T, H_v, d_k, d_v));
}

}  // namespace

hipError_t launch_split_states(float *S_in, const float *S0, const float *seg_states, int B, int H_v, int nseg,
                               int dkdv, hipStream_t st) {
  hipLaunchKernelGGL(split_states_kernel, dim3(B * nseg * H_v), dim3(256), 0, st, S_in, S0, seg_states, B, H_v, nseg,
                     dkdv);
  return hipGetLastError();
}

// The per-token backward all at once: unsplit, or the split plan's.
size_t per_token_workspace_bytes(int B, int T, int H_qk, int H_v, int d_k, int d_v, bool bf16) {
  const BwdSplit sp = backward_split_plan(B, T, H_qk, H_v, d_k, d_v, bf16);
  return sp.nseg < 2 ? backward_workspace_bytes(B, (size_t)B * T, H_v, d_k, d_v)
                     : split_layout(B, T, H_v, d_k, d_v, sp).total;
}

size_t backward_workspace_bytes_split(int B, int T, int H_qk, int H_v, int d_k, int d_v, bool bf16) {
  // Where the chunk form applies to the shape (bf16, d_k = d_v = 128): its
  // workspace, and at least the per-token backward's smallest in rounds
  // (what other gate forms, and chunks that decay too fast for the chunk
  // form, run in). Elsewhere the per-token backward's.
  // (GDN2_BACKWARD_CHUNKED=0, read at each call: the per-token backward's)
  const char *cenv = getenv("GDN2_BACKWARD_CHUNKED");
  const bool chunk_shape = bf16 && d_k == 128 && d_v == 128 && B > 0 && T > 0 && !(cenv && atoi(cenv) == 0);
  if (!chunk_shape) return per_token_workspace_bytes(B, T, H_qk, H_v, d_k, d_v, bf16);
  const size_t chunked = backward_chunked_workspace_bytes(B, T, H_qk, H_v);
  const size_t rounds = backward_rounds_min_bytes(B, T, H_qk, H_v, d_k, d_v, bf16);
  return chunked > rounds ? chunked : rounds;
}

// Checkpoints: per (head, column block) BT / kSub + B slots of d_k x CB fp32
// (each sequence needs at most ceil(T_n / kSub) <= T_n / kSub + 1 of them);
// key-side sums: ncb x BT x H_v x 4 x d_k fp32; k-reads: BT x H_v x d_v fp32;
// coupled gates' value-side sums: ncb x BT x H_v fp32.
// BT = B * T, or T for packed sequences.
size_t backward_workspace_bytes(int B, size_t BT, int H_v, int d_k, int d_v) {
  if (BT == 0) return 0;  // no tokens: only dS0 = dS_T, no scratch
  const size_t ncb = (size_t)d_v / bwd_cb(d_v);
  const size_t ck = (BT / kSub + B) * (size_t)H_v * d_k * d_v * 4;
  const size_t part = ncb * BT * H_v * 4 * d_k * 4;
  const size_t rk = BT * H_v * d_v * 4;
  const size_t ws = ncb * BT * H_v * 4;
  return align256(ck) + align256(part) + align256(rk) + align256(ws);
}

hipError_t launch_backward(const BackwardArgs &a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  // GDN2_BACKWARD_CHUNKED, read at each call: 0 never runs the chunk form, 2
  // requires it (hipErrorNotSupported where it cannot run), else it runs
  // wherever it applies
  const char *cenv = getenv("GDN2_BACKWARD_CHUNKED");
  const int cmode = cenv ? atoi(cenv) : 1;
  if (cmode != 0 && backward_chunked_eligible(a)) {
    bool ran = false;
    const hipError_t e = launch_backward_chunked(a, st, &ran);
    if (e != hipSuccess || ran) return e;
  }
  if (cmode == 2) return hipErrorNotSupported;
  if (!a.cu_seqlens &&
      a.workspace_bytes < per_token_workspace_bytes(a.B, a.T, a.H_qk, a.H_v, a.d_k, a.d_v, a.bf16))
    return launch_backward_rounds(a, st);
  if (!a.cu_seqlens) {
    const BwdSplit sp = backward_split_plan(a.B, a.T, a.H_qk, a.H_v, a.d_k, a.d_v, a.bf16);
    if (sp.nseg > 1) return launch_backward_split(a, sp, st);
  }
  return launch_backward_per_token(a, st);
}

#endif

}  // namespace gdn2
