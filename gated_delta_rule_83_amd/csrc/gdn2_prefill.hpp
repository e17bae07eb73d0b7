// gdn2_prefill.hpp -- chunk-parallel prefill of the Gated DeltaNet-2
// recurrence (template; instantiated per dtype in gdn2_prefill_*.hip).
//
// The recurrence per token (Gated DeltaNet-2 post on tilnote.io, GDN-2
// design section; delta-rule tutorial on ai-systems-engineering.com, "record
// the difference" and beta sections):
//   S_t = diag(a_t) S_{t-1} - (b_t * k_t) r_t^T + k_t (w_t * v_t)^T,
//   r_t = (diag(a_t) S_{t-1})^T k_t,   o_t = S_t^T q_t.
//
// Chunk form. Unrolling C tokens from the entering state S0 with
// gamma_t = prod_{s<=t} a_s (channel-wise), beta_s = b_s * k_s, u_s = w_s * v_s:
//   Akk[t,s] = sum_i (k_t gamma_t)_i (k_s / gamma_s)_i      s < t
//   Akb[t,s] = sum_i (k_t gamma_t)_i (beta_s / gamma_s)_i   s < t
//   Mqk[t,s] = sum_i (q_t gamma_t)_i (k_s / gamma_s)_i      s <= t
//   Mqb[t,s] = sum_i (q_t gamma_t)_i (beta_s / gamma_s)_i   s <= t
//   (I + Akb) R = (gamma * K) S0 + Akk U          (row t of R is the key read r_t)
//   O  = (gamma * Q) S0 + Mqk U - Mqb R
//   S_C = diag(gamma_C) (S0 + (K / gamma)^T U - (beta / gamma)^T R)
// The factor gamma_t / gamma_s <= 1 is split against the chunk start (the
// anchor), so each MFMA operand carries one factor. Both factors only rescale
// elements, so bf16/fp32 rounding stays relative; the only risk is range,
// which is bounded by requiring gamma_C >= e^-60 on every channel. A chunk
// that fails this test (very strong decay) is stepped token by token, which
// is exact for any decay. Rescaling cumulative gates against an in-block
// anchor so that no ratio explodes is the device the FiX analysis on
// iplexlaw.co.kr describes for its block-wise kernel (section 5); here the
// blocks are the prefill's chunks.
//
// Workgroup = one (sequence, value head, block of 16*NCT value columns);
// one wave per 16-column tile of the state. Value columns of S evolve
// independently, so the split is exact. Per chunk:
//   1. all waves: cumulative decay (two-level product scan over the chunk),
//      scaled operands K*gamma | Q*gamma and K/gamma | beta/gamma into LDS;
//   2. all waves: the four Gram matrices as 16x16 MFMA tiles (lower
//      triangles only), masked and stored to LDS;
//   3. the 16x16 diagonal blocks of (I + Akb) inverted by forward
//      substitution (one wave per block);
//   4. each wave, in registers, for its own 16 columns: (gamma*K|Q) S0,
//      Z = X + Akk U, blocked forward solve for R, outputs O, and the state
//      carry -- every product chained through MFMA accumulators with no
//      further LDS traffic for the state, U or R.
#pragma once

#include "gdn2_device.hpp"
#include "gdn2_internal.hpp"

namespace gdn2 {

template <int DK_, int C_, int NCT_, bool BF16_>
struct PrefillCfg {
  static constexpr int DK = DK_, C = C_, NCT = NCT_;
  static constexpr bool BF16 = BF16_;
  static constexpr int NW = NCT;           // waves per workgroup
  static constexpr int NT = 64 * NW;       // threads
  static constexpr int DVB = 16 * NCT;     // value columns per workgroup
  static constexpr int NRT = DK / 16;      // 16-row tiles of the state
  static constexpr int NCH = C / 16;       // 16-token tiles of a chunk
  static constexpr int PAD = BF16 ? 8 : 4; // 16 bytes of row padding
  static constexpr int LDK = DK + PAD;     // row stride of sKQg / sKBi
  static constexpr int LDC = C + PAD;      // row stride of sAkk / sAkbN
  static constexpr int LDM = 2 * C + PAD;  // row stride of sM = [Mqk | Mqb]
  static constexpr int LDD = 16 + PAD;     // row stride of the diagonal inverses
  static constexpr int CP = DK / 2;        // channel pairs in the build
  static constexpr int RG0 = NT / CP;
  static constexpr int RG = RG0 < C ? RG0 : C;  // row groups of the build
  static constexpr int RPG = C / RG;            // rows per group
  static constexpr int NTRI = NCH * (NCH + 1) / 2;
  static constexpr int NGT = 4 * NTRI;          // Gram tiles computed per chunk
  static_assert(DK % 16 == 0 && C % 16 == 0, "16-aligned tiles");
  static_assert(NT % CP == 0 && C % RG == 0, "build layout");
};

template <class Cf>
struct PrefillSmem {
  typedef typename Op<Cf::BF16>::T OT;
  OT kqg[2 * Cf::C * Cf::LDK];   // rows 0..C-1: k*gamma; rows C..2C-1: q*gamma
  OT kbi[2 * Cf::C * Cf::LDK];   // rows 0..C-1: k/gamma; rows C..2C-1: (b*k)/gamma
  OT akk[Cf::C * Cf::LDC];       // Akk, strictly lower blocks
  OT akbn[Cf::C * Cf::LDC];      // -Akb, off-diagonal lower blocks
  OT m[Cf::C * Cf::LDM];         // [Mqk | Mqb], lower blocks incl. diagonal
  OT dinv[Cf::NCH * 16 * Cf::LDD];     // (I + Akb_rr)^-1 per diagonal block
  float akbd[Cf::NCH * 16 * 17];       // Akb diagonal blocks (fp32) for the inverses
  float gamc[Cf::DK];                  // gamma_C per key channel
  float tot[Cf::RG * Cf::DK];          // per-group decay products of the scan
};

struct PrefillParams {
  const void *q, *k, *v;
  const float *a, *b, *w, *S0;
  void *o;
  float *S_T;
  int T, H_qk, H_v, d_v;
};

template <int DK, int C, int NCT, bool BF16>
__global__ __launch_bounds__(64 * NCT) void prefill_kernel(PrefillParams p) {
  using Cf = PrefillCfg<DK, C, NCT, BF16>;
  using E = Elem<BF16>;
  using O = Op<BF16>;
  using ET = typename E::T;
  using Frag = typename O::Frag;
  constexpr int NRT = Cf::NRT, NCH = Cf::NCH, LDK = Cf::LDK, LDC = Cf::LDC, LDM = Cf::LDM,
                LDD = Cf::LDD;

  __shared__ PrefillSmem<Cf> sm;

  const int cb = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int g = h / (p.H_v / p.H_qk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  const int d_v = p.d_v;
  const int col = cb * Cf::DVB + wave * 16 + lc;  // this lane's value column

  const size_t qk_tok = (size_t)p.H_qk * DK, ab_tok = (size_t)p.H_v * DK;
  const size_t vw_tok = (size_t)p.H_v * d_v;
  const size_t tok0 = (size_t)n * p.T;
  const ET *qh = (const ET *)p.q + tok0 * qk_tok + (size_t)g * DK;
  const ET *kh = (const ET *)p.k + tok0 * qk_tok + (size_t)g * DK;
  const ET *vh = (const ET *)p.v + tok0 * vw_tok + (size_t)h * d_v + col;
  const float *ah = p.a + tok0 * ab_tok + (size_t)h * DK;
  const float *bh = p.b + tok0 * ab_tok + (size_t)h * DK;
  const float *wh = p.w + tok0 * vw_tok + (size_t)h * d_v + col;
  ET *oh = (ET *)p.o + tok0 * vw_tok + (size_t)h * d_v + col;
  const size_t s_off = ((size_t)n * p.H_v + h) * (size_t)DK * d_v + col;

  // State tiles: S[rt][j] = S[16*rt + 4*lg + j][col] (accumulator layout).
  floatx4 S[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[rt][j] = p.S0 ? p.S0[s_off + (size_t)(16 * rt + 4 * lg + j) * d_v] : 0.f;

  // Token-by-token steps on this wave's columns (exact for any decay).
  auto token_steps = [&](int tb, int te) {
    for (int t = tb; t < te; ++t) {
      const float *at = ah + (size_t)t * ab_tok;
      const float *bt = bh + (size_t)t * ab_tok;
      const ET *kt = kh + (size_t)t * qk_tok;
      const ET *qt = qh + (size_t)t * qk_tok;
      float part = 0.f;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int i0 = 16 * rt + 4 * lg;
        const floatx4 av = *reinterpret_cast<const floatx4 *>(at + i0);
        const floatx4 kv = E::ld4(kt + i0);
        S[rt] *= av;
        part += S[rt][0] * kv[0] + S[rt][1] * kv[1] + S[rt][2] * kv[2] + S[rt][3] * kv[3];
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);  // key read r for this column
      const float u = wh[(size_t)t * vw_tok] * E::ld(vh + (size_t)t * vw_tok);
      float po = 0.f;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int i0 = 16 * rt + 4 * lg;
        const floatx4 bv = *reinterpret_cast<const floatx4 *>(bt + i0);
        const floatx4 kv = E::ld4(kt + i0);
        const floatx4 qv = E::ld4(qt + i0);
        S[rt] = S[rt] - (bv * kv) * part + kv * u;
        po += S[rt][0] * qv[0] + S[rt][1] * qv[1] + S[rt][2] * qv[2] + S[rt][3] * qv[3];
      }
      po += __shfl_xor(po, 16, 64);
      po += __shfl_xor(po, 32, 64);
      if (lg == 0) E::st(oh + (size_t)t * vw_tok, po);
    }
  };

  const int nfull = p.T / C;
  const int cp = tid % Cf::CP, rgi = tid / Cf::CP, ch0 = 2 * cp;

  for (int chk = 0; chk < nfull; ++chk) {
    const int t0 = chk * C;
    // ---------------------------------------------------------------- 1. build
    floatx2 gl[Cf::RPG];
    if (rgi < Cf::RG) {
      floatx2 pr = {1.f, 1.f};
#pragma unroll
      for (int r = 0; r < Cf::RPG; ++r) {
        const int t = t0 + rgi * Cf::RPG + r;
        pr *= *reinterpret_cast<const floatx2 *>(ah + (size_t)t * ab_tok + ch0);
        gl[r] = pr;
      }
      *reinterpret_cast<floatx2 *>(&sm.tot[rgi * DK + ch0]) = pr;
    }
    __syncthreads();
    int bad = 0;
    if (rgi < Cf::RG) {
      floatx2 pre = {1.f, 1.f}, tot = {1.f, 1.f};
#pragma unroll
      for (int gg = 0; gg < Cf::RG; ++gg) {
        const floatx2 x = *reinterpret_cast<const floatx2 *>(&sm.tot[gg * DK + ch0]);
        if (gg < rgi) pre *= x;
        tot *= x;
      }
      if (rgi == 0) {
        *reinterpret_cast<floatx2 *>(&sm.gamc[ch0]) = tot;
        bad = !(tot[0] >= kMinChunkDecay) || !(tot[1] >= kMinChunkDecay);
      }
#pragma unroll
      for (int r = 0; r < Cf::RPG; ++r) {
        const int tl = rgi * Cf::RPG + r;
        const size_t t = (size_t)(t0 + tl);
        const floatx2 gm = pre * gl[r];
        const floatx2 gi = {__builtin_amdgcn_rcpf(gm[0]), __builtin_amdgcn_rcpf(gm[1])};
        const floatx2 kv = E::ld2(kh + t * qk_tok + ch0);
        const floatx2 qv = E::ld2(qh + t * qk_tok + ch0);
        const floatx2 bv = *reinterpret_cast<const floatx2 *>(bh + t * ab_tok + ch0);
        O::st2(&sm.kqg[tl * LDK + ch0], kv[0] * gm[0], kv[1] * gm[1]);
        O::st2(&sm.kqg[(C + tl) * LDK + ch0], qv[0] * gm[0], qv[1] * gm[1]);
        O::st2(&sm.kbi[tl * LDK + ch0], kv[0] * gi[0], kv[1] * gi[1]);
        O::st2(&sm.kbi[(C + tl) * LDK + ch0], bv[0] * kv[0] * gi[0], bv[1] * kv[1] * gi[1]);
      }
    }
    bad = __syncthreads_or(bad);
    if (bad) {
      token_steps(t0, t0 + C);
      __syncthreads();  // nothing shared was touched; keeps waves in step
      continue;
    }

    // ---------------------------------------------------------------- 2. Gram tiles
    for (int tile = wave; tile < Cf::NGT; tile += Cf::NW) {
      const int quad = tile / Cf::NTRI;
      int idx = tile - quad * Cf::NTRI, r = 0;
      while ((r + 1) * (r + 2) / 2 <= idx) ++r;
      const int c = idx - r * (r + 1) / 2;
      const int arow = ((quad >= 2) ? C : 0) + 16 * r;
      const int brow = ((quad & 1) ? C : 0) + 16 * c;
      floatx4 acc = zero4();
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        const Frag fa = O::ld_row(&sm.kqg[(arow + lc) * LDK + 16 * kt + 4 * lg]);
        const Frag fb = O::ld_row(&sm.kbi[(brow + lc) * LDK + 16 * kt + 4 * lg]);
        acc = O::mma(acc, fa, fb);
      }
      const int s = 16 * c + lc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * r + 4 * lg + j;
        const float x = acc[j];
        if (quad == 0) {
          sm.akk[t * LDC + s] = O::cvt(t > s ? x : 0.f);
        } else if (quad == 1) {
          if (c == r)
            sm.akbd[r * 16 * 17 + (4 * lg + j) * 17 + lc] = (t > s) ? x : 0.f;
          else
            sm.akbn[t * LDC + s] = O::cvt(-x);
        } else if (quad == 2) {
          sm.m[t * LDM + s] = O::cvt(t >= s ? x : 0.f);
        } else {
          sm.m[t * LDM + C + s] = O::cvt(t >= s ? x : 0.f);
        }
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- 3. diagonal inverses
    for (int r = wave; r < NCH; r += Cf::NW) {
      if (lane < 16) {
        const float *A = &sm.akbd[r * 16 * 17];
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = (i == lane) ? 1.f : 0.f;
#pragma unroll
          for (int si = 0; si < i; ++si) s -= A[i * 17 + si] * x[si];
          x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.dinv[r * 16 * LDD + i * LDD + lane] = O::cvt(x[i]);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- 4. per-wave columns
    Frag Uf[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      floatx4 u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t t = (size_t)(t0 + 16 * c + 4 * lg + j);
        u[j] = wh[t * vw_tok] * E::ld(vh + t * vw_tok);
      }
      Uf[c] = O::from_acc(u);
    }
    Frag Sf[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) Sf[rt] = O::from_acc(S[rt]);

    // X = (gamma * K) S0 and Y = (gamma * Q) S0
    floatx4 X[NCH], Y[NCH];
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      X[r] = zero4();
      Y[r] = zero4();
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt) {
        X[r] = O::mma(X[r], O::ld_row(&sm.kqg[(16 * r + lc) * LDK + 16 * kt + 4 * lg]), Sf[kt]);
        Y[r] = O::mma(Y[r], O::ld_row(&sm.kqg[(C + 16 * r + lc) * LDK + 16 * kt + 4 * lg]), Sf[kt]);
      }
    }
    // Z = X + Akk U, then (I + Akb) R = Z by blocked forward substitution.
    Frag Rf[NCH], Rn[NCH];
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      floatx4 acc = X[r];
#pragma unroll
      for (int c = 0; c <= r; ++c)
        acc = O::mma(acc, O::ld_row(&sm.akk[(16 * r + lc) * LDC + 16 * c + 4 * lg]), Uf[c]);
#pragma unroll
      for (int c = 0; c < r; ++c)
        acc = O::mma(acc, O::ld_row(&sm.akbn[(16 * r + lc) * LDC + 16 * c + 4 * lg]), Rf[c]);
      const floatx4 R =
          O::mma(zero4(), O::ld_row(&sm.dinv[r * 16 * LDD + lc * LDD + 4 * lg]), O::from_acc(acc));
      Rf[r] = O::from_acc(R);
      Rn[r] = O::from_acc_neg(R);
    }
    // O = Y + Mqk U - Mqb R
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      floatx4 acc = Y[r];
#pragma unroll
      for (int c = 0; c <= r; ++c) {
        acc = O::mma(acc, O::ld_row(&sm.m[(16 * r + lc) * LDM + 16 * c + 4 * lg]), Uf[c]);
        acc = O::mma(acc, O::ld_row(&sm.m[(16 * r + lc) * LDM + C + 16 * c + 4 * lg]), Rn[c]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) E::st(oh + (size_t)(t0 + 16 * r + 4 * lg + j) * vw_tok, acc[j]);
    }
    // S_C = diag(gamma_C) (S0 + (K/gamma)^T U - (beta/gamma)^T R)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      floatx4 acc = S[rt];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        acc = O::mma(acc, O::ld_col(&sm.kbi[(16 * c + 4 * lg) * LDK + 16 * rt + lc], LDK), Uf[c]);
        acc = O::mma(acc, O::ld_col(&sm.kbi[(C + 16 * c + 4 * lg) * LDK + 16 * rt + lc], LDK), Rn[c]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] *= sm.gamc[16 * rt + 4 * lg + j];
      S[rt] = acc;
    }
    __syncthreads();  // LDS is rebuilt by the next chunk
  }

  if (nfull * C < p.T) token_steps(nfull * C, p.T);

  if (p.S_T) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) p.S_T[s_off + (size_t)(16 * rt + 4 * lg + j) * d_v] = S[rt][j];
  }
}

template <int DK, int C, int NCT, bool BF16>
hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t st) {
  PrefillParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.a = a.a; p.b = a.b; p.w = a.w; p.S0 = a.S0;
  p.o = a.o; p.S_T = a.S_T;
  p.T = a.T; p.H_qk = a.H_qk; p.H_v = a.H_v; p.d_v = a.d_v;
  const dim3 grid(a.d_v / (16 * NCT), a.H_v, a.B);
  hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16>), grid, dim3(64 * NCT), 0, st, p);
  return hipGetLastError();
}

template <int DK, int C, bool BF16>
hipError_t dispatch_prefill_nct(const PrefillArgs &a, hipStream_t st) {
  switch (a.nct) {
    case 1: return launch_prefill_t<DK, C, 1, BF16>(a, st);
    case 4: return launch_prefill_t<DK, C, 4, BF16>(a, st);
    case 8: return launch_prefill_t<DK, C, 8, BF16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn2
