// gdn2_prefill.hpp -- chunk-parallel prefill of the Gated DeltaNet-2
// recurrence (template; instantiated per dtype and d_k in gdn2_prefill_inst.hip).
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
// one wave per 16-column tile of the state (at least four waves: any beyond
// the column tiles only help with the build and the Gram tiles). Value columns of S evolve
// independently, so the split is exact. Per chunk:
//   1. all waves: cumulative decay (two-level product scan over the chunk),
//      scaled operands K*gamma | Q*gamma and K/gamma | beta/gamma into LDS
//      (the latter also transposed, for the carry), and each wave's U tile;
//      then the next chunk's raw inputs are requested into registers;
//   2. all waves: the four Gram matrices as MFMA tiles (lower triangles
//      only, a static balanced split of the tiles over the waves);
//   3. the 16x16 diagonal blocks of (I + Akb) inverted (one wave per block);
//   4. each wave, in registers, for its own 16 columns: (gamma*K|Q) S0,
//      Z = X + Akk U, blocked forward solve for R, outputs O, and the state
//      carry -- every product chained through MFMA accumulators (an
//      accumulator tile is already the next product's B operand).
#pragma once

#include <utility>

#include "gdn2_device.hpp"
#include "gdn2_internal.hpp"

namespace gdn2 {

template <int DK_, int C_, int NCT_, bool BF16_>
struct PrefillCfg {
  static constexpr int DK = DK_, C = C_, NCT = NCT_;
  static constexpr bool BF16 = BF16_;
  static constexpr int NW = NCT < 4 ? 4 : NCT;  // waves (>= 4: the build needs the threads)
  static constexpr int NT = 64 * NW;       // threads
  static constexpr int DVB = 16 * NCT;     // value columns per workgroup
  static constexpr int NRT = DK / 16;      // 16-row tiles of the state
  static constexpr int NCH = C / 16;       // 16-token tiles of a chunk
  static constexpr int PAD = BF16 ? 8 : 4; // 16 bytes of row padding
  static constexpr int PADT = BF16 ? 4 : 2;// 8 bytes of row padding (transposed copy)
  static constexpr int LDK = DK + PAD;     // row stride of kqg / kbi
  static constexpr int LDT = 2 * C + PADT; // row stride of kbiT
  static constexpr int LDC = C + PAD;      // row stride of akk / akbn
  static constexpr int LDM = 2 * C + PAD;  // row stride of m = [Mqk | Mqb]
  static constexpr int LDD = 16 + PAD;     // row stride of the diagonal inverses
  static constexpr int CP = DK / 2;        // channel pairs in the build
  static constexpr int RG0 = NT / CP;
  static constexpr int RG = RG0 < C / 2 ? RG0 : C / 2;  // row groups of the build
  static constexpr int RPG = C / RG;                    // rows per group (even)
  static_assert(DK % 16 == 0 && C % 16 == 0, "16-aligned tiles");
  static_assert(NT % CP == 0 && C % RG == 0 && RPG % 2 == 0, "build layout");
};

// Static split of the Gram tiles over the waves. A "half-row" is one
// 16-row block r of one quadrant (Akk, Akb, Mqk, Mqb) with its r+1 lower
// tiles; half-rows are dealt largest first to the least-loaded wave.
template <int NCH, int NW>
struct GramSchedule {
  static constexpr int MAXH = 4 * NCH;
  int nh[NW];            // half-rows per wave
  int quad[NW][MAXH];
  int row[NW][MAXH];
  constexpr GramSchedule() : nh(), quad(), row() {
    int load[NW] = {};
    for (int r = NCH - 1; r >= 0; --r)
      for (int q = 0; q < 4; ++q) {
        int best = 0;
        for (int w = 1; w < NW; ++w)
          if (load[w] < load[best]) best = w;
        quad[best][nh[best]] = q;
        row[best][nh[best]] = r;
        ++nh[best];
        load[best] += r + 1;
      }
  }
};

template <class Cf>
struct PrefillSmem {
  typedef typename Op<Cf::BF16>::T OT;
  OT kqg[2 * Cf::C * Cf::LDK];   // rows 0..C-1: k*gamma; rows C..2C-1: q*gamma
  OT kbi[2 * Cf::C * Cf::LDK];   // rows 0..C-1: k/gamma; rows C..2C-1: (b*k)/gamma
  OT kbiT[Cf::DK * Cf::LDT];     // kbi transposed: [channel][token (K part | beta part)]
  OT akk[Cf::C * Cf::LDC];       // Akk, lower blocks (strictly lower inside diagonal blocks)
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
  int B, T, H_qk, H_v, d_v;
};

// Load of type V at a wave-uniform base plus a 32-bit byte offset.
template <class V>
__device__ __forceinline__ V ldg(const void *base, uint32_t byte_off) {
  return *reinterpret_cast<const V *>(reinterpret_cast<const char *>(base) + byte_off);
}

// Chain a contraction over 16-deep blocks kb0..kb1-1 into acc, pairing blocks
// into K32 steps (see the operand convention in gdn2_device.hpp). An odd
// last block is padded with a zero half where the chain must keep one shape.
template <class O, int KB0, int KB1, class FA, class FB>
__device__ __forceinline__ floatx4 chain(floatx4 acc, FA fa, FB fb) {
#pragma unroll
  for (int kb = KB0; kb + 1 < KB1; kb += 2) acc = O::mma32(acc, fa(kb), fa(kb + 1), fb(kb), fb(kb + 1));
  if constexpr (((KB1 - KB0) & 1) != 0) {
    if constexpr (O::kK32Only)
      acc = O::mma32(acc, fa(KB1 - 1), O::zero(), fb(KB1 - 1), O::zero());
    else
      acc = O::mma16(acc, fa(KB1 - 1), fb(KB1 - 1));
  }
  return acc;
}

// Gram tiles of wave W: products of kqg rows with kbi rows over the channels.
template <class Cf, int W>
__device__ __forceinline__ void gram_wave(PrefillSmem<Cf> &sm, int lg, int lc) {
  using O = Op<Cf::BF16>;
  using Frag = typename O::Frag;
  constexpr int C = Cf::C, NRT = Cf::NRT, LDK = Cf::LDK, LDC = Cf::LDC, LDM = Cf::LDM;
  constexpr GramSchedule<Cf::NCH, Cf::NW> S{};
  constexpr int NH = S.nh[W];
  constexpr int NTILE = [] {
    int n = 0;
    for (int i = 0; i < S.nh[W]; ++i) n += S.row[W][i] + 1;
    return n;
  }();
  if constexpr (NTILE > 0) {
    floatx4 acc[NTILE];
#pragma unroll
    for (int i = 0; i < NTILE; ++i) acc[i] = zero4();
    auto frag = [&](const typename O::T *base, int row, int kb) -> Frag {
      return O::ld(base + (row + lc) * LDK + 16 * kb + 4 * lg);
    };
#pragma unroll
    for (int kb = 0; kb < NRT; kb += 2) {
      int ti = 0;
#pragma unroll
      for (int hr = 0; hr < NH; ++hr) {
        const int q = S.quad[W][hr], r = S.row[W][hr];
        const int arow = ((q >= 2) ? C : 0) + 16 * r;
        const Frag a0 = frag(sm.kqg, arow, kb);
        const Frag a1 = (kb + 1 < NRT) ? frag(sm.kqg, arow, kb + 1) : a0;
#pragma unroll
        for (int c = 0; c <= r; ++c, ++ti) {
          const int brow = ((q & 1) ? C : 0) + 16 * c;
          const Frag b0 = frag(sm.kbi, brow, kb);
          if (kb + 1 < NRT)
            acc[ti] = O::mma32(acc[ti], a0, a1, b0, frag(sm.kbi, brow, kb + 1));
          else if constexpr (O::kK32Only)
            acc[ti] = O::mma32(acc[ti], a0, O::zero(), b0, O::zero());
          else
            acc[ti] = O::mma16(acc[ti], a0, b0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // bound the operand loads in flight
    }
    int ti = 0;
#pragma unroll
    for (int hr = 0; hr < NH; ++hr) {
      const int q = S.quad[W][hr], r = S.row[W][hr];
#pragma unroll
      for (int c = 0; c <= r; ++c, ++ti) {
        const int s = 16 * c + lc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 16 * r + 4 * lg + j;
          const float x = acc[ti][j];
          if (q == 0) {
            sm.akk[t * LDC + s] = O::cvt(t > s ? x : 0.f);
          } else if (q == 1) {
            if (c == r)
              sm.akbd[r * 16 * 17 + (4 * lg + j) * 17 + lc] = (t > s) ? x : 0.f;
            else
              sm.akbn[t * LDC + s] = O::cvt(-x);
          } else if (q == 2) {
            sm.m[t * LDM + s] = O::cvt(t >= s ? x : 0.f);
          } else {
            sm.m[t * LDM + C + s] = O::cvt(t >= s ? x : 0.f);
          }
        }
      }
    }
  }
}

template <class Cf, int... Ws>
__device__ __forceinline__ void gram_dispatch(PrefillSmem<Cf> &sm, int wave, int lg, int lc,
                                              std::integer_sequence<int, Ws...>) {
  ((wave == Ws ? gram_wave<Cf, Ws>(sm, lg, lc) : void()), ...);
}

// Block -> (sequence, value head, column block). Workgroups are dealt
// round-robin to the 8 XCDs by linear id; the column blocks of one value
// head and the value heads sharing one query/key head re-read the same q, k,
// a, b rows, so they are placed on the same XCD (one L2) when a full group
// of 8 such units exists.
__device__ __forceinline__ void map_block(int L, int B, int H_qk, int H_v, int ncb, int &n, int &h,
                                          int &cb) {
  const int G = H_v / H_qk;
  const int U = G * ncb;               // workgroups sharing one query/key head
  const int nsh = B * H_qk;            // query/key heads in the batch
  const int full = (nsh / 8) * 8 * U;  // blocks covered by full groups of 8
  int sh, u;
  if (L < full) {
    sh = (L / (8 * U)) * 8 + (L & 7);
    u = (L >> 3) % U;
  } else {
    const int L2 = L - full;
    sh = (nsh / 8) * 8 + L2 / U;
    u = L2 % U;
  }
  n = sh / H_qk;
  h = (sh - n * H_qk) * G + u / ncb;
  cb = u % ncb;
}

template <int DK, int C, int NCT, bool BF16>
__global__ __launch_bounds__((PrefillCfg<DK, C, NCT, BF16>::NT)) void prefill_kernel(PrefillParams p) {
  using Cf = PrefillCfg<DK, C, NCT, BF16>;
  using E = Elem<BF16>;
  using O = Op<BF16>;
  using ET = typename E::T;
  using OT = typename O::T;
  using Frag = typename O::Frag;
  using Pair = typename std::conditional<BF16, uint32_t, floatx2>::type;  // two q/k elements
  constexpr int NRT = Cf::NRT, NCH = Cf::NCH, LDK = Cf::LDK, LDT = Cf::LDT, LDC = Cf::LDC,
                LDM = Cf::LDM, LDD = Cf::LDD, RPG = Cf::RPG;
  static_assert(sizeof(PrefillSmem<Cf>) <= 160 * 1024, "LDS working set exceeds one CU");

  __shared__ PrefillSmem<Cf> sm;

  int n, h, cb;
  map_block(blockIdx.x, p.B, p.H_qk, p.H_v, p.d_v / Cf::DVB, n, h, cb);
  const int g = h / (p.H_v / p.H_qk);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int lg = lane >> 4, lc = lane & 15;
  const int d_v = p.d_v;
  const bool colwave = wave < NCT;                 // owns a 16-column state tile
  const int col = cb * Cf::DVB + (colwave ? wave : 0) * 16 + lc;  // this lane's value column

  // Token strides in bytes, and this (sequence, head)'s token-0 bases.
  const uint32_t qk_tb = (uint32_t)(p.H_qk * DK) * sizeof(ET);
  const uint32_t ab_tb = (uint32_t)(p.H_v * DK) * 4u;
  const uint32_t v_tb = (uint32_t)(p.H_v * d_v) * sizeof(ET);
  const uint32_t w_tb = (uint32_t)(p.H_v * d_v) * 4u;
  const size_t tok0 = (size_t)n * p.T;
  const ET *qh = (const ET *)p.q + tok0 * p.H_qk * DK + (size_t)g * DK;
  const ET *kh = (const ET *)p.k + tok0 * p.H_qk * DK + (size_t)g * DK;
  const ET *vh = (const ET *)p.v + tok0 * p.H_v * d_v + (size_t)h * d_v;
  const float *ah = p.a + tok0 * p.H_v * DK + (size_t)h * DK;
  const float *bh = p.b + tok0 * p.H_v * DK + (size_t)h * DK;
  const float *wh = p.w + tok0 * p.H_v * d_v + (size_t)h * d_v;
  ET *oh = (ET *)p.o + tok0 * p.H_v * d_v + (size_t)h * d_v;
  const size_t s_off = ((size_t)n * p.H_v + h) * (size_t)DK * d_v + col;

  // State tiles: S[rt][j] = S[16*rt + 4*lg + j][col] (accumulator layout).
  floatx4 S[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[rt][j] = (p.S0 && colwave) ? p.S0[s_off + (size_t)(16 * rt + 4 * lg + j) * d_v] : 0.f;

  // Token-by-token steps on this wave's columns (exact for any decay).
  auto token_steps = [&](int tb, int te) {
    if (!colwave) return;
    for (int t = tb; t < te; ++t) {
      const float *at = ah + (size_t)t * (ab_tb / 4);
      const float *bt = bh + (size_t)t * (ab_tb / 4);
      const ET *kt = kh + (size_t)t * (qk_tb / sizeof(ET));
      const ET *qt = qh + (size_t)t * (qk_tb / sizeof(ET));
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
      const float u = wh[(size_t)t * (w_tb / 4) + col] * E::ld(vh + (size_t)t * (v_tb / sizeof(ET)) + col);
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
      if (lg == 0) E::st(oh + (size_t)t * (v_tb / sizeof(ET)) + col, po);
    }
  };

  const int nfull = p.T / C;
  const int cp = tid % Cf::CP, rgi = tid / Cf::CP, ch0 = 2 * cp;
  const bool builder = rgi < Cf::RG;
  // Byte offsets of this thread's build rows/channels within a chunk, and of
  // this lane's U elements (token 16c + 4lg + j, column col).
  const uint32_t ab_off = (uint32_t)(rgi * RPG) * ab_tb + (uint32_t)ch0 * 4u;
  const uint32_t qk_off = (uint32_t)(rgi * RPG) * qk_tb + (uint32_t)ch0 * sizeof(ET);
  const uint32_t v_off = (uint32_t)(4 * lg) * v_tb + (uint32_t)col * sizeof(ET);
  const uint32_t w_off = (uint32_t)(4 * lg) * w_tb + (uint32_t)col * 4u;

  // Raw inputs of one chunk, held in registers (prefetched one chunk ahead).
  floatx2 ra[RPG], rb[RPG];
  Pair rk[RPG], rq[RPG];
  float rw[NCH * 4];
  ET rv[NCH * 4];
  // Bytes from a chunk's first token to the end of this sequence's rows, for
  // the buffer descriptors' range (a chunk never reads past its sequence).
  auto rows_left = [&](int t0, uint32_t tb) -> uint32_t { return (uint32_t)(p.T - t0) * tb; };
  auto load_raw = [&](int t0) {
    if (builder) {
      const rsrc_t ra_ = make_rsrc((const char *)ah + (size_t)t0 * ab_tb, rows_left(t0, ab_tb));
      const rsrc_t rb_ = make_rsrc((const char *)bh + (size_t)t0 * ab_tb, rows_left(t0, ab_tb));
      const rsrc_t rk_ = make_rsrc((const char *)kh + (size_t)t0 * qk_tb, rows_left(t0, qk_tb));
      const rsrc_t rq_ = make_rsrc((const char *)qh + (size_t)t0 * qk_tb, rows_left(t0, qk_tb));
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        ra[r] = bload<floatx2>(ra_, ab_off, r * ab_tb);
        rb[r] = bload<floatx2>(rb_, ab_off, r * ab_tb);
        rk[r] = bload<Pair>(rk_, qk_off, r * qk_tb);
        rq[r] = bload<Pair>(rq_, qk_off, r * qk_tb);
      }
    }
    if (colwave) {
      const rsrc_t rv_ = make_rsrc((const char *)vh + (size_t)t0 * v_tb, rows_left(t0, v_tb));
      const rsrc_t rw_ = make_rsrc((const char *)wh + (size_t)t0 * w_tb, rows_left(t0, w_tb));
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rv[4 * c + j] = bload<ET>(rv_, v_off, (16 * c + j) * v_tb);
          rw[4 * c + j] = bload<float>(rw_, w_off, (16 * c + j) * w_tb);
        }
    }
  };
  auto pair_f = [](Pair x) -> floatx2 {
    if constexpr (BF16)
      return floatx2{__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u)};
    else
      return x;
  };

  if (nfull > 0) load_raw(0);

  for (int chk = 0; chk < nfull; ++chk) {
    const int t0 = chk * C;
    // ---------------------------------------------------------------- 1. build
    floatx2 gl[RPG];
    if (builder) {
      floatx2 pr = {1.f, 1.f};
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        pr *= ra[r];
        gl[r] = pr;
      }
      *reinterpret_cast<floatx2 *>(&sm.tot[rgi * DK + ch0]) = pr;
    }
    // this wave's U tile: U[16c + 4lg + j][col] = w * v
    Frag Uf[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      floatx4 u;
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = rw[4 * c + j] * E::f(rv[4 * c + j]);
      Uf[c] = O::from_acc(u);
    }
    __syncthreads();
    int bad = 0;
    if (builder) {
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
      for (int r = 0; r < RPG; r += 2) {
        const int tl = rgi * RPG + r;
        floatx2 kb[2], bk[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const floatx2 gm = pre * gl[r + e];
          const floatx2 gi = {__builtin_amdgcn_rcpf(gm[0]), __builtin_amdgcn_rcpf(gm[1])};
          const floatx2 kv = pair_f(rk[r + e]);
          const floatx2 qv = pair_f(rq[r + e]);
          O::st2(&sm.kqg[(tl + e) * LDK + ch0], kv[0] * gm[0], kv[1] * gm[1]);
          O::st2(&sm.kqg[(C + tl + e) * LDK + ch0], qv[0] * gm[0], qv[1] * gm[1]);
          kb[e] = kv * gi;
          bk[e] = rb[r + e] * kv * gi;
          O::st2(&sm.kbi[(tl + e) * LDK + ch0], kb[e][0], kb[e][1]);
          O::st2(&sm.kbi[(C + tl + e) * LDK + ch0], bk[e][0], bk[e][1]);
        }
        // transposed copy: two consecutive tokens per channel
        O::st2(&sm.kbiT[ch0 * LDT + tl], kb[0][0], kb[1][0]);
        O::st2(&sm.kbiT[(ch0 + 1) * LDT + tl], kb[0][1], kb[1][1]);
        O::st2(&sm.kbiT[ch0 * LDT + C + tl], bk[0][0], bk[1][0]);
        O::st2(&sm.kbiT[(ch0 + 1) * LDT + C + tl], bk[0][1], bk[1][1]);
      }
    }
    bad = __syncthreads_or(bad);
    if (bad) {
      token_steps(t0, t0 + C);
      if (chk + 1 < nfull) load_raw(t0 + C);
      __syncthreads();
      continue;
    }
    if (chk + 1 < nfull) load_raw(t0 + C);  // next chunk's inputs stream in meanwhile

    // ---------------------------------------------------------------- 2. Gram tiles
    gram_dispatch<Cf>(sm, wave, lg, lc, std::make_integer_sequence<int, Cf::NW>{});
    __syncthreads();

    // ---------------------------------------------------------------- 3. diagonal inverses
    for (int r = wave; r < NCH; r += Cf::NW) {
      if (lane < 16) {
        const float *A = &sm.akbd[r * 16 * 17];
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == lane) ? 1.f : 0.f;
        // column `lane` of (I + A)^-1 by forward substitution, axpy form
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
          for (int i2 = i + 1; i2 < 16; ++i2) x[i2] -= A[i2 * 17 + i] * x[i];
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.dinv[r * 16 * LDD + i * LDD + lane] = O::cvt(x[i]);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- 4. per-wave columns
    if (colwave) {
      Frag Sf[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) Sf[rt] = O::from_acc(S[rt]);
      auto rowfrag = [&](const OT *base, int ld, int row, int colblk) -> Frag {
        return O::ld(base + (row + lc) * ld + 16 * colblk + 4 * lg);
      };
      auto sfrag = [&](int kb) { return Sf[kb]; };

      // X = (gamma * K) S0, Y = (gamma * Q) S0
      floatx4 X[NCH], Y[NCH];
#pragma unroll
      for (int r = 0; r < NCH; ++r) {
        X[r] = chain<O, 0, NRT>(zero4(), [&](int kb) { return rowfrag(sm.kqg, LDK, 16 * r, kb); }, sfrag);
        Y[r] = chain<O, 0, NRT>(zero4(), [&](int kb) { return rowfrag(sm.kqg, LDK, C + 16 * r, kb); }, sfrag);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Z = X + Akk U, then (I + Akb) R = Z by blocked forward substitution:
      // R_r = D_r (Z_r - sum_{c<r} Akb_rc R_c), as one chain over
      // [Akk blocks 0..r with U] ++ [-Akb blocks 0..r-1 with R].
      Frag Rf[NCH], Rn[NCH];
      static_for<NCH>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        auto fa = [&](int kb) {
          return kb <= r ? rowfrag(sm.akk, LDC, 16 * r, kb) : rowfrag(sm.akbn, LDC, 16 * r, kb - r - 1);
        };
        auto fb = [&](int kb) { return kb <= r ? Uf[kb] : Rf[kb - r - 1]; };
        const floatx4 acc = chain<O, 0, 2 * r + 1>(X[r], fa, fb);
        const floatx4 R = chain<O, 0, 1>(
            zero4(), [&](int) { return rowfrag(sm.dinv + r * 16 * LDD, LDD, 0, 0); },
            [&](int) { return O::from_acc(acc); });
        Rf[r] = O::from_acc(R);
        Rn[r] = O::from_acc(-R);
      });
      // O = Y + Mqk U - Mqb R, one chain over [Mqk blocks 0..r | Mqb blocks 0..r]
      const rsrc_t ro_ = make_rsrc((const char *)oh + (size_t)t0 * v_tb, rows_left(t0, v_tb));
      static_for<NCH>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        auto fa = [&](int kb) {
          return kb <= r ? rowfrag(sm.m, LDM, 16 * r, kb) : rowfrag(sm.m, LDM, 16 * r, NCH + kb - r - 1);
        };
        auto fb = [&](int kb) { return kb <= r ? Uf[kb] : Rn[kb - r - 1]; };
        const floatx4 acc = chain<O, 0, 2 * r + 2>(Y[r], fa, fb);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (BF16)
            bstore(f32_to_bf16(acc[j]), ro_, v_off, (16 * r + j) * v_tb);
          else
            bstore(acc[j], ro_, v_off, (16 * r + j) * v_tb);
        }
      });
      // S_C = diag(gamma_C) (S0 + (K/gamma)^T U - (beta/gamma)^T R)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        auto fa = [&](int kb) { return rowfrag(sm.kbiT, LDT, 16 * rt, kb); };
        auto fb = [&](int kb) { return kb < NCH ? Uf[kb] : Rn[kb - NCH]; };
        const floatx4 acc = chain<O, 0, 2 * NCH>(S[rt], fa, fb);
        const floatx4 gc = *reinterpret_cast<const floatx4 *>(&sm.gamc[16 * rt + 4 * lg]);
        S[rt] = acc * gc;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // LDS is rebuilt by the next chunk
  }

  if (nfull * C < p.T) token_steps(nfull * C, p.T);

  if (p.S_T && colwave) {
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
  p.B = a.B; p.T = a.T; p.H_qk = a.H_qk; p.H_v = a.H_v; p.d_v = a.d_v;
  const int blocks = (a.d_v / (16 * NCT)) * a.H_v * a.B;
  hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16>), dim3(blocks),
                     dim3(PrefillCfg<DK, C, NCT, BF16>::NT), 0, st, p);
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
