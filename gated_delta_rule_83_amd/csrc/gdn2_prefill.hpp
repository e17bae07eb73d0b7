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
// Everything that does not depend on the entering state (scaled operands,
// the Gram matrices, the inverses of the diagonal blocks of I + Akb) is
// computed one chunk ahead by four producer waves, while four consumer
// waves run the state-dependent part of the previous chunk. A workgroup of
// 8 waves handles one (sequence, value head, block of 16*NCT value columns,
// NCT = 1, 2 or 4); consumer wave w < NCT owns the 16-column state tile w.
// Value columns of S evolve independently, so the column split is exact.
// Step s of the pipeline (chunk s produced into LDS buffer s%2, chunk s-1
// consumed from buffer (s-1)%2), with one workgroup barrier after each phase:
//   A. producers: decay scan (wave-local, across lanes), scaled operands
//      K*gamma | Q*gamma, K/gamma | beta/gamma (also transposed), U = w*v;
//      then the next chunk's raw inputs are requested into registers.
//      consumers: X = (gamma*K) S0, Y = (gamma*Q) S0.
//   B. producer wave q: Gram quadrant q (Akk, Akb, Mqk, Mqb), lower tiles.
//      consumers: Z = X + Akk U and the blocked forward solve for R.
//   C. producer wave 0: inverses of the 16x16 diagonal blocks of I + Akb.
//      consumers: outputs O and the state carry.
// Consumer products are chained through MFMA accumulators: an accumulator
// tile is already the next product's B operand.
#pragma once

#include <utility>

#include "gdn2_device.hpp"
#include "gdn2_internal.hpp"

namespace gdn2 {

template <int DK_, int C_, int NCT_, bool BF16_>
struct PrefillCfg {
  static constexpr int DK = DK_, C = C_, NCT = NCT_;
  static constexpr bool BF16 = BF16_;
  static constexpr int NP = 4;             // producer waves
  static constexpr int NW = 8;             // waves per workgroup (4 producers + 4 consumers)
  static constexpr int NT = 64 * NW;       // threads
  static constexpr int DVB = 16 * NCT;     // value columns per workgroup (one consumer wave per 16)
  static constexpr int NRT = DK / 16;      // 16-row tiles of the state
  static constexpr int NCH = C / 16;       // 16-token tiles of a chunk
  static constexpr int NTRI = NCH * (NCH + 1) / 2;  // lower 16x16 tiles of a C x C matrix
  static constexpr int PAD = BF16 ? 8 : 4; // 16 bytes of row padding
  static constexpr int PADT = BF16 ? 4 : 2;// 8 bytes of row padding
  static constexpr int LDK = DK + PAD;     // row stride of kqg / kbi
  static constexpr int LDT = 2 * C + PADT; // row stride of kbiT
  static constexpr int LDC = C + PAD;      // row stride of akk / akbn
  static constexpr int LDM = 2 * C + PAD;  // row stride of m = [Mqk | Mqb]
  static constexpr int LDD = 16 + PAD;     // row stride of the diagonal inverses
  static constexpr int LDU = C + PADT;     // row stride of uT
  // producer build: wave pw owns key channels [pw*DK/4, (pw+1)*DK/4); a lane
  // owns 4 adjacent channels (quad cq) on RPG consecutive tokens (group rg)
  static constexpr int QPW = DK / 16;              // channel quads per producer wave
  static constexpr int RGW = 64 / QPW;             // row groups a wave can hold
  static constexpr int RGE = RGW < C ? RGW : C;    // row groups used
  static constexpr int RPG = C / RGE;              // tokens per row group
  static constexpr int RGL = 64 / QPW;             // lanes per channel quad (>= RGE)
  // U staging over the 256 producer threads: 4 value columns x TPT tokens
  static constexpr int UCQ = DVB / 4;
  static constexpr int UTG = (256 / UCQ) < C ? (256 / UCQ) : C;
  static constexpr int TPT = C / UTG;
  static_assert(NCT == 1 || NCT == 2 || NCT == 4, "one to four column waves");
  static_assert(DK % 16 == 0 && C % 16 == 0, "16-aligned tiles");
  static_assert(C % RGE == 0 && C % UTG == 0, "build layout");
  static_assert(TPT == 1 || TPT == 2 || TPT == 4, "U staging layout");
};

// Operands of one chunk (double-buffered: produced for chunk s while chunk
// s-1 is consumed).
template <class Cf>
struct ChunkBuf {
  typedef typename Op<Cf::BF16>::T OT;
  OT kqg[2 * Cf::C * Cf::LDK];   // rows 0..C-1: k*gamma; rows C..2C-1: q*gamma
  OT kbi[2 * Cf::C * Cf::LDK];   // rows 0..C-1: k/gamma; rows C..2C-1: (b*k)/gamma
  OT kbiT[Cf::DK * Cf::LDT];     // kbi transposed: [channel][token (K part | beta part)]
  OT akk[Cf::C * Cf::LDC];       // Akk, lower blocks (strictly lower inside diagonal blocks)
  OT akbn[Cf::C * Cf::LDC];      // -Akb, off-diagonal lower blocks
  OT m[Cf::C * Cf::LDM];         // [Mqk | Mqb], lower blocks incl. diagonal
  OT dinv[Cf::NCH * 16 * Cf::LDD];   // (I + Akb_rr)^-1 per diagonal block
  OT uT[Cf::DVB * Cf::LDU];          // U = w * v, transposed: [value column][token]
  float gamc[Cf::DK];                // gamma_C per key channel
  int bad[Cf::NP];                   // per producer wave: chunk must be stepped token by token
};

template <class Cf>
struct PrefillSmem {
  ChunkBuf<Cf> buf[2];
  float akbd[Cf::NCH * 16 * 20];     // Akb diagonal blocks (fp32, 16-byte rows), Gram -> inverses
};

template <class Cf>
constexpr size_t prefill_smem_bytes() {
  return sizeof(PrefillSmem<Cf>);
}

// Optional per-phase cycle counters for kernel development, compiled only
// with -DGDN2_PHASE_TIMING: the first 8 workgroups accumulate s_memtime
// deltas per phase into gdn2_phase_cycles[block][wave][phase].
#ifdef GDN2_PHASE_TIMING
__device__ unsigned long long gdn2_phase_cycles[8][8][8];
#define GDN2_TIMER_INIT unsigned long long tm_acc[8] = {}, tm_prev = __builtin_amdgcn_s_memtime();
#define GDN2_MARK(i)                                                \
  do {                                                              \
    const unsigned long long tm_now = __builtin_amdgcn_s_memtime(); \
    tm_acc[i] += tm_now - tm_prev;                                  \
    tm_prev = tm_now;                                               \
  } while (0)
#define GDN2_TIMER_STORE \
  if (blockIdx.x < 8 && lane == 0) \
    for (int i = 0; i < 8; ++i) gdn2_phase_cycles[blockIdx.x][wave][i] = tm_acc[i];
#else
#define GDN2_TIMER_INIT
#define GDN2_MARK(i) ((void)0)
#define GDN2_TIMER_STORE
#endif

struct PrefillParams {
  const void *q, *k, *v;
  const float *a, *b, *w, *S0;
  void *o;
  float *S_T;
  int B, T, H_qk, H_v, d_v;
};

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

// One quadrant of the chunk's Gram matrix (q = 0 Akk, 1 Akb, 2 Mqk, 3 Mqb):
// rows of kqg times rows of kbi over the key channels. Per K32 step the wave
// loads each row block's and each column block's fragments once and reuses
// them across the quadrant's lower tiles.
template <class Cf, int q>
__device__ __forceinline__ void gram_quadrant(ChunkBuf<Cf> &cb, float *akbd, int lg, int lc) {
  using O = Op<Cf::BF16>;
  using Frag = typename O::Frag;
  constexpr int C = Cf::C, NRT = Cf::NRT, NCH = Cf::NCH, LDK = Cf::LDK, LDC = Cf::LDC,
                LDM = Cf::LDM;
  const int arow0 = (q >= 2) ? C : 0, brow0 = (q & 1) ? C : 0;
  floatx4 acc[Cf::NTRI];
#pragma unroll
  for (int i = 0; i < Cf::NTRI; ++i) acc[i] = zero4();
  auto frag = [&](const typename O::T *base, int row, int kb) -> Frag {
    return O::ld(base + (row + lc) * LDK + 16 * kb + 4 * lg);
  };
#pragma unroll
  for (int kb = 0; kb < NRT; kb += 2) {
    Frag a0[NCH], a1[NCH], b0[NCH], b1[NCH];
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      a0[r] = frag(cb.kqg, arow0 + 16 * r, kb);
      a1[r] = (kb + 1 < NRT) ? frag(cb.kqg, arow0 + 16 * r, kb + 1) : O::zero();
      b0[r] = frag(cb.kbi, brow0 + 16 * r, kb);
      b1[r] = (kb + 1 < NRT) ? frag(cb.kbi, brow0 + 16 * r, kb + 1) : O::zero();
    }
#pragma unroll
    for (int r = 0, ti = 0; r < NCH; ++r)
#pragma unroll
      for (int c = 0; c <= r; ++c, ++ti) {
        if constexpr (O::kK32Only || NRT % 2 == 0)
          acc[ti] = O::mma32(acc[ti], a0[r], a1[r], b0[c], b1[c]);
        else if (kb + 1 < NRT)
          acc[ti] = O::mma32(acc[ti], a0[r], a1[r], b0[c], b1[c]);
        else
          acc[ti] = O::mma16(acc[ti], a0[r], b0[c]);
      }
  }
#pragma unroll
  for (int r = 0, ti = 0; r < NCH; ++r)
#pragma unroll
    for (int c = 0; c <= r; ++c, ++ti) {
      const int s = 16 * c + lc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * r + 4 * lg + j;
        const float x = acc[ti][j];
        if constexpr (q == 0) {
          cb.akk[t * LDC + s] = O::cvt(t > s ? x : 0.f);
        } else if constexpr (q == 1) {
          if (c != r)
            cb.akbn[t * LDC + s] = O::cvt(-x);
          else  // diagonal block, strictly lower part, fp32 for the inverse
            akbd[r * 16 * 20 + (4 * lg + j) * 20 + lc] = (t > s) ? x : 0.f;
        } else if constexpr (q == 2) {
          cb.m[t * LDM + s] = O::cvt(t >= s ? x : 0.f);
        } else {
          cb.m[t * LDM + C + s] = O::cvt(t >= s ? x : 0.f);
        }
      }
    }
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
__global__ __launch_bounds__(512) void prefill_kernel(PrefillParams p) {
  using Cf = PrefillCfg<DK, C, NCT, BF16>;
  using E = Elem<BF16>;
  using O = Op<BF16>;
  using ET = typename E::T;
  using OT = typename O::T;
  using Frag = typename O::Frag;
  // four q/k (or v) elements in their stored type
  using Quad = typename std::conditional<BF16, uint2, floatx4>::type;
  constexpr int NRT = Cf::NRT, NCH = Cf::NCH, LDK = Cf::LDK, LDT = Cf::LDT, LDC = Cf::LDC,
                LDM = Cf::LDM, LDD = Cf::LDD, LDU = Cf::LDU, RPG = Cf::RPG, TPT = Cf::TPT,
                QPW = Cf::QPW, RGE = Cf::RGE;
  static_assert(sizeof(PrefillSmem<Cf>) <= 160 * 1024, "LDS working set exceeds one CU");

  __shared__ PrefillSmem<Cf> sm;
  GDN2_TIMER_INIT

  int n, h, cb;
  map_block(blockIdx.x, p.B, p.H_qk, p.H_v, p.d_v / Cf::DVB, n, h, cb);
  const int g = h / (p.H_v / p.H_qk);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int lg = lane >> 4, lc = lane & 15;
  const int d_v = p.d_v;
  const bool producer = wave < Cf::NP;
  const int cw = wave - Cf::NP;                 // consumer index
  const bool consumer = !producer && cw < NCT;  // owns a 16-column state tile
  const int col = cb * Cf::DVB + (consumer ? cw : 0) * 16 + lc;  // consumer lane's value column

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
  auto rows_left = [&](int t0, uint32_t tb) -> uint32_t { return (uint32_t)(p.T - t0) * tb; };

  // ---------------------------------------------------------------- producer layout
  // build: lane = (row group rg, channel quad cq) of producer wave `wave`,
  // row group fastest so that a quad's prefix product runs across adjacent lanes
  const int rg = lane % Cf::RGL, cq = lane / Cf::RGL;
  const bool brow = (RGE == Cf::RGL) || rg < RGE;  // lane holds build rows
  const int ch0 = wave * (DK / 4) + 4 * cq;
  const uint32_t ab_off = (uint32_t)(rg * RPG) * ab_tb + (uint32_t)ch0 * 4u;
  const uint32_t qk_off = (uint32_t)(rg * RPG) * qk_tb + (uint32_t)ch0 * sizeof(ET);
  // U staging: producer thread tid = (token group utq, column quad ucq)
  const int ucq = tid % Cf::UCQ, utq = tid / Cf::UCQ, ucol = 4 * ucq;
  const bool ustager = (Cf::UTG * Cf::UCQ == 256) || utq < Cf::UTG;
  const uint32_t v_off = (uint32_t)(utq * TPT) * v_tb + (uint32_t)(cb * Cf::DVB + ucol) * sizeof(ET);
  const uint32_t w_off = (uint32_t)(utq * TPT) * w_tb + (uint32_t)(cb * Cf::DVB + ucol) * 4u;

  // Raw inputs of the next chunk to build, held in producer registers.
  floatx4 ra[RPG], rb[RPG];
  Quad rk[RPG], rq[RPG];
  floatx4 uw[TPT];
  Quad uv[TPT];
  // The next chunk's inputs are requested in two parts (decay and erase gate
  // after the build; keys, queries, values and write gate after the Gram
  // tiles) so that no single phase waits for the whole request to issue.
  auto load_raw_ab = [&](int t0) {
    if (brow) {
      const rsrc_t ra_ = make_rsrc((const char *)ah + (size_t)t0 * ab_tb, rows_left(t0, ab_tb));
      const rsrc_t rb_ = make_rsrc((const char *)bh + (size_t)t0 * ab_tb, rows_left(t0, ab_tb));
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        ra[r] = bload<floatx4>(ra_, ab_off, r * ab_tb);
        rb[r] = bload<floatx4>(rb_, ab_off, r * ab_tb);
      }
    }
  };
  auto load_raw_kqvw = [&](int t0) {
    if (brow) {
      const rsrc_t rk_ = make_rsrc((const char *)kh + (size_t)t0 * qk_tb, rows_left(t0, qk_tb));
      const rsrc_t rq_ = make_rsrc((const char *)qh + (size_t)t0 * qk_tb, rows_left(t0, qk_tb));
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        rk[r] = bload<Quad>(rk_, qk_off, r * qk_tb);
        rq[r] = bload<Quad>(rq_, qk_off, r * qk_tb);
      }
    }
    if (ustager) {
      const rsrc_t rv_ = make_rsrc((const char *)vh + (size_t)t0 * v_tb, rows_left(t0, v_tb));
      const rsrc_t rw_ = make_rsrc((const char *)wh + (size_t)t0 * w_tb, rows_left(t0, w_tb));
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        uv[i] = bload<Quad>(rv_, v_off, i * v_tb);
        uw[i] = bload<floatx4>(rw_, w_off, i * w_tb);
      }
    }
  };
  auto quad_f = [](Quad x) -> floatx4 {
    if constexpr (BF16)
      return floatx4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                     __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
    else
      return x;
  };
  auto shfl4 = [](floatx4 x, int src) {
    return floatx4{__shfl(x[0], src, 64), __shfl(x[1], src, 64), __shfl(x[2], src, 64),
                   __shfl(x[3], src, 64)};
  };

  // Build chunk operands into buffer cbuf (producer waves; no workgroup sync
  // inside: the decay scan runs across the lanes of one wave).
  auto build = [&](ChunkBuf<Cf> &cbuf) {
    // cumulative decay within the lane's RPG tokens
    floatx4 gl[RPG];
    floatx4 pr = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
      if (brow) pr *= ra[r];
      gl[r] = pr;
    }
    // inclusive prefix product over the row groups (adjacent lanes): DPP row
    // shifts when a quad's groups fit in one 16-lane row, lane shuffles else
    floatx4 inc = pr, pre;
    if constexpr (RGE <= 16) {
      static_for<4>([&](auto li) {
        constexpr int d = 1 << decltype(li)::value;
        if constexpr (d < RGE) {
          floatx4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = row_shr<d>(inc[e], 1.f);
          if (rg >= d) inc *= y;
        }
      });
#pragma unroll
      for (int e = 0; e < 4; ++e) pre[e] = row_shr<1>(inc[e], 1.f);
    } else {
#pragma unroll
      for (int d = 1; d < RGE; d <<= 1) {
        const floatx4 y = shfl4(inc, lane - d);
        if (rg >= d) inc *= y;
      }
      pre = shfl4(inc, lane - 1);
    }
    if (rg == 0) pre = floatx4{1.f, 1.f, 1.f, 1.f};
    // the last row group holds gamma_C of the lane's 4 channels
    const bool last = rg == RGE - 1;
    const bool lane_bad = last && (!(inc[0] >= kMinChunkDecay) || !(inc[1] >= kMinChunkDecay) ||
                                   !(inc[2] >= kMinChunkDecay) || !(inc[3] >= kMinChunkDecay));
    const bool any_bad = __any(lane_bad);
    if (lane == 0) cbuf.bad[wave] = any_bad ? 1 : 0;
    if (last) *reinterpret_cast<floatx4 *>(&cbuf.gamc[ch0]) = inc;
    if (brow) {
      floatx4 kbq[4], bkq[4];
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        const int tl = rg * RPG + r;
        const floatx4 gm = pre * gl[r];
        const floatx4 gi = {__builtin_amdgcn_rcpf(gm[0]), __builtin_amdgcn_rcpf(gm[1]),
                            __builtin_amdgcn_rcpf(gm[2]), __builtin_amdgcn_rcpf(gm[3])};
        const floatx4 kv = quad_f(rk[r]);
        const floatx4 qv = quad_f(rq[r]);
        const floatx4 kb = kv * gi;
        const floatx4 bk = rb[r] * kb;
        *reinterpret_cast<Frag *>(&cbuf.kqg[tl * LDK + ch0]) = O::from_acc(kv * gm);
        *reinterpret_cast<Frag *>(&cbuf.kqg[(C + tl) * LDK + ch0]) = O::from_acc(qv * gm);
        *reinterpret_cast<Frag *>(&cbuf.kbi[tl * LDK + ch0]) = O::from_acc(kb);
        *reinterpret_cast<Frag *>(&cbuf.kbi[(C + tl) * LDK + ch0]) = O::from_acc(bk);
        // transposed copy: 4 (or 2) consecutive tokens per channel at once
        if constexpr (RPG % 4 == 0) {
          kbq[r & 3] = kb;
          bkq[r & 3] = bk;
          if ((r & 3) == 3) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              *reinterpret_cast<Frag *>(&cbuf.kbiT[(ch0 + c) * LDT + tl - 3]) =
                  O::from_acc(floatx4{kbq[0][c], kbq[1][c], kbq[2][c], kbq[3][c]});
              *reinterpret_cast<Frag *>(&cbuf.kbiT[(ch0 + c) * LDT + C + tl - 3]) =
                  O::from_acc(floatx4{bkq[0][c], bkq[1][c], bkq[2][c], bkq[3][c]});
            }
          }
        } else if constexpr (RPG % 2 == 0) {
          if (r & 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              O::st2(&cbuf.kbiT[(ch0 + c) * LDT + tl - 1], kbq[0][c], kb[c]);
              O::st2(&cbuf.kbiT[(ch0 + c) * LDT + C + tl - 1], bkq[0][c], bk[c]);
            }
          }
          kbq[0] = kb;
          bkq[0] = bk;
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            cbuf.kbiT[(ch0 + c) * LDT + tl] = O::cvt(kb[c]);
            cbuf.kbiT[(ch0 + c) * LDT + C + tl] = O::cvt(bk[c]);
          }
        }
      }
    }
    if (ustager) {  // U = w * v, stored transposed for the consumers' B fragments
      floatx4 u[TPT];
#pragma unroll
      for (int i = 0; i < TPT; ++i) u[i] = uw[i] * quad_f(uv[i]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        OT *dst = &cbuf.uT[(ucol + c) * LDU + utq * TPT];
        if constexpr (TPT == 4) {
          *reinterpret_cast<Frag *>(dst) = O::from_acc(floatx4{u[0][c], u[1][c], u[2][c], u[3][c]});
        } else if constexpr (TPT == 2) {
          O::st2(dst, u[0][c], u[1][c]);
        } else {
          dst[0] = O::cvt(u[0][c]);
        }
      }
    }
  };

  const int nfull = p.T / C;

  // The two roles run separate loops (the branch is wave-uniform); each loop
  // step executes exactly three workgroup barriers, so the barrier counts of
  // producer and consumer waves always match.
  if (producer) {
    if (nfull > 0) {
      load_raw_ab(0);
      load_raw_kqvw(0);
    }
    for (int s = 0; s <= nfull; ++s) {
      ChunkBuf<Cf> &pb = sm.buf[s & 1];  // produced this step (chunk s)
      const bool produce = s < nfull;
      // phase A: operands of chunk s, then request chunk s+1's inputs
      if (produce) {
        build(pb);
        if (s + 1 < nfull) load_raw_ab((s + 1) * C);
      }
      GDN2_MARK(0);
      __syncthreads();
      GDN2_MARK(7);
      // phase B: Gram quadrant `wave`
      if (produce) {
        switch (wave) {
          case 0: gram_quadrant<Cf, 0>(pb, sm.akbd, lg, lc); break;
          case 1: gram_quadrant<Cf, 1>(pb, sm.akbd, lg, lc); break;
          case 2: gram_quadrant<Cf, 2>(pb, sm.akbd, lg, lc); break;
          default: gram_quadrant<Cf, 3>(pb, sm.akbd, lg, lc); break;
        }
        if (s + 1 < nfull) load_raw_kqvw((s + 1) * C);
      }
      GDN2_MARK(2);
      __syncthreads();
      GDN2_MARK(7);
      // phase C: inverses of the diagonal blocks of I + Akb, one block per
      // producer wave. Lane = (column c, row quarter qq): it holds rows
      // 4qq..4qq+3 of column c of (I + Akb_rr)^-1 and of Akb_rr. Forward
      // substitution: at step i the lane owning row i passes the final x_i to
      // its quad by DPP, and every lane updates its rows below i.
      for (int r = wave; r < NCH && produce; r += Cf::NP) {
        const int c = lane >> 2, qq = lane & 3;
        floatx4 arow[4][4];  // arow[j][k4] = Akb_rr[4qq + j][4k4 .. 4k4+3]
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4)
            arow[j][k4] = *reinterpret_cast<const floatx4 *>(&sm.akbd[r * 16 * 20 + (4 * qq + j) * 20 + 4 * k4]);
        floatx4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (4 * qq + j == c) ? 1.f : 0.f;
        static_for<15>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          const float xi = quad_bcast<i / 4>(x[i % 4]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * qq + j > i) x[j] -= arow[j][i / 4][i % 4] * xi;
        });
#pragma unroll
        for (int j = 0; j < 4; ++j) pb.dinv[r * 16 * LDD + (4 * qq + j) * LDD + c] = O::cvt(x[j]);
      }
      GDN2_MARK(4);
      __syncthreads();  // buffer s&1 is now complete for the consumers
      GDN2_MARK(7);
    }
    GDN2_TIMER_STORE
    return;
  }

  // ---------------------------------------------------------------- consumer waves
  // S[rt][j] = S[16*rt + 4*lg + j][col] (accumulator layout).
  floatx4 S[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[rt][j] = (p.S0 && consumer) ? p.S0[s_off + (size_t)(16 * rt + 4 * lg + j) * d_v] : 0.f;

  // Token-by-token steps on this wave's columns (exact for any decay).
  auto token_steps = [&](int tb, int te) {
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

  // consumer registers carried across the phases of one step
  Frag Uf[NCH], Rf[NCH], Rn[NCH];
  floatx4 X[NCH], Y[NCH];
  auto rowfrag = [&](const OT *base, int ld, int row, int colblk) -> Frag {
    return O::ld(base + (row + lc) * ld + 16 * colblk + 4 * lg);
  };
  for (int s = 0; s <= nfull; ++s) {
    ChunkBuf<Cf> &cbf = sm.buf[(s + 1) & 1];  // consumed this step (chunk s-1)
    const bool work = consumer && s >= 1;
    const int tc = (s - 1) * C;               // first token of the consumed chunk
    const bool cbad = work && (cbf.bad[0] | cbf.bad[1] | cbf.bad[2] | cbf.bad[3]) != 0;
    const bool fast = work && !cbad;
    // ---------------------------------------------------------------- phase A
    if (cbad) {
      token_steps(tc, tc + C);
    } else if (fast) {
      // X = (gamma * K) S0, Y = (gamma * Q) S0
      Frag Sf[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) Sf[rt] = O::from_acc(S[rt]);
#pragma unroll
      for (int c = 0; c < NCH; ++c) Uf[c] = O::ld(&cbf.uT[(cw * 16 + lc) * LDU + 16 * c + 4 * lg]);
      auto sfrag = [&](int kb) { return Sf[kb]; };
#pragma unroll
      for (int r = 0; r < NCH; ++r) {
        X[r] = chain<O, 0, NRT>(zero4(), [&](int kb) { return rowfrag(cbf.kqg, LDK, 16 * r, kb); }, sfrag);
        Y[r] = chain<O, 0, NRT>(zero4(), [&](int kb) { return rowfrag(cbf.kqg, LDK, C + 16 * r, kb); }, sfrag);
      }
    }
    GDN2_MARK(1);
    __syncthreads();
    GDN2_MARK(7);
    // ---------------------------------------------------------------- phase B
    if (fast) {
      // Z = X + Akk U, then (I + Akb) R = Z by blocked forward substitution:
      // R_r = D_r (Z_r - sum_{c<r} Akb_rc R_c), one chain over
      // [Akk blocks 0..r with U] ++ [-Akb blocks 0..r-1 with R].
      static_for<NCH>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        auto fa = [&](int kb) {
          return kb <= r ? rowfrag(cbf.akk, LDC, 16 * r, kb) : rowfrag(cbf.akbn, LDC, 16 * r, kb - r - 1);
        };
        auto fb = [&](int kb) { return kb <= r ? Uf[kb] : Rf[kb - r - 1]; };
        const floatx4 acc = chain<O, 0, 2 * r + 1>(X[r], fa, fb);
        const floatx4 R = chain<O, 0, 1>(
            zero4(), [&](int) { return rowfrag(cbf.dinv + r * 16 * LDD, LDD, 0, 0); },
            [&](int) { return O::from_acc(acc); });
        Rf[r] = O::from_acc(R);
        Rn[r] = O::from_acc(-R);
      });
    }
    GDN2_MARK(3);
    __syncthreads();
    GDN2_MARK(7);
    // ---------------------------------------------------------------- phase C
    if (fast) {
      // O = Y + Mqk U - Mqb R, one chain over [Mqk blocks 0..r | Mqb blocks 0..r]
      const rsrc_t ro_ = make_rsrc((const char *)oh + (size_t)tc * v_tb, rows_left(tc, v_tb));
      const uint32_t o_off = (uint32_t)(4 * lg) * v_tb + (uint32_t)col * sizeof(ET);
      static_for<NCH>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        auto fa = [&](int kb) {
          return kb <= r ? rowfrag(cbf.m, LDM, 16 * r, kb) : rowfrag(cbf.m, LDM, 16 * r, NCH + kb - r - 1);
        };
        auto fb = [&](int kb) { return kb <= r ? Uf[kb] : Rn[kb - r - 1]; };
        const floatx4 acc = chain<O, 0, 2 * r + 2>(Y[r], fa, fb);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (BF16)
            bstore(f32_to_bf16(acc[j]), ro_, o_off, (16 * r + j) * v_tb);
          else
            bstore(acc[j], ro_, o_off, (16 * r + j) * v_tb);
        }
      });
      // S_C = diag(gamma_C) (S0 + (K/gamma)^T U - (beta/gamma)^T R)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        auto fa = [&](int kb) { return rowfrag(cbf.kbiT, LDT, 16 * rt, kb); };
        auto fb = [&](int kb) { return kb < NCH ? Uf[kb] : Rn[kb - NCH]; };
        const floatx4 acc = chain<O, 0, 2 * NCH>(S[rt], fa, fb);
        const floatx4 gc = *reinterpret_cast<const floatx4 *>(&cbf.gamc[16 * rt + 4 * lg]);
        S[rt] = acc * gc;
      }
    }
    GDN2_MARK(5);
    __syncthreads();  // buffer (s+1)&1 may now be rebuilt by the producers
    GDN2_MARK(7);
  }
  GDN2_TIMER_STORE

  if (consumer) {
    if (nfull * C < p.T) token_steps(nfull * C, p.T);
    if (p.S_T) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) p.S_T[s_off + (size_t)(16 * rt + 4 * lg + j) * d_v] = S[rt][j];
    }
  }
}

// Largest chunk (<= the requested one) whose double-buffered working set
// fits one CU's LDS.
template <int DK, int NCT, bool BF16>
constexpr int fitting_chunk(int requested) {
  return (requested >= 64 && prefill_smem_bytes<PrefillCfg<DK, 64, NCT, BF16>>() <= 160 * 1024) ? 64
         : (requested >= 32 && prefill_smem_bytes<PrefillCfg<DK, 32, NCT, BF16>>() <= 160 * 1024) ? 32
                                                                                                  : 16;
}

template <int DK, int C, int NCT, bool BF16>
hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t st) {
  PrefillParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.a = a.a; p.b = a.b; p.w = a.w; p.S0 = a.S0;
  p.o = a.o; p.S_T = a.S_T;
  p.B = a.B; p.T = a.T; p.H_qk = a.H_qk; p.H_v = a.H_v; p.d_v = a.d_v;
  const int blocks = (a.d_v / (16 * NCT)) * a.H_v * a.B;
  hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16>), dim3(blocks), dim3(512), 0, st, p);
  return hipGetLastError();
}

template <int DK, int NCT, bool BF16>
hipError_t dispatch_prefill_chunk(const PrefillArgs &a, hipStream_t st) {
  switch (fitting_chunk<DK, NCT, BF16>(a.chunk)) {
    case 64:
      if constexpr (prefill_smem_bytes<PrefillCfg<DK, 64, NCT, BF16>>() <= 160 * 1024)
        return launch_prefill_t<DK, 64, NCT, BF16>(a, st);
      else
        return hipErrorInvalidValue;
    case 32:
      if constexpr (prefill_smem_bytes<PrefillCfg<DK, 32, NCT, BF16>>() <= 160 * 1024)
        return launch_prefill_t<DK, 32, NCT, BF16>(a, st);
      else
        return hipErrorInvalidValue;
    default:
      return launch_prefill_t<DK, 16, NCT, BF16>(a, st);
  }
}

template <int DK, bool BF16>
hipError_t dispatch_prefill(const PrefillArgs &a, hipStream_t st) {
  switch (a.nct) {
    case 1: return dispatch_prefill_chunk<DK, 1, BF16>(a, st);
    case 2: return dispatch_prefill_chunk<DK, 2, BF16>(a, st);
    case 4: return dispatch_prefill_chunk<DK, 4, BF16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn2
