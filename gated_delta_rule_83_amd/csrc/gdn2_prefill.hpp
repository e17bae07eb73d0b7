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
//   Akk[t,s] = sum_i k_t,i k_s,i gamma_t,i / gamma_s,i      s < t
//   Akb[t,s] = sum_i k_t,i beta_s,i gamma_t,i / gamma_s,i   s < t
//   Mqk[t,s] = sum_i q_t,i k_s,i gamma_t,i / gamma_s,i      s <= t
//   Mqb[t,s] = sum_i q_t,i beta_s,i gamma_t,i / gamma_s,i   s <= t
//   (I + Akb) R = (gamma * K) S0 + Akk U          (row t of R is the key read r_t)
//   O  = (gamma * Q) S0 + Mqk U - Mqb R
//   S_C = diag(gamma_C) S0 + (rho * K)^T U - (rho * beta)^T R,  rho_s = gamma_C / gamma_s
// Anchors. The ratio gamma_t / gamma_s <= 1 is split between the two MFMA
// operands against an anchor token with cumulative decay A: the left
// operands carry lam_t = gamma_t / A, the right ones mu_s = A / gamma_s.
// Rescaling cumulative gates against an in-block anchor so that ratios
// cannot explode is the device the FiX analysis on iplexlaw.co.kr describes
// for its block-wise kernel (section 5). (gamma * K) S0 is formed as
// (lam * K)(diag(A) S0), and the carry as
//   S_C = diag(gamma_C / A) (diag(A) S0 + (mu * K)^T U - (mu * beta)^T R).
// The anchor is chosen per chunk: the chunk start (A = 1, lam = gamma_t <= 1)
// while the whole chunk's decay is at least e^-60 on every channel (the
// right factors are then below e^60); for d_k = 128 otherwise the middle
// token m = C/2 - 1 (A = gamma_m) while each half chunk's decay is at least
// e^-60: in the off-diagonal block (second half x first half) both factors
// are then <= 1 and elsewhere one factor is bounded by the inverse decay of
// half a chunk. Every factor only rescales elements, so bf16 rounding stays
// relative; the only risk is range. A chunk that fails the test (for
// d_k = 128 a decay below ~e^-3.75 per token throughout half a chunk) is
// stepped token by token, which is exact for any decay.
//
// Everything that does not depend on the entering state (scaled operands,
// the Gram matrices, the diagonal inverses) is computed one chunk ahead by
// four producer waves, while four consumer waves run the state-dependent
// part of the previous chunk. A workgroup of 8 waves handles one (sequence,
// value head, block of 16*NCT value columns, NCT = 1, 2 or 4); consumer wave
// w < NCT owns the 16-column state tile w. Value columns of S evolve
// independently, so the column split is exact. Step s of the pipeline
// (chunk s produced into LDS buffer s%2, chunk s-1 consumed from buffer
// (s-1)%2), with one workgroup barrier after each phase:
//   A. producers: decay scan (wave-local, across lanes), scaled operands
//      K*lam | Q*lam, K*mu | beta*mu (also transposed); then the
//      decay and erase gates of chunk s+2 are requested into registers.
//      consumers: U = w*v of chunk s-1 (requested two steps earlier) into an
//      LDS staging array, the previous chunk's outputs stored, v and w of
//      chunk s+1 requested, X = (lam*K) diag(A) S0, Y = (lam*Q) diag(A) S0.
//   B. producers: the Gram tiles (Akk, Akb, Mqk, Mqb, lower tiles) split
//      over the waves, the inverses of the 16x16 diagonal blocks of I + Akb;
//      then the keys and queries of chunk s+2 are requested.
//      consumers: U fragments from the staging array, Z = X + Akk U, the
//      blocked forward solve for R, the outputs O and the state carry.
// A launch may also run segments of the sequences (split sequences): see
// PrefillParams and launch_prefill_t.
// Consumer products are chained through MFMA accumulators: an accumulator
// tile is already the next product's B operand.
#pragma once

#include <stdlib.h>

#include <type_traits>
#include <utility>

#include "gdn2_device.hpp"
#include "gdn2_internal.hpp"
#include "gdn2_range.hpp"

namespace gdn2 {

// LDS row layout of an MFMA operand array. A row holds W elements of the
// contraction index k; a lane's K16 fragment is k = 16kb + 4g .. +3 (lane
// group g). For bf16 the two K16 blocks of a K32 step are interleaved so
// that a lane's whole K32 fragment is one 16-byte unit: unit 4P + g of a row
// holds k = 32P + 4g .. +3 in its first 8 bytes and k = 32P + 16 + 4g .. +3
// in its second. For fp32 one unit is one K16 fragment (unit 4kb + g).
// The units of row R are XOR-permuted by (R >> 2) & SW and rows are NU + 2
// units apart. With the LDS serving 16-byte reads of 16 lanes as one 64-bank
// pass and 8-byte accesses of 16 consecutive lanes as one 32-bank pass,
// this keeps the kernel's patterns free of bank conflicts: operand reads
// (16 lanes on 16 consecutive rows, one unit) and the build's writes (lanes
// on 8 rows 4 apart, both halves of one unit).
template <bool BF16, int W>
struct RowLayout {
  static constexpr int EPU = BF16 ? 8 : 4;                 // elements per unit
  static constexpr int NU = (W / EPU) < 4 ? 4 : (W / EPU);  // units per row
  static constexpr int SW = (NU < 8 ? NU : 8) - 1;
  static constexpr int STRIDE = 16 * (NU + 2);             // bytes per row
  static __device__ __forceinline__ uint32_t off(int row, int k) {
    const int unit = BF16 ? (((k >> 5) << 2) | ((k >> 2) & 3)) : (k >> 2);
    const int sub = BF16 ? ((((k >> 4) & 1) << 3) | ((k & 3) << 1)) : ((k & 3) << 2);
    return (uint32_t)(row * STRIDE + ((unit ^ ((row >> 2) & SW)) << 4) + sub);
  }
};

// Fragment loads and stores in RowLayout L (O = Op<BF16>).
template <class L, bool BF16>
__device__ __forceinline__ typename Op<BF16>::Frag frag16(const char *base, int row, int kb, int g) {
  return *reinterpret_cast<const typename Op<BF16>::Frag *>(base + L::off(row, 16 * kb + 4 * g));
}
// K32 step p (K16 blocks 2p, 2p+1); `single` = only block 2p exists
template <class L, bool BF16, bool single = false>
__device__ __forceinline__ Pair<BF16> frag32(const char *base, int row, int p, int g) {
  using O = Op<BF16>;
  if constexpr (single) {
    return Pair<BF16>{frag16<L, BF16>(base, row, 2 * p, g), O::zero()};
  } else if constexpr (BF16) {
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(base + L::off(row, 32 * p + 4 * g));
    return Pair<BF16>{__builtin_shufflevector(x, x, 0, 1, 2, 3), __builtin_shufflevector(x, x, 4, 5, 6, 7)};
  } else {
    return Pair<BF16>{frag16<L, BF16>(base, row, 2 * p, g), frag16<L, BF16>(base, row, 2 * p + 1, g)};
  }
}
template <class L, bool BF16>
__device__ __forceinline__ void st4(char *base, int row, int k, floatx4 v) {
  *reinterpret_cast<typename Op<BF16>::Frag *>(base + L::off(row, k)) = Op<BF16>::from_acc(v);
}
template <class L, bool BF16>
__device__ __forceinline__ void st2(char *base, int row, int k, float x0, float x1) {
  Op<BF16>::st2(reinterpret_cast<typename Op<BF16>::T *>(base + L::off(row, k)), x0, x1);
}
template <class L, bool BF16>
__device__ __forceinline__ void st1(char *base, int row, int k, float x) {
  *reinterpret_cast<typename Op<BF16>::T *>(base + L::off(row, k)) = Op<BF16>::cvt(x);
}
// acc += a * b over one K32 step; a zero upper half costs nothing extra on
// the fp32 path (one K16 step), and keeps one MFMA shape on the bf16 path.
template <bool BF16, bool single = false>
__device__ __forceinline__ floatx4 mma(floatx4 acc, const Pair<BF16> &a, const Pair<BF16> &b) {
  using O = Op<BF16>;
  if constexpr (single && !O::kK32Only)
    return O::mma16(acc, a.lo, b.lo);
  else
    return O::mma32(acc, a.lo, a.hi, b.lo, b.hi);
}

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
  static constexpr int NKP = (NRT + 1) / 2;          // K32 steps over the key channels
  typedef RowLayout<BF16, DK> LK;                     // kqg / kbi rows (channels)
  typedef RowLayout<BF16, 2 * C> LT;                  // kbiT / ab / m rows (tokens)
  static constexpr int LDD = 20;           // row stride (elements) of the diagonal inverses
  // producer build: wave pw owns key channels [pw*DK/4, (pw+1)*DK/4); a lane
  // owns 4 adjacent channels (quad cq) on RPG consecutive tokens (group rg)
  static constexpr int QPW = DK / 16;              // channel quads per producer wave
  static constexpr int RGW = 64 / QPW;             // row groups a wave can hold
  static constexpr int RGE = RGW < C ? RGW : C;    // row groups used
  static constexpr int RPG = C / RGE;              // tokens per row group
  static constexpr int RGL = 64 / QPW;             // lanes per channel quad (>= RGE)
  // lane -> channel quad: with 8 quads per wave, the two quads that share a
  // 16-byte operand unit (q and q + 4) are written by the same 16-lane pass
  // U = w * v staging: the column waves share the chunk's tokens; a lane
  // loads 8 adjacent columns of one token
  static constexpr int ULPT = DVB / 8;                  // lanes per token
  static constexpr int UTPI = 64 / ULPT;                // tokens per load
  static constexpr int UTPW = C / NCT;                  // tokens per column wave
  static constexpr int UNI = (UTPW + UTPI - 1) / UTPI;  // loads per wave and array
  // row stride (bytes) of the staged U: rows 4 apart in banks for the
  // transposing reads (4 consecutive rows per 16-lane pass)
  static constexpr int UROW = DVB * (BF16 ? 2 : 4) + (DVB * (BF16 ? 2 : 4) >= 64 ? 32 : 0);
  // token-major build (d_k = 128): producer wave w builds tokens
  // w*C/4 .. +C/4 for all key channels, so that every raw request covers
  // whole token rows (see the kernel's producer layout)
  static constexpr bool TOKM = DK == 128;
  // bf16: the carry's operands (mu K | mu b*K per key channel) are read from
  // the kbi rows with transposing LDS reads, so kbi is kept per chunk buffer
  // and no transposed copy is built; fp32 keeps the transposed copy kbiT
  static constexpr bool TRC = BF16;
  // output staging: rows of DVB output elements plus 8 bytes, so that the
  // 16 rows of one 8-byte column slice written together fall on distinct
  // bank pairs; the stores then write whole rows, 8 bytes per lane
  static constexpr int OES = BF16 ? 2 : 4;               // output element bytes
  static constexpr int OROW = DVB * OES + 8;             // row stride (bytes)
  static constexpr int OLPR = DVB * OES / 8;             // lanes per row in a store
  static constexpr int ORPI = 64 / OLPR;                 // rows per store instruction
  static constexpr int ORPW = C / NCT;                   // rows stored by each column wave
  static constexpr int ONI = ORPW / ORPI;                // store instructions per wave
  static_assert(ORPW % ORPI == 0, "whole store instructions");
  static_assert(NCT == 1 || NCT == 2 || NCT == 4, "one to four column waves");
  static_assert(DK % 16 == 0 && C % 16 == 0, "16-aligned tiles");
  static_assert(C % RGE == 0, "build layout");
};

// Operands of one chunk (double-buffered: produced for chunk s while chunk
// s-1 is consumed). Operand arrays are byte arrays in RowLayout order.
template <class Cf>
struct ChunkBuf {
  typedef typename Cf::LK LK;
  typedef typename Cf::LT LT;
  alignas(16) char kqg[2 * Cf::C * LK::STRIDE];  // rows 0..C-1: k*lam; rows C..2C-1: q*lam
  // bf16: rows 0..C-1: k*mu; rows C..2C-1: (b*k)*mu (read by this chunk's
  // Gram tiles and, one step later, by the carry)
  alignas(16) char kbi[Cf::TRC ? 2 * Cf::C * LK::STRIDE : 16];
  // fp32: kbi transposed, [channel][token (K part | beta part)], for the carry
  alignas(16) char kbiT[Cf::TRC ? 16 : Cf::DK * LT::STRIDE];
  // ab: row t, 16-column block 2c = Akk block (t, c) (strictly lower inside
  // diagonal blocks), block 2c + 1 = -Akb block (t, c) (off-diagonal only);
  // m: block 2c = Mqk block, 2c + 1 = Mqb block (lower incl. diagonal)
  alignas(16) char ab[Cf::C * LT::STRIDE];
  alignas(16) char m[Cf::C * LT::STRIDE];
  alignas(16) typename Op<Cf::BF16>::T dinv[Cf::NCH * 16 * Cf::LDD];  // (I + Akb_rr)^-1 per diagonal block
  alignas(16) float gamc[Cf::DK];                // gamma_C / A (A: the anchor's cumulative decay) per key channel
  alignas(16) float gamm[Cf::TOKM ? Cf::DK : 4];  // gamma_m (the Gram anchor) per key channel
  alignas(16) int bad[Cf::NP];                   // per producer wave: chunk must be stepped token by token
};

template <class Cf>
struct PrefillSmem {
  ChunkBuf<Cf> buf[2];
  // fp32: rows 0..C-1: k*mu; rows C..2C-1: (b*k)*mu of the chunk being
  // produced (written by the build, read by the Gram tiles of the same step:
  // one buffer; bf16 keeps them per chunk buffer)
  alignas(16) char kbi[Cf::TRC ? 16 : 2 * Cf::C * Cf::LK::STRIDE];
  // Akb diagonal blocks (fp32, 80-byte rows), Gram -> inverses; row i of a
  // block is stored at position 4 (i % 4) + i / 4 so that the inverse's
  // reads of rows 4qq + j (qq = 0..3) fall on distinct banks
  alignas(16) float akbd[Cf::NCH * 16 * 20];
  // U = w * v of the chunk being consumed, [token][column of the workgroup]
  // in the operand type (written in the first phase of a step, read in the
  // second)
  alignas(16) char ubuf[Cf::C * Cf::UROW];
  // outputs of the chunk consumed last, [token][column of the workgroup] in
  // the output type (written in the second phase of a step, stored to memory
  // in the first phase of the next)
  alignas(16) char obuf[Cf::C * Cf::OROW];
  // token-major build: per producer wave, the product of the decays of its
  // tokens per key channel, for the next chunk to build
  alignas(16) float tot[Cf::NP][Cf::TOKM ? Cf::DK : 4];
  // coupled gates: beta per token of the chunk in buffer b (last, so that
  // the other members keep their offsets)
  alignas(16) float beta[2][Cf::C];
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
#ifndef GDN2_TIMER_BLOCK0
#define GDN2_TIMER_BLOCK0 0  // first of the 8 workgroups recorded
#endif
#define GDN2_TIMER_STORE \
  if (blockIdx.x >= GDN2_TIMER_BLOCK0 && blockIdx.x < GDN2_TIMER_BLOCK0 + 8 && lane == 0) \
    for (int i = 0; i < 8; ++i) gdn2_phase_cycles[blockIdx.x - GDN2_TIMER_BLOCK0][wave][i] = tm_acc[i];
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
  // Split sequences. Segment s of a sequence is tokens [s * seg_len,
  // min((s + 1) * seg_len, T)) (seg_len a multiple of the chunk, >= T when
  // unsplit); the launch runs segments seg_first .. seg_first + nseg - 1,
  // the r-th of them (r = s - seg_first) as its own workgroups. Per head
  // there are ncb_val value column blocks and ncb_id identity column blocks:
  // an identity block runs the recurrence on the key-axis identity (entering
  // state I restricted to its columns, no writes, no outputs), so that its
  // final state is the segment's transition matrix, stored in M_T.
  int seg_len, seg_first, nseg, ncb_val, ncb_id;
  // Per-segment strides (elements) of S0, S_T and M_T. S0 with stride 0 is
  // the entering state of the launch's first segment only (later segments
  // start from zero).
  size_t s0_stride, sT_stride, m_stride;
  float *M_T;
  bool o_first_only;   // only the launch's first segment writes outputs
  bool sT_last_only;   // only the launch's last segment writes S_T
  // packed sequences: sequence n is tokens cu[n] .. cu[n+1]-1 of T (one
  // segment each); null: sequence n is tokens n*T .. n*T + T-1
  const int32_t *cu;
  // outputs of the identity column blocks, [B*T][H_v][d_k] in the output
  // type, d_k == d_v (null: not written): for token t of a segment, the query read of
  // the segment's transition, (Phi_t)^T q_t, where Phi_t maps the segment's
  // entering state to the state after t
  void *oI;
  // state at every chunk boundary (the backward's checkpoints), in the
  // output type, [B * H_v][ceil(T / C) + 1][d_v][d_k]: entry e of a
  // (sequence, head) is the state entering chunk e (e = 0: S0; the last
  // entry: the final state). Unsplit, unpacked launches only; null: none.
  // With cst_segs > 1 the launch's sequences are consecutive segments of
  // equal length, cst_segs to a sequence of the layout (n = m * cst_segs + j:
  // segment j of sequence m), and segment j writes that sequence's entries
  // j * nc .. j * nc + nc - 1 (nc chunks per segment), the last segment also
  // the final entry.
  void *cst;
  int cst_segs;
};

// Lower 16x16 tiles (r, c), c <= r, of the chunk's Gram matrices over the
// key channels; tile (r, c) has index r (r + 1) / 2 + c in the bit masks
// KK (Akk), KB (Akb), QK (Mqk), QB (Mqb). Tiles are computed transposed: the
// A operand is rows of kbi (column index s), the B operand rows of kqg (row
// index t), so acc[j] = G[t = 16r + lc][s = 16c + 4g + j] and each lane
// stores four consecutive columns of one row. Every fragment the tiles need
// is read once, before the first product, so that the LDS latencies overlap.
constexpr bool tile_in(unsigned m, int r, int c) { return ((m >> (r * (r + 1) / 2 + c)) & 1u) != 0; }
constexpr bool tile_row_used(unsigned m, int r) {
  bool u = false;
  for (int c = 0; c <= r; ++c) u = u || tile_in(m, r, c);
  return u;
}
constexpr bool tile_col_used(unsigned m, int c, int nch) {
  bool u = false;
  for (int r = c; r < nch; ++r) u = u || tile_in(m, r, c);
  return u;
}
// CPLT (coupled gates, b = beta per token): B = diag(beta) K, so Akb and
// Mqb are Akk and Mqk with column s scaled by beta_s; each Akk and Mqk tile
// is then also written, scaled, as the Akb / Mqb tile (KB and QB are empty).
template <class Cf, unsigned KK, unsigned KB, unsigned QK, unsigned QB, bool CPLT = false>
__device__ __forceinline__ void gram_tiles(ChunkBuf<Cf> &cb, const char *kbi, float *akbd, const float *beta, int lg,
                                           int lc) {
  constexpr bool BF16 = Cf::BF16;
  using LK = typename Cf::LK;
  using LT = typename Cf::LT;
  constexpr int C = Cf::C, NCH = Cf::NCH, NKP = Cf::NKP, NRT = Cf::NRT;
  constexpr unsigned ALL = KK | KB | QK | QB;
  Pair<BF16> tk[NKP][NCH], tq[NKP][NCH], sk[NKP][NCH], sb[NKP][NCH];
  static_for<NKP>([&](auto pc) {
    constexpr int pp = decltype(pc)::value;
    constexpr bool single = 2 * pp + 1 >= NRT;
    static_for<NCH>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (tile_row_used(KK | KB, i)) tk[pp][i] = frag32<LK, BF16, single>(cb.kqg, 16 * i + lc, pp, lg);
      if constexpr (tile_row_used(QK | QB, i)) tq[pp][i] = frag32<LK, BF16, single>(cb.kqg, C + 16 * i + lc, pp, lg);
      if constexpr (tile_col_used(KK | QK, i, NCH)) sk[pp][i] = frag32<LK, BF16, single>(kbi, 16 * i + lc, pp, lg);
      if constexpr (tile_col_used(KB | QB, i, NCH)) sb[pp][i] = frag32<LK, BF16, single>(kbi, C + 16 * i + lc, pp, lg);
    });
  });
  static_for<NCH>([&](auto rc) {
    constexpr int r = decltype(rc)::value;
    static_for<r + 1>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      static_for<4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        constexpr unsigned M = q == 0 ? KK : q == 1 ? KB : q == 2 ? QK : QB;
        if constexpr (tile_in(M, r, c)) {
          floatx4 x = zero4();
          static_for<NKP>([&](auto pc) {
            constexpr int pp = decltype(pc)::value;
            constexpr bool single = 2 * pp + 1 >= NRT;
            const Pair<BF16> &a = (q & 1) ? sb[pp][c] : sk[pp][c];
            const Pair<BF16> &b = (q >= 2) ? tq[pp][r] : tk[pp][r];
            x = mma<BF16, single>(x, a, b);
          });
          const int t = 16 * r + lc, s0 = 16 * c + 4 * lg;
          if constexpr (q == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = t > s0 + j ? x[j] : 0.f;
            st4<LT, BF16>(cb.ab, t, 32 * c + 4 * lg, x);
            if constexpr (CPLT) {
              const floatx4 y = x * *reinterpret_cast<const floatx4 *>(&beta[s0]);
              if constexpr (c != r)
                st4<LT, BF16>(cb.ab, t, 32 * c + 16 + 4 * lg, -y);
              else
                *reinterpret_cast<floatx4 *>(&akbd[r * 16 * 20 + (4 * (lc & 3) + (lc >> 2)) * 20 + 4 * lg]) = y;
            }
          } else if constexpr (q == 1) {
            if constexpr (c != r) {
              st4<LT, BF16>(cb.ab, t, 32 * c + 16 + 4 * lg, -x);
            } else {  // diagonal block, strictly lower part, fp32 for the inverse
#pragma unroll
              for (int j = 0; j < 4; ++j) x[j] = t > s0 + j ? x[j] : 0.f;
              *reinterpret_cast<floatx4 *>(&akbd[r * 16 * 20 + (4 * (lc & 3) + (lc >> 2)) * 20 + 4 * lg]) = x;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = t >= s0 + j ? x[j] : 0.f;
            st4<LT, BF16>(cb.m, t, 32 * c + (q == 3 ? 16 : 0) + 4 * lg, x);
            if constexpr (CPLT && q == 2)
              st4<LT, BF16>(cb.m, t, 32 * c + 16 + 4 * lg, x * *reinterpret_cast<const floatx4 *>(&beta[s0]));
          }
        }
      });
    });
  });
  (void)ALL;
}

// Work split of the Gram tiles and diagonal inverses over the 4 producer
// waves (masks of lower tiles per wave; INV: diagonal blocks the wave
// inverts, always blocks whose Akb tile the same wave computes, so no
// synchronisation is needed). The inverses are the longest serial part, so
// with two row blocks the waves that invert compute only the diagonal Akb
// tile they need and the other two waves take the remaining ten tiles. With
// one block waves 0 and 1 take Akk and Akb, 2 and 3 Mqk and Mqb; with more
// blocks wave 0 takes all of Akk, wave 1 all of Akb and the inverses.
// Coupled gates (Akb and Mqb as scaled Akk and Mqk): with two row blocks
// waves 0 and 1 compute the diagonal Akk tile they invert, wave 2 the
// off-diagonal Akk tile and Mqk (0,0), wave 3 the other two Mqk tiles; with
// one block, or more, wave 0 takes Akk (and the inverses) and wave 2 Mqk.
template <int NCH>
struct GramSplitCpl {
  static constexpr unsigned FULL = (1u << (NCH * (NCH + 1) / 2)) - 1u;
  static constexpr bool TWO = NCH == 2;  // tiles 0 = (0,0), 1 = (1,0), 2 = (1,1)
  static constexpr unsigned KK[4] = {TWO ? 1u : FULL, TWO ? 4u : 0u, TWO ? 2u : 0u, 0u};
  static constexpr unsigned KB[4] = {0u, 0u, 0u, 0u};
  static constexpr unsigned QK[4] = {0u, 0u, TWO ? 1u : FULL, TWO ? 6u : 0u};
  static constexpr unsigned QB[4] = {0u, 0u, 0u, 0u};
  static constexpr unsigned INV[4] = {TWO ? 1u : (1u << NCH) - 1u, TWO ? 2u : 0u, 0u, 0u};
};

template <int NCH>
struct GramSplit {
  static constexpr unsigned FULL = (1u << (NCH * (NCH + 1) / 2)) - 1u;
  static constexpr bool TWO = NCH == 2;  // tiles 0 = (0,0), 1 = (1,0), 2 = (1,1)
  static constexpr unsigned KK[4] = {TWO ? 0u : NCH == 1 ? 1u : FULL, 0u, TWO ? 3u : 0u, TWO ? 4u : 0u};
  static constexpr unsigned KB[4] = {TWO ? 1u : 0u, TWO ? 4u : NCH == 1 ? 1u : FULL, TWO ? 2u : 0u, 0u};
  static constexpr unsigned QK[4] = {0u, 0u, TWO ? 3u : FULL, TWO ? 4u : 0u};
  static constexpr unsigned QB[4] = {0u, 0u, 0u, FULL};
  static constexpr unsigned INV[4] = {TWO ? 1u : 0u, TWO ? 2u : (1u << NCH) - 1u, 0u, 0u};
};

// Inverses of the diagonal blocks r0 .. r0+NB-1 of I + Akb (strictly lower
// Akb_rr, fp32, from the Gram step) into dinv; the NB independent
// substitutions run interleaved. Lane = (column c, row quarter qq): it holds
// rows 4qq..4qq+3 of column c of (I + Akb_rr)^-1 and of Akb_rr. Forward
// substitution: at step i the lane owning row i passes the final x_i to its
// quad by DPP, and every lane updates its rows; the coefficients
// Akb_rr[row][i] of rows <= i are zero, so no row needs masking.
template <class Cf, int NB>
__device__ __forceinline__ void invert_diag(const float *akbd, typename Op<Cf::BF16>::T *dinv, int r0, int lane) {
  using O = Op<Cf::BF16>;
  constexpr int LDD = Cf::LDD;
  const int c = lane >> 2, qq = lane & 3;
  floatx4 arow[NB][4][4];  // arow[b][j][k4] = Akb_rr[4qq + j][4k4 .. 4k4+3], r = r0 + b
  floatx4 x[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        arow[b][j][k4] = *reinterpret_cast<const floatx4 *>(&akbd[(r0 + b) * 16 * 20 + (4 * j + qq) * 20 + 4 * k4]);
      x[b][j] = (4 * qq + j == c) ? 1.f : 0.f;
    }
  }
  static_for<15>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    float xi[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xi[b] = quad_bcast<i / 4>(x[b][i % 4]);
    // the element the next step broadcasts is updated first: it is the only
    // one on the dependency chain
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int jj = 1; jj <= 4; ++jj) {
        const int j = (i + jj) & 3;
        x[b][j] -= arow[b][j][i / 4][i % 4] * xi[b];
      }
  });
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) dinv[(r0 + b) * 16 * LDD + (4 * qq + j) * LDD + c] = O::cvt(x[b][j]);
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

// CPL: coupled gates (b = w = beta, one scalar per token and value head,
// passed as both p.b and p.w, [.., T, H_v]); otherwise b is per key channel
// and w per value channel. SCA: scalar decay (a one scalar per token and
// value head, [.., T, H_v]); otherwise a is per key channel. PRE: per-channel
// gates given as pre-activations x in the input dtype, activated here
// (decay a = exp(-softplus(x)) = 1 / (1 + e^x), erase and write gates
// b, w = sigmoid(x)).
// CST: store the state at every chunk boundary (PrefillParams::cst)
template <int DK, int C, int NCT, bool BF16, bool CPL, bool SCA, bool PRE, bool CST = false>
__global__ __launch_bounds__(512) void prefill_kernel(PrefillParams p) {
  using Cf = PrefillCfg<DK, C, NCT, BF16>;
  using E = Elem<BF16>;
  using O = Op<BF16>;
  using ET = typename E::T;
  using OT = typename O::T;
  using Frag = typename O::Frag;
  // four q/k (or v) elements in their stored type
  using Quad = typename std::conditional<BF16, uint2, floatx4>::type;
  using LK = typename Cf::LK;
  using LT = typename Cf::LT;
  constexpr int NRT = Cf::NRT, NCH = Cf::NCH, NKP = Cf::NKP, LDD = Cf::LDD, RPG = Cf::RPG,
                RGE = Cf::RGE;
  // Coupled gates (b = beta per token): the carry's erase term is
  // (mu beta K)^T R = (mu K)^T diag(beta) R, so the carry contracts the
  // mu K rows once with U - diag(beta) R (half the products) and the
  // mu beta K rows are not built (the Gram tiles derive Akb, Mqb from Akk,
  // Mqk). With an odd number of 16-token blocks a K32 step would pair the
  // two halves, so that case keeps both; so does the launch that stores the
  // chunk-boundary states for the backward, whose states are then those of
  // the per-channel form on the broadcast gates.
  constexpr bool HCARRY = CPL && NCH % 2 == 0 && !CST;
  // Pre-activations with the token-major build: the erase gates are
  // activated by the column waves (idle while the producers build) and handed
  // to the producers in LDS, fp32, double-buffered by chunk parity; the
  // producers activate only the decays.
  constexpr bool CBG = PRE && Cf::TOKM;
  static_assert(sizeof(PrefillSmem<Cf>) <= 160 * 1024, "LDS working set exceeds one CU");

  __shared__ PrefillSmem<Cf> sm;
  // CBG: activated erase gates of the chunks with parity 0 and 1, [token][channel]
  __shared__ __attribute__((aligned(16))) float bgl[CBG ? 2 * C * DK : 4];
  static_assert(sizeof(PrefillSmem<Cf>) + sizeof(bgl) <= 160 * 1024, "LDS working set exceeds one CU");
  GDN2_TIMER_INIT

  // workgroup -> (segment, sequence, value head, column block)
  const int ncbt = p.ncb_val + p.ncb_id;
  const int per_seg = p.B * p.H_v * ncbt;
  const int rel = blockIdx.x / per_seg;  // segment within the launch
  int n, h, cb;
  map_block(blockIdx.x - rel * per_seg, p.B, p.H_qk, p.H_v, ncbt, n, h, cb);
  size_t tok0;  // first token of the segment in the token axis of the inputs
  int Tl;       // tokens in the segment
  if (p.cu) {
    const int t0 = min(max(p.cu[n], 0), p.T), t1 = min(max(p.cu[n + 1], t0), p.T);
    tok0 = (size_t)t0;
    Tl = t1 - t0;
  } else {
    const int tseg = (p.seg_first + rel) * p.seg_len;  // first token of the segment
    tok0 = (size_t)n * p.T + tseg;
    Tl = min(p.seg_len, p.T - tseg);
  }
  const bool ident = cb >= p.ncb_val;  // identity column block
  // (uniform over the workgroup) nothing to do past the end of the
  // sequence, nor for the transition of a sequence's first segment, whose
  // entering state is known
  if ((!p.cu && p.T > 0 && Tl <= 0) || (ident && p.seg_first + rel == 0)) return;
  const int g = h / (p.H_v / p.H_qk);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int lg = lane >> 4, lc = lane & 15;
  const int d_v = p.d_v;
  const bool producer = wave < Cf::NP;
  const int cw = wave - Cf::NP;                 // consumer index
  const bool consumer = !producer && cw < NCT;  // owns a 16-column state tile
  // consumer lane's column: a value column, or for an identity block the
  // key channel whose unit vector the column starts from
  const int col = (ident ? cb - p.ncb_val : cb) * Cf::DVB + (consumer ? cw : 0) * 16 + lc;
  const bool write_o = ident ? p.oI != nullptr : (p.o && !(p.o_first_only && rel > 0));

  // Token strides in bytes, and this (sequence, head)'s token-0 bases. GT:
  // the stored type of the per-channel gates.
  static_assert(!PRE || (!CPL && !SCA), "pre-activations for per-channel gates");
  using GT = typename std::conditional<PRE, ET, float>::type;
  constexpr uint32_t GS = sizeof(GT);
  const uint32_t qk_tb = (uint32_t)(p.H_qk * DK) * sizeof(ET);
  const uint32_t ab_tb = (uint32_t)(p.H_v * DK) * GS;
  const uint32_t v_tb = (uint32_t)(p.H_v * d_v) * sizeof(ET);
  const uint32_t w_tb = (uint32_t)(p.H_v * d_v) * GS;
  const uint32_t at_tb = SCA ? (uint32_t)p.H_v * 4u : ab_tb;  // token strides of a, b and w
  const uint32_t bt_tb = CPL ? (uint32_t)p.H_v * 4u : ab_tb;
  const uint32_t wt_tb = CPL ? (uint32_t)p.H_v * 4u : w_tb;
  const ET *qh = (const ET *)p.q + tok0 * p.H_qk * DK + (size_t)g * DK;
  const ET *kh = (const ET *)p.k + tok0 * p.H_qk * DK + (size_t)g * DK;
  const ET *vh = (const ET *)p.v + tok0 * p.H_v * d_v + (size_t)h * d_v;
  const GT *ga = (const GT *)p.a, *gb = (const GT *)p.b, *gw = (const GT *)p.w;
  const GT *ah = SCA ? ga + tok0 * p.H_v + h : ga + tok0 * p.H_v * DK + (size_t)h * DK;
  const GT *bh = CPL ? gb + tok0 * p.H_v + h : gb + tok0 * p.H_v * DK + (size_t)h * DK;
  const GT *wh = CPL ? gw + tok0 * p.H_v + h : gw + tok0 * p.H_v * d_v + (size_t)h * d_v;
  // activated gates from pre-activations (four channels: the raw values are
  // the register's first two words as bf16 pairs, or all four as fp32)
  auto gate_unpack = [](floatx4 raw) -> floatx4 {
    if constexpr (BF16) {
      const uint32_t x = __float_as_uint(raw[0]), y = __float_as_uint(raw[1]);
      return floatx4{__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u), __uint_as_float(y << 16),
                     __uint_as_float(y & 0xffff0000u)};
    } else {
      return raw;
    }
  };
  auto decay4 = [](floatx4 x) {
    return floatx4{decay_from_pre(x[0]), decay_from_pre(x[1]), decay_from_pre(x[2]), decay_from_pre(x[3])};
  };
  auto gate4 = [](floatx4 x) {
    return floatx4{gate_from_pre(x[0]), gate_from_pre(x[1]), gate_from_pre(x[2]), gate_from_pre(x[3])};
  };
  // outputs: value blocks write o, identity blocks oI (written only when
  // d_v == d_k: the same token stride)
  ET *oh = (ET *)(ident ? p.oI : p.o) + tok0 * p.H_v * d_v + (size_t)h * d_v;
  const int ocb = ident ? cb - p.ncb_val : cb;  // column block within the output row
  // entering and final state of this lane's column: value blocks use S0 /
  // S_T ([B][H_v][d_k][d_v] per segment), identity blocks start from the
  // unit vector and end in M_T ([B][H_v][d_k][d_k] per segment)
  const int ld_s = ident ? DK : d_v;
  const size_t s_off = ((size_t)n * p.H_v + h) * (size_t)DK * ld_s + col;
  const float *S0p = (ident || !p.S0 || (rel > 0 && p.s0_stride == 0)) ? nullptr : p.S0 + rel * p.s0_stride;
  float *STp = ident ? p.M_T + rel * p.m_stride
               : (!p.S_T || (p.sT_last_only && rel != p.nseg - 1)) ? nullptr : p.S_T + rel * p.sT_stride;
  // byte range of a descriptor based at token t0: the C tokens of the chunk
  // starting there, fewer at the end of the segment, 0 past it (a buffer
  // access beyond the range returns 0 without touching memory). Every
  // request and store of a chunk stays inside its own C tokens.
  auto rows_left = [&](int t0, uint32_t tb) -> uint32_t { return window_bytes(t0, Tl, C, tb); };

  // ---------------------------------------------------------------- producer layout
  // Token-major (d_k = 128): producer wave w builds tokens w*C/4 .. +C/4 of
  // the chunk for all key channels; lane = (half rg, channel quad cq) holds
  // tokens w*C/4 + rg*RPG + r (r < RPG) of channels 4cq .. 4cq+3, so every
  // raw request covers two whole token rows. The decay's cumulative product
  // runs within the lane, across the halves by a lane exchange, and across
  // the waves through per-wave totals in LDS computed one step ahead.
  // Channel-major (d_k < 128): lane = (row group rg, channel quad cq) of the
  // wave's d_k/4 channels, row group fastest so that a quad's prefix product
  // runs across adjacent lanes.
  constexpr bool TOKM = Cf::TOKM;
  const int rg = TOKM ? lane >> 5 : lane % Cf::RGL;
  const int cq = TOKM ? lane & 31
                      : Cf::QPW == 8 ? (((lane / Cf::RGL) >> 1) | (((lane / Cf::RGL) & 1) << 2)) : lane / Cf::RGL;
  const bool brow = TOKM || (RGE == Cf::RGL) || rg < RGE;  // lane holds build rows
  const int ch0 = TOKM ? 4 * cq : wave * (DK / 4) + 4 * cq;
  const int tb0 = TOKM ? wave * (C / 4) + rg * RPG : rg * RPG;  // the lane's first token
  static_assert(!TOKM || RPG * 8 == C, "token-major: C/8 tokens per lane");
  const uint32_t ab_off = (uint32_t)tb0 * ab_tb + (uint32_t)ch0 * GS;
  const uint32_t qk_off = (uint32_t)tb0 * qk_tb + (uint32_t)ch0 * sizeof(ET);

  // Raw inputs of the chunks to build, held in two register sets (chunk s
  // in set s % 2) and requested two chunks ahead so that a request has more
  // than a full step to complete: decay and erase gate after the build,
  // keys and queries after the Gram tiles, so that neither burst of
  // requests delays the other phase's work.
  floatx4 ra[2][RPG], rb[2][RPG];
  Quad rk[2][RPG], rq[2][RPG];
  struct RawSrc {
    rsrc_t a, b, k, q;
  };
  auto raw_src = [&](int t0) {
    return RawSrc{make_rsrc((const char *)ah + (size_t)t0 * at_tb, rows_left(t0, at_tb)),
                  make_rsrc((const char *)bh + (size_t)t0 * bt_tb, rows_left(t0, bt_tb)),
                  make_rsrc((const char *)kh + (size_t)t0 * qk_tb, rows_left(t0, qk_tb)),
                  make_rsrc((const char *)qh + (size_t)t0 * qk_tb, rows_left(t0, qk_tb))};
  };
  auto load_ab = [&](auto P, const RawSrc &src) {
    if (brow) {
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        if constexpr (SCA) {
          const float aa = bload<float>(src.a, (uint32_t)tb0 * at_tb, r * at_tb);
          ra[P][r] = floatx4{aa, aa, aa, aa};
        } else if constexpr (PRE && BF16) {  // raw bf16 quads in the first two words
          const uint2 u = bload<uint2>(src.a, ab_off, r * ab_tb);
          ra[P][r] = floatx4{__uint_as_float(u.x), __uint_as_float(u.y), 0.f, 0.f};
        } else {
          ra[P][r] = bload<floatx4>(src.a, ab_off, r * ab_tb);
        }
        if constexpr (CBG) {
          // erase gates come from LDS (activated by the column waves)
        } else if constexpr (CPL) {
          const float bb = bload<float>(src.b, (uint32_t)tb0 * bt_tb, r * bt_tb);
          rb[P][r] = floatx4{bb, bb, bb, bb};
        } else if constexpr (PRE && BF16) {
          const uint2 u = bload<uint2>(src.b, ab_off, r * ab_tb);
          rb[P][r] = floatx4{__uint_as_float(u.x), __uint_as_float(u.y), 0.f, 0.f};
        } else {
          rb[P][r] = bload<floatx4>(src.b, ab_off, r * ab_tb);
        }
      }
    }
  };
  auto load_kq = [&](auto P, const RawSrc &src) {
    if (brow) {
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        rk[P][r] = bload<Quad>(src.k, qk_off, r * qk_tb);
        rq[P][r] = bload<Quad>(src.q, qk_off, r * qk_tb);
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

  // Pre-activations of register set P -> activated decay and erase gate, in
  // place (before the set's first use: its wave totals, then its build).
  auto activate_ab = [&](auto P) {
    if constexpr (PRE) {
      if (brow) {
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
          ra[P][r] = decay4(gate_unpack(ra[P][r]));
          if constexpr (!CBG) rb[P][r] = gate4(gate_unpack(rb[P][r]));
        }
      }
    }
  };

  // Token-major: this wave's total decay per channel for the chunk in raw
  // set P, for the next build (published by the barrier before it).
  auto wave_totals = [&](auto P) {
    if constexpr (TOKM) {
      floatx4 pr = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int r = 0; r < RPG; ++r) pr *= ra[P][r];
      const floatx4 lo = shfl4(pr, lane ^ 32);
      if (rg == 0) *reinterpret_cast<floatx4 *>(&sm.tot[wave][ch0]) = pr * lo;
    }
  };

  // Build chunk operands into buffer cbuf (producer waves; no workgroup sync
  // inside: the decay scan runs across the lanes of one wave).
  auto build = [&](auto P, ChunkBuf<Cf> &cbuf) {
    // token-major: all waves' totals of this chunk (LDS, one step ahead),
    // requested first so that they arrive while the gates are awaited
    floatx4 tw[TOKM ? Cf::NP : 1];
    if constexpr (TOKM) {
#pragma unroll
      for (int w2 = 0; w2 < Cf::NP; ++w2) tw[w2] = *reinterpret_cast<const floatx4 *>(&sm.tot[w2][ch0]);
    }
    // cumulative decay within the lane's RPG tokens
    floatx4 gl[RPG];
    floatx4 pr = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
      if (brow) pr *= ra[P][r];
      gl[r] = pr;
    }

    floatx4 inc = pr, pre;
    // factors of the operands (see the kernel's header): lam (left: keys and
    // queries) and mu (right: the Gram matrices' and the carry's keys and
    // erase keys), as lam = gl[r] * cL, mu = sl[r] * cR with the lane's
    // prefix gl and suffix sl of its own tokens' decays
    floatx4 cL, cR;
    const floatx4 one = {1.f, 1.f, 1.f, 1.f};
    int flag = 0;
    if constexpr (TOKM) {
      // the other lane half's product (lane exchange) and the chunk's decay
      const floatx4 lo = shfl4(pr, lane ^ 32);
      const floatx4 gC = (tw[0] * tw[1]) * (tw[2] * tw[3]);
      floatx4 before = one;  // the waves before this one
#pragma unroll
      for (int w2 = 0; w2 < Cf::NP - 1; ++w2)
        if (w2 < wave) before *= tw[w2];
      pre = rg ? before * lo : before;  // tokens before the lane's first
      inc = pre * pr;
      auto rcp4 = [](floatx4 x) {
        return floatx4{__builtin_amdgcn_rcpf(x[0]), __builtin_amdgcn_rcpf(x[1]), __builtin_amdgcn_rcpf(x[2]),
                       __builtin_amdgcn_rcpf(x[3])};
      };
      // The anchor, the same on every producer wave (lanes 0..31 hold every
      // channel once): the chunk start while the whole chunk's decay is at
      // least kMinChunkDecay on every channel, else the middle token while
      // both half chunks' are at least kMinHalfDecay, else token by token.
      // (The test also reads the lane's own product, which is never
      // negative: the decision then waits for this chunk's gates rather than
      // holding back the products that use them.)
      const bool mild = __all(gC[0] >= kMinChunkDecay && gC[1] >= kMinChunkDecay && gC[2] >= kMinChunkDecay &&
                              gC[3] >= kMinChunkDecay && inc[0] >= 0.f);
      if (mild) {  // chunk start: lam = gamma_t, mu = 1 / gamma_t
        cL = pre;
        cR = rcp4(inc);
        if (wave == Cf::NP - 1 && rg == 1) *reinterpret_cast<floatx4 *>(&cbuf.gamc[ch0]) = inc;  // gamma_C
      } else {
        constexpr int HW = Cf::NP / 2;  // waves of the first half (tokens 0 .. m)
        floatx4 half_before = one, half_after = one;  // within the lane's own half of the chunk
#pragma unroll
        for (int w2 = 0; w2 < Cf::NP; ++w2) {
          if (w2 < wave && (w2 >= HW) == (wave >= HW)) half_before *= tw[w2];
          if (w2 > wave && (w2 >= HW) == (wave >= HW)) half_after *= tw[w2];
        }
        const floatx4 h1 = tw[0] * tw[1], h2 = tw[2] * tw[3];  // half-chunk decays
        flag = __all(h1[0] >= kMinHalfDecay && h1[1] >= kMinHalfDecay && h1[2] >= kMinHalfDecay &&
                     h1[3] >= kMinHalfDecay && h2[0] >= kMinHalfDecay && h2[1] >= kMinHalfDecay &&
                     h2[2] >= kMinHalfDecay && h2[3] >= kMinHalfDecay)
                   ? kChunkMid
                   : kChunkSteps;
        if (wave < HW) {  // t <= m: lam = 1 / (decays t+1 .. m), mu = decays t+1 .. m
          const floatx4 p1 = rg ? half_after : lo * half_after;  // lane's last token .. m
          cL = rcp4(pr * p1);
          cR = p1;
        } else {  // t > m: lam = decays m+1 .. t, mu = 1 / lam
          cL = rg ? half_before * lo : half_before;
          cR = rcp4(pr * cL);
        }
        // the carry's factor on the gamma_m-scaled entering state, and
        // gamma_m (wave 0's first lane half holds every channel once)
        if (wave == 0 && rg == 0) {
          *reinterpret_cast<floatx4 *>(&cbuf.gamc[ch0]) = h2;
          *reinterpret_cast<floatx4 *>(&cbuf.gamm[ch0]) = h1;
        }
      }
    } else {
      if constexpr (RGE <= 16) {
        // inclusive prefix product over the row groups (adjacent lanes): DPP
        // row shifts when a quad's groups fit in one 16-lane row
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
      if (rg == 0) pre = one;
      // channel-major build: the anchor is the chunk start (lam = gamma_t,
      // mu = 1 / gamma_t), which bounds every factor by 1 / gamma_C: the
      // whole chunk's decay is checked against kMinChunkDecay
      cL = pre;
      cR = floatx4{__builtin_amdgcn_rcpf(inc[0]), __builtin_amdgcn_rcpf(inc[1]), __builtin_amdgcn_rcpf(inc[2]),
                   __builtin_amdgcn_rcpf(inc[3])};
      const bool last = rg == RGE - 1;
      const bool lane_bad = last && (!(inc[0] >= kMinChunkDecay) || !(inc[1] >= kMinChunkDecay) ||
                                     !(inc[2] >= kMinChunkDecay) || !(inc[3] >= kMinChunkDecay));
      if (last) *reinterpret_cast<floatx4 *>(&cbuf.gamc[ch0]) = inc;
      flag = __any(lane_bad) ? kChunkSteps : 0;
    }
    if (lane == 0) cbuf.bad[wave] = flag;
    if constexpr (CPL) {  // beta of the lane's tokens, for the Gram tiles
      if (brow && cq == 0 && (TOKM || wave == 0)) {
#pragma unroll
        for (int r = 0; r < RPG; ++r) sm.beta[P][tb0 + r] = rb[P][r][0];
      }
    }
    if (brow) {
      // suffix products of the lane's own decays: sl[r] = a_{r+1} ... a_{RPG-1}
      floatx4 sl[RPG];
      sl[RPG - 1] = one;
#pragma unroll
      for (int r = RPG - 2; r >= 0; --r) sl[r] = sl[r + 1] * ra[P][r + 1];
      floatx4 kbq[4], bkq[4];
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        const int tl = tb0 + r;
        const floatx4 lam = gl[r] * cL;
        const floatx4 mu = sl[r] * cR;
        const floatx4 kv = quad_f(rk[P][r]);
        const floatx4 qv = quad_f(rq[P][r]);
        const floatx4 kr = kv * mu;
        const floatx4 bg = CBG ? *reinterpret_cast<const floatx4 *>(&bgl[((int)decltype(P)::value * C + tl) * DK + ch0])
                               : rb[P][r];
        const floatx4 bkr = bg * kr;
        st4<LK, BF16>(cbuf.kqg, tl, ch0, kv * lam);
        st4<LK, BF16>(cbuf.kqg, C + tl, ch0, qv * lam);
        char *kbi_b = Cf::TRC ? cbuf.kbi : sm.kbi;
        st4<LK, BF16>(kbi_b, tl, ch0, kr);
        if constexpr (!HCARRY) st4<LK, BF16>(kbi_b, C + tl, ch0, bkr);
        // fp32: the carry's operands transposed, 4 (or 2) consecutive tokens
        // per channel at once
        if constexpr (!Cf::TRC) {
          if constexpr (RPG % 4 == 0) {
            kbq[r & 3] = kr;
            bkq[r & 3] = bkr;
            if ((r & 3) == 3) {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                st4<LT, BF16>(cbuf.kbiT, ch0 + c, tl - 3, floatx4{kbq[0][c], kbq[1][c], kbq[2][c], kbq[3][c]});
                if constexpr (!HCARRY)
                  st4<LT, BF16>(cbuf.kbiT, ch0 + c, C + tl - 3, floatx4{bkq[0][c], bkq[1][c], bkq[2][c], bkq[3][c]});
              }
            }
          } else if constexpr (RPG % 2 == 0) {
            if (r & 1) {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                st2<LT, BF16>(cbuf.kbiT, ch0 + c, tl - 1, kbq[0][c], kr[c]);
                if constexpr (!HCARRY) st2<LT, BF16>(cbuf.kbiT, ch0 + c, C + tl - 1, bkq[0][c], bkr[c]);
              }
            }
            kbq[0] = kr;
            bkq[0] = bkr;
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              st1<LT, BF16>(cbuf.kbiT, ch0 + c, tl, kr[c]);
              if constexpr (!HCARRY) st1<LT, BF16>(cbuf.kbiT, ch0 + c, C + tl, bkr[c]);
            }
          }
        }
      }
    }
  };

  const int nfull = Tl / C;
  // pipeline steps: chunk s is produced in step s and consumed in step s+1;
  // the count is rounded up to even so that the producers' two-step loop
  // body has no conditional part (the extra step only passes the barriers)
  const int nsteps = (nfull + 2) & ~1;

  // The two roles run separate loops (the branch is wave-uniform) of nsteps
  // steps each; every step executes exactly two workgroup barriers, so the
  // barrier counts of producer and consumer waves always match.
  if (producer) {
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    {  // chunks 0 and 1, unconditional and in the loop's request order
       // (the scheduling barriers keep that order)
      const RawSrc src0 = raw_src(nfull > 0 ? 0 : Tl);
      const RawSrc src1 = raw_src(nfull > 1 ? C : Tl);
      load_ab(I0(), src0);
      __builtin_amdgcn_sched_barrier(0);
      load_kq(I0(), src0);
      __builtin_amdgcn_sched_barrier(0);
      load_ab(I1(), src1);
      __builtin_amdgcn_sched_barrier(0);
      load_kq(I1(), src1);
      __builtin_amdgcn_sched_barrier(0);
      activate_ab(I0());
      if constexpr (TOKM) {
        // chunk 0's wave totals; the barrier publishes them (the other waves
        // execute a matching one before their loop)
        wave_totals(I0());
        __syncthreads();
      }
    }
    // One pipeline step; chunk s uses raw register set P = s % 2. The
    // requests for chunk s+2 are issued unconditionally (past the last
    // chunk they read nothing): every path through the loop then has the
    // same request order, so the compiler's waits before the build only
    // cover set P.
    auto pstep = [&](auto P, int s) {
      ChunkBuf<Cf> &pb = sm.buf[P];  // produced this step (chunk s)
      const bool produce = s < nfull;
      const int tn = s + 2 < nfull ? (s + 2) * C : Tl;
      // phase A: operands of chunk s, then request chunk s+2's gates
      if (produce) build(P, pb);
      load_ab(P, raw_src(tn));
      GDN2_MARK(0);
      __syncthreads();
      GDN2_MARK(7);
      // phase B: Gram tiles (and diagonal inverses), then chunk s+2's keys
      // and queries
      if (produce) {
        using GS = typename std::conditional<CPL, GramSplitCpl<NCH>, GramSplit<NCH>>::type;
        // the diagonal blocks whose Akb tile this wave has just written
        auto invert_set = [&](auto mask) {
          static_for<NCH>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            if constexpr (((decltype(mask)::value >> r) & 1u) != 0) invert_diag<Cf, 1>(sm.akbd, pb.dinv, r, lane);
          });
        };
        auto gram_wave = [&](auto wc) {
          constexpr int w = decltype(wc)::value;
          gram_tiles<Cf, GS::KK[w], GS::KB[w], GS::QK[w], GS::QB[w], CPL>(pb, Cf::TRC ? pb.kbi : sm.kbi, sm.akbd,
                                                                          sm.beta[P], lg, lc);
          invert_set(std::integral_constant<unsigned, GS::INV[w]>());
        };
        switch (wave) {
          case 0: gram_wave(std::integral_constant<int, 0>()); break;
          case 1: gram_wave(std::integral_constant<int, 1>()); break;
          case 2: gram_wave(std::integral_constant<int, 2>()); break;
          default: gram_wave(std::integral_constant<int, 3>()); break;
        }
      }
      GDN2_MARK(4);
      activate_ab(std::integral_constant<int, decltype(P)::value ^ 1>());
      wave_totals(std::integral_constant<int, decltype(P)::value ^ 1>());  // chunk s+1
      GDN2_MARK(6);
      load_kq(P, raw_src(tn));
      GDN2_MARK(2);
      __syncthreads();  // buffer P is now complete for the consumers
      GDN2_MARK(7);
    };
    for (int s = 0; s < nsteps; s += 2) {
      pstep(I0(), s);
      pstep(I1(), s + 1);
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
      S[rt][j] = !consumer ? 0.f
                 : ident  ? (16 * rt + 4 * lg + j == col ? 1.f : 0.f)
                 : S0p    ? S0p[s_off + (size_t)(16 * rt + 4 * lg + j) * d_v]
                          : 0.f;
  // The entering state is complete before the chunk loop: otherwise the
  // compiler, merging loop entry and back edge, waits for every outstanding
  // load (including the next chunk's prefetch) at each first use of S.
  __builtin_amdgcn_s_waitcnt(0);

  // Chunk-boundary states (see PrefillParams::cst): this lane's column,
  // four consecutive key channels per tile.
  const int cst_nc = (Tl + C - 1) / C;           // entries of this segment: 0 .. cst_nc
  const int cst_j = CST ? n % p.cst_segs : 0;     // segment within its sequence
  const bool cst_last = cst_j == p.cst_segs - 1;  // writes the final entry
  ET *const cstp =
      (CST && consumer && !ident)
          ? (ET *)p.cst + ((((size_t)(n / p.cst_segs) * p.H_v + h) * (size_t)(cst_nc * p.cst_segs + 1) +
                            (size_t)cst_j * cst_nc) * d_v + col) * DK + 4 * lg
          : nullptr;
  auto store_cst = [&](int e) {
    if constexpr (!CST) return;
    if (e == cst_nc && !cst_last) return;  // the next segment's entry 0
    ET *dst = cstp + (size_t)e * d_v * DK;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      if constexpr (BF16) {
        *reinterpret_cast<bf16x4 *>(dst + 16 * rt) = __builtin_convertvector(S[rt], bf16x4);
      } else {
        *reinterpret_cast<floatx4 *>(dst + 16 * rt) = S[rt];
      }
    }
  };
  if (CST && cstp) store_cst(0);

  // Token-by-token steps on this wave's columns (exact for any decay).
  auto token_steps = [&](int tb, int te) __attribute__((always_inline)) {
    for (int t = tb; t < te; ++t) {
      const GT *at = ah + (size_t)t * (at_tb / GS);
      const GT *bt = bh + (size_t)t * (bt_tb / GS);
      const ET *kt = kh + (size_t)t * (qk_tb / sizeof(ET));
      const ET *qt = qh + (size_t)t * (qk_tb / sizeof(ET));
      float part = 0.f;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int i0 = 16 * rt + 4 * lg;
        floatx4 av;
        if constexpr (PRE)
          av = decay4(E::ld4(at + i0));
        else
          av = SCA ? floatx4{at[0], at[0], at[0], at[0]} : *reinterpret_cast<const floatx4 *>(at + i0);
        const floatx4 kv = E::ld4(kt + i0);
        S[rt] *= av;
        part += S[rt][0] * kv[0] + S[rt][1] * kv[1] + S[rt][2] * kv[2] + S[rt][3] * kv[3];
      }
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);  // key read r for this column
      float wg;
      if constexpr (PRE)
        wg = gate_from_pre(E::ld(wh + (size_t)t * (wt_tb / GS) + col));
      else
        wg = wh[(size_t)t * (wt_tb / GS) + (CPL ? 0 : col)];
      const float u = ident ? 0.f : wg * E::ld(vh + (size_t)t * (v_tb / sizeof(ET)) + col);
      float po = 0.f;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int i0 = 16 * rt + 4 * lg;
        floatx4 bv;
        if constexpr (PRE)
          bv = gate4(E::ld4(bt + i0));
        else
          bv = CPL ? floatx4{bt[0], bt[0], bt[0], bt[0]} : *reinterpret_cast<const floatx4 *>(bt + i0);
        const floatx4 kv = E::ld4(kt + i0);
        const floatx4 qv = E::ld4(qt + i0);
        S[rt] = S[rt] - (bv * kv) * part + kv * u;
        po += S[rt][0] * qv[0] + S[rt][1] * qv[1] + S[rt][2] * qv[2] + S[rt][3] * qv[3];
      }
      po += __shfl_xor(po, 16, 64);
      po += __shfl_xor(po, 32, 64);
      if (lg == 0 && write_o) E::st(oh + (size_t)t * (v_tb / sizeof(ET)) + col, po);
    }
    // Drain every memory operation of this path here: the fast path reuses
    // these registers, and an operation left in flight across the merge would
    // make the compiler wait for all outstanding loads (including the next
    // chunk's prefetch) at the first such reuse.
    __builtin_amdgcn_s_waitcnt(0);
  };

  // U = w * v. The column waves split the chunk's tokens: lane (ut, uc) of
  // column wave cw requests token cw * UTPW + i * UTPI + ut, columns
  // 8 uc .. 8 uc + 7 of the workgroup's block, as 16-byte loads. Chunk c's
  // raw values (register set c % 2) are requested two steps before they are
  // used: in step c - 1 (chunk 0 before the loop); in step c + 1 their
  // products are staged in LDS ([token][column], operand type) and each wave
  // reads its own columns back as MFMA fragments.
  constexpr int UNI = Cf::UNI, UTPI = Cf::UTPI, UTPW = Cf::UTPW, UROW = Cf::UROW;
  constexpr int NVL = BF16 ? 1 : 2;  // 16-byte loads of v per 8 columns
  floatx4 rv[2][UNI][NVL], rw[2][UNI][2];
  const int ut = lane / Cf::ULPT, uc = lane % Cf::ULPT;
  const int utok = cw * UTPW + ut;  // first token of this lane (i = 0)
  const uint32_t uv_off = (uint32_t)utok * v_tb + (uint32_t)(cb * Cf::DVB + 8 * uc) * sizeof(ET);
  const uint32_t uw_off = CPL ? (uint32_t)utok * wt_tb : (uint32_t)utok * w_tb + (uint32_t)(cb * Cf::DVB + 8 * uc) * GS;
  auto load_u = [&](auto P, int t0) {
    const rsrc_t rv_ = make_rsrc((const char *)vh + (size_t)t0 * v_tb, rows_left(t0, v_tb));
    const rsrc_t rw_ = make_rsrc((const char *)wh + (size_t)t0 * wt_tb, rows_left(t0, wt_tb));
#pragma unroll
    for (int i = 0; i < UNI; ++i) {
#pragma unroll
      for (int e = 0; e < NVL; ++e)
        rv[P][i][e] = bload<floatx4>(rv_, uv_off + 16u * e, (uint32_t)(i * UTPI) * v_tb);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if constexpr (CPL) {  // one gate per token, for all 8 columns
          if (e == 0) {
            const float bb = bload<float>(rw_, uw_off, (uint32_t)(i * UTPI) * wt_tb);
            rw[P][i][0] = rw[P][i][1] = floatx4{bb, bb, bb, bb};
          }
        } else if constexpr (PRE && BF16) {  // 8 bf16 pre-activations in one 16-byte load
          if (e == 0) {
            rw[P][i][0] = bload<floatx4>(rw_, uw_off, (uint32_t)(i * UTPI) * w_tb);
            rw[P][i][1] = zero4();
          }
        } else {
          rw[P][i][e] = bload<floatx4>(rw_, uw_off + 16u * e, (uint32_t)(i * UTPI) * w_tb);
        }
    }
  };
  // products of register set PP into the staging rows (lanes past the
  // wave's share of tokens hold duplicates and write nothing)
  auto stage_u = [&](auto PP) {
#pragma unroll
    for (int i = 0; i < UNI; ++i) {
      if (UTPW % UTPI == 0 || i * UTPI + ut < UTPW) {
        floatx4 v8[2];
        if constexpr (BF16) {
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 raw = __builtin_bit_cast(u32x4, rv[PP][i][0]);
          v8[0] = floatx4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                          __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
          v8[1] = floatx4{__uint_as_float(raw.z << 16), __uint_as_float(raw.z & 0xffff0000u),
                          __uint_as_float(raw.w << 16), __uint_as_float(raw.w & 0xffff0000u)};
        } else {
          v8[0] = rv[PP][i][0];
          v8[1] = rv[PP][i][NVL - 1];
        }
        floatx4 w8[2] = {rw[PP][i][0], rw[PP][i][1]};
        if constexpr (PRE && BF16) {  // 8 bf16 pre-activations -> write gates
          const floatx4 raw = rw[PP][i][0];
          w8[0] = gate4(gate_unpack(floatx4{raw[0], raw[1], 0.f, 0.f}));
          w8[1] = gate4(gate_unpack(floatx4{raw[2], raw[3], 0.f, 0.f}));
        } else if constexpr (PRE) {
          w8[0] = gate4(w8[0]);
          w8[1] = gate4(w8[1]);
        }
        char *dst = sm.ubuf + (utok + i * UTPI) * UROW + 8 * uc * (int)sizeof(OT);
        if constexpr (BF16) {
          const bf16x4 lo = __builtin_convertvector(w8[0] * v8[0], bf16x4);
          const bf16x4 hi = __builtin_convertvector(w8[1] * v8[1], bf16x4);
          *reinterpret_cast<bf16x8 *>(dst) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          *reinterpret_cast<floatx4 *>(dst) = w8[0] * v8[0];
          *reinterpret_cast<floatx4 *>(dst + 16) = w8[1] * v8[1];
        }
      }
    }
  };
  // The carry's A operand for key-channel tile rt and K32 block pp: rows =
  // channels 16 rt .. +15, k = the columns [K part (tokens) | beta part] of
  // the transposed kbi, i.e. kbi row 32 pp + k. bf16: two transposing reads
  // of the kbi rows (lane j of a 16-lane group addresses kbi row
  // 32 pp + 16 h + 4 lg + j / 4, channels 16 rt + 4 (j % 4) .. +3, 8 bytes;
  // lane (lc, lg) then holds rows 4 lg .. 4 lg + 3 (+16 h) of channel
  // 16 rt + lc); fp32: rows of the transposed copy.
  auto carry_frag = [&](const ChunkBuf<Cf> &cb, int rt, int pp) -> Pair<BF16> {
    if constexpr (Cf::TRC) {
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      auto rd = [&](int h) {
        const char *src = cb.kbi + Cf::LK::off(32 * pp + 16 * h + 4 * lg + (lc >> 2), 16 * rt + 4 * (lc & 3));
        const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16 *)(__attribute__((address_space(3))) const char *)src);
        return __builtin_bit_cast(Frag, r);
      };
      return Pair<BF16>{rd(0), rd(1)};
    } else {
      return frag32<LT, BF16>(cb.kbiT, 16 * rt + lc, pp, lg);
    }
  };
  // this wave's U fragment of 16-token block c: lane (lc, lg) gets tokens
  // 16c + 4lg .. +3 of column lc. bf16: one transposing read per fragment
  // (within a 16-lane group, lane 4a + b receives element b of the 8-byte
  // rows addressed by lanes a, a + 4, a + 8, a + 12; lane j addresses token
  // 16c + 4lg + j / 4, columns 4 (j % 4) .. +3); fp32: four element reads.
  auto read_u = [&](int c) -> Frag {
    if constexpr (BF16) {
      const char *src = sm.ubuf + (16 * c + 4 * lg + (lc >> 2)) * UROW + (cw * 16 + 4 * (lc & 3)) * 2;
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16 *)(__attribute__((address_space(3))) const char *)src);
      return __builtin_bit_cast(Frag, r);
    } else {
      const float *src = reinterpret_cast<const float *>(sm.ubuf + (16 * c + 4 * lg) * UROW) + cw * 16 + lc;
      return Frag{src[0], src[UROW / 4], src[2 * (UROW / 4)], src[3 * (UROW / 4)]};
    }
  };

  // Outputs. Each column wave writes its 16-column tile of the chunk's
  // outputs to the staging rows; in the next step the waves store whole rows
  // (the workgroup's DVB columns of a token, 8 bytes per lane), so every
  // output line is written by one instruction. Column wave cw stores rows
  // cw * ORPW + i * ORPI + lane / OLPR, bytes 8 (lane % OLPR) .. +7.
  constexpr int OROW = Cf::OROW, OLPR = Cf::OLPR, ORPI = Cf::ORPI, ORPW = Cf::ORPW, ONI = Cf::ONI;
  int otc = -1;  // first token of the staged outputs (-1: none)
  const int orow0 = (consumer ? cw : 0) * ORPW + lane / OLPR;
  const uint32_t o_off = (uint32_t)orow0 * v_tb + (uint32_t)(ocb * Cf::DVB * Cf::OES + 8 * (lane % OLPR));
  uint2 ox[ONI];
  auto read_o = [&]() {
#pragma unroll
    for (int i = 0; i < ONI; ++i)
      ox[i] = *reinterpret_cast<const uint2 *>(sm.obuf + (orow0 + i * ORPI) * OROW + 8 * (lane % OLPR));
  };
  // The stores are issued on every call (with nothing pending, into an empty
  // range: dropped without a memory access) so that the number of memory
  // operations between a request and its use is the same on every path,
  // which keeps the compiler's waits for the U requests exact.
  auto store_o = [&]() {
    const bool pend = otc >= 0 && write_o;
    const int t = pend ? otc : 0;
    const rsrc_t ro_ = make_rsrc((const char *)oh + (size_t)t * v_tb, pend ? rows_left(t, v_tb) : 0u);
#pragma unroll
    for (int i = 0; i < ONI; ++i) bstore(ox[i], ro_, o_off, (uint32_t)(i * ORPI) * v_tb);
    otc = -1;
  };

  // CBG: erase-gate pre-activations. Column wave cw (all four, consumers or
  // not) requests tokens cw C/4 + 4 i + lane/16 (i < C/16), channels
  // 8 (lane % 16) .. +7 (one 16-byte load in bf16, two in fp32), into
  // register set c % 2 for chunk c, two steps before the set is activated and
  // written to LDS buffer c % 2 (at the end of step c - 1, or before the loop
  // for c = 0).
  constexpr int BGI = CBG ? C / 16 : 1, BGL = BF16 ? 1 : 2;
  floatx4 rbg[2][BGI][BGL];
  const int bg_tok = (cw & 3) * (C / 4) + (lane >> 4), bg_ch = 8 * (lane & 15);
  const uint32_t bg_off = (uint32_t)bg_tok * bt_tb + (uint32_t)bg_ch * GS;
  auto load_bg = [&](auto S, int t0) {
    if constexpr (CBG) {
      const rsrc_t rs = make_rsrc((const char *)bh + (size_t)t0 * bt_tb, rows_left(t0, bt_tb));
#pragma unroll
      for (int i = 0; i < BGI; ++i)
#pragma unroll
        for (int e = 0; e < BGL; ++e)
          rbg[decltype(S)::value][i][e] = bload<floatx4>(rs, bg_off + 16u * e, (uint32_t)(4 * i) * bt_tb);
    }
  };
  auto stage_bg = [&](auto S) {
    if constexpr (CBG) {
      constexpr int b = decltype(S)::value;
#pragma unroll
      for (int i = 0; i < BGI; ++i) {
        floatx4 g8[2];
        if constexpr (BF16) {
          const floatx4 raw = rbg[b][i][0];
          g8[0] = gate4(gate_unpack(floatx4{raw[0], raw[1], 0.f, 0.f}));
          g8[1] = gate4(gate_unpack(floatx4{raw[2], raw[3], 0.f, 0.f}));
        } else {
          g8[0] = gate4(rbg[b][i][0]);
          g8[1] = gate4(rbg[b][i][BGL - 1]);
        }
        float *dst = &bgl[(b * C + bg_tok + 4 * i) * DK + bg_ch];
        *reinterpret_cast<floatx4 *>(dst) = g8[0];
        *reinterpret_cast<floatx4 *>(dst + 4) = g8[1];
      }
    }
  };
  if constexpr (CBG) load_bg(std::integral_constant<int, 0>(), nfull > 0 ? 0 : Tl);

  // consumer registers carried across the phases of one step
  Frag Uf[NCH], Rf[NCH], Rn[NCH], Wf[HCARRY ? NCH : 1];
  floatx4 X[NCH], Y[NCH];
  // One pipeline step (chunk s-1 consumed from set PP, which then receives
  // chunk s+1); the loop runs two steps per iteration so that both U
  // register sets have fixed registers (no copies that would wait for the
  // requests).
  auto cstep = [&](auto P, int s) {
    constexpr int PP = decltype(P)::value ^ 1;  // set of the consumed chunk
    ChunkBuf<Cf> &cbf = sm.buf[(s + 1) & 1];  // consumed this step (chunk s-1)
    const int tc = (s - 1) * C;               // first token of the consumed chunk
    const bool live = s >= 1 && s <= nfull;   // a chunk is consumed this step
    // ---------------------------------------------------------------- phase A
    // The operand reads of X and Y and the chunk's flags are issued first
    // (reading a buffer that holds no chunk is harmless), so that their LDS
    // latency overlaps the U conversion, the output stores and the U requests;
    // the scheduling barriers keep that order.
    read_o();  // first: its wait then covers only these reads
    Pair<BF16> kf[NCH][NKP], qf[NCH][NKP];
    static_for<NKP>([&](auto pc) {
      constexpr int pp = decltype(pc)::value;
      constexpr bool single = 2 * pp + 1 >= NRT;
#pragma unroll
      for (int r = 0; r < NCH; ++r) {
        kf[r][pp] = frag32<LK, BF16, single>(cbf.kqg, 16 * r + lc, pp, lg);
        qf[r][pp] = frag32<LK, BF16, single>(cbf.kqg, C + 16 * r + lc, pp, lg);
      }
    });
    const int flags = cbf.bad[0] | cbf.bad[1] | cbf.bad[2] | cbf.bad[3];
    __builtin_amdgcn_sched_barrier(0);
    // U of the consumed chunk (requested two steps ago) into the staging rows
    if (consumer) stage_u(std::integral_constant<int, PP>());
    store_o();
    // unconditional (reads nothing past the last chunk): one request order on
    // every path keeps the compiler's waits exact
    load_u(std::integral_constant<int, PP>(), consumer && !ident && s + 1 < nfull ? (s + 1) * C : Tl);
    __builtin_amdgcn_sched_barrier(0);
    // the same flags are read by every wave: the chunk's path is workgroup-uniform
    const bool chunk_bad = live && (flags & kChunkSteps) != 0;
    const bool cbad = consumer && live && chunk_bad;
    const bool fast = consumer && live && !chunk_bad;
    if (cbad) {
      token_steps(tc, tc + C);
    } else if (fast) {
      // X = (lam * K) diag(A) S0, Y = (lam * Q) diag(A) S0 (the held state
      // is already diag(A) S0: see the end of the step). Y is formed
      // transposed (operands swapped): lane (lc, lg) holds Y[t = lc] at
      // columns 4lg..4lg+3, the layout of the output store.
      Pair<BF16> Sp[NKP];
#pragma unroll
      for (int pp = 0; pp < NKP; ++pp)
        Sp[pp] = Pair<BF16>{O::from_acc(S[2 * pp]), 2 * pp + 1 < NRT ? O::from_acc(S[(2 * pp + 1) % NRT]) : O::zero()};
#pragma unroll
      for (int r = 0; r < NCH; ++r) {
        X[r] = zero4();
        Y[r] = zero4();
        static_for<NKP>([&](auto pc) {
          constexpr int pp = decltype(pc)::value;
          constexpr bool single = 2 * pp + 1 >= NRT;
          X[r] = mma<BF16, single>(X[r], kf[r][pp], Sp[pp]);
          Y[r] = mma<BF16, single>(Y[r], Sp[pp], qf[r][pp]);  // transposed
        });
      }
    }
    GDN2_MARK(1);
    __syncthreads();
    GDN2_MARK(7);
    // ---------------------------------------------------------------- phase B
    if (fast) {
      // All of this phase's LDS operands are read up front: U, the diagonal
      // inverses and Gram blocks of the solve and the outputs, then the
      // transposed keys and gamma_C of the carry.
      Frag df[NCH];
      Pair<BF16> af[NCH][NCH], mf[NCH][NCH], tf[NRT][NCH];
      floatx4 gc[NRT];
#pragma unroll
      for (int r = 0; r < NCH; ++r) {
        Uf[r] = read_u(r);
        df[r] = O::ld(cbf.dinv + r * 16 * LDD + lc * LDD + 4 * lg);
#pragma unroll
        for (int c = 0; c <= r; ++c) {
          // pair c: [Akk block c | -Akb block c]; the last pair only has Akk
          af[r][c] = c < r ? frag32<LT, BF16>(cbf.ab, 16 * r + lc, c, lg)
                           : frag32<LT, BF16, true>(cbf.ab, 16 * r + lc, c, lg);
          mf[r][c] = frag32<LT, BF16>(cbf.m, 16 * r + lc, c, lg);  // [Mqk block c | Mqb block c]
        }
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
        for (int pp = 0; pp < (HCARRY ? NCH / 2 : NCH); ++pp) tf[rt][pp] = carry_frag(cbf, rt, pp);
        gc[rt] = *reinterpret_cast<const floatx4 *>(&cbf.gamc[16 * rt + 4 * lg]);
      }
      // Z = X + Akk U, then (I + Akb) R = Z by blocked forward substitution:
      // R_r = D_r (Z_r - sum_{c<r} Akb_rc R_c), one chain over the pairs
      // ([Akk_rc | -Akb_rc], [U_c ; R_c]) for c < r and (Akk_rr, U_r).
      static_for<NCH>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        floatx4 acc = X[r];
#pragma unroll
        for (int c = 0; c < r; ++c) acc = mma<BF16>(acc, af[r][c], Pair<BF16>{Uf[c], Rf[c]});
        acc = mma<BF16, true>(acc, af[r][r], Pair<BF16>{Uf[r], O::zero()});
        const floatx4 R = mma<BF16, true>(zero4(), Pair<BF16>{df[r], O::zero()}, Pair<BF16>{O::from_acc(acc), O::zero()});
        Rf[r] = O::from_acc(R);
        Rn[r] = O::from_acc(-R);
        if constexpr (HCARRY) {  // U - diag(beta) R of this lane's tokens 16 r + 4 lg ..
          const floatx4 b4 = *reinterpret_cast<const floatx4 *>(&sm.beta[PP][16 * r + 4 * lg]);
          Wf[r] = O::from_acc(__builtin_convertvector(Uf[r], floatx4) - b4 * R);
        }
      });
      GDN2_MARK(3);
      // O^T = Y^T + U^T Mqk^T - R^T Mqb^T, one chain over the pairs
      // ([U_c ; -R_c]^T, [Mqk_rc | Mqb_rc]); U and R tiles are already A
      // operands of the transposed product. The outputs go to the staging
      // rows and are stored to memory in the next step.
      static_for<NCH>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        floatx4 acc = Y[r];
#pragma unroll
        for (int c = 0; c <= r; ++c) acc = mma<BF16>(acc, Pair<BF16>{Uf[c], Rn[c]}, mf[r][c]);
        char *dst = sm.obuf + (16 * r + lc) * OROW + (cw * 16 + 4 * lg) * Cf::OES;
        if constexpr (BF16) {
          *reinterpret_cast<bf16x4 *>(dst) = __builtin_convertvector(acc, bf16x4);
        } else {
          *reinterpret_cast<floatx2 *>(dst) = floatx2{acc[0], acc[1]};
          *reinterpret_cast<floatx2 *>(dst + 8) = floatx2{acc[2], acc[3]};
        }
      });
      otc = tc;
      // S_C = diag(gamma_C / A) (diag(A) S0 + (mu K)^T U - (mu beta)^T R)
      // with the anchor's cumulative decay A (1 at the chunk start, gamma_m
      // in the middle) and mu_s = A / gamma_s: kbiT columns are
      // [K part | beta part], K16 block kb pairs with U_kb or -R_(kb - NCH)
      // (coupled gates: only the K part, paired with U - diag(beta) R)
      auto ub = [&](int kb) { return kb < NCH ? Uf[kb % NCH] : Rn[(kb - NCH) % NCH]; };
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        floatx4 acc = S[rt];
        if constexpr (HCARRY) {
#pragma unroll
          for (int pp = 0; pp < NCH / 2; ++pp) acc = mma<BF16>(acc, tf[rt][pp], Pair<BF16>{Wf[2 * pp], Wf[2 * pp + 1]});
        } else {
#pragma unroll
          for (int pp = 0; pp < NCH; ++pp) acc = mma<BF16>(acc, tf[rt][pp], Pair<BF16>{ub(2 * pp), ub(2 * pp + 1)});
        }
        S[rt] = acc * gc[rt];
      }
    }
    if (CST && cstp && live) store_cst(s);  // the state entering chunk s
    // The state enters a chunk with the middle anchor (built in this step's
    // first phase, consumed in the next step) as diag(gamma_m) S: scaled
    // here, after the carry, so that the other chunks need no scaling.
    if constexpr (Cf::TOKM) {
      const ChunkBuf<Cf> &nb = sm.buf[s & 1];
      if (consumer && s < nfull && ((nb.bad[0] | nb.bad[1] | nb.bad[2] | nb.bad[3]) & kChunkMid)) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) S[rt] *= *reinterpret_cast<const floatx4 *>(&nb.gamm[16 * rt + 4 * lg]);
      }
    }
    // chunk s+1's erase gates into LDS buffer PP (the producers build from it
    // in the next step), then chunk s+3's requested: in the second phase,
    // which the column waves finish before the producers (they activate the
    // write gates in the first)
    if constexpr (CBG) {
      stage_bg(std::integral_constant<int, PP>());
      load_bg(std::integral_constant<int, PP>(), s + 3 < nfull ? (s + 3) * C : Tl);
    }
    GDN2_MARK(5);
    __syncthreads();  // buffer (s+1)&1 may now be rebuilt by the producers
    GDN2_MARK(7);
  };
  load_u(std::integral_constant<int, 0>(), consumer && !ident && nfull > 0 ? 0 : Tl);
  if constexpr (CBG) {  // erase gates of chunks 0 and 1 requested, chunk 0's staged, chunk 2's requested
    load_bg(std::integral_constant<int, 1>(), nfull > 1 ? C : Tl);
    stage_bg(std::integral_constant<int, 0>());
    load_bg(std::integral_constant<int, 0>(), nfull > 2 ? 2 * C : Tl);
  }
  if constexpr (Cf::TOKM) __syncthreads();  // matches the producers' barrier before their loop
  for (int s = 0; s < nsteps; s += 2) {
    cstep(std::integral_constant<int, 0>(), s);
    cstep(std::integral_constant<int, 1>(), s + 1);
  }
  GDN2_TIMER_STORE

  if (consumer) {
    read_o();
    store_o();
    if (nfull * C < Tl) {
      token_steps(nfull * C, Tl);
      if (CST && cstp) store_cst(nfull + 1);
    }
    if (STp) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) STp[s_off + (size_t)(16 * rt + 4 * lg + j) * ld_s] = S[rt][j];
    }
  }
}

// A chunk size is usable when its double-buffered working set fits one CU's
// LDS and the K32 operand pairs a consumer wave prefetches for its second
// phase (solve and output blocks, transposed keys) fit its registers.
template <int DK, int C, int NCT, bool BF16>
constexpr bool chunk_fits() {
  using Cf = PrefillCfg<DK, C, NCT, BF16>;
  return prefill_smem_bytes<Cf>() <= 160 * 1024 && Cf::NCH * (Cf::NCH + 1) + Cf::NRT * Cf::NCH <= 24;
}

// Largest usable chunk <= the requested one.
template <int DK, int NCT, bool BF16>
constexpr int fitting_chunk(int requested) {
  return (requested >= 64 && chunk_fits<DK, 64, NCT, BF16>()) ? 64
         : (requested >= 32 && chunk_fits<DK, 32, NCT, BF16>()) ? 32
                                                                 : 16;
}

// Split plan. Sequences are cut into segments when an unsplit launch would
// occupy few workgroups (few sequences and heads) and the sequence is long:
// segments of at least 16 chunks, the largest power of two of them that
// keeps the first pass (value blocks of every segment, identity blocks of
// all but the first) within PrefillArgs::split_wgs workgroups (default: one
// per compute unit, i.e. one round). Every round of the first pass is as
// deep as its segments, so more segments than one round holds only add
// identity work and a longer combine and correction. GDN2_PREFILL_SPLIT=<n>
// forces n segments (1: never split).
template <int DK, int C, int NCT, bool BF16>
PrefillPlan plan_t(const PrefillArgs &a) {
  constexpr int DVB = 16 * NCT;
  PrefillPlan pl{C, 1, a.T, 0, false};
  const int ncb = a.d_v / DVB;
  const int nfull = a.T / C;
  if (a.cu_seqlens || DK % DVB != 0 || nfull < 2) return pl;
  long P = 1;
  if (a.force_nseg > 0) {
    P = a.force_nseg;
  } else if (const char *env = getenv("GDN2_PREFILL_SPLIT")) {
    P = atol(env);
  } else if ((long)a.B * a.H_v * ncb < 128) {
    const long val = (long)a.B * a.H_v * ncb, idb = (long)a.B * a.H_v * (DK / DVB);
    const long cap = a.split_wgs > 0 ? a.split_wgs : kNumCU;
    // the largest power of two with val P + idb (P - 1) <= cap (powers of two
    // give equal segments of the usual power-of-two lengths)
    while (val * (2 * P) + idb * (2 * P - 1) <= cap) P *= 2;
    P = P < nfull / 16 ? P : nfull / 16;
  }
  P = P < nfull ? P : nfull;
  if (P < 2) return pl;
  const int seg_chunks = (int)((nfull + P - 1) / P);
  const int seg_len = seg_chunks * C;
  const int nseg = (a.T + seg_len - 1) / seg_len;
  if (nseg < 2) return pl;
  pl.nseg = nseg;
  pl.seg_len = seg_len;
  // segment states and transitions; with the output correction also the
  // identity columns' outputs, one row of d_k per token and value head
  const size_t states = (size_t)nseg * a.B * a.H_v * DK * (size_t)(a.d_v + DK) * sizeof(float);
  const size_t corr = ((states + 255) & ~(size_t)255) + (size_t)a.B * a.T * a.H_v * DK * (BF16 ? 2 : 4);
  pl.correct = a.d_v == DK && (a.ws_cap == 0 || corr <= a.ws_cap);
  pl.ws_bytes = pl.correct ? corr : states;
  return pl;
}

// Unsplit: one launch over whole sequences. Split (nseg segments):
//  1. every segment from a zero entering state (the first from S0), value
//     blocks ending in state[s] and writing their outputs o_zero, identity
//     blocks (segments >= 1) ending in trans[s] and writing their query
//     reads oI to the workspace: the segment maps an entering state X to
//     trans[s] X + state[s], and its outputs to o_zero + X^T oI;
//  2. state[s] = trans[s] state[s - 1] + state[s] in order: the exact state
//     after each segment, the last one also into S_T;
//  3. o += oI . state[s - 1] on segments 1 .. nseg - 1 (launch_split_correct).
// When the workspace is capped below what oI needs, the first pass writes
// only the first segment's outputs, step 2 stops at segment nseg - 2, and
// segments 1 .. nseg - 1 run again from their exact entering states, the
// last one writing S_T. The chunk boundaries of every segment are those of
// the unsplit run.
template <int DK, int C, int NCT, bool BF16>
hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t st, PrefillPlan *plan_only) {
  auto kernel = [&](int blocks, const PrefillParams &kp) {
    if constexpr (DK == 128 && BF16) {
      if (kp.cst) {  // the chunk-form backward's states
        if (a.scalar_decay)
          hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16, true, true, false, true>), dim3(blocks), dim3(512), 0,
                             st, kp);
        else if (a.coupled)
          hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16, true, false, false, true>), dim3(blocks), dim3(512), 0,
                             st, kp);
        else if (a.preact)
          hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16, false, false, true, true>), dim3(blocks), dim3(512), 0,
                             st, kp);
        else
          hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16, false, false, false, true>), dim3(blocks), dim3(512), 0,
                             st, kp);
        return;
      }
    }
    if (a.scalar_decay)  // scalar decay comes with coupled gates (Gated DeltaNet)
      hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16, true, true, false>), dim3(blocks), dim3(512), 0, st, kp);
    else if (a.coupled)
      hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16, true, false, false>), dim3(blocks), dim3(512), 0, st, kp);
    else if (a.preact)
      hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16, false, false, true>), dim3(blocks), dim3(512), 0, st, kp);
    else
      hipLaunchKernelGGL((prefill_kernel<DK, C, NCT, BF16, false, false, false>), dim3(blocks), dim3(512), 0, st, kp);
  };
  const PrefillPlan pl = plan_t<DK, C, NCT, BF16>(a);
  if (plan_only) {
    *plan_only = pl;
    return hipSuccess;
  }
  constexpr int DVB = 16 * NCT;
  const int ncb = a.d_v / DVB;
  PrefillParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.a = a.a; p.b = a.b; p.w = a.w;
  p.B = a.B; p.T = a.T; p.H_qk = a.H_qk; p.H_v = a.H_v; p.d_v = a.d_v;
  p.o = a.o;
  p.seg_len = pl.seg_len;
  p.seg_first = 0;
  p.nseg = pl.nseg;
  p.ncb_val = ncb;
  p.ncb_id = 0;
  p.S0 = a.S0; p.s0_stride = 0;
  p.S_T = a.S_T; p.sT_stride = 0;
  p.M_T = nullptr; p.m_stride = 0;
  p.o_first_only = false;
  p.sT_last_only = false;
  p.cu = a.cu_seqlens;
  p.oI = nullptr;
  p.cst = nullptr;
  p.cst_segs = a.cst_segs > 1 ? a.cst_segs : 1;
  const int units = a.B * a.H_v;
  if (a.chunk_states && (pl.nseg > 1 || a.cu_seqlens || DK != 128 || !BF16 || a.B % p.cst_segs != 0))
    return hipErrorInvalidValue;
  if (pl.nseg <= 1) {
    p.cst = a.chunk_states;
    kernel(units * ncb, p);
    return hipGetLastError();
  }
  const size_t sstate = (size_t)units * DK * a.d_v, strans = (size_t)units * DK * DK;
  float *state, *trans;
  if (a.seg_states) {  // states only: the caller's state array, transitions in the workspace
    if (!a.workspace || a.workspace_bytes < (size_t)pl.nseg * strans * sizeof(float)) return hipErrorInvalidValue;
    state = a.seg_states;
    trans = static_cast<float *>(a.workspace);
    p.o = nullptr;
  } else {
    if (!a.workspace || a.workspace_bytes < pl.ws_bytes) return hipErrorInvalidValue;
    state = static_cast<float *>(a.workspace);
    trans = state + (size_t)pl.nseg * sstate;
  }
  const bool correct = pl.correct && !a.seg_states;
  void *oI = nullptr;
  if (correct) {
    const size_t states = (size_t)pl.nseg * (sstate + strans) * sizeof(float);
    oI = static_cast<char *>(a.workspace) + ((states + 255) & ~(size_t)255);
  }
  // 1.
  p.ncb_id = DK / DVB;
  p.S_T = state; p.sT_stride = sstate;
  p.M_T = trans; p.m_stride = strans;
  p.o_first_only = !correct;
  p.oI = oI;
  kernel(pl.nseg * units * (ncb + p.ncb_id), p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2.
  e = launch_split_combine(state, trans, correct ? pl.nseg - 1 : pl.nseg - 2, units, DK, a.d_v,
                           correct ? a.S_T : nullptr, st);
  if (e != hipSuccess || a.seg_states) return e;
  if (correct)  // 3.
    return launch_split_correct(a.o, oI, state, a.B, a.T, a.H_v, DK, a.d_v, pl.seg_len, pl.nseg, BF16, st);
  // 3.
  p.seg_first = 1;
  p.nseg = pl.nseg - 1;
  p.ncb_id = 0;
  p.S0 = state; p.s0_stride = sstate;
  p.S_T = a.S_T; p.sT_stride = 0; p.sT_last_only = true;
  p.M_T = nullptr; p.m_stride = 0;
  p.o_first_only = false;
  kernel(p.nseg * units * ncb, p);
  return hipGetLastError();
}

template <int DK, int NCT, bool BF16>
hipError_t dispatch_prefill_chunk(const PrefillArgs &a, hipStream_t st, PrefillPlan *plan_only) {
  switch (fitting_chunk<DK, NCT, BF16>(a.chunk)) {
    case 64:
      if constexpr (chunk_fits<DK, 64, NCT, BF16>())
        return launch_prefill_t<DK, 64, NCT, BF16>(a, st, plan_only);
      else
        return hipErrorInvalidValue;
    case 32:
      if constexpr (chunk_fits<DK, 32, NCT, BF16>())
        return launch_prefill_t<DK, 32, NCT, BF16>(a, st, plan_only);
      else
        return hipErrorInvalidValue;
    default:
      return launch_prefill_t<DK, 16, NCT, BF16>(a, st, plan_only);
  }
}

template <int DK, bool BF16>
hipError_t dispatch_prefill(const PrefillArgs &a, hipStream_t st, PrefillPlan *plan_only) {
  switch (a.nct) {
    case 1: return dispatch_prefill_chunk<DK, 1, BF16>(a, st, plan_only);
    case 2: return dispatch_prefill_chunk<DK, 2, BF16>(a, st, plan_only);
    case 4: return dispatch_prefill_chunk<DK, 4, BF16>(a, st, plan_only);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn2
