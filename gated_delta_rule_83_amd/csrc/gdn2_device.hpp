// gdn2_device.hpp -- device helpers for the libgdn2 kernels (gfx950 only).
//
// Element types, bf16 rounding, and the 16x16 MFMA tile primitive that every
// contraction of the prefill uses.
//
// MFMA tile conventions (CDNA 16x16 output tiles, wave of 64 lanes; lane l,
// g = l >> 4 in 0..3, c = l & 15; K16 steps):
//   accumulator  floatx4 acc:  acc[j] = D[4*g + j][c]
//   A fragment (16 x K16):     lane holds A[c][k0 + 4*g + 0..3]
//   B fragment (K16 x 16):     lane holds B[k0 + 4*g + 0..3][c]
// so an accumulator tile, read as rows = k, is already a B fragment for the
// next product: no data movement is needed to chain products through the
// reduction dimension. For bf16 one K16 step is one
// v_mfma_f32_16x16x16_bf16; for fp32 it is four v_mfma_f32_16x16x4_f32, the
// j-th taking element j of both fragments (A and B pair up k = 4*g + j).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace gdn2 {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950); NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Storage type of q, k, v, o.
template <bool BF16> struct Elem;
template <> struct Elem<true> {
  typedef uint16_t T;
  static __device__ __forceinline__ float ld(const T *p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ float f(T x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ void st(T *p, float x) { *p = f32_to_bf16(x); }
  static __device__ __forceinline__ floatx2 ld2(const T *p) {
    uint32_t u = *reinterpret_cast<const uint32_t *>(p);
    return floatx2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
  }
  static __device__ __forceinline__ floatx4 ld4(const T *p) {
    uint2 u = *reinterpret_cast<const uint2 *>(p);
    return floatx4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
  }
};
template <> struct Elem<false> {
  typedef float T;
  static __device__ __forceinline__ float ld(const T *p) { return *p; }
  static __device__ __forceinline__ float f(T x) { return x; }
  static __device__ __forceinline__ void st(T *p, float x) { *p = x; }
  static __device__ __forceinline__ floatx2 ld2(const T *p) {
    return *reinterpret_cast<const floatx2 *>(p);
  }
  static __device__ __forceinline__ floatx4 ld4(const T *p) {
    return *reinterpret_cast<const floatx4 *>(p);
  }
};

// ---------------------------------------------------------------- MFMA operands
// Operand type held in LDS and fragments: bf16 for the bf16 path, fp32 for
// the fp32 path (full-precision contractions).
//
// K32 steps pair two 16-deep blocks: slot j of lane group g carries
// k = 4g + j (j < 4, first block) or 16 + 4g + (j - 4) (second block). The
// MFMA only requires A and B to agree on which k each slot holds, so two
// accumulator tiles (rows 0-15 and 16-31 of a K32 block) concatenate into a
// B operand with no data movement, and an A operand is two 4-element reads.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool BF16> struct Op;

template <> struct Op<true> {
  typedef __bf16 T;      // one element in LDS
  typedef bf16x4 Frag;   // 4 consecutive k of one row (A) or column (B)
  // Accumulation chains use one MFMA shape only (K32): chains that mixed
  // 16x16x32 and 16x16x16 steps on one accumulator gave wrong results in
  // the prefill; an odd leftover block is a K32 step with a zero half.
  static constexpr bool kK32Only = true;
  static __device__ __forceinline__ Frag zero() { return Frag{0, 0, 0, 0}; }
  static __device__ __forceinline__ void st2(T *p, float x0, float x1) {
    *reinterpret_cast<bf16x2 *>(p) = __builtin_convertvector(floatx2{x0, x1}, bf16x2);
  }
  static __device__ __forceinline__ Frag ld(const T *p) { return *reinterpret_cast<const Frag *>(p); }
  static __device__ __forceinline__ Frag from_acc(floatx4 x) {
    return __builtin_convertvector(x, bf16x4);
  }
  static __device__ __forceinline__ T cvt(float x) { return (T)x; }
  static __device__ __forceinline__ floatx4 mma16(floatx4 acc, Frag a, Frag b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a),
                                                     __builtin_bit_cast(shortx4, b), acc, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 mma32(floatx4 acc, Frag a0, Frag a1, Frag b0, Frag b1) {
    const bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
};

template <> struct Op<false> {
  typedef float T;
  typedef floatx4 Frag;
  static constexpr bool kK32Only = false;
  static __device__ __forceinline__ Frag zero() { return Frag{0.f, 0.f, 0.f, 0.f}; }
  static __device__ __forceinline__ void st2(T *p, float x0, float x1) {
    *reinterpret_cast<floatx2 *>(p) = floatx2{x0, x1};
  }
  static __device__ __forceinline__ Frag ld(const T *p) { return *reinterpret_cast<const Frag *>(p); }
  static __device__ __forceinline__ Frag from_acc(floatx4 x) { return x; }
  static __device__ __forceinline__ T cvt(float x) { return x; }
  static __device__ __forceinline__ floatx4 mma16(floatx4 acc, Frag a, Frag b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
  }
  static __device__ __forceinline__ floatx4 mma32(floatx4 acc, Frag a0, Frag a1, Frag b0, Frag b1) {
    return mma16(mma16(acc, a0, b0), a1, b1);
  }
};

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// K32 operand: the fragments of two consecutive K16 blocks.
template <bool BF16>
struct Pair {
  typename Op<BF16>::Frag lo, hi;
};

// ---------------------------------------------------------------- buffer access
// Raw buffer loads/stores: a wave-uniform base (the descriptor, in SGPRs), a
// per-lane 32-bit byte offset (VGPR) and a wave-uniform byte offset (SGPR).
// Keeping the uniform part of an address in SGPRs saves one 64-bit VALU
// address per access and keeps loop-invariant per-row offsets out of VGPRs.
// Accesses at or beyond `bytes` read 0 / are dropped by the hardware.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)(bytes > 0x7fffffffu ? 0x7fffffffu : bytes),
                                           0x00020000);
}
template <class V> __device__ __forceinline__ V bload(rsrc_t r, uint32_t voff, uint32_t soff);
template <> __device__ __forceinline__ float bload<float>(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
template <> __device__ __forceinline__ uint32_t bload<uint32_t>(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
template <> __device__ __forceinline__ uint16_t bload<uint16_t>(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
template <> __device__ __forceinline__ floatx2 bload<floatx2>(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(floatx2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
template <> __device__ __forceinline__ uint2 bload<uint2>(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
template <> __device__ __forceinline__ floatx4 bload<floatx4>(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ void bstore(uint16_t x, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b16(x, r, voff, soff, 0);
}
__device__ __forceinline__ void bstore(float x, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, voff, soff, 0);
}
__device__ __forceinline__ void bstore(uint2 x, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), x), r, voff, soff, 0);
}
__device__ __forceinline__ void bstore(floatx4 x, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), x), r, voff, soff, 0);
}

// ---------------------------------------------------------------- gate activations
// Decay from its pre-activation: exp(-softplus(x)) = 1 / (1 + e^x); erase and
// write gates: sigmoid(x) = 1 / (1 + e^-x). e^x as 2^(x log2 e) (v_exp_f32),
// then one reciprocal: relative error a few ulp; e^x overflowing to infinity
// gives 0, underflowing gives 1.
__device__ __forceinline__ float decay_from_pre(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * 1.44269504088896341f));
}
__device__ __forceinline__ float gate_from_pre(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}

// ---------------------------------------------------------------- lane shifts
// x from lane (l - D) of the same 16-lane row (DPP row_shr:D); lanes whose
// source is outside the row get `fill`. The empty asm keeps each component's
// shift a separate instruction: when shifts of the components of one vector
// were left to the optimizer, a single shifted component was reused for all
// of them (wrong results).
template <int D>
__device__ __forceinline__ float row_shr(float x, float fill) {
  static_assert(D >= 1 && D < 16, "row shift");
  asm volatile("" : "+v"(x));
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                               __builtin_bit_cast(int, x),
                                                               0x110 + D, 0xf, 0xf, false));
}

// x from lane S of this lane's group of 4 (DPP quad_perm [S,S,S,S]), as one
// asm statement: independent broadcasts issued together cannot be merged by
// the optimizer (see row_shr), and the asm costs no copy of x. The leading
// s_nop covers the wait a DPP read needs after a VALU write of its source,
// which the compiler does not see through the asm.
template <int S>
__device__ __forceinline__ float quad_bcast(float x) {
  static_assert(S >= 0 && S < 4, "quad lane");
  float y;
  asm volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 quad_perm:[%2,%2,%2,%2] row_mask:0xf bank_mask:0xf"
               : "=v"(y)
               : "v"(x), "i"(S));
  return y;
}

// Empty asm on every 32-bit part of x: the value counts as used and
// redefined here, so its computation cannot move past this point.
template <class V>
__device__ __forceinline__ void pin_regs(V &x) {
  static_assert(sizeof(V) % 4 == 0, "32-bit parts");
  uint32_t w[sizeof(V) / 4];
  __builtin_memcpy(w, &x, sizeof(V));
#pragma unroll
  for (unsigned i = 0; i < sizeof(V) / 4; ++i) asm volatile("" : "+v"(w[i]));
  __builtin_memcpy(&x, w, sizeof(V));
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace gdn2
