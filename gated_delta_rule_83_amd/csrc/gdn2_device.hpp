// gdn2_device.hpp -- device helpers for the libgdn2 kernels (gfx950 only).
//
// Element types, bf16 rounding, and the 16x16 MFMA tile primitive that every
// contraction of the prefill uses.
//
// MFMA tile conventions (CDNA 16x16 output tiles, wave of 64 lanes; lane l,
// g = l >> 4 in 0..3, c = l & 15):
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

namespace gdn2 {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest even; NaN stays NaN (quietened).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Storage type of q, k, v, o.
template <bool BF16> struct Elem;
template <> struct Elem<true> {
  typedef uint16_t T;
  static __device__ __forceinline__ float ld(const T *p) { return bf16_to_f32(*p); }
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
  static __device__ __forceinline__ void st(T *p, float x) { *p = x; }
  static __device__ __forceinline__ floatx2 ld2(const T *p) {
    return *reinterpret_cast<const floatx2 *>(p);
  }
  static __device__ __forceinline__ floatx4 ld4(const T *p) {
    return *reinterpret_cast<const floatx4 *>(p);
  }
};

// ---------------------------------------------------------------- MFMA operands
// Operand type held in LDS and fragments: bf16 bits for the bf16 path, fp32
// for the fp32 path (full-precision contractions).
template <bool BF16> struct Op;

template <> struct Op<true> {
  typedef uint16_t T;    // one element in LDS
  typedef shortx4 Frag;  // 4 consecutive k
  static __device__ __forceinline__ T cvt(float x) { return f32_to_bf16(x); }
  static __device__ __forceinline__ void st2(T *p, float x0, float x1) {
    *reinterpret_cast<uint32_t *>(p) = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
  }
  static __device__ __forceinline__ Frag ld_row(const T *p) {  // 4 consecutive elements
    return *reinterpret_cast<const Frag *>(p);
  }
  static __device__ __forceinline__ Frag ld_col(const T *p, int stride) {  // 4 strided elements
    return Frag{(short)p[0], (short)p[stride], (short)p[2 * stride], (short)p[3 * stride]};
  }
  static __device__ __forceinline__ Frag from_acc(floatx4 x) {
    return Frag{(short)f32_to_bf16(x[0]), (short)f32_to_bf16(x[1]), (short)f32_to_bf16(x[2]),
                (short)f32_to_bf16(x[3])};
  }
  static __device__ __forceinline__ Frag from_acc_neg(floatx4 x) {
    return Frag{(short)f32_to_bf16(-x[0]), (short)f32_to_bf16(-x[1]), (short)f32_to_bf16(-x[2]),
                (short)f32_to_bf16(-x[3])};
  }
  static __device__ __forceinline__ floatx4 mma(floatx4 acc, Frag a, Frag b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
  }
};

template <> struct Op<false> {
  typedef float T;
  typedef floatx4 Frag;
  static __device__ __forceinline__ T cvt(float x) { return x; }
  static __device__ __forceinline__ void st2(T *p, float x0, float x1) {
    *reinterpret_cast<floatx2 *>(p) = floatx2{x0, x1};
  }
  static __device__ __forceinline__ Frag ld_row(const T *p) {
    return *reinterpret_cast<const Frag *>(p);
  }
  static __device__ __forceinline__ Frag ld_col(const T *p, int stride) {
    return Frag{p[0], p[stride], p[2 * stride], p[3 * stride]};
  }
  static __device__ __forceinline__ Frag from_acc(floatx4 x) { return x; }
  static __device__ __forceinline__ Frag from_acc_neg(floatx4 x) { return -x; }
  static __device__ __forceinline__ floatx4 mma(floatx4 acc, Frag a, Frag b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
  }
};

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace gdn2
