// Device-side building blocks shared by the gfx950 kernels of this library.
//
// Decode of an NVFP4 weight into bf16, exactly: w = E2M1(code) * E4M3(S). The product has at
// most 6 significant bits and lies in [2^-10, 2688], so it is exact in f32 and in bf16.
//  - v_cvt_scalef32_pk_f32_fp4 turns two E2M1 nibbles of a selected byte into two f32 values.
//    Its scale operand contributes only its exponent (a power of two), so it is called with
//    1.0 and the E4M3 scale is applied with an exact f32 multiply.
//  - v_cvt_f32_fp8 decodes the E4M3 scale byte (OCP "FN" format on gfx950).
//  - the two exact f32 products are packed into a bf16 pair by taking their high halves
//    (truncation is exact because the low 16 bits are zero).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssn {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// E4M3 byte (in the low byte of b) -> f32
__device__ __forceinline__ float e4m3_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8(b, 0); }

// byte `sel` (0..3) of word `w` as E4M3 -> f32
template <int SEL>
__device__ __forceinline__ float e4m3_f32_sel(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8(w, SEL); }

// Pack the high halves of two f32 values (exactly representable in bf16) into a bf16 pair.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Two E2M1 nibbles (byte SEL of w, low nibble first) times s -> packed bf16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_bf16(uint32_t w, float s) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return pack_hi16(v[0] * s, v[1] * s);
}

// Eight E2M1 nibbles (little-endian nibble order) times s -> 8 bf16 as a u32x4.
__device__ __forceinline__ u32x4 fp4x8_bf16(uint32_t w, float s) {
  u32x4 r;
  r[0] = fp4x2_bf16<0>(w, s);
  r[1] = fp4x2_bf16<1>(w, s);
  r[2] = fp4x2_bf16<2>(w, s);
  r[3] = fp4x2_bf16<3>(w, s);
  return r;
}

// Two E2M1 nibbles of byte SEL -> two f32 (unscaled)
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x16 as_bf16x16(u32x8 v) { return __builtin_bit_cast(bf16x16, v); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 -> bf16 bits, round to nearest even (inputs are finite), on the conversion instruction
// (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// two f32 -> a packed bf16 pair (lo in the low half), round to nearest even, one instruction
__device__ __forceinline__ uint32_t pk_bf16_rne(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }

}  // namespace ssn
