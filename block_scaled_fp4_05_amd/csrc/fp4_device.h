// Device-side helpers for NVFP4 on gfx950 (CDNA4).
//
// Element format E2M1 (OCP MX v1.0), block scale E4M3 (OCP OFP8 v1.0), one
// scale per 16 elements along K, two elements per byte with element 2i in the
// low nibble ("Peering into the CUTLASS SharedStorage", section "Input
// Knowledge", item 3, for the packing and the 16-element FP8 block).
//
// Dequantisation is exact in FP16: an E2M1 value times an E4M3 value has at
// most 6 significant bits and lies in [2^-10, 2688], inside FP16's normal
// range, so the products fed to the FP16 MFMA equal the real values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_fp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Two E4M3 scale bytes (bits 0-7 and 8-15 of `d`, or 16-31 when HI) as a pair
// of FP16 values, each equal to the E4M3 value times 2^-8.  Placing the byte's
// exponent and mantissa at FP16 bit 7 maps E4M3 exponent e to FP16 exponent
// e (bias 15 vs 7: a factor 2^-8) and E4M3 subnormals onto FP16 subnormals,
// so the map is exact for every finite code; the sign bit moves to bit 15.
template <bool HI>
__device__ __forceinline__ half2_t scale_pair_x2m8(uint32_t d) {
  uint32_t x = HI ? (d >> 16) : d;
  uint32_t lo = ((x & 0x7Fu) << 7) | ((x & 0x80u) << 8);
  uint32_t hi = ((x & 0x7F00u) << 15) | ((x & 0x8000u) << 16);
  return __builtin_bit_cast(half2_t, lo | hi);
}

// Eight packed E2M1 codes (one dword, element 0 in the low nibble) times one
// block scale, as eight exact FP16 values.  The hardware conversion applies
// only the exponent of its FP32 scale operand, so it is given 2^8 and the
// scale itself (carried as value * 2^-8) is applied with a packed multiply.
__device__ __forceinline__ half8_t dequant8(uint32_t codes, _Float16 scale_x2m8) {
  const half2_t s2 = {scale_x2m8, scale_x2m8};
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * s2;
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * s2;
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * s2;
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * s2;
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ u32x4_t load_16B(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ uint32_t load_4B(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

}  // namespace moe_fp4
