// MFMA helpers shared by the router and expert kernels: the 128-element
// reduction block of the router's logit tiles and the MXFP4 element decoding
// (OCP MX: E2M1 element, E8M0 scale of 32 elements).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kSplitWaves = 4;                     // wavefronts splitting a reduction
constexpr int kBlockThreads = kSplitWaves * kWave;
constexpr int kKBlock = 128;

// --------------------------------------------------------------------------
// MXFP4 decoding (OCP MX: E2M1 element, E8M0 scale of 32 elements)
// --------------------------------------------------------------------------

// E2M1 code -> f32: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3f000000u : 0u);
  return __uint_as_float(mag | ((c & 8u) << 28));
}

// E8M0 -> 2^(s-127) as f32 (s = 0 is the subnormal 2^-127; 255 is not used).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// 8 codes (4 bytes; element 2j in the low nibble of byte j) -> 8 bf16 values
// times the block scale.  Every product is a power-of-two multiple of an E2M1
// value, exact in f32 and in bf16.  gfx950 converts one byte (two codes) per
// instruction, scaling by an f32 factor; the result is the exact product
// (checked bit for bit against the arithmetic decode e2m1_to_f32 * scale).
__device__ __forceinline__ u32x4_t decode_e2m1x8(uint32_t codes, float scale) {
  return u32x4_t{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3))};
}

// The same decode by arithmetic (reference for the instruction above).
__device__ __forceinline__ u32x4_t decode_e2m1x8_arith(uint32_t codes, float scale) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t byte = (codes >> (8 * j)) & 0xffu;
    const float lo = e2m1_to_f32(byte & 15u) * scale;
    const float hi = e2m1_to_f32(byte >> 4) * scale;
    o[j] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  return u32x4_t{o[0], o[1], o[2], o[3]};
}

}  // namespace moe
