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

// E8M0 -> 2^(s-127) as f32, by ldexp (s = 0 gives the subnormal 2^-127); s =
// 255 is NaN in OCP MX, and a NaN scale makes its whole block NaN.  One
// select beside the ldexp: a form with a second select (for s = 0) slowed the
// MXFP4 decode loops by 12-16%.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __builtin_amdgcn_ldexpf(s == 255u ? __uint_as_float(0x7fc00000u) : 1.0f, (int)s - 127);
}

// 8 codes (4 bytes; element 2j in the low nibble of byte j) -> 8 bf16 values
// times the block scale.  Every product is a power-of-two multiple of an E2M1
// value (sign, two exponent bits with bias 1, one mantissa bit), exact in f32
// and in bf16.  gfx950 converts one byte (two codes) per instruction, scaling
// by an f32 factor; the MXFP4 parity cases, whose oracle decodes through the
// OCP table, pin the result (scales from 2^-40 to 2^20 included).
__device__ __forceinline__ u32x4_t decode_e2m1x8(uint32_t codes, float scale) {
  return u32x4_t{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3))};
}

// --------------------------------------------------------------------------
// Direct-to-LDS loads
// --------------------------------------------------------------------------

// 16 bytes per lane from global memory straight into LDS: the wavefront's 64
// lanes fill 1 KB at `l` (uniform across the wavefront), lane i at l + 16 i.
// Counted by the vector-memory counter like any other load.
__device__ __forceinline__ void dma16(const char *g, u32x4_t *l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)l, 16, 0, 0);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// workgroup barrier that the compiler does not move memory operations across
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace moe
