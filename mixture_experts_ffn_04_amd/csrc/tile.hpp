// Weight-streaming MFMA tile: one workgroup of kSplitWaves wavefronts computes
// a 16-column x (MT*16)-row output tile (times NS column sub-tiles) over the
// full reduction dimension.  Each wavefront takes every kSplitWaves-th block
// of the reduction; the partial sums meet in LDS and are added in wave order,
// so the result does not depend on timing.
//
// Operand roles: the weight rows (output columns) are MFMA operand A, the
// activation rows (tokens) operand B, so lane l receives output columns
// 4*(l/16)+q of token row (l % 16): four adjacent outputs of one row, which
// the epilogues store with one vector store.
//
// Reduction index layout inside a block of 128: lane group g = l/16 reads 32
// contiguous elements starting at 32*g and feeds them to 4 MFMAs (8 each).
// Weights and activations use the same layout, so each MFMA pairs matching
// elements.  A reduction length that is a multiple of 32 but not of 128 ends
// with single 32-element steps (lane group g reads 8 elements at 8*g).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kSplitWaves = 4;
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

// --------------------------------------------------------------------------
// Accumulation over this wavefront's share of the reduction dimension.
//   wrow[s]  : this lane's weight row of column sub-tile s (bf16)
//   arow[mt] : this lane's activation row of row tile mt (bf16)
//   acc[mt][s] += W_s . A_mt^T for mt < mt_count
// --------------------------------------------------------------------------
template <int MT, int NS>
__device__ __forceinline__ void accum_bf16(const uint16_t *const (&wrow)[NS],
                                           const uint16_t *const (&arow)[MT], int mt_count,
                                           int kdim, int wave, f32x4_t (&acc)[MT][NS]) {
  const int lg = (threadIdx.x & 63) >> 4;
  const int nblk = kdim / kKBlock;
  for (int b = wave; b < nblk; b += kSplitWaves) {
    const int k = b * kKBlock + 32 * lg;
    u32x4_t w[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[s][i] = load_stream16(wrow[s] + k + 8 * i);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
        u32x4_t av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = load16(arow[mt] + k + 8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s][i], av[i], acc[mt][s]);
      }
    }
  }
  const int ntail = (kdim % kKBlock) / 32;
  for (int t = wave; t < ntail; t += kSplitWaves) {
    const int k = nblk * kKBlock + 32 * t + 8 * lg;
    u32x4_t w[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) w[s] = load_stream16(wrow[s] + k);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
        const u32x4_t av = load16(arow[mt] + k);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s], av, acc[mt][s]);
      }
    }
  }
}

// Pipelined variant.  Reduction layout per 128-block: MFMA step i (0..3) uses
// elements [32i, 32i+32) of the block with the standard operand layout (lane
// group g holds elements 32i + 8g .. 32i + 8g + 7), so each load
// instruction reads 64 contiguous bytes of every row it touches.  The next
// block's weights (and, with PFA, activations) are loaded before the MFMAs of
// the current block, so HBM latency overlaps the matrix work.
template <int MT, int NS, bool PFA, int SW = kSplitWaves, bool LO = false>
__device__ __forceinline__ void accum_bf16_pf(const uint16_t *const (&wrow)[NS],
                                              const uint16_t *const (&arow)[MT], int mt_count,
                                              int kdim, int wave, f32x4_t (&acc)[MT][NS],
                                              int b0 = 0, int b1 = -1, bool tail = true,
                                              const uint16_t *const *arow_lo = nullptr) {
  const int lg = (threadIdx.x & 63) >> 4;
  const int nblk = kdim / kKBlock;
  if (b1 < 0) b1 = nblk;
  auto load_w = [&](u32x4_t (&w)[NS][4], int b) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) w[s][i] = load_stream16(wrow[s] + b * kKBlock + 32 * i + 8 * lg);
  };
  auto load_a = [&](u32x4_t (&a)[MT][4], int b) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mt_count)
#pragma unroll
        for (int i = 0; i < 4; ++i) a[mt][i] = load16(arow[mt] + b * kKBlock + 32 * i + 8 * lg);
  };
  auto mma = [&](const u32x4_t (&w)[NS][4], const u32x4_t (&a)[MT][4], int b) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mt_count)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s][i], a[mt][i], acc[mt][s]);
    if constexpr (LO) {  // the low halves of the activations, same weights
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < mt_count)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4_t al = load16(arow_lo[mt] + b * kKBlock + 32 * i + 8 * lg);
#pragma unroll
            for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s][i], al, acc[mt][s]);
          }
    }
  };
  int b = b0 + wave;
  if (b < b1) {
    u32x4_t w0[NS][4], a0[MT][4];
    load_w(w0, b);
    if constexpr (PFA) load_a(a0, b);
    while (true) {
      const int bn = b + SW;
      if (bn < b1) {
        u32x4_t w1[NS][4], a1[MT][4];
        load_w(w1, bn);
        if constexpr (PFA) {
          load_a(a1, bn);
        } else {
          load_a(a0, b);
        }
        mma(w0, a0, b);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) w0[s][i] = w1[s][i];
        if constexpr (PFA) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) a0[mt][i] = a1[mt][i];
        }
        b = bn;
      } else {
        if constexpr (!PFA) load_a(a0, b);
        mma(w0, a0, b);
        break;
      }
    }
  }
  const int ntail = tail ? (kdim % kKBlock) / 32 : 0;
  for (int t = wave; t < ntail; t += SW) {
    const int k = nblk * kKBlock + 32 * t + 8 * lg;
    u32x4_t w[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) w[s] = load_stream16(wrow[s] + k);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
        const u32x4_t av = load16(arow[mt] + k);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s], av, acc[mt][s]);
        if constexpr (LO) {
          const u32x4_t al = load16(arow_lo[mt] + k);
#pragma unroll
          for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s], al, acc[mt][s]);
        }
      }
    }
  }
}

// Same with MXFP4 weights: crow[s] = this lane's code row (bytes, two
// elements per byte), srow[s] = its E8M0 scale row (one byte per 32).
template <int MT, int NS>
__device__ __forceinline__ void accum_mxfp4(const uint8_t *const (&crow)[NS],
                                            const uint8_t *const (&srow)[NS],
                                            const uint16_t *const (&arow)[MT], int mt_count,
                                            int kdim, int wave, f32x4_t (&acc)[MT][NS]) {
  const int lg = (threadIdx.x & 63) >> 4;
  const int nblk = kdim / kKBlock;
  for (int b = wave; b < nblk; b += kSplitWaves) {
    const int k = b * kKBlock + 32 * lg;  // 32 elements: one scale block
    u32x4_t w[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4_t c = load_stream16(crow[s] + k / 2);
      const float sc = e8m0_to_f32(srow[s][k / 32]);
      w[s][0] = decode_e2m1x8(c.x, sc);
      w[s][1] = decode_e2m1x8(c.y, sc);
      w[s][2] = decode_e2m1x8(c.z, sc);
      w[s][3] = decode_e2m1x8(c.w, sc);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
        u32x4_t av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = load16(arow[mt] + k + 8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s][i], av[i], acc[mt][s]);
      }
    }
  }
  const int ntail = (kdim % kKBlock) / 32;
  for (int t = wave; t < ntail; t += kSplitWaves) {
    const int k = nblk * kKBlock + 32 * t + 8 * lg;
    u32x4_t w[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t c = *reinterpret_cast<const uint32_t *>(crow[s] + k / 2);
      w[s] = decode_e2m1x8(c, e8m0_to_f32(srow[s][k / 32]));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
        const u32x4_t av = load16(arow[mt] + k);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s], av, acc[mt][s]);
      }
    }
  }
}

// Pipelined MXFP4 variant with 256-element blocks.  Lane group g covers
// elements [64g, 64g+64) of a block: 32 contiguous code bytes and two E8M0
// scales per row; MFMA step i (0..7) takes elements 64g + 8i .. 64g + 8i + 7.
// Activations use the same layout (128 contiguous bytes per lane).  Codes and
// scales of the next block are loaded before the current block is decoded and
// multiplied.  A reduction length that is a multiple of 32 but not of 256 ends
// with 32-element steps as in accum_mxfp4.
constexpr int kKBlockMx = 256;

template <int MT, int NS, bool PFA, int SW = kSplitWaves, bool LO = false>
__device__ __forceinline__ void accum_mxfp4_pf(const uint8_t *const (&crow)[NS],
                                               const uint8_t *const (&srow)[NS],
                                               const uint16_t *const (&arow)[MT], int mt_count,
                                               int kdim, int wave, f32x4_t (&acc)[MT][NS],
                                               int b0 = 0, int b1 = -1, bool tail = true,
                                               const uint16_t *const *arow_lo = nullptr) {
  const int lg = (threadIdx.x & 63) >> 4;
  const int nblk = kdim / kKBlockMx;
  if (b1 < 0) b1 = nblk;
  struct Raw {
    u32x4_t c[NS][2];
    uint32_t s[NS];
  };
  auto load_w = [&](Raw &r, int b) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint8_t *cp = crow[s] + (b * kKBlockMx + 64 * lg) / 2;
      r.c[s][0] = load_stream16(cp);
      r.c[s][1] = load_stream16(cp + 16);
      const uint8_t *sp = srow[s] + (b * kKBlockMx + 64 * lg) / 32;  // rows may start at odd bytes
      r.s[s] = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
    }
  };
  auto load_a = [&](u32x4_t (&a)[MT][8], int b) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mt_count)
#pragma unroll
        for (int i = 0; i < 8; ++i) a[mt][i] = load16(arow[mt] + b * kKBlockMx + 64 * lg + 8 * i);
  };
  auto mma = [&](const Raw &r, const u32x4_t (&a)[MT][8], int b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4_t al[MT];
      if constexpr (LO) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (mt < mt_count) al[mt] = load16(arow_lo[mt] + b * kKBlockMx + 64 * lg + 8 * i);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4_t c = r.c[s][i >> 2];
        const uint32_t word = (i & 3) == 0 ? c.x : (i & 3) == 1 ? c.y : (i & 3) == 2 ? c.z : c.w;
        const u32x4_t w = decode_e2m1x8(word, e8m0_to_f32((r.s[s] >> (8 * (i >> 2))) & 0xffu));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (mt < mt_count) {
            acc[mt][s] = mfma_16x16x32(w, a[mt][i], acc[mt][s]);
            if constexpr (LO) acc[mt][s] = mfma_16x16x32(w, al[mt], acc[mt][s]);
          }
      }
    }
  };
  int b = b0 + wave;
  if (b < b1) {
    Raw r0;
    u32x4_t a0[MT][8];
    load_w(r0, b);
    if constexpr (PFA) load_a(a0, b);
    while (true) {
      const int bn = b + SW;
      if (bn < b1) {
        Raw r1;
        u32x4_t a1[MT][8];
        load_w(r1, bn);
        if constexpr (PFA) {
          load_a(a1, bn);
        } else {
          load_a(a0, b);
        }
        mma(r0, a0, b);
        r0 = r1;
        if constexpr (PFA) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 8; ++i) a0[mt][i] = a1[mt][i];
        }
        b = bn;
      } else {
        if constexpr (!PFA) load_a(a0, b);
        mma(r0, a0, b);
        break;
      }
    }
  }
  const int ntail = tail ? (kdim % kKBlockMx) / 32 : 0;
  for (int t = wave; t < ntail; t += SW) {
    const int k = nblk * kKBlockMx + 32 * t + 8 * lg;
    u32x4_t w[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t c = *reinterpret_cast<const uint32_t *>(crow[s] + k / 2);
      w[s] = decode_e2m1x8(c, e8m0_to_f32(srow[s][k / 32]));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
        const u32x4_t av = load16(arow[mt] + k);
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s], av, acc[mt][s]);
        if constexpr (LO) {
          const u32x4_t al = load16(arow_lo[mt] + k);
#pragma unroll
          for (int s = 0; s < NS; ++s) acc[mt][s] = mfma_16x16x32(w[s], al, acc[mt][s]);
        }
      }
    }
  }
}

// Split-reduction merge: every wave stores its partial tile to LDS, then wave
// w adds, in wave order, the partials of the row tiles mt with mt % kSplitWaves
// == w.  After the call acc[mt] of those tiles holds the full sums.
// `red` must hold kSplitWaves * MT * NS * 64 f32x4 values.
template <int MT, int NS, int SW = kSplitWaves>
__device__ __forceinline__ void splitk_merge(f32x4_t (&acc)[MT][NS], f32x4_t *red, int mt_count,
                                             int wave) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (mt < mt_count) red[((wave * MT + mt) * NS + s) * 64 + lane] = acc[mt][s];
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < mt_count && (mt % SW) == wave) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        f32x4_t sum = red[((0 * MT + mt) * NS + s) * 64 + lane];
#pragma unroll
        for (int w = 1; w < SW; ++w) sum += red[((w * MT + mt) * NS + s) * 64 + lane];
        acc[mt][s] = sum;
      }
    }
  }
}

}  // namespace moe
