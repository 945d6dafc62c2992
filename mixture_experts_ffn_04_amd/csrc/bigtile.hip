// Large-tile grouped expert GEMMs for experts that hold hundreds of rows
// (matrix-core bound: every weight element meets >= 256 token rows).
//
// Same operations as the streaming and tiled kernels (gate_up + SwiGLU,
// down + optional per-expert bias; bf16 or MXFP4 weights, bf16
// activations).  A workgroup of four wavefronts computes a 256-token x
// 256-weight-row tile; each wavefront a 128 x 128 sub-tile with 32x32x16 bf16
// MFMAs (weights as operand A, tokens as operand B: lane l holds output
// columns 8j + 4(l/32) + q, q < 4, of token l % 32 for j < 4).  Per
// workgroup and 16-deep reduction step the wavefronts read 32 KB of operands
// from LDS for 2 M multiply-adds, half the LDS traffic per MFMA of a
// 128 x 64 sub-tile.
//
// Reduction slices of 64 (32 with the low halves of h) are staged in LDS,
// double-buffered: the next slice's global loads are in flight while the
// current one is multiplied.  Rows of the LDS tiles are 16-byte chunks with
// an XOR swizzle, so the 16 lanes of an operand read (16 rows, one chunk)
// and of a store (two rows, eight chunks) touch 64 different banks.  This
// register-staged form serves MXFP4 weights when the direct-to-LDS form below
// does not apply (codes decoded to bf16 on their way into LDS).
//
// gate_up tiles hold 128 gate rows and the matching 128 up rows; wavefront
// column half wn takes gate rows 64 wn .. 64 wn + 63 and the same up rows, so
// a SwiGLU pair meets in one lane.
//
// [SF1073] SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own DSpark draft
// (stacked on #1035)": clamped SwiGLU; stacked gate_up_proj; FP4 experts two
// codes per byte (low nibble first), one E8M0 scale per 32 inputs.  [MI143]
// MoE-Infinity PR #143 "feat(dflash): converge DFlash spec-decode stack ->
// dev (supersedes #140)": output-major MXFP4 blocks, per-expert biases.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"
#include "tile.hpp"

namespace moe {

namespace {

constexpr int BM = 256;  // tokens per tile
constexpr int BN = 256;  // weight rows per tile
constexpr int kThreads = 256;


// 16-byte unit of (row, chunk) in a tile with CH chunks per row.  Rows
// that share a 256-byte bank window get different chunk permutations.
template <int CH>
__device__ __forceinline__ int unit(int row, int ch) {
  return row * CH + (ch ^ ((row / (16 / CH)) % CH));
}

struct BigCoord {
  int g, nrows, row0, m0, n0;
};

// tile -> (group, first token row, column tile).  Tiles of one expert run
// row tile fastest, so the workgroups sharing a weight tile are adjacent.
__device__ __forceinline__ void big_coord(const TiledGemmArgs &t, int tile, int n_tiles, BigCoord &c,
                                          int tm = BM) {
  const ExpertGemmArgs &a = t.g;
  if (!a.counts) {
    const int mt = (a.single_rows + tm - 1) / tm;
    c.g = 0;
    c.nrows = a.single_rows;
    c.row0 = 0;
    c.m0 = (tile % mt) * tm;
    c.n0 = tile / mt;
    return;
  }
  const int q = tile / n_tiles;  // global row-tile index over all experts
  int lo = 0, hi = t.n_active_all[0];
  while (hi - lo > 1) {  // mtile_prefix[lo] <= q < mtile_prefix[lo + 1]
    const int mid = (lo + hi) >> 1;
    if (t.mtile_prefix[mid] <= q) lo = mid;
    else hi = mid;
  }
  const int mt_e = t.mtile_prefix[lo + 1] - t.mtile_prefix[lo];
  const int local = tile - t.mtile_prefix[lo] * n_tiles;
  c.g = t.active_all[lo];
  c.nrows = a.counts[c.g];
  c.row0 = a.offsets[c.g];
  c.m0 = (local % mt_e) * tm;
  c.n0 = local / mt_e;
}

template <bool LO>
struct BigPlan {
  static constexpr int BK = LO ? 32 : 64;         // reduction slice
  static constexpr int CH = BK / 8;               // 16-byte chunks per row
  static constexpr int WU = BN * CH;              // units of the weight tile
  static constexpr int XU = BM * CH;              // units of one activation tile
  static constexpr int BUF = WU + XU * (LO ? 2 : 1);
  static constexpr size_t LDS_BYTES = (size_t)2 * BUF * 16;
};

}  // namespace

// Epilogue of a gate_up tile.  The matching gate and up columns of a lane
// sit in fragments nf and nf + 2 at the same register index, so SwiGLU runs
// on the accumulators directly.  The packed bf16 h (hi, and lo when out_lo
// is set) then passes once through LDS, where each wave turns its pieces of
// 4 columns x 32 tokens into 16-byte row runs for the global stores.  Staged
// token rows are 64 bf16 plus 16 bytes, so a half-wave's 8-byte writes (16
// tokens, one column group) spread over 16 different 16-byte bank groups.
constexpr int kEpiPitch = 144;  // bytes per staged token row
template <int MF>
constexpr size_t epi_gate_up_bytes() {
  return (size_t)4 * 2 * MF * 32 * kEpiPitch;
}

template <int MF>
__device__ __forceinline__ void big_epilogue_gate_up(const ExpertGemmArgs &a, const BigCoord &c, int col0,
                                                     f32x16_t (&acc)[MF][4], char *lds) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int wcol0 = col0 + wn * 64;  // first h column of the wave
  char *hi_s = lds + (size_t)wave * 2 * MF * 32 * kEpiPitch;
  char *lo_s = hi_s + MF * 32 * kEpiPitch;
  const bool want_lo = a.out_lo != nullptr;
  const uint16_t *bp = a.bias ? static_cast<const uint16_t *>(a.bias) + (size_t)c.g * a.bias_stride : nullptr;
  // lane: token l32 of each fragment, columns 32 p + 8 j + 4 lh + q
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cl = 32 * p + 8 * j + 4 * lh;  // column within the wave's 64
        float gb[4] = {0.f, 0.f, 0.f, 0.f}, ub[4] = {0.f, 0.f, 0.f, 0.f};
        if (bp && wcol0 + cl < a.N) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gb[q] = bf16_to_f32(bp[wcol0 + cl + q]);
            ub[q] = bf16_to_f32(bp[a.N + wcol0 + cl + q]);
          }
        }
        float h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          h[q] = swiglu_fast(acc[mf][p][4 * j + q] + gb[q], acc[mf][p + 2][4 * j + q] + ub[q], a.limit, a.act);
        const uint32_t h01 = pack_bf16x2(h[0], h[1]), h23 = pack_bf16x2(h[2], h[3]);
        const int off = (mf * 32 + l32) * kEpiPitch + cl * 2;
        *reinterpret_cast<uint2 *>(hi_s + off) = make_uint2(h01, h23);
        if (want_lo)  // h = hi + lo to ~16 bits (h - hi is exact in f32)
          *reinterpret_cast<uint2 *>(lo_s + off) =
              make_uint2(pack_bf16x2(h[0] - bf16_lo(h01), h[1] - bf16_hi(h01)),
                         pack_bf16x2(h[2] - bf16_lo(h23), h[3] - bf16_hi(h23)));
      }
    }
  }
  // a wave reads back only what it wrote (LDS operations of a wave complete
  // in order): 8 lanes per token row, 16 bytes (8 columns) each
  const int ch = lane & 7;
  const bool cok = wcol0 + 8 * ch < a.N;  // N is a multiple of 32
  const int trow0 = c.m0 + wm * (MF * 32);
#pragma unroll 2
  for (int i = 0; i < MF * 4; ++i) {
    const int r = i * 8 + (lane >> 3);
    const u32x4_t vh = *reinterpret_cast<const u32x4_t *>(hi_s + r * kEpiPitch + ch * 16);
    u32x4_t vl = {0u, 0u, 0u, 0u};
    if (want_lo) vl = *reinterpret_cast<const u32x4_t *>(lo_s + r * kEpiPitch + ch * 16);
    const int row = trow0 + r;
    if (cok && row < c.nrows) {
      const size_t off = (size_t)(c.row0 + row) * a.N + wcol0 + 8 * ch;
      *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(a.out) + off) = vh;
      if (want_lo) *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(a.out_lo) + off) = vl;
    }
  }
}

// Epilogue of a down tile through LDS (the stage buffers must be free: at
// least 4 x 32 x 132 floats).  The wave's sub-tile is MF fragment rows of 32
// tokens x 128 columns.  Each wave writes one fragment row of its sub-tile
// to its own padded region, then reads it back one token row at a time, so
// its stores cover contiguous column runs of one row: (+ bias) -> y f32, or
// out[token] = weight * y with direct_out.
template <int MF>
__device__ __forceinline__ void big_epilogue_down(const ExpertGemmArgs &a, const BigCoord &c, int col0,
                                                  f32x16_t (&acc)[MF][4], float *lds) {
  constexpr int EP = 128 + 4;  // padded row (floats): the 16 rows of a float4 write hit distinct banks
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  float *Ew = lds + wave * 32 * EP;
  const int ccol0 = col0 + wn * 128;  // first output column of the wave
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4 *>(Ew + l32 * EP + nf * 32 + 8 * j + 4 * lh) =
            make_float4(acc[mf][nf][4 * j], acc[mf][nf][4 * j + 1], acc[mf][nf][4 * j + 2], acc[mf][nf][4 * j + 3]);
    const int rbase = c.m0 + wm * MF * 32 + mf * 32;  // token row (in the group) of fragment row 0
    // every lane owns output columns 2 lane, 2 lane + 1 of each row
    const int col = ccol0 + 2 * lane;
    const bool cok = col < a.N;
    float b0 = 0.f, b1 = 0.f;
    if (a.bias && cok) {
      const uint16_t *bp = static_cast<const uint16_t *>(a.bias) + (size_t)c.g * a.bias_stride;
      b0 = bf16_to_f32(bp[col]);
      b1 = bf16_to_f32(bp[col + 1]);
    }
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      const int row = rbase + r;
      if (!cok || row >= c.nrows) continue;
      const float2 v = *reinterpret_cast<const float2 *>(Ew + r * EP + 2 * lane);
      const float y0 = v.x + b0, y1 = v.y + b1;
      if (a.direct_out) {  // one expert per token: out = weight * y
        const int slot = a.perm[c.row0 + row];
        const float wt = a.weights[slot];
        *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(a.direct_out) + (size_t)slot * a.N + col) =
            pack_bf16x2(wt * y0, wt * y1);
      } else {
        *reinterpret_cast<float2 *>(static_cast<float *>(a.out) + (size_t)(c.row0 + row) * a.N + col) =
            make_float2(y0, y1);
      }
    }
  }
}

template <bool GATE_UP, int MF = 4>
__device__ __forceinline__ void big_epilogue(const ExpertGemmArgs &a, const BigCoord &c, int col0,
                                             f32x16_t (&acc)[MF][4], void *lds) {
  if constexpr (GATE_UP) big_epilogue_gate_up<MF>(a, c, col0, acc, static_cast<char *>(lds));
  else big_epilogue_down<MF>(a, c, col0, acc, static_cast<float *>(lds));
}

template <bool GATE_UP, int WF, bool GATHER, bool LO>
__global__ __launch_bounds__(kThreads, 1) void expert_bigtile(TiledGemmArgs ta) {
  using P = BigPlan<LO>;
  constexpr int BK = P::BK, CH = P::CH, WU = P::WU, XU = P::XU, BUF = P::BUF;
  constexpr int XL = XU / kThreads;                        // activation loads per thread per tile
  constexpr int WL = WF == W_MXFP4 ? BN * (BK / 32) / kThreads : WU / kThreads;  // weight loads
  const ExpertGemmArgs &a = ta.g;
  extern __shared__ u32x4_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int l32 = lane & 31, lh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;

  const int cols_per_tile = GATE_UP ? BN / 2 : BN;
  const int n_tiles = (a.N + cols_per_tile - 1) / cols_per_tile;
  const int total = a.counts ? ta.mtile_prefix[ta.n_active_all[0]] * n_tiles
                             : ((a.single_rows + BM - 1) / BM) * n_tiles;
  const uint16_t *A = static_cast<const uint16_t *>(a.A);
  const int nks = (a.Kdim + BK - 1) / BK;

  // XCD-contiguous ranges of the tile list (workgroups go to the 8 XCDs
  // round-robin), so the workgroups of one XCD share weight and token tiles
  // through its L2.
  const int nx = gridDim.x % 8 == 0 ? 8 : 1;
  const int xcd = blockIdx.x % nx, per = gridDim.x / nx;
  const int span = (total + nx - 1) / nx;
  for (int local = blockIdx.x / nx; local < span; local += per) {
    const int tile = xcd * span + local;
    if (tile >= total) break;
    BigCoord c;
    big_coord(ta, tile, n_tiles, c);
    const int col0 = c.n0 * cols_per_tile;

    // ---- global sources of this thread's loads -----------------------------
    // 32-bit byte offsets from workgroup-uniform bases (the launcher checks
    // that activations and one expert's weights span less than 4 GiB).
    // activation unit j*256 + tid -> tile row (j*256 + tid) / CH, chunk tid % CH
    const int xc = tid % CH;
    const char *xbase = static_cast<const char *>(a.A);
    const char *xlbase = static_cast<const char *>(a.A_lo);
    uint32_t xo[XL], xlo[LO ? XL : 1];
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      const int r = min(c.m0 + (j * kThreads + tid) / CH, c.nrows - 1);
      uint32_t ar;
      if constexpr (GATHER)
        ar = (uint32_t)(a.perm[c.row0 + r] / a.topk);
      else
        ar = (uint32_t)(c.row0 + r);
      xo[j] = (ar * (uint32_t)a.Kdim + xc * 8) * 2u;
      if constexpr (LO) xlo[j] = ((uint32_t)(c.row0 + r) * (uint32_t)a.Kdim + xc * 8) * 2u;
    }
    // weight tile row -> weight row of the expert (clamped into the matrix)
    auto wrow = [&](int r) {
      int g, lim;
      if constexpr (GATE_UP) {
        g = r < BN / 2 ? col0 + r : a.N + col0 + (r - BN / 2);
        lim = r < BN / 2 ? a.N - 1 : 2 * a.N - 1;
      } else {
        g = col0 + r;
        lim = a.N - 1;
      }
      return (uint32_t)min(g, lim);
    };
    // bf16: unit j*256 + tid -> row (j*256 + tid) / CH, chunk tid % CH
    // MXFP4: one 32-element block (16 code bytes + a scale) per load:
    //        load j*256 + tid -> row (j*256 + tid) / (BK/32), block tid % (BK/32)
    const char *wbase = static_cast<const char *>(a.W) + (size_t)c.g * a.w_stride * (WF == W_MXFP4 ? 1 : 2);
    const uint8_t *sbase = WF == W_MXFP4 ? a.Wscale + (size_t)c.g * a.s_stride : nullptr;
    uint32_t wo[WL], so[WF == W_MXFP4 ? WL : 1];
    const int wb = tid % (BK / 32);
#pragma unroll
    for (int j = 0; j < WL; ++j) {
      if constexpr (WF == W_MXFP4) {
        const uint32_t gr = wrow((j * kThreads + tid) / (BK / 32));
        wo[j] = gr * (uint32_t)(a.Kdim / 2) + wb * 16;
        so[j] = gr * (uint32_t)(a.Kdim / 32) + wb;
      } else {
        wo[j] = (wrow((j * kThreads + tid) / CH) * (uint32_t)a.Kdim + xc * 8) * 2u;
      }
    }

    u32x4_t xv[XL], xlv[LO ? XL : 1], wv[WL];
    uint32_t sv[WF == W_MXFP4 ? WL : 1];
    auto gload = [&](int ks) {
      const int k0 = ks * BK;
      const bool xin = k0 + xc * 8 < a.Kdim;
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        xv[j] = xin ? load16(xbase + xo[j] + k0 * 2) : u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (LO) xlv[j] = xin ? load16(xlbase + xlo[j] + k0 * 2) : u32x4_t{0u, 0u, 0u, 0u};
      }
      if constexpr (WF == W_MXFP4) {
        const bool win = k0 + wb * 32 < a.Kdim;
#pragma unroll
        for (int j = 0; j < WL; ++j) {
          wv[j] = win ? load16(wbase + wo[j] + k0 / 2) : u32x4_t{0u, 0u, 0u, 0u};
          sv[j] = win ? sbase[so[j] + k0 / 32] : 127u;
        }
      } else {
#pragma unroll
        for (int j = 0; j < WL; ++j) wv[j] = xin ? load16(wbase + wo[j] + k0 * 2) : u32x4_t{0u, 0u, 0u, 0u};
      }
    };
    auto lstore = [&](int buf) {
      u32x4_t *Wt = smem + buf * BUF, *Xt = Wt + WU;
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        const int r = (j * kThreads + tid) / CH;
        Xt[unit<CH>(r, xc)] = xv[j];
        if constexpr (LO) Xt[XU + unit<CH>(r, xc)] = xlv[j];
      }
      if constexpr (WF == W_MXFP4) {
#pragma unroll
        for (int j = 0; j < WL; ++j) {
          const int r = (j * kThreads + tid) / (BK / 32);
          const float sc = e8m0_to_f32(sv[j]);
          Wt[unit<CH>(r, 4 * wb + 0)] = decode_e2m1x8(wv[j].x, sc);
          Wt[unit<CH>(r, 4 * wb + 1)] = decode_e2m1x8(wv[j].y, sc);
          Wt[unit<CH>(r, 4 * wb + 2)] = decode_e2m1x8(wv[j].z, sc);
          Wt[unit<CH>(r, 4 * wb + 3)] = decode_e2m1x8(wv[j].w, sc);
        }
      } else {
#pragma unroll
        for (int j = 0; j < WL; ++j) Wt[unit<CH>((j * kThreads + tid) / CH, xc)] = wv[j];
      }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mf][nf][i] = 0.f;

    // LDS weight row of fragment nf of this wavefront
    auto wfrag = [&](int nf) {
      if constexpr (GATE_UP) return nf < 2 ? wn * 64 + nf * 32 : BN / 2 + wn * 64 + (nf - 2) * 32;
      else return wn * 128 + nf * 32;
    };
    // 32-row token fragments of this wave that hold rows of the group (the
    // others are skipped: a group's last row tile is often nearly empty)
    const int mf_count = min(4, max(0, (c.nrows - c.m0 - wm * 128 + 31) / 32));
    // Operand fragments of reduction step kk + 1 are read from LDS while the
    // MFMAs of step kk run (two register sets).
    // `full` (a std::bool_constant): every fragment holds rows, no guards (a
    // guard per MFMA group becomes an exec-mask branch that stalls the
    // matrix pipe, so full tiles, the common case, take an unguarded copy)
    auto compute = [&](int buf, auto full) {
      constexpr bool FULL = decltype(full)::value;
      const u32x4_t *Wt = smem + buf * BUF, *Xt = Wt + WU;
      constexpr int KS = BK / 16;
      constexpr int NB = LO ? 8 : 4;  // token fragments per step (hi, then lo)
      u32x4_t af[2][4], bf[2][NB];
      auto fetch = [&](int set, int kk) {
        const int ch = 2 * kk + lh;
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) af[set][nf] = Wt[unit<CH>(wfrag(nf) + l32, ch)];
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
          if (FULL || mf < mf_count) {
            bf[set][mf] = Xt[unit<CH>(wm * 128 + mf * 32 + l32, ch)];
            if constexpr (LO) bf[set][4 + mf] = Xt[XU + unit<CH>(wm * 128 + mf * 32 + l32, ch)];
          }
        }
      };
      fetch(0, 0);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < KS) fetch(cur ^ 1, kk + 1);
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
          if (FULL || mf < mf_count) {
#pragma unroll
            for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma_32x32x16(af[cur][nf], bf[cur][mf], acc[mf][nf]);
            if constexpr (LO) {  // the same weight fragments times the low halves of h
#pragma unroll
              for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma_32x32x16(af[cur][nf], bf[cur][4 + mf], acc[mf][nf]);
            }
          }
        }
      }
    };

    auto run = [&](auto full) {
      gload(0);
      lstore(0);
      __syncthreads();
      for (int ks = 0; ks < nks; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nks) gload(ks + 1);
        compute(buf, full);
        if (ks + 1 < nks) lstore(buf ^ 1);
        __syncthreads();
      }
    };
    if (c.nrows - c.m0 >= BM) run(std::true_type{});
    else run(std::false_type{});

    big_epilogue<GATE_UP>(a, c, col0, acc, smem);
    __syncthreads();  // the next tile's first slice overwrites buffer 0
  }
}

// ---------------------------------------------------------------------------
// The same tile fed by direct-to-LDS loads (bf16 weights, and the MXFP4
// gate_up whose scale array starts on 16 bytes and whose reduction is at most
// 5120 deep).  Each load
// instruction of a wavefront writes 64 x 16 bytes to consecutive LDS
// addresses without passing through registers, so the workgroup keeps up to
// four 32-deep stages in flight beyond the one being multiplied (a ring of
// five; of three with the low halves of h) instead of one register-staged
// slice.  A lane chooses which global chunk it
// fetches so that the data lands at its swizzled LDS position.  The compiler
// does not track these loads: the waits on the vector-memory counter and the
// barriers are explicit.
// ---------------------------------------------------------------------------
namespace {

// MXFP4 weights: a stage holds each weight row's 16 code bytes (32 codes) in
// one unit; the block scales of the tile's 256 weight rows over the whole
// reduction sit in a table after the ring, loaded once per tile (the gate and
// up rows' scales are two contiguous runs of 128 * K/32 bytes); fragments are
// decoded to bf16 when read from LDS.
template <bool LO, int TM, int WF = W_BF16>
struct DmaPlan {
  static constexpr bool MX = WF == W_MXFP4;
  static constexpr int BK = 32, CH = 4;
  static constexpr int WUN = MX ? BN : BN * CH;             // 16-byte units of the weight part
  static constexpr int XUN = TM * CH;                       // 16-byte units of one activation tile
  static constexpr int XI = XUN / 256;                      // activation load instructions per wave
  static constexpr int NXS = LO ? 2 : 1;
  static constexpr int SLOT = WUN + NXS * XUN;
  static constexpr int NSTAGE = std::min(6, (160 * 1024) / (SLOT * 16));
  static constexpr int OPS = (MX ? 1 : 4) + XI * NXS;       // load instructions per wave and stage
  static constexpr size_t LDS_BYTES = (size_t)NSTAGE * SLOT * 16;
  // MXFP4 scale table: 256 rows x K/32 bytes = K/2 units, in whole 64-unit
  // load instructions, after the ring
  static constexpr int MAX_K = 5120;
  static __host__ __device__ constexpr int table_units(int K) { return (K / 2 + 63) & ~63; }
  static_assert(NSTAGE >= 3 && LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(NSTAGE * SLOT * 16 >= 4 * 32 * 132 * 4, "epilogue staging fits the ring");
  static_assert((NSTAGE - 1) * OPS < 64, "vmcnt range");
};

// Scheduling order of a region with NREAD LDS reads (next step's operands)
// and NMFMA MFMAs (this step's): an MFMA, then two reads, until every read is
// issued, then the remaining MFMAs.  The reads go out early, behind a
// single MFMA each, so their latency is covered by the rest of the step.
template <int NREAD, int NMFMA, int I = 0>
__device__ __forceinline__ void interleave_reads() {
  if constexpr (I < NREAD) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD - I >= 2 ? 2 : 1, 0);  // up to two LDS reads
    interleave_reads<NREAD, NMFMA - 1, I + 2>();
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);                   // the other MFMAs
  }
}

// The same with VALU work between the later MFMAs (the MXFP4 decode of the
// next step's weight fragments): after the reads, each MFMA is followed by
// an even share of NVALU vector instructions.
template <int NREAD, int NMFMA, int NVALU, int I = 0>
__device__ __forceinline__ void interleave_reads_valu() {
  if constexpr (I < NREAD) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD - I >= 2 ? 2 : 1, 0);  // up to two LDS reads
    interleave_reads_valu<NREAD, NMFMA - 1, NVALU, I + 2>();
  } else if constexpr (NMFMA > 0) {
    constexpr int V = (NVALU + NMFMA - 1) / NMFMA;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);                       // its share of VALU work
    interleave_reads_valu<NREAD, NMFMA - 1, NVALU - V, I>();
  }
}

}  // namespace

template <bool GATE_UP, bool GATHER, bool LO, int TM, int WF>
__global__ __launch_bounds__(kThreads, 1) void expert_bigtile_dma(TiledGemmArgs ta, int32_t *queue) {
  using P = DmaPlan<LO, TM, WF>;
  constexpr bool MX = P::MX;
  constexpr int CH = P::CH, WUN = P::WUN, XUN = P::XUN, SLOT = P::SLOT, NSTAGE = P::NSTAGE, OPS = P::OPS;
  constexpr int XI = P::XI, MF = TM / 64;  // wave sub-tile: MF fragments of 32 tokens x 128 columns
  static_assert(!MX || (GATE_UP && !LO), "MXFP4 weights: gate_up only");
  const ExpertGemmArgs &a = ta.g;
  extern __shared__ u32x4_t smem[];

  const int tid = threadIdx.x;
  // the wave index is uniform across the wave; saying so keeps every branch
  // on it a scalar branch
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;

  const int cols_per_tile = GATE_UP ? BN / 2 : BN;
  const int n_tiles = (a.N + cols_per_tile - 1) / cols_per_tile;
  const int total = a.counts ? ta.mtile_prefix[ta.n_active_all[0]] * n_tiles
                             : ((a.single_rows + TM - 1) / TM) * n_tiles;
  const int nst = a.Kdim / P::BK;  // the reduction is a multiple of 32

  // XCD-contiguous ranges of the tile list; inside its range a workgroup
  // takes the next tile from the XCD's counter when it is free (the thin
  // tail tiles of the experts cost less than full ones, so a fixed stride
  // leaves some workgroups idle at the end)
  const int nx = gridDim.x % 8 == 0 ? 8 : 1;
  const int xcd = blockIdx.x % nx;
  const int span = (total + nx - 1) / nx;
  int *next = reinterpret_cast<int *>(smem);  // the ring is free between tiles
  // once its own range is done, a workgroup of a launch over many experts
  // takes tiles left in the other XCDs' ranges (gpt-oss MXFP4 gate_up at
  // T=2048: 481 -> 456 us); a single group's equal tiles stay in their
  // range (stealing slowed the shared expert's gate_up by 12%: a stolen
  // tile's operands sit in another XCD's L2)
  const int sources = a.single_rows == 0 ? nx : 1;
  int from = 0;  // (thread 0) the counter drawn from: own XCD's, then the others'
  for (;;) {
    __syncthreads();
    if (tid == 0) {
      int got = -1;
      for (; from < sources; ++from) {
        const int x2 = (xcd + from) % nx;
        const int local = atomicAdd(queue + x2, 1);
        if (local < span && x2 * span + local < total) {
          got = x2 * span + local;
          break;
        }
      }
      next[0] = got;
    }
    __syncthreads();
    const int tile = next[0];
    __syncthreads();
    if (tile < 0) break;
    BigCoord c;
    big_coord(ta, tile, n_tiles, c, TM);
    const int col0 = c.n0 * cols_per_tile;

    // ---- this lane's chunk of each of the wave's load instructions ---------
    // instruction i writes units (wave*4 + i)*64 + lane = row*4 + cs of a tile,
    // row = (wave*4 + i)*16 + lane/4; the unit holds logical chunk cs ^ f(row)
    const char *xbase = static_cast<const char *>(a.A);
    const char *xlbase = static_cast<const char *>(a.A_lo);
    // weight tile row -> weight row of the expert (clamped into the matrix)
    auto wrow = [&](int row) {
      int wr, lim;
      if constexpr (GATE_UP) {
        wr = row < BN / 2 ? col0 + row : a.N + col0 + (row - BN / 2);
        lim = row < BN / 2 ? a.N - 1 : 2 * a.N - 1;
      } else {
        wr = col0 + row;
        lim = a.N - 1;
      }
      return (uint32_t)min(wr, lim);
    };
    const char *wbase = static_cast<const char *>(a.W) + (size_t)c.g * a.w_stride * (MX ? 1 : 2);
    constexpr int NW = MX ? 1 : 4;  // weight load instructions per wave and stage
    uint32_t wof[NW], xof[XI], xlof[LO ? XI : 1];
    if constexpr (MX) {  // lane -> weight row wave * 64 + lane: its 16 code bytes
      wof[0] = wrow(wave * 64 + lane) * (uint32_t)(a.Kdim / 2);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (wave * 4 + i) * 16 + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 2) & 3);
        wof[i] = (wrow(row) * (uint32_t)a.Kdim + ch * 8) * 2u;
      }
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int row = (wave * XI + i) * 16 + (lane >> 2);
      const int ch = (lane & 3) ^ ((row >> 2) & 3);
      const int r = min(c.m0 + row, c.nrows - 1);
      uint32_t ar;
      if constexpr (GATHER)
        ar = (uint32_t)(a.perm[c.row0 + r] / a.topk);
      else
        ar = (uint32_t)(c.row0 + r);
      xof[i] = (ar * (uint32_t)a.Kdim + ch * 8) * 2u;
      if constexpr (LO) xlof[i] = ((uint32_t)(c.row0 + r) * (uint32_t)a.Kdim + ch * 8) * 2u;
    }
    auto issue = [&](int st) {  // stage st into ring slot st % NSTAGE
      u32x4_t *sl = smem + (st % NSTAGE) * SLOT;
      const uint32_t kb = (uint32_t)st * (P::BK * 2);
      if constexpr (MX) {
        dma16(wbase + wof[0] + (uint32_t)st * (P::BK / 2), sl + wave * 64);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(wbase + wof[i] + kb, sl + (wave * 4 + i) * 64);
      }
#pragma unroll
      for (int i = 0; i < XI; ++i) dma16(xbase + xof[i] + kb, sl + WUN + (wave * XI + i) * 64);
      if constexpr (LO) {
#pragma unroll
        for (int i = 0; i < XI; ++i) dma16(xlbase + xlof[i] + kb, sl + WUN + XUN + (wave * XI + i) * 64);
      }
    };

    f32x16_t acc[MF][4];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mf][nf][i] = 0.f;

    // 32-row token fragments of this wave that hold rows of the group.  The
    // main loop is compiled once per count (no guards inside it: a guard per
    // MFMA group would break the interleaved schedule); a wave with fewer
    // rows skips the empty fragments' reads and MFMAs but still issues its
    // share of the tile's loads and meets every barrier.
    const int mf_count = min(MF, max(0, (c.nrows - c.m0 - wm * (TM / 2) + 31) / 32));
    auto wfrag = [&](int nf) {
      if constexpr (GATE_UP) return nf < 2 ? wn * 64 + nf * 32 : BN / 2 + wn * 64 + (nf - 2) * 32;
      else return wn * 128 + nf * 32;
    };
    // Operand fragments of one 16-deep step, two register sets: the MFMAs of
    // step t run while the fragments of step t + 1 are read from LDS.
    constexpr int NB = LO ? 2 * MF : MF;
    u32x4_t af[2][4], bf[2][NB];
    // MXFP4: byte of the scale table where the scales of fragment nf's row
    // start; the scales of the stage being read (both of its 16-deep steps)
    const uint8_t *stab = reinterpret_cast<const uint8_t *>(smem + NSTAGE * SLOT);
    int srow[MX ? 4 : 1];
    float scl[MX ? 4 : 1];
    if constexpr (MX) {
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) srow[nf] = (wfrag(nf) + l32) * (a.Kdim / 32);
    }
    auto fetch = [&](int set, int stg, int kk, auto cnt) {
      constexpr int C = decltype(cnt)::value;
      const u32x4_t *Wt = smem + (stg % NSTAGE) * SLOT, *Xt = Wt + WUN;
      const int ch = 2 * kk + lh;
      if constexpr (C > 0) {
        if constexpr (MX) {  // codes 16 kk + 8 lh .. + 7 of the row: dword 2 kk + lh of its unit
          const uint32_t *Wd = reinterpret_cast<const uint32_t *>(Wt);
          if (kk == 0) {  // a new stage: its scale bytes
#pragma unroll
            for (int nf = 0; nf < 4; ++nf) scl[nf] = e8m0_to_f32(stab[srow[nf] + stg]);
          }
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) af[set][nf] = decode_e2m1x8(Wd[(wfrag(nf) + l32) * 4 + ch], scl[nf]);
        } else {
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) af[set][nf] = Wt[unit<CH>(wfrag(nf) + l32, ch)];
        }
      }
#pragma unroll
      for (int mf = 0; mf < C; ++mf) {
        bf[set][mf] = Xt[unit<CH>(wm * (TM / 2) + mf * 32 + l32, ch)];
        if constexpr (LO) bf[set][MF + mf] = Xt[XUN + unit<CH>(wm * (TM / 2) + mf * 32 + l32, ch)];
      }
    };
    auto mma = [&](int set, auto cnt) {
      constexpr int C = decltype(cnt)::value;
#pragma unroll
      for (int mf = 0; mf < C; ++mf) {
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma_32x32x16(af[set][nf], bf[set][mf], acc[mf][nf]);
        if constexpr (LO) {
#pragma unroll
          for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma_32x32x16(af[set][nf], bf[set][MF + mf], acc[mf][nf]);
        }
      }
    };
    // fetch of the next step and MFMAs of this one in one scheduling region,
    // the reads spread between the MFMAs
    auto step = [&](int next_set, int next_stg, int next_kk, int set, auto cnt) {
      constexpr int C = decltype(cnt)::value;
      fetch(next_set, next_stg, next_kk, cnt);
      mma(set, cnt);
      if constexpr (C > 0) {
        if constexpr (MX)  // 4 code reads + C token reads; 4 decodes of 4 converts and their scale work
          interleave_reads_valu<4 + C, C * 4, 20>();
        else
          interleave_reads<4 + (LO ? 2 * C : C), C * 4 * (LO ? 2 : 1)>();
      }
    };
    // wait until the stage `after` stages before the newest issued one has landed
    auto wait_stage = [&](int after) {
      switch (after) {
        case 0: wait_vmem<0>(); break;
        case 1: wait_vmem<OPS>(); break;
        case 2: wait_vmem<(NSTAGE >= 3 ? 2 : 0) * OPS>(); break;
        case 3: wait_vmem<(NSTAGE >= 4 ? 3 : 0) * OPS>(); break;
        case 4: wait_vmem<(NSTAGE >= 5 ? 4 : 0) * OPS>(); break;
        default: wait_vmem<(NSTAGE >= 6 ? 5 : 0) * OPS>(); break;
      }
    };

    // ---- pipeline over 32-deep stages (two 16-deep steps each).  The ring
    // holds NSTAGE stages.  In the second step of stage s every wave waits
    // for stage s + 1, one barrier follows (after it nobody reads slot s any
    // more), stage s + NSTAGE is issued into slot s, and the first fragments
    // of stage s + 1 are read while the second step's MFMAs run.
    auto run = [&](auto cnt) {
      if constexpr (MX) {
        // the tile's scale table: LDS unit p holds bytes 16 q .. 16 q + 15 of
        // the gate rows' run (p < K/4, q = p) or of the up rows' run (q = p -
        // K/4); units past a run's valid rows (a partial last column tile) and
        // the padding read the run's start instead and are never used.  These
        // loads precede stage 0's, so stage 0's wait covers them.
        const int hu = a.Kdim / 4;  // units per run of 128 rows
        const int nv = min(BN / 2, a.N - col0) * (a.Kdim / 32) / 16;  // units of the valid rows
        const char *gs = reinterpret_cast<const char *>(a.Wscale) + (size_t)c.g * a.s_stride;
        const char *g0 = gs + (size_t)col0 * (a.Kdim / 32), *u0 = gs + (size_t)(a.N + col0) * (a.Kdim / 32);
        u32x4_t *tab = smem + NSTAGE * SLOT;
        const int n_inst = P::table_units(a.Kdim) / 64;
        for (int j = wave; j < n_inst; j += 4) {
          const int p = j * 64 + lane;
          const int q = p < hu ? p : p - hu;
          const char *src = (p < hu ? g0 : u0) + (p < 2 * hu && q < nv ? q * 16 : 0);
          dma16(src, tab + j * 64);
        }
      }
#pragma unroll
      for (int d = 0; d < NSTAGE; ++d)
        if (d < nst) issue(d);
      wait_stage(min(NSTAGE - 1, nst - 1));
      barrier_lds();
      fetch(0, 0, 0, cnt);
      for (int s = 0; s < nst - 1; ++s) {
        step(1, s, 1, 0, cnt);
        wait_stage(min(NSTAGE - 2, nst - 2 - s));
        barrier_lds();
        if (s + NSTAGE < nst) issue(s + NSTAGE);
        step(0, s + 1, 0, 1, cnt);
      }
      fetch(1, nst - 1, 1, cnt);
      mma(0, cnt);
      mma(1, cnt);
    };
    static_assert(MF == 4 || MF == 2, "fragment counts");
    if (mf_count == MF) run(std::integral_constant<int, MF>{});  // uniform per wave
    else if (mf_count == 0) run(std::integral_constant<int, 0>{});
    else if (mf_count == 1) run(std::integral_constant<int, 1>{});
    else if constexpr (MF == 4) {
      if (mf_count == 2) run(std::integral_constant<int, 2>{});
      else run(std::integral_constant<int, 3>{});
    }
    barrier_lds();  // every wave is done with the ring
    big_epilogue<GATE_UP, MF>(a, c, col0, acc, smem);
    barrier_lds();  // the next tile's first loads overwrite the ring
  }
}

// ---------------------------------------------------------------------------
// MXFP4 gate_up on the block-scaled matrix cores of gfx950
// (v_mfma_scale_f32_32x32x64_f8f6f4: E2M1 codes times E4M3 values, every
// 32-element block of either operand with its own E8M0 scale), so the expert
// weights enter the multiplication as they are stored.  The activations are
// first split (mxfp8_split) into two MXFP8 terms x = hi + lo: per block of 32
// the scale 2^(floor(log2 max|x|) - 7) keeps every |x| / scale at or below
// 256 (no E4M3 saturation), hi is x / scale rounded to E4M3, lo the remainder
// rounded to E4M3 under a scale of its own.  A bf16 value has 8 significant
// bits and each term carries 4, so hi + lo reproduces x up to remainders
// below the smallest E4M3 subnormal of their block; each stage multiplies
// the codes by both terms.
//
// Operand layouts (measured on the GPU): lane l of the FP4 operand holds row
// l % 32 with reduction index 32 (l / 32) + p in nibble p (byte p / 2, low
// nibble first); lane l of the FP8 operand holds column l % 32 with index
// 16 (l / 32) + j in byte j < 16 and 32 + 16 (l / 32) + (j - 16) in byte
// j >= 16; the A scale of lane l scales its own block, the B scale of lane l
// block l / 32 of column l % 32; the result has the layout of the 32x32 bf16
// instruction.
//
// Tile and epilogue as in the direct-to-LDS big tile (256 tokens x 256 weight
// rows, four wavefronts of 128 x 128), stages of 64 reduction elements (one
// MFMA step) in a ring of three.  A stage holds the weight codes as two planes
// (reduction halves) of 256 rows x 16 bytes, the activations as eight planes
// of 256 rows x 16 bytes ([hi | lo] of its two blocks, 16 bytes each) and the
// activation scales as 256 rows x 4 bytes; each plane is read by 32 lanes at
// consecutive rows.  The tile's weight-scale table follows the ring.
// ---------------------------------------------------------------------------
namespace {

struct MxsPlan {
  static constexpr int BK = 64;
  static constexpr int WUN = 2 * BN;             // weight code planes
  static constexpr int XUN = 8 * BM;             // activation planes
  static constexpr int SUN = BM * 4 / 16;        // activation scales
  static constexpr int SLOT = WUN + XUN + SUN;   // 2624 units (41 KB)
  static constexpr int NSTAGE = 3;
  static constexpr int OPS = WUN / 256 + XUN / 256 + 1;  // load instructions per wave and stage
  static constexpr int MAX_K = 4096;             // the scale table beside the ring
  static constexpr size_t RING_BYTES = (size_t)NSTAGE * SLOT * 16;
  static __host__ __device__ constexpr int table_units(int K) { return (K / 2 + 63) & ~63; }
  static_assert((NSTAGE - 1) * OPS < 64, "vmcnt range");
};
static_assert(MxsPlan::RING_BYTES + (size_t)MxsPlan::table_units(MxsPlan::MAX_K) * 16 <= 160 * 1024, "LDS");

// 4 bytes per lane from global memory straight into LDS (lane i at l + 4 i)
__device__ __forceinline__ void dma4(const char *g, void *l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)l, 4, 0, 0);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16_t mfma_mx(i32x8_t a_fp4, i32x8_t b_fp8, f32x16_t c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a_fp4, b_fp8, c, 4, 0, 0, scale_a, 0, scale_b);
}

}  // namespace

template <bool GATHER>
__global__ __launch_bounds__(kThreads, 1) void expert_bigtile_mxs(TiledGemmArgs ta, MxActs xa) {
  using P = MxsPlan;
  constexpr int SLOT = P::SLOT, NSTAGE = P::NSTAGE, OPS = P::OPS, MF = 4;
  const ExpertGemmArgs &a = ta.g;
  extern __shared__ u32x4_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;

  const int cols_per_tile = BN / 2;
  const int n_tiles = (a.N + cols_per_tile - 1) / cols_per_tile;
  const int total = a.counts ? ta.mtile_prefix[ta.n_active_all[0]] * n_tiles
                             : ((a.single_rows + BM - 1) / BM) * n_tiles;
  const int nst = a.Kdim / P::BK;   // the launcher checks Kdim % 64 == 0
  const int nblk = a.Kdim / 32;     // blocks of 32 per row

  const int nx = gridDim.x % 8 == 0 ? 8 : 1;
  const int xcd = blockIdx.x % nx, per = gridDim.x / nx;
  const int span = (total + nx - 1) / nx;
  for (int local = blockIdx.x / nx; local < span; local += per) {
    const int tile = xcd * span + local;
    if (tile >= total) break;
    BigCoord c;
    big_coord(ta, tile, n_tiles, c, BM);
    const int col0 = c.n0 * cols_per_tile;

    // weight tile row -> weight row of the expert (clamped into the matrix)
    auto wrow = [&](int row) {
      const int wr = row < BN / 2 ? col0 + row : a.N + col0 + (row - BN / 2);
      const int lim = row < BN / 2 ? a.N - 1 : 2 * a.N - 1;
      return (uint32_t)min(wr, lim);
    };
    const char *wbase = static_cast<const char *>(a.W) + (size_t)c.g * a.w_stride;
    // this lane's sources.  Load instruction g (of 8 weight, 32 activation
    // and 4 scale instructions per stage, spread over the waves) covers tile
    // rows (g % 4) * 64 + lane of plane g / 4; the scale instruction of wave w
    // rows w * 64 + lane.
    uint32_t wof[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = wave * 2 + i;
      wof[i] = wrow((g & 3) * 64 + lane) * (uint32_t)(a.Kdim / 2) + (g >> 2) * 16;
    }
    uint32_t xrow[4];  // activation row of tile rows rg * 64 + lane
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int r = min(c.m0 + rg * 64 + lane, c.nrows - 1);
      xrow[rg] = GATHER ? (uint32_t)(a.perm[c.row0 + r] / a.topk) : (uint32_t)(c.row0 + r);
    }
    const uint32_t srow = xrow[wave];
    const char *xq = reinterpret_cast<const char *>(xa.q);
    const char *xs = reinterpret_cast<const char *>(xa.s);
    const uint32_t xrow_bytes = (uint32_t)a.Kdim * 2u;  // [hi | lo] of every block: 64 bytes per block

    auto issue = [&](int st) __attribute__((always_inline)) {  // stage st into ring slot st % NSTAGE
      u32x4_t *sl = smem + (st % NSTAGE) * SLOT;
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(wbase + wof[i] + (uint32_t)st * 32u, sl + (wave * 2 + i) * 64);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int g = wave * 8 + i;  // plane g / 4, row group g % 4
        dma16(xq + xrow[g & 3] * xrow_bytes + (uint32_t)st * 128u + (g >> 2) * 16, sl + P::WUN + g * 64);
      }
      dma4(xs + (srow * (uint32_t)nblk + 2u * st) * 2u, reinterpret_cast<char *>(sl + P::WUN + P::XUN) + wave * 256);
    };

    f32x16_t acc[MF][4];
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mf][nf][i] = 0.f;

    const int mf_count = min(MF, max(0, (c.nrows - c.m0 - wm * (BM / 2) + 31) / 32));
    auto wfrag = [&](int nf) { return nf < 2 ? wn * 64 + nf * 32 : BN / 2 + wn * 64 + (nf - 2) * 32; };
    const uint8_t *stab = reinterpret_cast<const uint8_t *>(smem + NSTAGE * SLOT);

    // one stage: its fragments read from LDS, then its MFMAs (a second
    // register set, to read the next stage under these MFMAs, does not fit
    // beside the accumulators: it spills)
    auto compute = [&](int st, auto cnt) __attribute__((always_inline)) {
      constexpr int C = decltype(cnt)::value;
      const u32x4_t *sl = smem + (st % NSTAGE) * SLOT;
      const u32x4_t *Wt = sl, *Xt = sl + P::WUN;
      const uint32_t *St = reinterpret_cast<const uint32_t *>(sl + P::WUN + P::XUN);
      i32x8_t af[4];
      int sa[4];
      if constexpr (C > 0) {
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          const int row = wfrag(nf) + l32;
          const u32x4_t v = Wt[lh * 256 + row];
          af[nf] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          sa[nf] = stab[row * nblk + 2 * st + lh];
        }
      }
#pragma unroll
      for (int mf = 0; mf < C; ++mf) {
        const int tr = wm * (BM / 2) + mf * 32 + l32;
        const u32x4_t h0 = Xt[(0 + lh) * 256 + tr], h1 = Xt[(4 + lh) * 256 + tr];
        const u32x4_t o0 = Xt[(2 + lh) * 256 + tr], o1 = Xt[(6 + lh) * 256 + tr];
        const uint32_t sc = St[tr];
        const i32x8_t bh = {(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
        const i32x8_t bl = {(int)o0.x, (int)o0.y, (int)o0.z, (int)o0.w, (int)o1.x, (int)o1.y, (int)o1.z, (int)o1.w};
        const int sbh = (int)((sc >> (16 * lh)) & 0xffu), sbl = (int)((sc >> (16 * lh + 8)) & 0xffu);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
          acc[mf][nf] = mfma_mx(af[nf], bh, acc[mf][nf], sa[nf], sbh);
          acc[mf][nf] = mfma_mx(af[nf], bl, acc[mf][nf], sa[nf], sbl);
        }
      }
    };

    auto run = [&](auto cnt) __attribute__((always_inline)) {
      // the tile's weight-scale table: LDS unit p holds bytes 16 q .. 16 q + 15
      // of the gate rows' run (p < K/4, q = p) or of the up rows' run (q = p -
      // K/4); units past a run's valid rows (a partial last column tile) and
      // the padding read the run's start instead and are never used.  These
      // loads precede stage 0's, so stage 0's wait covers them.
      const int hu = a.Kdim / 4;
      const int nv = min(BN / 2, a.N - col0) * nblk / 16;
      const char *gs = reinterpret_cast<const char *>(a.Wscale) + (size_t)c.g * a.s_stride;
      const char *g0 = gs + (size_t)col0 * nblk, *u0 = gs + (size_t)(a.N + col0) * nblk;
      u32x4_t *tab = smem + NSTAGE * SLOT;
      const int n_inst = P::table_units(a.Kdim) / 64;
      for (int j = wave; j < n_inst; j += 4) {
        const int p = j * 64 + lane;
        const int q = p < hu ? p : p - hu;
        const char *src = (p < hu ? g0 : u0) + (p < 2 * hu && q < nv ? q * 16 : 0);
        dma16(src, tab + j * 64);
      }
#pragma unroll
      for (int d = 0; d < NSTAGE - 1; ++d)
        if (d < nst) issue(d);
      for (int st = 0; st < nst; ++st) {
        // stage st + 1, issued before, may stay in flight
        if (st + 1 < nst) wait_vmem<OPS>();
        else wait_vmem<0>();
        barrier_lds();
        if (st + NSTAGE - 1 < nst) issue(st + NSTAGE - 1);  // into the slot stage st - 1 used
        compute(st, cnt);
      }
    };
    if (mf_count == MF) run(std::integral_constant<int, MF>{});  // uniform per wave
    else if (mf_count == 0) run(std::integral_constant<int, 0>{});
    else if (mf_count == 1) run(std::integral_constant<int, 1>{});
    else if (mf_count == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 3>{});
    barrier_lds();  // every wave is done with the ring
    big_epilogue<true, MF>(a, c, col0, acc, smem);
    barrier_lds();  // the next tile's first loads overwrite the ring
  }
}

// x (bf16 [rows, K]) -> two MXFP8 terms per block of 32: q[rows][K/32][hi 32
// bytes | lo 32 bytes] (E4M3) and s[rows][K/32] = hi scale | lo scale << 8
// (E8M0).  One thread per block.
__global__ __launch_bounds__(256) void mxfp8_split(const uint16_t *x, long n_blocks, uint8_t *q, uint16_t *s) {
  const long b = blockIdx.x * 256L + threadIdx.x;
  if (b >= n_blocks) return;
  float v[32];
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + b * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_t w = src[i];
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[i * 8 + 2 * j] = __uint_as_float(d[j] << 16);
      v[i * 8 + 2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
    }
  }
  // one term: scale exponent e = floor(log2 max|t|) - 7 (0 for an all-zero
  // block), codes of t / 2^e, and what they leave over
  auto term = [&](float (&t)[32], uint32_t (&out)[8]) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(t[j]));
    int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 8 : 0;  // frexp: amax = m 2^E, m in [0.5, 1)
    e = min(127, max(-127, e));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(t[4 * j], -e),
                                              __builtin_amdgcn_ldexpf(t[4 * j + 1], -e), 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(t[4 * j + 2], -e),
                                          __builtin_amdgcn_ldexpf(t[4 * j + 3], -e), w, true);
      out[j] = (uint32_t)w;
      // the remainder is exact in f32
      t[4 * j] -= __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 0), e);
      t[4 * j + 1] -= __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 1), e);
      t[4 * j + 2] -= __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 2), e);
      t[4 * j + 3] -= __builtin_amdgcn_ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 3), e);
    }
    return e + 127;
  };
  uint32_t hi[8], lo[8];
  const int sh = term(v, hi);
  const int sl = term(v, lo);
  u32x4_t *dst = reinterpret_cast<u32x4_t *>(q + b * 64);
  dst[0] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
  dst[1] = u32x4_t{hi[4], hi[5], hi[6], hi[7]};
  dst[2] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
  dst[3] = u32x4_t{lo[4], lo[5], lo[6], lo[7]};
  s[b] = (uint16_t)(sh | (sl << 8));
}

namespace {

template <bool GATE_UP, bool GATHER, bool LO, int TM = BM, int WF = W_BF16>
hipError_t launch_dma_t(const TiledGemmArgs &t, long tiles_bound, int32_t *queue, hipStream_t st) {
  using P = DmaPlan<LO, TM, WF>;
  auto kern = expert_bigtile_dma<GATE_UP, GATHER, LO, TM, WF>;
  // the ring (+ the MXFP4 scale table), or the gate_up epilogue's staging if
  // that is larger
  constexpr size_t lds_max = 160 * 1024;
  const size_t ring = P::LDS_BYTES + (P::MX ? (size_t)P::table_units(t.g.Kdim) * 16 : 0);
  const size_t lds = std::max(ring, GATE_UP ? epi_gate_up_bytes<TM / 64>() : (size_t)0);
  if (lds > lds_max) return hipErrorInvalidValue;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
  if (attr != hipSuccess) return attr;
  const int grid = (int)std::max(1L, std::min(tiles_bound, 256L));  // one per CU
  enqueue_kernel(kern, dim3(grid), dim3(kThreads), lds, st, t, queue);
  return hipGetLastError();
}

template <bool GATE_UP, int WF, bool GATHER, bool LO>
hipError_t launch_big_t(const TiledGemmArgs &t, long tiles_bound, int32_t *queue, hipStream_t st) {
  if constexpr (WF == W_BF16) {
    return launch_dma_t<GATE_UP, GATHER, LO>(t, tiles_bound, queue, st);
  } else {
    if constexpr (GATE_UP && !LO) {
      // MXFP4 gate_up: codes and the tile's scale table fed by direct-to-LDS
      // loads (16-byte loads: the scale array starts on 16 bytes; the table
      // fits beside the ring up to a reduction of MAX_K)
      if ((reinterpret_cast<uintptr_t>(t.g.Wscale) & 15) == 0 && t.g.Kdim <= DmaPlan<LO, BM, W_MXFP4>::MAX_K)
        return launch_dma_t<GATE_UP, GATHER, LO, BM, W_MXFP4>(t, tiles_bound, queue, st);
    }
    // otherwise codes are decoded on their way into LDS (register-staged)
    auto kern = expert_bigtile<GATE_UP, WF, GATHER, LO>;
    constexpr size_t lds = std::max(BigPlan<LO>::LDS_BYTES, GATE_UP ? epi_gate_up_bytes<4>() : (size_t)0);
    static_assert(lds <= 160 * 1024, "LDS");
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    const int grid = (int)std::max(1L, std::min(tiles_bound, 256L));  // one per CU
    enqueue_kernel(kern, dim3(grid), dim3(kThreads), lds, st, t);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_bigtile(const TiledGemmArgs &t, bool gate_up, WFormat wf, long max_rows_total, int max_groups,
                          int32_t *queue, hipStream_t st) {
  if (!queue) return hipErrorInvalidValue;
  const ExpertGemmArgs &a = t.g;
  const int cols_per_tile = gate_up ? BN / 2 : BN;
  const long n_tiles = (a.N + cols_per_tile - 1) / cols_per_tile;
  const long tiles_bound = ((max_rows_total + BM - 1) / BM + max_groups) * n_tiles;
  const bool gather = gate_up && a.perm != nullptr;
  if (gate_up) {
    if (wf == W_MXFP4)
      return gather ? launch_big_t<true, W_MXFP4, true, false>(t, tiles_bound, queue, st)
                    : launch_big_t<true, W_MXFP4, false, false>(t, tiles_bound, queue, st);
    return gather ? launch_big_t<true, W_BF16, true, false>(t, tiles_bound, queue, st)
                  : launch_big_t<true, W_BF16, false, false>(t, tiles_bound, queue, st);
  }
  if (a.A_lo) {
    if (wf == W_MXFP4) return launch_big_t<false, W_MXFP4, false, true>(t, tiles_bound, queue, st);
    return launch_big_t<false, W_BF16, false, true>(t, tiles_bound, queue, st);
  }
  if (wf == W_MXFP4) return launch_big_t<false, W_MXFP4, false, false>(t, tiles_bound, queue, st);
  return launch_big_t<false, W_BF16, false, false>(t, tiles_bound, queue, st);
}

int bigtile_rows() { return BM; }

bool bigtile_mx_scaled_applies(const TiledGemmArgs &t) {
  const ExpertGemmArgs &a = t.g;
  return a.Kdim % MxsPlan::BK == 0 && a.Kdim <= MxsPlan::MAX_K && (reinterpret_cast<uintptr_t>(a.Wscale) & 15) == 0;
}

hipError_t launch_mxfp8_split(const uint16_t *x, long rows, int K, const MxActs &xa, hipStream_t st) {
  if (K % 32) return hipErrorInvalidValue;
  const long nb = rows * (K / 32);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_split, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, x, nb, xa.q, xa.s);
  return hipGetLastError();
}

hipError_t launch_bigtile_mx_scaled(const TiledGemmArgs &t, const MxActs &xa, long max_rows_total, int max_groups,
                                    hipStream_t st) {
  const ExpertGemmArgs &a = t.g;
  if (!bigtile_mx_scaled_applies(t)) return hipErrorInvalidValue;
  const long n_tiles = (a.N + BN / 2 - 1) / (BN / 2);
  const long tiles_bound = ((max_rows_total + BM - 1) / BM + max_groups) * n_tiles;
  auto kern = a.perm ? expert_bigtile_mxs<true> : expert_bigtile_mxs<false>;
  constexpr size_t lds_max = 160 * 1024;
  const size_t ring = MxsPlan::RING_BYTES + (size_t)MxsPlan::table_units(a.Kdim) * 16;
  const size_t lds = std::max(ring, epi_gate_up_bytes<4>());
  if (lds > lds_max) return hipErrorInvalidValue;
  static const hipError_t attr1 = hipFuncSetAttribute(reinterpret_cast<const void *>(expert_bigtile_mxs<true>),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
  static const hipError_t attr0 = hipFuncSetAttribute(reinterpret_cast<const void *>(expert_bigtile_mxs<false>),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
  if (attr1 != hipSuccess) return attr1;
  if (attr0 != hipSuccess) return attr0;
  const int grid = (int)std::max(1L, std::min(tiles_bound, 256L));  // one per CU
  enqueue_kernel(kern, dim3(grid), dim3(kThreads), lds, st, t, xa);
  return hipGetLastError();
}

}  // namespace moe
