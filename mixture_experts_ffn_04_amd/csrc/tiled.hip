// Tiled grouped expert GEMMs for large token counts (matrix-core bound).
//
// Same operations as the streaming kernels in experts.hip (gate_up + SwiGLU,
// down + optional per-expert bias; bf16 or MXFP4 weights, bf16 activations),
// organised for operand reuse: a workgroup computes a 128-token x TBN-weight-
// row tile, staging TBK-deep slices of both operands in LDS (double-buffered:
// the next slice's global loads are issued before the current slice's MFMAs
// and stored to the other buffer afterwards).  Four waves each compute a
// 64-token x TBN/2-weight-row sub-tile with 16x16x32 bf16 MFMAs (weights as
// operand A, tokens as operand B, so a lane ends with four adjacent output
// columns of one token).  gate_up tiles hold TBN/2 gate rows and the matching
// up rows, and each wave takes half of each, so SwiGLU pairs meet in one
// lane.  MXFP4 codes are decoded to bf16 on their way into LDS.
//
// Tile shapes: 256 x 32, and 128 x 64 for bf16 gate_up when experts hold
// about one row tile: its weight slice visits each of 128 rows 128 bytes at
// a time instead of 256 rows 64 bytes at a time (the same 16 KB), and HBM
// streams many rows at once better in longer runs.
//
// A persistent grid walks the (expert, column tile, row tile) list built from
// the per-expert row counts (mtile_prefix); row tiles of one column tile are
// consecutive (in blocks of at most eight), so the weight tile is reused from
// L2.
//
// [SF1073] SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own DSpark draft
// (stacked on #1035)" (clamped SwiGLU; stacked gate_up_proj; FP4 experts two
// codes per byte, low nibble first, E8M0 scale per 32 inputs) and [MI143]
// MoE-Infinity PR #143 (output-major MXFP4 blocks, expert biases).
#include <type_traits>

#include "kernels.hpp"
#include "tile.hpp"

namespace moe {

namespace {

constexpr int TBM = 128;          // tokens per tile
// weight rows per tile and reduction slice
constexpr int kTN = 256, kTK = 32;
constexpr int kTNg = 128, kTKg = 64;    // bf16 gate_up of experts with about one row tile
constexpr int TTHREADS = 256;

// Tile order inside an expert: its row tiles fastest, in blocks of at most
// kRowBlock.  Measured on the selection-bias qwen3_5_moe drafter at T=4096
// (collapsed routing, experts of up to 32 row tiles): gate_up 746 -> 712 us,
// down 636 -> 596 us against every row tile per column tile; walking column
// tiles fastest everywhere instead slowed the DeepSeek-V4 gate_up by 9%.
constexpr int kRowBlock = 8;

struct TileCoord {
  int g, nrows, row0;  // group
  int m0, n0;          // first token row (in the group) and first column
};

__device__ __forceinline__ bool tile_coord(const TiledGemmArgs &t, int tile, int n_tiles, TileCoord &c) {
  const ExpertGemmArgs &a = t.g;
  if (!a.counts) {  // one group of single_rows rows
    const int mt = (a.single_rows + TBM - 1) / TBM;
    c.g = 0;
    c.nrows = a.single_rows;
    c.row0 = 0;
    c.m0 = (tile % mt) * TBM;
    c.n0 = tile / mt;  // column tile index; scaled by the caller
    return true;
  }
  const int q = tile / n_tiles;  // global row-tile index (of all experts)
  // binary search: mtile_prefix[ai] <= q < mtile_prefix[ai + 1]
  int lo = 0, hi = t.n_active_all[0];
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (t.mtile_prefix[mid] <= q) lo = mid;
    else hi = mid;
  }
  const int mt_e = t.mtile_prefix[lo + 1] - t.mtile_prefix[lo];
  const int local = tile - t.mtile_prefix[lo] * n_tiles;
  c.g = t.active_all[lo];
  c.nrows = a.counts[c.g];
  c.row0 = a.offsets[c.g];
  if (mt_e <= kRowBlock) {  // every row tile of the expert per column tile
    c.m0 = (local % mt_e) * TBM;
    c.n0 = local / mt_e;  // column tile index; scaled by the caller
    return true;
  }
  // an expert with many row tiles (collapsed routing): row tiles fastest
  // within blocks of kRowBlock, every column tile per block, so the tiles
  // in flight on an XCD share both token and weight tiles
  const int nfb = mt_e / kRowBlock;  // full blocks
  const int in_full = nfb * kRowBlock * n_tiles;
  int rb, w, bh;
  if (local < in_full) {
    bh = kRowBlock;
    rb = local / (kRowBlock * n_tiles);
    w = local - rb * kRowBlock * n_tiles;
  } else {
    bh = mt_e - nfb * kRowBlock;
    rb = nfb;
    w = local - in_full;
  }
  c.m0 = (rb * kRowBlock + w % bh) * TBM;
  c.n0 = w / bh;
  return true;
}

}  // namespace

template <bool GATE_UP, int WF, bool GATHER, bool LO, int TBN, int TBK>
__global__ __launch_bounds__(TTHREADS, 2) void expert_tiled(TiledGemmArgs ta, int32_t *queue) {
  constexpr int TLD = TBK + 8;  // padded LDS row: conflict-free 16-byte fragment reads
  constexpr int CF = TBN / 32;  // 16-row weight fragments per wave (half the tile's weight rows)
  static_assert(WF != W_MXFP4 || (TBN == 256 && TBK == 32), "MXFP4 tiles: 256 rows, 32-deep slices");
  const ExpertGemmArgs &a = ta.g;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t *Xs = smem;                         // [2][TBM][TLD]
  uint16_t *Ws = smem + 2 * TBM * TLD;         // [2][TBN][TLD]
  uint16_t *Xl = Ws + 2 * TBN * TLD;           // [2][TBM][TLD] low halves of h (down, LO)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;

  // column tiles: gate_up covers 128 gate columns per tile, down 256 columns
  const int cols_per_tile = GATE_UP ? TBN / 2 : TBN;
  const int n_tiles = (a.N + cols_per_tile - 1) / cols_per_tile;
  int total;
  if (a.counts) total = ta.mtile_prefix[ta.n_active_all[0]] * n_tiles;
  else total = ((a.single_rows + TBM - 1) / TBM) * n_tiles;

  const uint16_t *A = static_cast<const uint16_t *>(a.A);
  const int nks = (a.Kdim + TBK - 1) / TBK;

  // Workgroups are dispatched to the 8 XCDs round-robin; the tile list is cut
  // into 8 contiguous chunks so that the workgroups of one XCD walk one chunk
  // and share its weight and token tiles through their L2.  Inside a chunk a
  // workgroup takes the next tile from the XCD's counter when it is free, so
  // the tiles in flight on an XCD stay neighbours in the list (an expert's
  // tiles, which share token rows and weights) however long each tile took;
  // with a fixed stride they drift apart over the rounds.  Every tile is
  // computed the same way by whichever workgroup takes it.
  const int nx = gridDim.x % 8 == 0 ? 8 : 1;
  const int xcd = blockIdx.x % nx;
  const int chunk = (total + nx - 1) / nx;
  int *next = reinterpret_cast<int *>(smem);  // the LDS is free between tiles
  // Once its XCD's chunk is done, a workgroup of a routed gate_up (many
  // experts, tiles of unequal cost) takes tiles left in the other XCDs'
  // chunks: gate_up 1-3% faster.  The down calls were as often slower as
  // faster, and a single group's equal tiles only lose (a stolen tile's
  // operands sit in another XCD's L2), so those stay on their own chunk.
  const int sources = a.single_rows == 0 ? nx : 1;
  int from = 0;  // (thread 0) the counter drawn from: own XCD's, then the others'
  for (;;) {
    __syncthreads();  // the previous tile's LDS reads are done
    int tile;
    if constexpr (GATE_UP) {
      if (tid == 0) {
        int got = -1;
        for (; from < sources; ++from) {
          const int x2 = (xcd + from) % nx;
          const int local = atomicAdd(queue + x2, 1);
          if (local < chunk && x2 * chunk + local < total) {
            got = x2 * chunk + local;
            break;
          }
        }
        next[0] = got;
      }
      __syncthreads();
      tile = next[0];
      __syncthreads();  // read before the tile's first LDS stores
      if (tile < 0) break;
    } else {
      if (tid == 0) next[0] = atomicAdd(queue + xcd, 1);
      __syncthreads();
      const int local = next[0];
      __syncthreads();  // read before the tile's first LDS stores
      if (local >= chunk) break;
      tile = xcd * chunk + local;
      if (tile >= total) break;
    }
    TileCoord c;
    tile_coord(ta, tile, n_tiles, c);
    const int col0 = c.n0 * cols_per_tile;

    // ---- per-thread global source rows for the loads of every slice ----
    // X: 128 rows x 4 chunks of 16 B: chunk id = tid + 256 i, i < 2
    constexpr int XCH = TBM * (TBK / 8) / TTHREADS;
    const uint16_t *xsrc[XCH];
    int xrow[XCH], xkc[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int cid = tid + TTHREADS * i;
      xrow[i] = cid / (TBK / 8);
      xkc[i] = cid % (TBK / 8);
      const int r = min(c.m0 + xrow[i], c.nrows - 1);
      size_t ar;
      if constexpr (GATHER)
        ar = (size_t)(a.perm[c.row0 + r] / a.topk);
      else
        ar = (size_t)(c.row0 + r);
      xsrc[i] = A + ar * a.Kdim;
    }
    const uint16_t *xlsrc[XCH];
    if constexpr (LO) {
#pragma unroll
      for (int i = 0; i < XCH; ++i)
        xlsrc[i] = static_cast<const uint16_t *>(a.A_lo) +
                   (size_t)(c.row0 + min(c.m0 + xrow[i], c.nrows - 1)) * a.Kdim;
    }
    // W rows of this tile: LDS row r -> global weight row
    auto wrow_of = [&](int r) {
      int g;
      if constexpr (GATE_UP) g = r < TBN / 2 ? col0 + r : a.N + col0 + (r - TBN / 2);
      else g = col0 + r;
      const int lim = GATE_UP ? (r < TBN / 2 ? a.N - 1 : 2 * a.N - 1) : a.N - 1;
      return min(g, lim);
    };

    // W: bf16 256 rows x 4 chunks of 8 elements; MXFP4 256 rows x one 32-element
    // block (16 code bytes + 1 scale)
    constexpr int WCH = (WF == W_MXFP4) ? TBN / TTHREADS : TBN * (TBK / 8) / TTHREADS;
    u32x4_t xbuf[XCH], xlbuf[XCH], wbuf[WCH];
    uint32_t sbuf[WCH] = {};
    static_assert(WF != W_MXFP4 || TBK == 32, "one MXFP4 scale block per slice: slice ks reads block ks");
    int wr_l[WCH], wkc[WCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int cid = tid + TTHREADS * i;
      if constexpr (WF == W_MXFP4) {
        wr_l[i] = cid;
        wkc[i] = 0;
      } else {
        wr_l[i] = cid / (TBK / 8);
        wkc[i] = cid % (TBK / 8);
      }
    }
    const size_t wbase_rows = (size_t)c.g;
    // MXFP4 scales: with an even number of blocks per row (and the array on 2
    // bytes), one 16-bit load brings a row's scales of two consecutive
    // slices (a slice is one block deep), halving the scale loads, each of
    // which touches a cache line per lane
    const bool spair = WF == W_MXFP4 && (a.Kdim / 32) % 2 == 0 && (reinterpret_cast<uintptr_t>(a.Wscale) & 1) == 0;

    auto gload = [&](int ks) {
      const int k0 = ks * TBK;
#pragma unroll
      for (int i = 0; i < XCH; ++i) {
        const int k = k0 + xkc[i] * 8;
        xbuf[i] = k < a.Kdim ? load16(xsrc[i] + k) : u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (LO) xlbuf[i] = k < a.Kdim ? load16(xlsrc[i] + k) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        const int grow = wrow_of(wr_l[i]);
        if constexpr (WF == W_MXFP4) {
          if (k0 < a.Kdim) {
            const uint8_t *cp = static_cast<const uint8_t *>(a.W) + wbase_rows * a.w_stride +
                                (size_t)grow * (a.Kdim / 2) + k0 / 2;
            wbuf[i] = load_stream16(cp);
            const uint8_t *sp = a.Wscale + wbase_rows * a.s_stride + (size_t)grow * (a.Kdim / 32) + ks;
            if (!spair) sbuf[i] = *sp;
            else if ((ks & 1) == 0)  // the last slice of an odd count reads its byte alone
              sbuf[i] = ks + 1 < nks ? (uint32_t)*reinterpret_cast<const uint16_t *>(sp) : (uint32_t)*sp;
          } else {
            wbuf[i] = u32x4_t{0u, 0u, 0u, 0u};
            sbuf[i] = 127u;
          }
        } else {
          const int k = k0 + wkc[i] * 8;
          const uint16_t *wp = static_cast<const uint16_t *>(a.W) + wbase_rows * a.w_stride + (size_t)grow * a.Kdim;
          wbuf[i] = k < a.Kdim ? load16(wp + k) : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };
    auto lstore = [&](int buf) {
      uint16_t *xs = Xs + buf * TBM * TLD;
      uint16_t *ws = Ws + buf * TBN * TLD;
#pragma unroll
      for (int i = 0; i < XCH; ++i) *reinterpret_cast<u32x4_t *>(xs + xrow[i] * TLD + xkc[i] * 8) = xbuf[i];
      if constexpr (LO) {
        uint16_t *xl = Xl + buf * TBM * TLD;
#pragma unroll
        for (int i = 0; i < XCH; ++i) *reinterpret_cast<u32x4_t *>(xl + xrow[i] * TLD + xkc[i] * 8) = xlbuf[i];
      }
#pragma unroll
      for (int i = 0; i < WCH; ++i) {
        if constexpr (WF == W_MXFP4) {
          // the buffer index is the slice's parity
          const float sc = e8m0_to_f32(spair ? (sbuf[i] >> (8 * buf)) & 255u : sbuf[i]);
          uint16_t *dst = ws + wr_l[i] * TLD;
          *reinterpret_cast<u32x4_t *>(dst + 0) = decode_e2m1x8(wbuf[i].x, sc);
          *reinterpret_cast<u32x4_t *>(dst + 8) = decode_e2m1x8(wbuf[i].y, sc);
          *reinterpret_cast<u32x4_t *>(dst + 16) = decode_e2m1x8(wbuf[i].z, sc);
          *reinterpret_cast<u32x4_t *>(dst + 24) = decode_e2m1x8(wbuf[i].w, sc);
        } else {
          *reinterpret_cast<u32x4_t *>(ws + wr_l[i] * TLD + wkc[i] * 8) = wbuf[i];
        }
      }
    };

    f32x4_t acc[CF][4];
#pragma unroll
    for (int cf = 0; cf < CF; ++cf)
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) acc[cf][tf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // LDS row of this wave's column fragment cf
    auto wfrag_row = [&](int cf) {
      if constexpr (GATE_UP)
        return cf < CF / 2 ? wn * (TBN / 4) + cf * 16 : TBN / 2 + wn * (TBN / 4) + (cf - CF / 2) * 16;
      else return wn * (TBN / 2) + cf * 16;
    };

    // 16-row token fragments of this wave that hold rows of the group
    // (uniform); the loop is compiled once per count, so a thin last row
    // tile skips the empty fragments' reads and MFMAs with no guard inside
    // the loop.  Loads, LDS stores and barriers are the same for every wave.
    const int tf_count = min(4, max(0, (c.nrows - c.m0 - wm * 64 + 15) / 16));
    auto compute = [&](int buf, auto tfc_c) {
      constexpr int TFC = decltype(tfc_c)::value;
      const uint16_t *xs = Xs + buf * TBM * TLD;
      const uint16_t *ws = Ws + buf * TBN * TLD;
#pragma unroll
      for (int kk = 0; kk < TBK / 32; ++kk) {
        u32x4_t xf[4], wf[CF];
#pragma unroll
        for (int tf = 0; tf < TFC; ++tf)
          xf[tf] = *reinterpret_cast<const u32x4_t *>(xs + (wm * 64 + tf * 16 + lr) * TLD + kk * 32 + lg * 8);
        if constexpr (TFC > 0) {
#pragma unroll
          for (int cf = 0; cf < CF; ++cf)
            wf[cf] = *reinterpret_cast<const u32x4_t *>(ws + (wfrag_row(cf) + lr) * TLD + kk * 32 + lg * 8);
        }
#pragma unroll
        for (int cf = 0; cf < CF; ++cf)
#pragma unroll
          for (int tf = 0; tf < TFC; ++tf) acc[cf][tf] = mfma_16x16x32(wf[cf], xf[tf], acc[cf][tf]);
        if constexpr (LO) {  // same weight fragments times the low halves of h
          const uint16_t *xl = Xl + buf * TBM * TLD;
#pragma unroll
          for (int tf = 0; tf < TFC; ++tf)
            xf[tf] = *reinterpret_cast<const u32x4_t *>(xl + (wm * 64 + tf * 16 + lr) * TLD + kk * 32 + lg * 8);
#pragma unroll
          for (int cf = 0; cf < CF; ++cf)
#pragma unroll
            for (int tf = 0; tf < TFC; ++tf) acc[cf][tf] = mfma_16x16x32(wf[cf], xf[tf], acc[cf][tf]);
        }
      }
    };

    // double-buffered LDS: the next slice's global loads are in flight while
    // the current slice is multiplied, then stored to the other buffer
    auto run = [&](auto tfc_c) {
      gload(0);
      lstore(0);
      __syncthreads();
      for (int ks = 0; ks < nks; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nks) gload(ks + 1);
        compute(buf, tfc_c);
        if (ks + 1 < nks) lstore(buf ^ 1);
        __syncthreads();
      }
    };
    switch (tf_count) {
      case 4: run(std::integral_constant<int, 4>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      default: run(std::integral_constant<int, 0>{}); break;
    }

    // ---- epilogue ----
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) {
      const int row = c.m0 + wm * 64 + tf * 16 + lr;
      if (row >= c.nrows) continue;
      if constexpr (GATE_UP) {
#pragma unroll
        for (int cf = 0; cf < CF / 2; ++cf) {
          const int col = col0 + wn * (TBN / 4) + cf * 16 + 4 * lg;
          if (col >= a.N) continue;
          float gb[4] = {0.f, 0.f, 0.f, 0.f}, ub[4] = {0.f, 0.f, 0.f, 0.f};
          if (a.bias) {
            const uint16_t *b = static_cast<const uint16_t *>(a.bias) + (size_t)c.g * a.bias_stride;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              gb[q] = bf16_to_f32(b[col + q]);
              ub[q] = bf16_to_f32(b[a.N + col + q]);
            }
          }
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = swiglu_fast(acc[cf][tf][q] + gb[q], acc[cf + CF / 2][tf][q] + ub[q], a.limit, a.act);
          const uint32_t h01 = pack_bf16x2(hv[0], hv[1]), h23 = pack_bf16x2(hv[2], hv[3]);
          const size_t off = (size_t)(c.row0 + row) * a.N + col;
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + off) = make_uint2(h01, h23);
          if (a.out_lo)  // h = hi + lo to ~16 bits (h - hi is exact in f32)
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out_lo) + off) =
                make_uint2(pack_bf16x2(hv[0] - bf16_lo(h01), hv[1] - bf16_hi(h01)),
                           pack_bf16x2(hv[2] - bf16_lo(h23), hv[3] - bf16_hi(h23)));
        }
      } else {
        int slot = 0;
        float wt = 0.f;
        if (a.direct_out) {
          slot = a.perm[c.row0 + row];
          wt = a.weights[slot];
        }
#pragma unroll
        for (int cf = 0; cf < CF; ++cf) {
          const int col = col0 + wn * (TBN / 2) + cf * 16 + 4 * lg;
          if (col >= a.N) continue;
          float4 v = make_float4(acc[cf][tf][0], acc[cf][tf][1], acc[cf][tf][2], acc[cf][tf][3]);
          if (a.bias) {
            const uint16_t *b = static_cast<const uint16_t *>(a.bias) + (size_t)c.g * a.bias_stride + col;
            v.x += bf16_to_f32(b[0]);
            v.y += bf16_to_f32(b[1]);
            v.z += bf16_to_f32(b[2]);
            v.w += bf16_to_f32(b[3]);
          }
          if (a.direct_out) {
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.direct_out) + (size_t)slot * a.N + col) =
                make_uint2(pack_bf16x2(wt * v.x, wt * v.y), pack_bf16x2(wt * v.z, wt * v.w));
          } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + (size_t)(c.row0 + row) * a.N + col) = v;
          }
        }
      }
    }
  }
}

template <int TN, int TK>
static size_t tiled_lds_bytes(bool lo) {
  return (size_t)2 * (TBM + TN + (lo ? TBM : 0)) * (TK + 8) * sizeof(uint16_t);
}

template <bool GATE_UP, int WF, bool GATHER, bool LO, int TN, int TK>
static hipError_t launch_tiled_t(const TiledGemmArgs &t, long mtiles_bound, int32_t *queue, hipStream_t st) {
  auto kern = expert_tiled<GATE_UP, WF, GATHER, LO, TN, TK>;
  const size_t lds = tiled_lds_bytes<TN, TK>(LO);
  static const hipError_t attr =  // LDS above 64 KB must be allowed once per kernel
      hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const long n_tiles = (t.g.N + (GATE_UP ? TN / 2 : TN) - 1) / (GATE_UP ? TN / 2 : TN);
  const int grid = (int)std::max(1L, std::min(mtiles_bound * n_tiles, 512L));  // two per CU
  enqueue_kernel(kern, dim3(grid), dim3(TTHREADS), lds, st, t, queue);
  return hipGetLastError();
}

hipError_t launch_tiled(const TiledGemmArgs &t, bool gate_up, WFormat wf, long max_rows_total,
                        int max_groups, int32_t *queue, hipStream_t st) {
  if (!queue) return hipErrorInvalidValue;
  const ExpertGemmArgs &a = t.g;
  const long mtiles_bound = (max_rows_total + TBM - 1) / TBM + max_groups;
  const bool gather = gate_up && a.perm != nullptr;
  if (gate_up) {
    if (wf == W_MXFP4)
      return gather ? launch_tiled_t<true, W_MXFP4, true, false, kTN, kTK>(t, mtiles_bound, queue, st)
                    : launch_tiled_t<true, W_MXFP4, false, false, kTN, kTK>(t, mtiles_bound, queue, st);
    // 128 x 64 tiles pay for themselves where experts hold about one row tile
    // (qwen3_5_moe at T=4096, 80 rows: gate_up 1254 -> 1162 us); with many
    // row tiles per expert (deepseek_v4 at T=4096: 128 on average, up to 602)
    // the doubled re-reads of their token rows cost more (2373 -> 2446 us)
    if (max_rows_total <= 96L * max_groups)
      return gather ? launch_tiled_t<true, W_BF16, true, false, kTNg, kTKg>(t, mtiles_bound, queue, st)
                    : launch_tiled_t<true, W_BF16, false, false, kTNg, kTKg>(t, mtiles_bound, queue, st);
    return gather ? launch_tiled_t<true, W_BF16, true, false, kTN, kTK>(t, mtiles_bound, queue, st)
                  : launch_tiled_t<true, W_BF16, false, false, kTN, kTK>(t, mtiles_bound, queue, st);
  }
  if (a.A_lo) {
    if (wf == W_MXFP4) return launch_tiled_t<false, W_MXFP4, false, true, kTN, kTK>(t, mtiles_bound, queue, st);
    return launch_tiled_t<false, W_BF16, false, true, kTN, kTK>(t, mtiles_bound, queue, st);
  }
  if (wf == W_MXFP4) return launch_tiled_t<false, W_MXFP4, false, false, kTN, kTK>(t, mtiles_bound, queue, st);
  return launch_tiled_t<false, W_BF16, false, false, kTN, kTK>(t, mtiles_bound, queue, st);
}

int tiled_tile_rows() { return TBM; }

}  // namespace moe
