// Weight-streaming grouped SwiGLU expert GEMMs for small token counts (every
// expert holds a few rows, so the GEMMs read each weight once and are bound
// by HBM bandwidth).
//
//   gate_up: g = rows . Wg^T, u = rows . Wu^T (+ per-expert bias),
//            h = silu(min(g, L)) * min(max(u, -L), L)          -> h (bf16, hi + lo)
//   down:    y = h . Wd^T (+ per-expert bias)                   -> y (f32), or
//            out[token] = weight * y (bf16) with one expert per token
//
// [SF1073] = SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own DSpark draft
// (stacked on #1035)": clamped SwiGLU of the DeepSeek-V4 family; the V4.1
// converter's fused gate_up_proj (gate rows, then up rows) and down_proj, FP4
// experts with two codes per byte (low nibble first) and one E8M0 scale per 32
// inputs.  [MI143] = MoE-Infinity PR #143 "feat(dflash): converge DFlash
// spec-decode stack -> dev (supersedes #140)": output-major MXFP4 codes
// [E,N,K/2] and scales [E,N,K/32] used without a transpose; per-expert
// linear biases.  [SGL48763] = sglang PR #48763 "[Feat] dflash: Serve MoE FFN
// drafts for DFlash and DSpark": DraftMLP commit note (gate-up and down
// linears with silu or the clamped SwiGLU).
//
// Work item = (row chunk, column tile): up to MT*16 rows of one expert (the
// chunk table written by the permutation) against NS*16 weight rows (NS/2
// sets of 16 gate rows and the matching up rows, or NS*16 down rows) over
// the whole reduction dimension.  MXFP4 items are twice as wide (NS = 4) as
// bf16 ones: their weights are four times smaller, and a wider item reads
// the chunk's activation rows once for more weight bytes.
//
// Memory path.  HBM delivers its best rate when each load instruction of a
// wavefront covers few rows with long contiguous runs; the MFMA operand
// layout wants the opposite (16 rows x 16 bytes per lane group).  So the
// workgroup loads each stage of the weight tile with 256-byte (bf16) or
// 128-byte (MXFP4 codes) runs per row into registers, kDepth stages ahead,
// writes it to LDS in an XOR-swizzled layout and reads the MFMA operands from
// there without bank conflicts.  The activation rows of the chunk take the
// same path (they are L2 hits after the first column tile).
//
// Second segment: with bf16 weights a launch may carry, besides the grouped
// items, the items of one more group with operands of its own (the shared
// expert's gate_up, whose few items would leave a launch of their own short
// of work: carried, they stream among the routed items, and one dependent
// launch goes away).
//
// Reduction split: the four wavefronts take the four 32-element MFMA steps
// of each bf16 stage (two steps each of an MXFP4 stage) and merge their
// partial sums in LDS in wave order at the end, so results do not depend on
// timing.
#include <type_traits>

#include "kernels.hpp"
#include "tile.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;

template <int WF, int NS>
struct Geom;
template <int NS>
struct Geom<W_BF16, NS> {
  static constexpr int ROWS = 16 * NS;                 // weight rows per work item
  static constexpr int SK = 128;                       // reduction elements per stage
  static constexpr int W_UNITS = ROWS * SK * 2 / 16;   // 16-byte units of the weight tile
  static constexpr int W_LOADS = W_UNITS / kThreads;   // per thread
  static constexpr int S_BYTES = 0;
  static constexpr int S_LOADS = 0;
};
template <int NS>
struct Geom<W_MXFP4, NS> {
  static constexpr int ROWS = 16 * NS;
  static constexpr int SK = 256;
  static constexpr int W_UNITS = ROWS * SK / 2 / 16;
  static constexpr int W_LOADS = W_UNITS / kThreads;
  static constexpr int S_BYTES = ROWS * SK / 32;       // E8M0 scales per stage
  static constexpr int S_LOADS = S_BYTES / kThreads;   // one byte each
};

// Swizzled 16-byte unit of (row, chunk) inside a stage tile.  Each of the
// 16 lanes of an MFMA operand read (16 rows, one chunk) lands on its own
// group of four banks.
__device__ __forceinline__ int unit16(int row, int ch) { return row * 16 + (ch ^ (row & 15)); }  // 16 chunks/row
__device__ __forceinline__ int unit32(int row, int ch) { return row * 32 + (ch ^ (row & 15)); }  // 32 chunks/row
__device__ __forceinline__ int unit8(int row, int ch) { return row * 8 + (ch ^ ((row >> 1) & 7)); }  // 8 chunks/row

struct Chunk {
  int g, row0, nrows;  // expert (group), first row in expert-sorted order, rows
  int first, count;    // the expert's chunks: index of the first, how many
};

__device__ __forceinline__ Chunk chunk_of(const ExpertGemmArgs &a, int c, int n_chunks) {
  Chunk r;
  if (a.chunks) {
    const int4 v = a.chunks[c];
    r.g = v.x;
    r.row0 = v.y;
    r.nrows = v.z & 0xffff;
    r.count = (int)((unsigned)v.z >> 16);
    r.first = v.w;
  } else {
    r.g = 0;
    r.row0 = c * a.chunk_rows;
    r.nrows = min(a.chunk_rows, a.single_rows - r.row0);
    r.first = 0;
    r.count = n_chunks;
  }
  return r;
}

// Work item -> (chunk, column tile).  Items run expert by expert (the
// expert's chunks are adjacent in the chunk table); inside an expert, blocks
// of kTileBlock column tiles, and inside a block all the expert's chunks, so
// the chunks that share a weight tile read it at about the same time.
constexpr int kTileBlock = 8;

// item `local` of a group of `count` chunks and n_tiles column tiles ->
// (chunk of the group, column tile)
__device__ __forceinline__ void blocked(int local, int count, int n_tiles, int &c, int &ct) {
  const int per_block = count * kTileBlock;
  const int b = local / per_block;
  const int rem = local - b * per_block;
  const int width = min(kTileBlock, n_tiles - b * kTileBlock);
  c = rem / width;
  ct = b * kTileBlock + (rem - c * width);
}

__device__ __forceinline__ void item_coords(const ExpertGemmArgs &a, int item, int n_chunks, Chunk &C,
                                            int &ct) {
  const Chunk C0 = chunk_of(a, item / a.n_tiles, n_chunks);
  if (C0.count == 1) {
    C = C0;
    ct = item - (item / a.n_tiles) * a.n_tiles;
    return;
  }
  int c;
  blocked(item - C0.first * a.n_tiles, C0.count, a.n_tiles, c, ct);
  C = chunk_of(a, C0.first + c, n_chunks);
}

// Item `local` of the second segment (one group of rows2 rows, chunks of
// chunk_rows rows, the same blocked order).
__device__ __forceinline__ void seg2_coords(const ExpertGemmArgs &a, int local, int chunks2, int chunk_rows,
                                            Chunk &C, int &ct) {
  int c;
  blocked(local, chunks2, a.n_tiles2, c, ct);
  C.g = 0;
  C.row0 = c * chunk_rows;
  C.nrows = min(chunk_rows, a.rows2 - C.row0);
  C.first = 0;
  C.count = chunks2;
}

// Per-variant layout: stage sizes, LDS carve-up and the load pipeline depth
// (stages in flight per thread, bounded by the registers they occupy).
template <int MT, int WF, int NS, bool LO>
struct Plan {
  using G = Geom<WF, NS>;
  static constexpr int SK = G::SK;
  static constexpr int XCH = SK / 8;               // 16-byte chunks per activation row per stage
  static constexpr int X_UNITS = MT * 16 * XCH;
  static constexpr int X_LOADS = X_UNITS / kThreads;
  static constexpr int NXS = LO ? 2 : 1;           // activation streams (hi, lo)
  static constexpr int LOADS = G::W_LOADS + NXS * X_LOADS + (G::S_LOADS > 0 ? 1 : 0);
  static constexpr int DEPTH = (WF == W_MXFP4 && NS == 4) ? 2 : (16 / LOADS >= 4 ? 4 : (16 / LOADS >= 3 ? 3 : 2));
  static constexpr int S_UNITS = (2 * G::S_BYTES * 4 + 15) / 16;  // f32 scales, two buffers
  static constexpr int MAIN_UNITS = 2 * G::W_UNITS + 2 * NXS * X_UNITS;
  static constexpr int RED_UNITS = 4 * MT * NS * 64;
  static constexpr size_t LDS_BYTES = (size_t)(MAIN_UNITS + S_UNITS) * 16;
  // resident wavefronts per SIMD the register allocation must allow (four
  // lets a 1024-item launch fit the chip in one round)
  static constexpr int MIN_WAVES = (WF == W_BF16 && MT == 1) ? 4 : (MT == 1 || WF == W_BF16 ? 3 : 2);
  static_assert(RED_UNITS <= MAIN_UNITS, "merge buffer aliases the stage buffers");
  static_assert(X_UNITS % kThreads == 0 && G::W_UNITS % kThreads == 0, "whole loads per thread");
  static_assert(G::S_BYTES % kThreads == 0, "whole scale loads per thread");
};

// TAB (MXFP4 gate_up, reduction <= 4096, scale array on 16 bytes): the
// item's block scales (its gate rows' and up rows' runs of HC * K/32 bytes)
// are loaded once per item into an LDS table with coalesced 16-byte loads,
// instead of one byte per lane and stage (one such load instruction touches
// about seven cache lines for 64 bytes).
template <int MT, int WF, int NS, bool GATHER, bool GATE_UP, bool LO, bool TAB>
__global__ __launch_bounds__(kThreads, (Plan<MT, WF, NS, LO>::MIN_WAVES)) void expert_lds_stream(ExpertGemmArgs a) {
  using P = Plan<MT, WF, NS, LO>;
  using G = typename P::G;
  constexpr int SK = P::SK;
  constexpr int XCH = P::XCH;
  constexpr int X_UNITS = P::X_UNITS;
  constexpr int X_LOADS = P::X_LOADS;
  constexpr int NXS = P::NXS;
  constexpr int kDepth = P::DEPTH;
  constexpr int MAIN_UNITS = P::MAIN_UNITS;
  constexpr int HC = 8 * NS;  // gate_up: h columns per item (NS/2 gate sets + NS/2 up sets)
  extern __shared__ u32x4_t lds[];
  u32x4_t *Wl = lds;                                // [2][W_UNITS]
  u32x4_t *Xl = lds + 2 * G::W_UNITS;               // [2][NXS][X_UNITS]
  float *Sl = reinterpret_cast<float *>(lds + MAIN_UNITS);      // [2][S_BYTES] block scales as f32
  uint8_t *tab = reinterpret_cast<uint8_t *>(lds + MAIN_UNITS);  // TAB: [2 HC][K/32] E8M0 scales
  static_assert(!TAB || (WF == W_MXFP4 && GATE_UP), "scale table: MXFP4 gate_up");
  f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n_chunks = a.chunks ? a.n_chunks[0] : (a.single_rows + a.chunk_rows - 1) / a.chunk_rows;
  const int items1 = n_chunks * a.n_tiles;
  // second segment (bf16 weights only): chunks of this kernel's chunk height
  const int chunks2 = (WF == W_BF16 && a.rows2 > 0) ? (a.rows2 + 16 * MT - 1) / (16 * MT) : 0;
  const int items2 = chunks2 * a.n_tiles2;

  // XCD-aware order: the items of one contiguous range run on one XCD, so
  // an XCD keeps the activation rows of only a few experts in its L2 while
  // the weights stream past (item_coords gives the order inside a range).
  // Each segment is cut into one range per XCD, so every XCD gets its share
  // of both; an XCD runs its second-segment items first (they may have the
  // longer reduction).
  const int nx = gridDim.x % 8 == 0 ? 8 : 1;
  const int xcd = blockIdx.x % nx, per = gridDim.x / nx;
  const int span1 = (items1 + nx - 1) / nx, span2 = (items2 + nx - 1) / nx;
  const int lo1 = min(xcd * span1, items1), n1 = min(span1, items1 - lo1);
  const int lo2 = min(xcd * span2, items2), n2 = min(span2, items2 - lo2);

  for (int local = blockIdx.x / nx; local < n1 + n2; local += per) {
    // the item's segment and operands (uniform across the workgroup)
    const bool seg2 = local < n2;
    Chunk C;
    int ct;
    if (!seg2) item_coords(a, lo1 + (local - n2), n_chunks, C, ct);
    else seg2_coords(a, lo2 + local, chunks2, 16 * MT, C, ct);
    const int mt_count = (C.nrows + 15) >> 4;
    const int Kd = seg2 ? a.Kdim2 : a.Kdim;
    const int N = seg2 ? a.N2 : a.N;
    const int nst = (Kd + SK - 1) / SK;
    const uint16_t *A = static_cast<const uint16_t *>(seg2 ? a.A2 : a.A);
    const uint16_t *Alo = static_cast<const uint16_t *>(seg2 ? a.A2_lo : a.A_lo);
    const void *Wb = seg2 ? a.W2 : a.W;
    const void *bias = seg2 ? nullptr : a.bias;
    void *out = seg2 ? a.out2 : a.out;
    void *out_lo = seg2 ? a.out2_lo : a.out_lo;
    void *direct_out = seg2 ? nullptr : a.direct_out;

    // ---- this thread's load sources ------------------------------------
    // weight rows of the thread's loads
    // weight row (in the expert's matrix) of tile row r
    auto wrow = [&](int r) {
      return GATE_UP ? (r < HC ? ct * HC + r : N + ct * HC + (r - HC)) : ct * G::ROWS + r;
    };
    const uint16_t *wp[G::W_LOADS];
    const uint8_t *cp[G::W_LOADS], *sp[G::S_LOADS > 0 ? G::S_LOADS : 1];
    int wch, sb = 0;
    if constexpr (WF == W_BF16) {
      wch = tid & 15;  // 16 chunks of 16 bytes per row and stage
#pragma unroll
      for (int j = 0; j < G::W_LOADS; ++j)
        wp[j] = static_cast<const uint16_t *>(Wb) + (size_t)C.g * a.w_stride +
                (size_t)wrow(j * 16 + (tid >> 4)) * Kd + wch * 8;
    } else {
      wch = tid & 7;  // 8 chunks of 32 codes per row and stage
      sb = tid & 7;   // 8 scales per row and stage
#pragma unroll
      for (int j = 0; j < G::W_LOADS; ++j)
        cp[j] = static_cast<const uint8_t *>(Wb) + (size_t)C.g * a.w_stride +
                (size_t)wrow(j * 32 + (tid >> 3)) * (Kd / 2) + wch * 16;
      if constexpr (!TAB) {
#pragma unroll
        for (int j = 0; j < G::S_LOADS; ++j)
          sp[j] = a.Wscale + (size_t)C.g * a.s_stride + (size_t)wrow(j * 32 + (tid >> 3)) * (Kd / 32) + sb;
      }
    }
    // TAB: this thread's 16-byte units of the item's scale table (unit u of
    // the gate run, then of the up run; lanes past the table load its last
    // unit again and store nothing)
    constexpr int TL = 2;  // units per thread: 2 HC * K/32 / 16 <= 512 for K <= 4096
    u32x4_t tv[TL];
    const int t_units = TAB ? 2 * HC * (Kd / 32) / 16 : 0;
    if constexpr (TAB) {
      const int run = t_units / 2;
      const char *gs = reinterpret_cast<const char *>(a.Wscale) + (size_t)C.g * a.s_stride;
      const char *g0 = gs + (size_t)(ct * HC) * (Kd / 32), *u0 = gs + (size_t)(N + ct * HC) * (Kd / 32);
#pragma unroll
      for (int j = 0; j < TL; ++j) {
        const int u = min(j * kThreads + tid, t_units - 1);
        tv[j] = load16(u < run ? g0 + u * 16 : u0 + (u - run) * 16);
      }
    }
    // activation rows of the thread's loads.  Lanes of rows past the chunk
    // read the chunk's last row (the same addresses as that row's lanes, so
    // no extra traffic): each output column depends only on its own
    // activation row, and the columns of those rows are not stored.
    const int xch = tid % XCH;
    const uint16_t *xp[X_LOADS], *xlp[LO ? X_LOADS : 1];
#pragma unroll
    for (int j = 0; j < X_LOADS; ++j) {
      const int r = (j * kThreads + tid) / XCH;
      const int rr = min(r, C.nrows - 1);
      size_t ar;
      if (GATHER && !seg2)
        ar = (size_t)(a.perm[C.row0 + rr] / a.topk);
      else
        ar = (size_t)(C.row0 + rr);
      xp[j] = A + ar * Kd + xch * 8;
      if constexpr (LO) xlp[j] = Alo + (size_t)(C.row0 + rr) * Kd + xch * 8;
    }

    // ---- register stages -------------------------------------------------
    // Every stage issues the same loads with no branches around them: the
    // compiler's wait counts are then exact and only the oldest stage is
    // waited for.  Chunks past the end of the reduction read the row start
    // instead (their LDS copies are never read), and the stages issued past
    // the last one repeat the last stage's addresses (cache hits, unused).
    u32x4_t wv[kDepth][G::W_LOADS];
    uint32_t sv[kDepth][G::S_LOADS > 0 ? G::S_LOADS : 1];
    u32x4_t xv[kDepth][NXS][X_LOADS];

    auto issue = [&](int d, int s) {
      const int k0 = s * SK, kv = min(SK, Kd - k0);
      if constexpr (WF == W_BF16) {
        const int kw = wch * 8 < kv ? k0 : -wch * 8;
#pragma unroll
        for (int j = 0; j < G::W_LOADS; ++j) wv[d][j] = load_stream16(wp[j] + kw);
      } else {
        // Code rows of K/2 bytes are not in general a whole number of
        // 128-byte lines, so a stage's run can end inside a line that the
        // next stage starts on: cached loads keep that line in L2 for it
        // (streaming loads would fetch it from HBM twice).
        const int kc = wch * 32 < kv ? k0 / 2 : -wch * 16;
#pragma unroll
        for (int j = 0; j < G::W_LOADS; ++j) wv[d][j] = load16(cp[j] + kc);
        if constexpr (!TAB) {
          const int ks = sb * 32 < kv ? k0 / 32 : -sb;
#pragma unroll
          for (int j = 0; j < G::S_LOADS; ++j) sv[d][j] = sp[j][ks];
        }
      }
      const int kx = xch * 8 < kv ? k0 : -xch * 8;
#pragma unroll
      for (int j = 0; j < X_LOADS; ++j) {
        xv[d][0][j] = load16(xp[j] + kx);
        if constexpr (LO) xv[d][NXS - 1][j] = load16(xlp[j] + kx);
      }
    };
    auto stash = [&](int d, int buf) {
      if constexpr (WF == W_BF16) {
#pragma unroll
        for (int j = 0; j < G::W_LOADS; ++j) Wl[buf * G::W_UNITS + unit16(j * 16 + (tid >> 4), wch)] = wv[d][j];
      } else {
#pragma unroll
        for (int j = 0; j < G::W_LOADS; ++j) Wl[buf * G::W_UNITS + unit8(j * 32 + (tid >> 3), wch)] = wv[d][j];
        if constexpr (!TAB) {
#pragma unroll
          for (int j = 0; j < G::S_LOADS; ++j) Sl[buf * G::S_BYTES + j * kThreads + tid] = e8m0_to_f32(sv[d][j] & 0xffu);
        }
      }
#pragma unroll
      for (int j = 0; j < X_LOADS; ++j) {
        const int r = (j * kThreads + tid) / XCH;
        const int u = XCH == 16 ? unit16(r, xch) : unit32(r, xch);
#pragma unroll
        for (int h = 0; h < NXS; ++h) Xl[(buf * NXS + h) * X_UNITS + u] = xv[d][h][j];
      }
    };

    f32x4_t acc[MT][NS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int sx = 0; sx < NS; ++sx) acc[mt][sx] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // `full` (a std::bool_constant): the stage spans SK reduction elements,
    // so no step is skipped (no exec-mask branches around the MFMAs)
    auto compute = [&](int buf, int s, auto full) {
      constexpr bool FULL = decltype(full)::value;
      const int kv = min(SK, Kd - s * SK);
      constexpr int STEPS = SK / 32 / 4;  // MFMA steps per wave per stage
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        const int q = wave * STEPS + i;
        if (FULL || 32 * q < kv) {
          u32x4_t wa[NS];
#pragma unroll
          for (int sx = 0; sx < NS; ++sx) {
            const int row = sx * 16 + lr;
            if constexpr (WF == W_BF16) {
              wa[sx] = Wl[buf * G::W_UNITS + unit16(row, 4 * q + lg)];
            } else {
              const uint32_t *u = reinterpret_cast<const uint32_t *>(&Wl[buf * G::W_UNITS + unit8(row, q)]);
              if constexpr (TAB)  // block s * 8 + q of tile row `row`
                wa[sx] = decode_e2m1x8(u[lg], e8m0_to_f32(tab[row * (Kd / 32) + s * 8 + q]));
              else
                wa[sx] = decode_e2m1x8(u[lg], Sl[buf * G::S_BYTES + row * 8 + q]);
            }
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if ((WF == W_MXFP4 && MT == 1) || mt < mt_count) {  // a chunk holds at least one row
              const int u = XCH == 16 ? unit16(mt * 16 + lr, 4 * q + lg) : unit32(mt * 16 + lr, 4 * q + lg);
#pragma unroll
              for (int h = 0; h < NXS; ++h) {
                const u32x4_t b = Xl[(buf * NXS + h) * X_UNITS + u];
#pragma unroll
                for (int sx = 0; sx < NS; ++sx) acc[mt][sx] = mfma_16x16x32(wa[sx], b, acc[mt][sx]);
              }
            }
          }
        }
      }
    };

    // ---- pipelined main loop ---------------------------------------------
    // Steady state: whole groups of kDepth stages in which every stage issues
    // the loads of the stage kDepth ahead, with no branch around them (the
    // compiler's wait counts then let the later stages stay in flight).  The
    // last 2*kDepth - 1 stages or fewer issue only what is left.
#pragma unroll
    for (int d = 0; d < kDepth; ++d) issue(d, min(d, nst - 1));
    if constexpr (TAB) {  // the previous item's last barrier is behind every wave
#pragma unroll
      for (int j = 0; j < TL; ++j)
        if (j * kThreads + tid < t_units) reinterpret_cast<u32x4_t *>(tab)[j * kThreads + tid] = tv[j];
    }
    const int nfull = nst >= 2 * kDepth ? (nst - kDepth) / kDepth : 0;
    for (int g = 0; g < nfull; ++g) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int s = g * kDepth + d;
        stash(d, s & 1);
        issue(d, s + kDepth);
        __syncthreads();
        // stages before the last are whole; the unguarded copy pays off for
        // MXFP4 (its decode sits between the guards), not for bf16
        compute(s & 1, s, std::integral_constant<bool, WF == W_MXFP4>{});
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * kDepth - 1; ++i) {
      const int s = nfull * kDepth + i;
      if (s < nst) {
        const int d = i % kDepth;
        stash(d, s & 1);
        if (s + kDepth < nst) issue(d, s + kDepth);
        __syncthreads();
        compute(s & 1, s, std::false_type{});
      }
    }

    // ---- merge the four partial sums in wave order, epilogue ---------------
    __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int sx = 0; sx < NS; ++sx) red[((wave * MT + mt) * NS + sx) * 64 + lane] = acc[mt][sx];
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count && (mt & 3) == wave) {
        f32x4_t v[NS];
#pragma unroll
        for (int sx = 0; sx < NS; ++sx) {
          v[sx] = red[((0 * MT + mt) * NS + sx) * 64 + lane];
#pragma unroll
          for (int w = 1; w < 4; ++w) v[sx] += red[((w * MT + mt) * NS + sx) * 64 + lane];
        }
        const int row = mt * 16 + lr;
        if (row < C.nrows) {
          if constexpr (GATE_UP) {
#pragma unroll
            for (int c2 = 0; c2 < NS / 2; ++c2) {
              const int col = ct * HC + c2 * 16 + 4 * lg;
              float gb[4] = {0.f, 0.f, 0.f, 0.f}, ub[4] = {0.f, 0.f, 0.f, 0.f};
              if (bias) {
                const uint16_t *b = static_cast<const uint16_t *>(bias) + (size_t)C.g * a.bias_stride;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  gb[q] = bf16_to_f32(b[col + q]);
                  ub[q] = bf16_to_f32(b[N + col + q]);
                }
              }
              uint32_t hb[4], lb[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float hv = swiglu_exact(v[c2][q] + gb[q], v[NS / 2 + c2][q] + ub[q], a.limit, a.act);
                hb[q] = f32_to_bf16(hv);
                lb[q] = f32_to_bf16(hv - bf16_to_f32(hb[q]));  // h = hi + lo to ~16 bits
              }
              const size_t off = (size_t)(C.row0 + row) * N + col;
              *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + off) =
                  make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
              if (out_lo)
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out_lo) + off) =
                    make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
            }
          } else {
            int slot = 0;
            float wt = 0.f;
            if (direct_out) {  // one expert per token: out = weight * y
              slot = a.perm[C.row0 + row];
              wt = a.weights[slot];
            }
#pragma unroll
            for (int sx = 0; sx < NS; ++sx) {
              const int col = ct * G::ROWS + sx * 16 + 4 * lg;
              float4 o = make_float4(v[sx][0], v[sx][1], v[sx][2], v[sx][3]);
              if (bias) {
                const uint16_t *b = static_cast<const uint16_t *>(bias) + (size_t)C.g * a.bias_stride + col;
                o.x += bf16_to_f32(b[0]);
                o.y += bf16_to_f32(b[1]);
                o.z += bf16_to_f32(b[2]);
                o.w += bf16_to_f32(b[3]);
              }
              if (direct_out) {
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(direct_out) + (size_t)slot * N + col) =
                    make_uint2(f32_to_bf16(wt * o.x) | (f32_to_bf16(wt * o.y) << 16),
                               f32_to_bf16(wt * o.z) | (f32_to_bf16(wt * o.w) << 16));
              } else {
                *reinterpret_cast<float4 *>(static_cast<float *>(out) + (size_t)(C.row0 + row) * N + col) = o;
              }
            }
          }
        }
      }
    }
    __syncthreads();  // the next item's first stage overwrites the merge buffer
  }
}

constexpr int kGridCap = 256 * 8;

template <int MT, int WF, int NS, bool GATHER, bool GATE_UP, bool LO, bool TAB>
void launch_one(ExpertGemmArgs a, long max_chunks, hipStream_t st) {
  using P = Plan<MT, WF, NS, LO>;
  // TAB: the scale table (2 HC rows x K/32 bytes) replaces the f32 stage scales
  const size_t lds = TAB ? (size_t)P::MAIN_UNITS * 16 + (size_t)2 * 8 * NS * (a.Kdim / 32) : P::LDS_BYTES;
  auto *k = expert_lds_stream<MT, WF, NS, GATHER, GATE_UP, LO, TAB>;
  if (lds > 64 * 1024) {
    static const hipError_t attr =
        hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)attr;
  }
  a.n_tiles = a.N / (GATE_UP ? 8 * NS : 16 * NS);
  a.n_tiles2 = WF == W_BF16 && a.rows2 > 0 ? a.N2 / (GATE_UP ? 8 * NS : 16 * NS) : 0;
  const long chunks2 = WF == W_BF16 && a.rows2 > 0 ? (a.rows2 + 16 * MT - 1) / (16 * MT) : 0;
  const long items = max_chunks * a.n_tiles + chunks2 * a.n_tiles2;
  const dim3 g((unsigned)std::max(1L, std::min(items, (long)kGridCap))), b(kThreads);
  enqueue_kernel(k, g, b, lds, st, a);
}

template <int MT, int WF, int NS, bool GATE_UP, bool TAB = false>
void launch_ns(const ExpertGemmArgs &a, bool gather, bool lo, long max_chunks, hipStream_t st) {
  if constexpr (GATE_UP) {
    if (gather) launch_one<MT, WF, NS, true, true, false, TAB>(a, max_chunks, st);
    else launch_one<MT, WF, NS, false, true, false, TAB>(a, max_chunks, st);
  } else {  // the down projection reads h rows in expert order: no gather
    static_assert(!TAB, "scale table: gate_up only");
    if (lo) launch_one<MT, WF, NS, false, false, true, false>(a, max_chunks, st);
    else launch_one<MT, WF, NS, false, false, false, false>(a, max_chunks, st);
  }
}

template <int MT, bool GATE_UP>
void launch_mt(const ExpertGemmArgs &a, WFormat wf, bool gather, bool lo, long max_chunks, hipStream_t st) {
  // MXFP4 items span 64 weight rows when the output columns allow it; so do
  // bf16 down items of 16-row chunks (half as many items, each streaming
  // twice the weight rows: measured 8-13% faster on down, slower on gate_up)
  const bool table = GATE_UP && a.Kdim <= 4096 && (reinterpret_cast<uintptr_t>(a.Wscale) & 15) == 0;
  if (wf == W_MXFP4 && a.N % (GATE_UP ? 32 : 64) == 0 && table) {
    if constexpr (GATE_UP) launch_ns<MT, W_MXFP4, 4, GATE_UP, true>(a, gather, lo, max_chunks, st);
  } else if (wf == W_MXFP4 && a.N % (GATE_UP ? 32 : 64) == 0)
    launch_ns<MT, W_MXFP4, 4, GATE_UP>(a, gather, lo, max_chunks, st);
  else if (wf == W_MXFP4)
    launch_ns<MT, W_MXFP4, 2, GATE_UP>(a, gather, lo, max_chunks, st);
  else if (!GATE_UP && MT == 1 && a.N % 64 == 0 && (a.rows2 == 0 || a.N2 % 64 == 0))
    launch_ns<MT, W_BF16, 4, GATE_UP>(a, gather, lo, max_chunks, st);
  else
    launch_ns<MT, W_BF16, 2, GATE_UP>(a, gather, lo, max_chunks, st);
}

}  // namespace

int stream_chunk_rows(long slots, int E) {
  // rows per chunk: 16 while experts hold about one MFMA tile of rows, 32 above
  const long active = std::max(1L, std::min<long>(E, slots));
  return slots / active > 24 ? 32 : 16;
}

hipError_t launch_stream(const ExpertGemmArgs &a, bool gate_up, WFormat wf, long max_chunks, hipStream_t st) {
  if (max_chunks <= 0) return hipSuccess;
  if (wf != W_BF16 && wf != W_MXFP4) return hipErrorInvalidValue;
  if (a.chunk_rows != 16 && a.chunk_rows != 32) return hipErrorInvalidValue;
  if (a.Kdim % 32 || a.N % (gate_up ? 16 : 32)) return hipErrorInvalidValue;
  if (a.rows2 > 0 && (wf != W_BF16 || !a.A2 || !a.W2 || !a.out2 || a.Kdim2 % 32 || a.N2 % (gate_up ? 16 : 32) ||
                      (!gate_up && !a.A_lo != !a.A2_lo)))
    return hipErrorInvalidValue;
  const bool gather = gate_up && a.perm != nullptr;
  const bool lo = !gate_up && a.A_lo != nullptr;
  if (a.chunk_rows == 16) {
    if (gate_up) launch_mt<1, true>(a, wf, gather, lo, max_chunks, st);
    else launch_mt<1, false>(a, wf, gather, lo, max_chunks, st);
  } else {
    if (gate_up) launch_mt<2, true>(a, wf, gather, lo, max_chunks, st);
    else launch_mt<2, false>(a, wf, gather, lo, max_chunks, st);
  }
  return hipGetLastError();
}

}  // namespace moe
